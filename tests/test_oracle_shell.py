"""Pins of the fp64 generation-shell reference (CPU only).

Its attention is the pinned oracle decode step; its other pieces are pinned
here to independent library routines (torch fp64 layer norm and GELU), and
the stack to two reductions it must satisfy.
"""
import numpy as np
import torch

from oracle import shell
from workloads import ShellConfig, draw_shell_weights, shell_teacher_tokens


def test_layer_norm_and_gelu_match_torch_fp64():
    x = np.random.default_rng(0).standard_normal((7, 512)) * 3
    g = np.random.default_rng(1).standard_normal(512)
    b = np.random.default_rng(2).standard_normal(512)
    ref = torch.nn.functional.layer_norm(torch.tensor(x), (512,), torch.tensor(g), torch.tensor(b), 1e-5).numpy()
    np.testing.assert_allclose(shell.layer_norm(x, g, b), ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(shell.gelu(x), torch.nn.functional.gelu(torch.tensor(x)).numpy(), rtol=1e-12,
                               atol=1e-14)


def _cfg(layers):
    return ShellConfig("t", layers=layers, steps=16, batch=3)


def test_zero_layers_is_embedding_then_head():
    cfg = _cfg(0)
    w = {k: v.double().numpy() for k, v in draw_shell_weights(cfg).items()}
    toks = shell_teacher_tokens(cfg, 3, 5, seed=1).numpy()
    got = shell.teacher_forced_logits(w, 0, 8, toks)
    for t in range(5):
        x = w["tok_emb"][toks[t]] + w["pos_emb"][t]
        want = shell.layer_norm(x, w["ln_f_g"], w["ln_f_b"]) @ w["head"]
        np.testing.assert_allclose(got[t], want, rtol=1e-12, atol=1e-12)


def test_first_step_attention_output_is_its_own_value():
    # At step 0 every attention state holds one token, so each layer's
    # attention output equals that token's v projection ("Why Replace
    # Attention?", §7.3: o_1 = v_1).  Rebuild the first step with that
    # substitution and compare.
    cfg = _cfg(2)
    w = {k: v.double().numpy() for k, v in draw_shell_weights(cfg).items()}
    toks = shell_teacher_tokens(cfg, 3, 1, seed=2).numpy()
    got = shell.teacher_forced_logits(w, 2, 8, toks)[0]
    x = w["tok_emb"][toks[0]] + w["pos_emb"][0]
    for l in range(2):
        h = shell.layer_norm(x, w[f"ln1_g{l}"], w[f"ln1_b{l}"])
        v = (h @ w[f"wqkv{l}"])[:, 1024:1536]
        x = x + v @ w[f"wo{l}"]
        h = shell.layer_norm(x, w[f"ln2_g{l}"], w[f"ln2_b{l}"])
        x = x + shell.gelu(h @ w[f"w1{l}"]) @ w[f"w2{l}"]
    want = shell.layer_norm(x, w["ln_f_g"], w["ln_f_b"]) @ w["head"]
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12)
