"""fp64 reference of the generation shell (TEST INFRASTRUCTURE ONLY).

A pre-norm stack of causal linear-attention layers run one token at a time:
layer norm, q/k/v projection, the recurrent attention step of the pages
("Why Replace Attention?", §7.2, through ``oracle.decode_step`` on an fp64
state), output projection with a residual, then a GELU feed-forward block
with a residual; a final layer norm and the output head give the logits.
Written in plain numpy, independently of the GPU package; layer norm and
GELU are pinned to torch's fp64 routines in tests/test_oracle_shell.py.
"""
from __future__ import annotations

import numpy as np
from scipy.special import erf

from . import decode_step


def layer_norm(x: np.ndarray, g: np.ndarray, b: np.ndarray, eps: float = 1e-5) -> np.ndarray:
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * g + b


def gelu(x: np.ndarray) -> np.ndarray:
    """GELU with the Gaussian CDF: x * Phi(x)."""
    return 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))


def teacher_forced_logits(weights: dict, layers: int, heads: int, tokens: np.ndarray, threads: int = 1) -> np.ndarray:
    """Logits [steps, B, vocab] when the inputs of step t are tokens[t] (shape [steps, B])."""
    w = {k: np.asarray(v, dtype=np.float64) for k, v in weights.items()}
    steps, B = tokens.shape
    D = w["tok_emb"].shape[1]
    S = [np.zeros((B * heads, 64, 64)) for _ in range(layers)]
    z = [np.zeros((B * heads, 64)) for _ in range(layers)]
    out = np.empty((steps, B, w["head"].shape[1]))
    for t in range(steps):
        x = w["tok_emb"][tokens[t]] + w["pos_emb"][t]
        for l in range(layers):
            h = layer_norm(x, w[f"ln1_g{l}"], w[f"ln1_b{l}"])
            qkv = h @ w[f"wqkv{l}"]
            q = np.ascontiguousarray(qkv[:, 0:D].reshape(B * heads, 64))
            k = np.ascontiguousarray(qkv[:, D:2 * D].reshape(B * heads, 64))
            v = np.ascontiguousarray(qkv[:, 2 * D:3 * D].reshape(B * heads, 64))
            o = decode_step(S[l], z[l], q, k, v, threads=threads)
            x = x + o.reshape(B, D) @ w[f"wo{l}"]
            h = layer_norm(x, w[f"ln2_g{l}"], w[f"ln2_b{l}"])
            x = x + gelu(h @ w[f"w1{l}"]) @ w[f"w2{l}"]
        out[t] = layer_norm(x, w["ln_f_g"], w["ln_f_b"]) @ w["head"]
    return out
