"""Seeded synthetic inputs shared by the tests, bench.py and the oracle checks.

This module holds only workload shapes and random-number recipes; it contains
none of linear attention's arithmetic, so both the HIP path and the oracle can
take their inputs from it without sharing any method code.

Every tensor is drawn on the CPU with ``torch.Generator("cpu")`` (deterministic
across machines), in float32 from N(0, 1), optionally multiplied by a power of
two (0.125 = 1/sqrt(64), exact in every float format), and rounded to the
workload's element type with round-to-nearest-even.  Draw order is Q, K, V.

The named workloads follow the shapes on the pages: CIFAR-10 autoregressive
generation is 32*32*3 = 3072 steps per image ("Transformers Are RNNs: Linear
Attention" knowledge note, "Why This Exists"); the running model has
d_model 512, h 8, d_k = d_v = 64 and scales to n = 128K tokens ("Why Replace
Attention?", "The Running Example").  No dataset is read: values are i.i.d.
Gaussian stand-ins for activations.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Tuple

import torch

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class ForwardWorkload:
    name: str
    causal: bool
    dtype: str
    B: int
    H: int
    N: int
    C: int = 64
    M: int = 64
    scale: float = 1.0
    seed: int = 0
    note: str = ""

    @property
    def tokens(self) -> int:
        return self.B * self.N


@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    dtype: str
    sequences: int
    H: int
    steps: int
    C: int = 64
    M: int = 64
    scale: float = 1.0
    seed: int = 0
    note: str = ""

    @property
    def heads(self) -> int:
        return self.sequences * self.H


WORKLOADS: Dict[str, object] = {
    "causal_f32_b1h1n256": ForwardWorkload(
        "causal_f32_b1h1n256", True, "f32", 1, 1, 256, seed=1001,
        note="small causal case the fp64 oracle finishes in well under a second"),
    "noncausal_bf16_b8h8n4096": ForwardWorkload(
        "noncausal_bf16_b8h8n4096", False, "bf16", 8, 8, 4096, scale=0.125, seed=1002,
        note="non-causal, bf16 storage, fp32 accumulation"),
    "causal_bf16_b16h8n3072": ForwardWorkload(
        "causal_bf16_b16h8n3072", True, "bf16", 16, 8, 3072, seed=1003,
        note="shaped like autoregressive 32x32x3 image generation, d_model 512"),
    "causal_bf16_b2h8n131072": ForwardWorkload(
        "causal_bf16_b2h8n131072", True, "bf16", 2, 8, 131072, scale=0.125, seed=1004,
        note="long-context causal forward, fp32 state"),
    "decode_f32_s256h8_3072steps": DecodeWorkload(
        "decode_f32_s256h8_3072steps", "f32", 256, 8, 3072, seed=1005,
        note="256 concurrent sequences x 8 heads, 3072 sequential steps"),
}


def draw_qkv(B: int, H: int, N: int, C: int, M: int, dtype: str, seed: int,
             scale: float = 1.0) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Q [B,H,N,C], K [B,H,N,C], V [B,H,N,M] on the CPU, drawn in that order."""
    g = torch.Generator("cpu").manual_seed(int(seed))
    out = []
    for last in (C, C, M):
        x = torch.randn((B, H, N, last), dtype=torch.float32, generator=g)
        if scale != 1.0:
            x.mul_(scale)
        out.append(x.to(DTYPES[dtype]).contiguous())
    return out[0], out[1], out[2]


def forward_inputs(w: ForwardWorkload):
    return draw_qkv(w.B, w.H, w.N, w.C, w.M, w.dtype, w.seed, w.scale)


def decode_step_seed(w: DecodeWorkload, t: int) -> int:
    return w.seed * 1_000_000 + int(t)


def draw_decode_step(heads: int, C: int, M: int, dtype: str, seed: int,
                     scale: float = 1.0) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """q [heads,C], k [heads,C], v [heads,M] for one decode step."""
    g = torch.Generator("cpu").manual_seed(int(seed))
    out = []
    for last in (C, C, M):
        x = torch.randn((heads, last), dtype=torch.float32, generator=g)
        if scale != 1.0:
            x.mul_(scale)
        out.append(x.to(DTYPES[dtype]).contiguous())
    return out[0], out[1], out[2]


def decode_inputs(w: DecodeWorkload, t: int):
    return draw_decode_step(w.heads, w.C, w.M, w.dtype, decode_step_seed(w, t), w.scale)


def to_oracle_array(t: torch.Tensor):
    """CPU tensor -> numpy array in a form the oracle reads (bf16 as raw uint16 bits)."""
    import numpy as np
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype in (torch.float32, torch.float64):
        return t.numpy()
    raise TypeError(f"unsupported dtype {t.dtype}")


def grad_output_seed(seed: int) -> int:
    return int(seed) * 1_000_000 + 999_999


def draw_grad_output(B: int, H: int, N: int, M: int, dtype: str, seed: int) -> torch.Tensor:
    """dL/dO [B,H,N,M] for the gradient workloads: N(0, 1) from its own seed."""
    g = torch.Generator("cpu").manual_seed(grad_output_seed(seed))
    x = torch.randn((B, H, N, M), dtype=torch.float32, generator=g)
    return x.to(DTYPES[dtype]).contiguous()


def backward_inputs(w: ForwardWorkload):
    """Q, K, V of the forward workload plus a dL/dO of V's shape."""
    q, k, v = forward_inputs(w)
    return q, k, v, draw_grad_output(w.B, w.H, w.N, w.M, w.dtype, w.seed)


# ---------------------------------------------------------------------------
# Generation shell: a random-weight stack of linear-attention layers that
# emits one pixel-channel per step, shaped like autoregressive CIFAR-10
# generation (3072 steps per image, 256 values per step; "Transformers Are
# RNNs: Linear Attention" knowledge note, "How we know") with the running
# model's d_model 512, h 8, 12 layers ("Why Replace Attention?", "The Running
# Example").  The weights are random: throughput does not depend on them, and
# no trained model is available.
# ---------------------------------------------------------------------------
@dataclass(frozen=True)
class ShellConfig:
    name: str
    layers: int = 12
    d_model: int = 512
    heads: int = 8
    d_ff: int = 2048
    vocab: int = 256
    steps: int = 3072
    batch: int = 256
    seed: int = 2001


SHELLS: Dict[str, ShellConfig] = {
    "shell_l12_d512_h8_b256_3072steps": ShellConfig("shell_l12_d512_h8_b256_3072steps"),
}


def draw_shell_weights(cfg: ShellConfig) -> Dict[str, torch.Tensor]:
    """float32 CPU weights: token and position embeddings, per layer the fused
    q/k/v projection, the output projection and the two feed-forward matrices
    (all N(0, 0.02^2), scaled by 1/sqrt(2 * layers) on the residual outputs),
    layer-norm gains 1 and biases 0, and the output head."""
    g = torch.Generator("cpu").manual_seed(int(cfg.seed))
    D, F, L = cfg.d_model, cfg.d_ff, cfg.layers

    def n(*shape, std=0.02):
        return (torch.randn(shape, dtype=torch.float32, generator=g) * std).contiguous()

    res = 0.02 / (2.0 * max(L, 1)) ** 0.5
    w = {"tok_emb": n(cfg.vocab, D), "pos_emb": n(cfg.steps, D), "head": n(D, cfg.vocab),
         "ln_f_g": torch.ones(D), "ln_f_b": torch.zeros(D)}
    for l in range(L):
        w[f"wqkv{l}"] = n(D, 3 * D)
        w[f"wo{l}"] = n(D, D, std=res)
        w[f"w1{l}"] = n(D, F)
        w[f"w2{l}"] = n(F, D, std=res)
        for k in ("ln1", "ln2"):
            w[f"{k}_g{l}"] = torch.ones(D)
            w[f"{k}_b{l}"] = torch.zeros(D)
    return w


def shell_teacher_tokens(cfg: ShellConfig, batch: int, steps: int, seed: int) -> torch.Tensor:
    """Fixed input tokens [steps, batch] for teacher-forced comparisons."""
    g = torch.Generator("cpu").manual_seed(int(seed))
    return torch.randint(0, cfg.vocab, (steps, batch), generator=g, dtype=torch.int64)


def draw_device(shape, dtype: str, seed: int, scale: float = 1.0, device="cuda") -> torch.Tensor:
    """N(0, 1) (times a power-of-two scale) drawn on the device with its own
    seeded generator, rounded to the element type: for tensors too large to
    draw on the host (the random stream differs from the CPU draws)."""
    g = torch.Generator(device=device).manual_seed(int(seed))
    x = torch.randn(shape, dtype=torch.float32, device=device, generator=g)
    if scale != 1.0:
        x.mul_(scale)
    return x.to(DTYPES[dtype]).contiguous()
