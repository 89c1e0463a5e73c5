"""Autoregressive generation with a stack of causal linear-attention layers.

Each step feeds one token per sequence through L pre-norm layers.  A layer's
attention is one ``linattn_decode_step``: the layer keeps a per-head state
(S, z) and updates it in constant work per token, with no key/value cache
("Why Replace Attention?", §7.2 and §7.4; "Transformers Are RNNs: Linear
Attention" knowledge note, "Putting It Together": project the token, update
the state, read it, then continue through the layer).  Around it sit the
dense parts of a transformer layer: layer norm, the q/k/v projection,
the output projection and a GELU feed-forward block.  Those are plain
library GEMMs and elementwise operations on the same stream.

A step is captured once in a HIP graph and replayed per token, so that the
step's ~100 small launches cost one graph launch.  The position index and the
fed-back token live in device memory and are advanced inside the graph.
"""
from __future__ import annotations

from typing import Dict, Optional

from . import decode_step_strided, LinattnError


class GenerationShell:
    """Greedy generation for ``batch`` sequences with the given weights
    (``workloads.draw_shell_weights``).  ``dtype`` is the activation and weight
    type of the dense parts (float32 or bfloat16); the attention state is
    always float32."""

    def __init__(self, weights: Dict, layers: int, d_model: int, heads: int, batch: int, device="cuda",
                 dtype=None):
        import torch

        self.torch = torch
        self.L, self.D, self.H, self.B = layers, d_model, heads, batch
        if d_model != 64 * heads:
            raise LinattnError(2, "d_model must be 64 * heads (head size 64)")
        self.dtype = dtype or torch.float32
        self.device = torch.device(device)
        self.w = {k: v.to(self.device, self.dtype).contiguous() for k, v in weights.items()}
        # One q/k/v projection per layer, its columns reordered from
        # ({q, k, v}, head, 64) to (head, {q, k, v}, 64): the output row of a
        # sequence is then [H][3][64], so head h's q, k, v are 192 elements
        # apart and feed the strided decode step without copies.
        for l in range(layers):
            wqkv = self.w.pop(f"wqkv{l}")
            self.w[f"wqkv{l}"] = wqkv.view(d_model, 3, heads, 64).permute(0, 2, 1, 3).reshape(d_model, 3 * d_model)
            self.w[f"wqkv{l}"] = self.w[f"wqkv{l}"].contiguous()
        self.steps_max = self.w["pos_emb"].shape[0]
        BH = batch * heads
        self.S = [torch.zeros(BH, 64, 64, dtype=torch.float32, device=self.device) for _ in range(layers)]
        self.z = [torch.zeros(BH, 64, dtype=torch.float32, device=self.device) for _ in range(layers)]
        self.o = [torch.empty(BH, 64, dtype=torch.float32, device=self.device) for _ in range(layers)]
        self.pos = torch.zeros(1, dtype=torch.int64, device=self.device)
        self.tokens = torch.zeros(batch, dtype=torch.int64, device=self.device)
        self.logits = torch.empty(batch, self.w["head"].shape[1], dtype=torch.float32, device=self.device)
        self.graph = None

    def reset(self, first_tokens=None):
        """Clears the attention states and the position; sets the first input tokens."""
        for t in self.S + self.z:
            t.zero_()
        self.pos.zero_()
        if first_tokens is None:
            self.tokens.zero_()
        else:
            self.tokens.copy_(first_tokens.to(self.device))

    def _layer_norm(self, x, g, b):
        return self.torch.nn.functional.layer_norm(x, (self.D,), g, b, 1e-5)

    def _step(self, teacher: Optional[object] = None):
        """One token for every sequence: logits into self.logits; the argmax
        becomes the next input token (unless teacher-forced)."""
        torch, w, D, H, B = self.torch, self.w, self.D, self.H, self.B
        x = w["tok_emb"].index_select(0, self.tokens) + w["pos_emb"].index_select(0, self.pos)
        for l in range(self.L):
            h = self._layer_norm(x, w[f"ln1_g{l}"], w[f"ln1_b{l}"])
            rows = (h @ w[f"wqkv{l}"]).view(B * H, 192)
            decode_step_strided(self.S[l], self.z[l], rows[:, 0:64], rows[:, 64:128], rows[:, 128:192],
                                out=self.o[l])
            x = torch.addmm(x, self.o[l].view(B, D).to(self.dtype), w[f"wo{l}"])
            h = self._layer_norm(x, w[f"ln2_g{l}"], w[f"ln2_b{l}"])
            x = torch.addmm(x, torch.nn.functional.gelu(h @ w[f"w1{l}"]), w[f"w2{l}"])
        logits = self._layer_norm(x, w["ln_f_g"], w["ln_f_b"]) @ w["head"]
        self.logits.copy_(logits)
        if teacher is None:
            self.tokens.copy_(torch.argmax(self.logits, dim=1))
        self.pos.add_(1)

    def step(self, tokens=None):
        """Eager step; with ``tokens`` given they are the inputs of this step
        (teacher forcing).  Returns the step's logits [B, vocab] (float32)."""
        if tokens is not None:
            self.tokens.copy_(tokens.to(self.device))
        self._step(teacher=tokens)
        return self.logits

    def capture(self, stream=None):
        """Captures one greedy step in a HIP graph (after one eager warm-up step
        that the caller then resets away)."""
        torch = self.torch
        stream = stream or torch.cuda.Stream()
        with torch.cuda.stream(stream):
            self._step()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            self._step()
        torch.cuda.synchronize()
        self.graph = g
        return g

    def generate(self, steps: int, first_tokens=None, use_graph: bool = True, record=None):
        """Greedy generation of ``steps`` tokens per sequence from zero states.
        ``record`` (optional [steps, B] int64 device tensor) receives the tokens."""
        if steps > self.steps_max:
            raise LinattnError(2, f"at most {self.steps_max} steps (positions)")
        if use_graph and self.graph is None:
            self.capture()
        self.reset(first_tokens)
        for t in range(steps):
            if use_graph:
                self.graph.replay()
            else:
                self._step()
            if record is not None:
                record[t].copy_(self.tokens)
        return self.tokens
