"""Parity over a fixed list of pseudo-random shapes (GPU tests).

Forty configurations drawn once from a seeded generator: batch, heads,
length (ragged, from one token to 9000), element type, causality,
the segment plan (the library's own, or a forced count that lands in the
in-walk prefix, the per-element scan or the grouped scan), and whether the
forward starts from a carried state.  Each is checked against the fp64
oracle, forward and backward, on the same bars as the other parity tests.
Unseeded cases also run the training pair (linattn_forward_train, whose
output must equal the forward's bit for bit, then linattn_backward_train),
its gradients on the same bars.
"""
import random

import pytest
import torch

import linear_attention_02_amd as la
import oracle
from tests.gpu_util import TOL, note, oracle_forward
from workloads import draw_grad_output, draw_qkv, to_oracle_array

pytestmark = pytest.mark.gpu


def _cases(n=40, seed=20240):
    rng = random.Random(seed)
    out = []
    for i in range(n):
        B = rng.choice([1, 1, 2, 3])
        H = rng.choice([1, 2, 3, 5])
        N = rng.choice([1, 2, 15, 63, 64, 65, 127, 300, 777, 1500, 2049, 3000, 9000])
        dtype = rng.choice(["f32", "bf16"])
        causal = rng.random() < 0.7
        segments = rng.choice([0, 0, 2, 7, 9, 40, 200])
        if N == 9000 and rng.random() < 0.5:
            segments = 141  # one chunk each: the grouped scan
        seeded = causal and rng.random() < 0.3
        out.append((i, B, H, N, dtype, causal, segments, seeded))
    return out


@pytest.fixture(autouse=True)
def _reset_segments():
    la.set_segments(0)
    yield
    la.set_segments(0)


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"case{c[0]}")
def test_random_shape_matches_oracle(case):
    i, B, H, N, dtype, causal, segments, seeded = case
    la.set_segments(segments)
    seed = 7000 + i
    q, k, v = draw_qkv(B, H, N, 64, 64, dtype, seed=seed)
    P = la.plan_segments(B, H, N, q.dtype, causal)
    note(f"[random] case {i}: B{B} H{H} N{N} {dtype} causal={causal} segments={P} seeded={seeded}")
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    if seeded:
        gen = torch.Generator().manual_seed(seed)
        S0 = torch.rand(B * H, 64, 64, generator=gen)
        z0 = torch.rand(B * H, 64, generator=gen) + 0.5
        o, _, _ = la.forward_state(qd, kd, vd, S0=S0.cuda(), z0=z0.cuda())
        (ref, _, _), mag = oracle_forward(q, k, v, True, S0=S0, z0=z0, return_state=True)
    else:
        o = la.forward(qd, kd, vd, causal=causal)
        ref, mag = oracle_forward(q, k, v, causal)
    torch.cuda.synchronize()
    err, stats = oracle.parity_error(o.float().cpu().double().numpy(), ref, mag)
    note(f"[random] case {i} forward err={err:.3e}")
    assert err <= TOL[dtype], (case, err, stats)
    if seeded:
        return  # the backward is defined for a zero initial state
    g = draw_grad_output(B, H, N, 64, dtype, seed)
    grads = la.backward(qd, kd, vd, g.cuda(), causal=causal)
    torch.cuda.synchronize()
    arrs = [to_oracle_array(t) for t in (q, k, v, g)]
    refs = oracle.backward_recurrent(*arrs, causal=causal)
    mags = oracle.backward_recurrent(*arrs, causal=causal, companion=True)
    for name, got, r, m in zip(("dq", "dk", "dv"), grads, refs, mags):
        err, stats = oracle.parity_error(got.float().cpu().double().numpy(), r, m)
        note(f"[random] case {i} {name} err={err:.3e}")
        assert err <= TOL[dtype], (case, name, err, stats)
    o_t, ws = la.forward_train(qd, kd, vd, causal=causal)
    assert torch.equal(o_t, o)
    grads_t = la.backward_train(qd, kd, vd, o_t, g.cuda(), ws, causal=causal)
    torch.cuda.synchronize()
    for name, got, r, m in zip(("dq", "dk", "dv"), grads_t, refs, mags):
        err, stats = oracle.parity_error(got.float().cpu().double().numpy(), r, m)
        note(f"[random] case {i} train {name} err={err:.3e}")
        assert err <= TOL[dtype], (case, "train", name, err, stats)
