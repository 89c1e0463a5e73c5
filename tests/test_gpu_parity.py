"""Parity of the HIP path against the fp64 oracle (GPU tests).

Small cases span several 64-token chunks, several segments and ragged tails;
the named workloads run at their full sizes in the launch configuration the
benchmark uses.  Each test prints its case before the GPU work starts.
"""
import numpy as np
import pytest
import torch

import linear_attention_02_amd as la
import oracle
from tests.gpu_util import TOL, check_forward, gpu_forward, note, oracle_forward
from workloads import WORKLOADS, decode_inputs, draw_decode_step, draw_qkv, forward_inputs, to_oracle_array

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _reset_segments():
    la.set_segments(0)
    yield
    la.set_segments(0)


SMALL = [(1, 1, 1), (1, 1, 17), (1, 2, 64), (2, 1, 65), (1, 3, 130), (2, 2, 300), (1, 1, 1000)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("B,H,N", SMALL)
def test_small_shapes(B, H, N, causal, dtype):
    q, k, v = draw_qkv(B, H, N, 64, 64, dtype, seed=7 + N + 13 * B + 101 * H)
    check_forward(q, k, v, causal, dtype, label=f"small B{B}H{H}N{N}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("segments", [1, 2, 3, 7, 16])
def test_segment_count_does_not_change_results(segments, dtype):
    q, k, v = draw_qkv(1, 2, 64 * 16 + 5, 64, 64, dtype, seed=99)
    la.set_segments(segments)
    check_forward(q, k, v, True, dtype, label=f"segments={segments}")
    check_forward(q, k, v, False, dtype, label=f"segments={segments} noncausal")


# The planner's short-segment regime (few heads, N up to 16K): one-chunk
# segments with in-walk prefixes (N = 512: 8 segments), one-chunk segments with
# the scan (N = 4096: 64), two-chunk segments with the scan (N = 8192: 64).
@pytest.mark.parametrize("N", [512, 4096, 8192])
def test_sequence_sweep_shapes(N):
    q, k, v = draw_qkv(1, 8, N, 64, 64, "bf16", seed=4000 + N)
    note(f"[parity] sweep shape N={N} segments={la.plan_segments(1, 8, N, torch.bfloat16, True)}")
    check_forward(q, k, v, True, "bf16", label=f"sweep B1H8N{N}")


# 301 one-chunk segments: the prefix and total scans take the grouped form
# (runs of records per thread group), here also seeded with a carried state.
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_many_segments_grouped_scan(dtype):
    N = 64 * 300 + 17
    q, k, v = draw_qkv(1, 2, N, 64, 64, dtype, seed=303)
    la.set_segments(N)
    assert la.plan_segments(1, 2, N, q.dtype, True) == 301
    check_forward(q, k, v, True, dtype, label="301 segments")
    check_forward(q, k, v, False, dtype, label="301 segments noncausal")
    g = torch.Generator().manual_seed(304)
    S0 = torch.rand(2, 64, 64, generator=g).cuda()
    z0 = (torch.rand(2, 64, generator=g) + 1.0).cuda()
    o, S1, z1 = la.forward_state(q.cuda(), k.cuda(), v.cuda(), S0=S0, z0=z0)
    torch.cuda.synchronize()
    got = o.float().cpu().double().numpy()
    (ref, S_ref, z_ref), mag = oracle_forward(q, k, v, True, S0=S0.cpu(), z0=z0.cpu(), return_state=True)
    err, stats = oracle.parity_error(got, ref, mag)
    note(f"[parity] 301 segments seeded {dtype} err={err:.3e} stats={stats}")
    assert err <= TOL[dtype]


def test_mixed_scales_and_large_magnitudes():
    # Inputs far from N(0, 1): both phi branches, large positive features.
    g = torch.Generator().manual_seed(5)
    q = (torch.randn(1, 2, 700, 64, generator=g) * 4).to(torch.bfloat16)
    k = (torch.randn(1, 2, 700, 64, generator=g) * 4).to(torch.bfloat16)
    v = (torch.randn(1, 2, 700, 64, generator=g) * 100).to(torch.bfloat16)
    check_forward(q, k, v, True, "bf16", label="scale x4")


def test_textbook_reduction_zero_queries_keys():
    # q = k = 0: phi = 1, so causal outputs are cumulative means of v.
    v = torch.randn(1, 1, 333, 64, generator=torch.Generator().manual_seed(3))
    z = torch.zeros_like(v)
    out = gpu_forward(z, z, v, True)
    cum = np.cumsum(v.double().numpy(), axis=2) / np.arange(1, 334)[None, None, :, None]
    assert np.max(np.abs(out - cum)) < 1e-5


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_run_to_run_bitwise_determinism(dtype):
    q, k, v = [t.cuda() for t in draw_qkv(2, 3, 2000, 64, 64, dtype, seed=11)]
    for causal in (True, False):
        a = la.forward(q, k, v, causal=causal)
        b = la.forward(q, k, v, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(a, b)


def test_last_causal_row_matches_noncausal():
    q, k, v = [t.cuda() for t in draw_qkv(2, 2, 777, 64, 64, "f32", seed=12)]
    c = la.forward(q, k, v, causal=True)
    n = la.forward(q, k, v, causal=False)
    torch.cuda.synchronize()
    assert torch.allclose(c[:, :, -1], n[:, :, -1], rtol=1e-5, atol=1e-6)


def test_heads_are_independent():
    q, k, v = draw_qkv(1, 4, 500, 64, 64, "bf16", seed=13)
    full = gpu_forward(q, k, v, True)
    q2, k2, v2 = q.clone(), k.clone(), v.clone()
    q2[:, 1:] = 0
    k2[:, 1:] = 3
    v2[:, 1:] = -7
    part = gpu_forward(q2, k2, v2, True)
    assert np.array_equal(full[:, 0], part[:, 0])


# ---------------------------------------------------------------------------
# Prefill -> decode handoff: forward_state and decode_step.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
# 4 segments: each walk sums the earlier segments' totals itself; 12 (11 for
# the 652-token part): the prefix scan, seeded with the carried state.
@pytest.mark.parametrize("segments", [1, 4, 12])
def test_forward_state_split_and_resume(dtype, segments):
    la.set_segments(segments)
    q, k, v = draw_qkv(2, 2, 1100, 64, 64, dtype, seed=21)
    n1 = 448
    dq, dk, dv = q.cuda(), k.cuda(), v.cuda()
    o1, S1, z1 = la.forward_state(dq[:, :, :n1].contiguous(), dk[:, :, :n1].contiguous(), dv[:, :, :n1].contiguous())
    o2, S2, z2 = la.forward_state(dq[:, :, n1:].contiguous(), dk[:, :, n1:].contiguous(), dv[:, :, n1:].contiguous(),
                                  S0=S1, z0=z1)
    torch.cuda.synchronize()
    got = torch.cat([o1, o2], dim=2).float().cpu().double().numpy()
    (ref, S_ref, z_ref), mag = oracle_forward(q, k, v, True, return_state=True)
    err, stats = oracle.parity_error(got, ref, mag)
    note(f"[parity] split/resume {dtype} segments={segments} err={err:.3e}")
    assert err <= TOL[dtype]
    # Final state against the fp64 state, on the scale of the sum of |terms|.
    # bf16 inputs: phi(k) enters the MFMA rounded to bf16 (relative 2^-9).
    _, S_mag, _ = oracle.forward_recurrent(*(to_oracle_array(t) for t in (q, k, v)), causal=True, absv=True,
                                           return_state=True)
    tol = 1e-5 if dtype == "f32" else 8e-3
    S_got = S2.cpu().double().numpy().reshape(S_ref.shape)
    z_got = z2.cpu().double().numpy().reshape(z_ref.shape)
    assert np.max(np.abs(S_got - S_ref) / S_mag) <= tol
    assert np.max(np.abs(z_got - z_ref) / z_ref) <= tol


def test_forward_state_in_place_and_empty():
    q, k, v = [t.cuda() for t in draw_qkv(1, 2, 0, 64, 64, "f32", seed=1)]
    S = torch.randn(2, 64, 64, device="cuda")
    z = torch.rand(2, 64, device="cuda")
    S_keep, z_keep = S.clone(), z.clone()
    o, S_out, z_out = la.forward_state(q, k, v, S0=S, z0=z)
    torch.cuda.synchronize()
    assert torch.equal(S_out, S_keep) and torch.equal(z_out, z_keep)
    q, k, v = [t.cuda() for t in draw_qkv(1, 2, 200, 64, 64, "f32", seed=2)]
    ref_o, ref_S, ref_z = la.forward_state(q, k, v, S0=S_keep, z0=z_keep)
    # In place (4 segments: the prefix scan reads S0, z0 before the walk writes them).
    o, S_out, z_out = la.forward_state(q, k, v, S0=S, z0=z, S_out=S, z_out=z)
    torch.cuda.synchronize()
    assert torch.equal(o, ref_o) and torch.equal(S, ref_S) and torch.equal(z, ref_z)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_steps_match_oracle_and_forward(dtype):
    heads, steps = 37, 70
    S = torch.zeros(heads, 64, 64, device="cuda")
    z = torch.zeros(heads, 64, device="cuda")
    S_ref = np.zeros((heads, 64, 64))
    z_ref = np.zeros((heads, 64))
    S_mag = np.zeros((heads, 64, 64))
    z_mag = np.zeros((heads, 64))
    qs, ks, vs = [], [], []
    worst = 0.0
    for t in range(steps):
        q, k, v = draw_decode_step(heads, 64, 64, dtype, seed=5000 + t)
        qs.append(q), ks.append(k), vs.append(v)
        o = la.decode_step(S, z, q.cuda(), k.cuda(), v.cuda())
        ref = oracle.decode_step(S_ref, z_ref, *(to_oracle_array(x) for x in (q, k, v)))
        mag = oracle.decode_step(S_mag, z_mag, *(to_oracle_array(x) for x in (q, k, v)), absv=True)
        err, _ = oracle.parity_error(o.cpu().double().numpy(), ref, mag)
        worst = max(worst, err)
    note(f"[parity] decode {dtype} heads={heads} steps={steps} worst={worst:.3e}")
    assert worst <= 1e-4 if dtype == "f32" else worst <= TOL["bf16"]
    # Final state against the fp64 state, on the scale of its |terms| sum.
    assert np.max(np.abs(S.cpu().double().numpy() - S_ref) / np.maximum(S_mag, 1e-30)) < 1e-5
    assert np.max(np.abs(z.cpu().double().numpy() - z_ref) / z_ref) < 1e-5
    # Decode from zero reproduces the causal forward row by row.
    q = torch.stack(qs, 1).reshape(1, heads, steps, 64)
    k = torch.stack(ks, 1).reshape(1, heads, steps, 64)
    v = torch.stack(vs, 1).reshape(1, heads, steps, 64)
    fwd = gpu_forward(q, k, v, True)
    ref, mag = oracle_forward(q, k, v, True)
    err, _ = oracle.parity_error(fwd, ref, mag)
    assert err <= TOL[dtype]


def test_prefill_then_decode_continues_the_sequence():
    q, k, v = draw_qkv(1, 8, 300, 64, 64, "f32", seed=31)
    n1 = 257
    o1, S, z = la.forward_state(q[:, :, :n1].contiguous().cuda(), k[:, :, :n1].contiguous().cuda(),
                                v[:, :, :n1].contiguous().cuda())
    outs = []
    for t in range(n1, 300):
        outs.append(la.decode_step(S, z, q[0, :, t].contiguous().cuda(), k[0, :, t].contiguous().cuda(),
                                   v[0, :, t].contiguous().cuda()))
    torch.cuda.synchronize()
    got = torch.cat([o1[0].float().cpu(), torch.stack(outs, 1).cpu()], dim=1).double().numpy()[None]
    ref, mag = oracle_forward(q, k, v, True)
    err, _ = oracle.parity_error(got, ref, mag)
    note(f"[parity] prefill+decode err={err:.3e}")
    assert err <= 1e-4


def test_decode_snapshot_and_resume_is_bitwise():
    heads = 16
    S = torch.zeros(heads, 64, 64, device="cuda")
    z = torch.zeros(heads, 64, device="cuda")
    S2, z2 = S.clone(), z.clone()
    inputs = [draw_decode_step(heads, 64, 64, "f32", seed=700 + t) for t in range(40)]
    for q, k, v in inputs:
        a = la.decode_step(S, z, q.cuda(), k.cuda(), v.cuda())
    for t, (q, k, v) in enumerate(inputs):
        if t == 20:  # checkpoint to the host and back
            S2 = S2.cpu().cuda()
            z2 = z2.cpu().cuda()
        b = la.decode_step(S2, z2, q.cuda(), k.cuda(), v.cuda())
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(S, S2) and torch.equal(z, z2)


# ---------------------------------------------------------------------------
# The named workloads at full size, in the benchmark's launch configuration.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["causal_f32_b1h1n256", "noncausal_bf16_b8h8n4096", "causal_bf16_b16h8n3072",
                                  "causal_bf16_b2h8n131072"])
def test_named_workload_full_size(name):
    w = WORKLOADS[name]
    q, k, v = forward_inputs(w)
    check_forward(q, k, v, w.causal, w.dtype, label=name)


def test_named_decode_workload_full_size_all_heads():
    # Every head at every step.  Decode from the zero state is the causal
    # forward row by row ("Why Replace Attention?", §7.2), so the oracle side
    # runs its recurrence over blocks of steps, carrying its fp64 state from
    # block to block, instead of one call per step.
    w = WORKLOADS["decode_f32_s256h8_3072steps"]
    heads, block = w.heads, 256
    S = torch.zeros(heads, 64, 64, device="cuda")
    z = torch.zeros(heads, 64, device="cuda")
    S_ref = z_ref = S_mag = None
    worst = 0.0
    note(f"[parity] {w.name}: {heads} heads x {w.steps} steps, every head at every step")
    for t0 in range(0, w.steps, block):
        steps = [decode_inputs(w, t) for t in range(t0, min(t0 + block, w.steps))]
        q, k, v = (torch.stack([s[i] for s in steps], 0) for i in range(3))  # [T, heads, 64]
        dq, dk, dv = q.cuda(), k.cuda(), v.cuda()
        outs = torch.empty(len(steps), heads, 64, device="cuda")
        for t in range(len(steps)):
            outs[t] = la.decode_step(S, z, dq[t], dk[t], dv[t])
        torch.cuda.synchronize()
        got = outs.cpu().double().numpy().transpose(1, 0, 2)[None]  # [1, heads, T, 64]
        qa, ka, va = (to_oracle_array(x.transpose(0, 1).contiguous()[None]) for x in (q, k, v))
        z_start = z_ref
        ref, S_ref, z_ref = oracle.forward_recurrent(qa, ka, va, causal=True, S0=S_ref, z0=z_start,
                                                     return_state=True)
        mag, S_mag, _ = oracle.forward_recurrent(qa, ka, va, causal=True, absv=True, S0=S_mag, z0=z_start,
                                                 return_state=True)
        err, _ = oracle.parity_error(got, ref, mag)
        worst = max(worst, err)
        note(f"[parity] {w.name} steps {t0}..{t0 + len(steps) - 1} err={err:.3e} worst so far {worst:.3e}")
    assert worst <= TOL["f32"]
    # Final state of every head against the fp64 state, on the scale of its |terms| sum.
    assert np.max(np.abs(S.cpu().double().numpy() - S_ref.reshape(heads, 64, 64)) /
                  S_mag.reshape(heads, 64, 64)) < 1e-4
    assert np.max(np.abs(z.cpu().double().numpy() - z_ref.reshape(heads, 64)) / z_ref.reshape(heads, 64)) < 1e-4


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_strided_decode_matches_packed_decode(dtype):
    # q, k, v as column slices of one [BH, 192] buffer give the same bits as
    # packed [BH, 64] operands.
    heads = 37
    g = torch.Generator().manual_seed(77)
    rows = torch.randn(heads, 192, generator=g).to(torch.bfloat16 if dtype == "bf16" else torch.float32).cuda()
    S0 = torch.randn(heads, 64, 64, generator=g).abs().cuda()
    z0 = torch.rand(heads, 64, generator=g).cuda() + 1.0
    S1, z1, S2, z2 = S0.clone(), z0.clone(), S0.clone(), z0.clone()
    note(f"[parity] strided decode {dtype} heads={heads}")
    a = la.decode_step(S1, z1, rows[:, 0:64].contiguous(), rows[:, 64:128].contiguous(),
                       rows[:, 128:192].contiguous())
    b = la.decode_step_strided(S2, z2, rows[:, 0:64], rows[:, 64:128], rows[:, 128:192])
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(S1, S2) and torch.equal(z1, z2)
