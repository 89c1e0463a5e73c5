"""Parity of the HIP gradients against the fp64 oracle (GPU tests).

The oracle's gradients are pinned on the CPU (tests/test_oracle_backward.py);
here the HIP path is compared with them element by element.  Error metric:
max |grad - grad_ref| / grad_mag, where grad_mag is the oracle's magnitude
companion (every signed term replaced by a bound of its absolute value), the
scale on which fp32 and bf16 rounding act.  Bars as for the forward: 1e-4 for
fp32 inputs, 2e-2 for bf16 inputs with fp32 accumulation.
"""
import numpy as np
import pytest
import torch

import linear_attention_02_amd as la
import oracle
from tests.gpu_util import TOL, note
from workloads import WORKLOADS, backward_inputs, draw_grad_output, draw_qkv, to_oracle_array

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _reset_segments():
    la.set_segments(0)
    yield
    la.set_segments(0)


def gpu_backward(q, k, v, g, causal):
    grads = la.backward(q.cuda(), k.cuda(), v.cuda(), g.cuda(), causal=causal)
    torch.cuda.synchronize()
    return [t.float().cpu().double().numpy() for t in grads]


def check_backward(q, k, v, g, causal, dtype, label=""):
    note(f"[grad] {label} q{tuple(q.shape)} {dtype} causal={causal}")
    got = gpu_backward(q, k, v, g, causal)
    arrs = [to_oracle_array(t) for t in (q, k, v, g)]
    ref = oracle.backward_recurrent(*arrs, causal=causal)
    mag = oracle.backward_recurrent(*arrs, causal=causal, companion=True)
    errs = []
    for name, a, r, m in zip(("dq", "dk", "dv"), got, ref, mag):
        err, stats = oracle.parity_error(a, r, m)
        errs.append(err)
        note(f"[grad] {label} {name} err={err:.3e} stats={stats}")
        assert err <= TOL[dtype], f"{label} {name}: err {err:.3e} > {TOL[dtype]:.0e} ({stats})"
    return errs


SMALL = [(1, 1, 1), (1, 1, 17), (1, 2, 64), (2, 1, 65), (1, 3, 130), (2, 2, 300), (1, 1, 1000)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("B,H,N", SMALL)
def test_small_shapes(B, H, N, causal, dtype):
    seed = 17 + N + 13 * B + 101 * H
    q, k, v = draw_qkv(B, H, N, 64, 64, dtype, seed=seed)
    g = draw_grad_output(B, H, N, 64, dtype, seed)
    check_backward(q, k, v, g, causal, dtype, label=f"small B{B}H{H}N{N}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("segments", [1, 2, 3, 7, 16])
def test_segment_count_does_not_change_results(segments, dtype):
    N = 64 * 16 + 37
    q, k, v = draw_qkv(1, 2, N, 64, 64, dtype, seed=199)
    g = draw_grad_output(1, 2, N, 64, dtype, 199)
    la.set_segments(segments)
    check_backward(q, k, v, g, True, dtype, label=f"segments={segments}")
    check_backward(q, k, v, g, False, dtype, label=f"segments={segments} noncausal")


@pytest.mark.parametrize("N", [512, 4096, 8192])  # the planner's short-segment regime
def test_sequence_sweep_shapes(N):
    q, k, v = draw_qkv(1, 8, N, 64, 64, "bf16", seed=5000 + N)
    g = draw_grad_output(1, 8, N, 64, "bf16", 5000 + N)
    note(f"[grad] sweep shape N={N} segments={la.plan_segments(1, 8, N, torch.bfloat16, True)}")
    check_backward(q, k, v, g, True, "bf16", label=f"sweep B1H8N{N}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_many_segments_grouped_scan(dtype):
    # 301 one-chunk segments: the prefix, suffix and total scans take the
    # grouped form.
    N = 64 * 300 + 17
    q, k, v = draw_qkv(1, 2, N, 64, 64, dtype, seed=305)
    g = draw_grad_output(1, 2, N, 64, dtype, 305)
    la.set_segments(N)
    check_backward(q, k, v, g, True, dtype, label="301 segments")
    check_backward(q, k, v, g, False, dtype, label="301 segments noncausal")


def test_mixed_scales():
    gen = torch.Generator().manual_seed(55)
    q = (torch.randn(1, 2, 700, 64, generator=gen) * 3).to(torch.bfloat16)
    k = (torch.randn(1, 2, 700, 64, generator=gen) * 3).to(torch.bfloat16)
    v = (torch.randn(1, 2, 700, 64, generator=gen) * 50).to(torch.bfloat16)
    g = (torch.randn(1, 2, 700, 64, generator=gen) * 0.01).to(torch.bfloat16)
    for causal in (True, False):
        check_backward(q, k, v, g, causal, "bf16", label="scales x3/x50/x0.01")


def test_zero_queries_and_keys_closed_form_for_dv():
    # phi(0) = 1: o_i is the mean of the visible values, so dv_j is the sum of
    # g_i / |J(i)| over the rows i that see token j.
    N = 333
    gen = torch.Generator().manual_seed(8)
    v = torch.randn(1, 1, N, 64, generator=gen)
    g = torch.randn(1, 1, N, 64, generator=gen)
    z = torch.zeros_like(v)
    dq, dk, dv = gpu_backward(z, z, v, g, True)
    G = g[0, 0].double().numpy()
    w = G / np.arange(1, N + 1)[:, None]
    want = np.cumsum(w[::-1], axis=0)[::-1]
    np.testing.assert_allclose(dv[0, 0], want, rtol=1e-5, atol=1e-6)
    assert np.max(np.abs(dq)) < 1e-4 * np.max(np.abs(G))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_run_to_run_bitwise_determinism(dtype):
    q, k, v = draw_qkv(2, 2, 900, 64, 64, dtype, seed=3)
    g = draw_grad_output(2, 2, 900, 64, dtype, 3)
    for causal in (True, False):
        a = la.backward(q.cuda(), k.cuda(), v.cuda(), g.cuda(), causal=causal)
        b = la.backward(q.cuda(), k.cuda(), v.cuda(), g.cuda(), causal=causal)
        torch.cuda.synchronize()
        for x, y in zip(a, b):
            assert torch.equal(x, y)


def test_backward_matches_forward_difference_quotient():
    # Directional derivative of sum(g * O) along a random direction, from two
    # fp32 forwards on the GPU, against the gradients' inner product with it.
    gen = torch.Generator().manual_seed(21)
    B, H, N = 1, 2, 200
    q, k, v = (torch.randn(B, H, N, 64, generator=gen) for _ in range(3))
    g = torch.randn(B, H, N, 64, generator=gen)
    dirs = [torch.randn(B, H, N, 64, generator=gen) for _ in range(3)]
    dq, dk, dv = gpu_backward(q, k, v, g, True)
    h = 1e-2
    qp, kp, vp = (x + h * d for x, d in zip((q, k, v), dirs))
    qm, km, vm = (x - h * d for x, d in zip((q, k, v), dirs))
    Lp = float((la.forward(qp.cuda(), kp.cuda(), vp.cuda(), causal=True).cpu().double() * g.double()).sum())
    Lm = float((la.forward(qm.cuda(), km.cuda(), vm.cuda(), causal=True).cpu().double() * g.double()).sum())
    fd = (Lp - Lm) / (2 * h)
    an = sum(float((torch.from_numpy(x) * d.double()).sum()) for x, d in zip((dq, dk, dv), dirs))
    note(f"[grad] directional derivative fd={fd:.6e} analytic={an:.6e}")
    assert abs(fd - an) <= 2e-3 * max(1.0, abs(an))


# ---------------------------------------------------------------------------
# Named forward workloads, backward at full size.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["causal_f32_b1h1n256", "noncausal_bf16_b8h8n4096", "causal_bf16_b16h8n3072",
                                  "causal_bf16_b2h8n131072"])
def test_named_workload_backward_full_size(name):
    w = WORKLOADS[name]
    q, k, v, g = backward_inputs(w)
    check_backward(q, k, v, g, w.causal, w.dtype, label=name)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("segments", [0, 5, 12])  # 12: records hold scanned prefixes
def test_backward_after_forward_is_bitwise_identical(dtype, causal, segments):
    # Reusing the segment states the forward left in the workspace gives the
    # same bits as recomputing them.
    B, H, N = 1, 3, 64 * 21 + 9
    q, k, v = (t.cuda() for t in draw_qkv(B, H, N, 64, 64, dtype, seed=404))
    g = draw_grad_output(B, H, N, 64, dtype, 404).cuda()
    la.set_segments(segments)
    note(f"[grad] after_forward {dtype} causal={causal} segments={la.plan_segments(B, H, N, q.dtype, causal)}")
    ws = torch.empty(la.backward_workspace_bytes(B, H, N, q.dtype, causal), dtype=torch.uint8, device="cuda")
    ref = la.backward(q, k, v, g, causal=causal)
    la.forward(q, k, v, causal=causal, workspace=ws)
    got = la.backward(q, k, v, g, causal=causal, workspace=ws, after_forward=True)
    torch.cuda.synchronize()
    for x, y in zip(got, ref):
        assert torch.equal(x, y)


@pytest.mark.parametrize("causal", [True, False])
def test_tensors_beyond_2_to_the_31_elements_sampled_heads(causal):
    # 32 x 1024 heads x 1100 tokens x 64: 2.3e9 elements per tensor, so element
    # offsets pass 2^31.  Forward and backward run on all heads; the oracle
    # checks sampled heads, among them the last ones (highest addresses).
    from workloads import draw_device
    B, H, N = 32, 1024, 1100
    note(f"[big] B{B} H{H} N{N} causal={causal}: drawing on the device")
    q = draw_device((B, H, N, 64), "bf16", seed=3101, scale=0.125)
    k = draw_device((B, H, N, 64), "bf16", seed=3102, scale=0.125)
    v = draw_device((B, H, N, 64), "bf16", seed=3103)
    g = draw_device((B, H, N, 64), "bf16", seed=3104)
    out = la.forward(q, k, v, causal=causal)
    grads = la.backward(q, k, v, g, causal=causal)
    torch.cuda.synchronize()
    note("[big] device work done; checking sampled heads")
    for head in (0, 12345, B * H - 2, B * H - 1):
        b, h = divmod(head, H)
        sl = lambda t: t[b:b + 1, h:h + 1].cpu()
        arrs = [to_oracle_array(sl(t)) for t in (q, k, v, g)]
        ref = oracle.forward_recurrent(*arrs[:3], causal=causal)
        mag = oracle.forward_recurrent(*arrs[:3], causal=causal, absv=True)
        err, _ = oracle.parity_error(sl(out).double().numpy(), ref, mag)
        gref = oracle.backward_recurrent(*arrs, causal=causal)
        gmag = oracle.backward_recurrent(*arrs, causal=causal, companion=True)
        gerr = [oracle.parity_error(sl(x).double().numpy(), r, m)[0] for x, r, m in zip(grads, gref, gmag)]
        note(f"[big] head {head}: forward err={err:.3e} grads err={[f'{e:.2e}' for e in gerr]}")
        assert err <= TOL["bf16"] and max(gerr) <= TOL["bf16"]
    del q, k, v, g, out, grads
    torch.cuda.empty_cache()
