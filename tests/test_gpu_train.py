"""The training pair linattn_forward_train / linattn_backward_train (GPU tests).

bf16 causal calls take the saved-forward backward: the forward saves 1/den_i,
one pass over Q, dO and O forms the reverse sums, and one left-to-right pass
writes dQ, dK and dV ("[Paper Review] Transformers are RNNs", §3.5: the
gradients are forward and reverse cumulative sums).  Its gradients are
compared element by element with the fp64 oracle's, on the oracle's
magnitude companion, at the bars of the other backward (2e-2 for bf16
inputs).  Other types and the non-causal form must equal
linattn_backward_after_forward bit for bit.  Each test prints its case before
the GPU work starts.
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


def gpu_train(q, k, v, g, causal):
    q, k, v, g = (t.cuda() for t in (q, k, v, g))
    o, ws = la.forward_train(q, k, v, causal=causal)
    grads = la.backward_train(q, k, v, o, g, ws, causal=causal)
    torch.cuda.synchronize()
    return o, grads


def check_train(q, k, v, g, causal, dtype, label=""):
    B, H, N = q.shape[:3]
    note(f"[train] {label} B{B}H{H}N{N} {dtype} causal={causal} "
         f"segments={la.plan_segments(B, H, N, q.dtype, causal)}")
    _, grads = gpu_train(q, k, v, g, causal)
    got = [t.float().cpu().double().numpy() for t in grads]
    arrs = [to_oracle_array(t) for t in (q, k, v, g)]
    ref = oracle.backward_recurrent(*arrs, causal=causal)
    mag = oracle.backward_recurrent(*arrs, causal=causal, companion=True)
    errs = []
    for name, a, r, m in zip(("dq", "dk", "dv"), got, ref, mag):
        err, stats = oracle.parity_error(a, r, m)
        errs.append(err)
        note(f"[train] {label} {name} err={err:.3e} stats={stats}")
        assert err <= TOL[dtype], f"{label} {name}: err {err:.3e} > {TOL[dtype]:.0e} ({stats})"
    return errs


SMALL = [(1, 1, 1), (1, 1, 17), (1, 1, 31), (1, 1, 32), (1, 1, 33), (1, 2, 64), (2, 1, 65), (1, 3, 130),
         (2, 2, 300), (1, 1, 1000), (3, 5, 777)]


@pytest.mark.parametrize("B,H,N", SMALL)
def test_small_shapes_bf16_causal(B, H, N):
    seed = 7017 + N + 13 * B + 101 * H
    q, k, v = draw_qkv(B, H, N, 64, 64, "bf16", seed=seed)
    g = draw_grad_output(B, H, N, 64, "bf16", seed)
    check_train(q, k, v, g, True, "bf16", label=f"small B{B}H{H}N{N}")


@pytest.mark.parametrize("segments", [1, 2, 3, 7, 8, 9, 16, 40])
def test_segment_counts(segments):
    # 8 or fewer segments per head: the walk sums the totals records itself;
    # more: the suffix scan runs.  The ragged last chunk is 37 tokens.
    N = 64 * 40 + 37
    q, k, v = draw_qkv(1, 2, N, 64, 64, "bf16", seed=7199)
    g = draw_grad_output(1, 2, N, 64, "bf16", 7199)
    la.set_segments(segments)
    check_train(q, k, v, g, True, "bf16", label=f"segments={segments}")


def test_many_segments_grouped_scan_and_grouped_walk():
    # 301 one-chunk segments on 2 heads: the suffix scan takes the grouped
    # form and each walk workgroup covers several forward segments.
    N = 64 * 300 + 17
    q, k, v = draw_qkv(1, 2, N, 64, 64, "bf16", seed=7305)
    g = draw_grad_output(1, 2, N, 64, "bf16", 7305)
    la.set_segments(N)
    check_train(q, k, v, g, True, "bf16", label="301 segments")


def test_many_heads_groups_forward_segments_per_walk():
    # 96 heads of 24 chunks: 8 forward segments per head (the walk sums the
    # records), several per walk workgroup.
    q, k, v = draw_qkv(4, 24, 64 * 24 - 5, 64, 64, "bf16", seed=7400)
    g = draw_grad_output(4, 24, 64 * 24 - 5, 64, "bf16", 7400)
    check_train(q, k, v, g, True, "bf16", label="96 heads")


@pytest.mark.parametrize("N", [512, 4096, 8192])
def test_sequence_sweep_shapes(N):
    q, k, v = draw_qkv(1, 8, N, 64, 64, "bf16", seed=7500 + N)
    g = draw_grad_output(1, 8, N, 64, "bf16", 7500 + N)
    check_train(q, k, v, g, True, "bf16", label=f"sweep B1H8N{N}")


def test_mixed_scales():
    gen = torch.Generator().manual_seed(7055)
    q = (torch.randn(1, 2, 700, 64, generator=gen) * 3).to(torch.bfloat16)
    k = (torch.randn(1, 2, 700, 64, generator=gen) * 3).to(torch.bfloat16)
    v = (torch.randn(1, 2, 700, 64, generator=gen) * 50).to(torch.bfloat16)
    g = (torch.randn(1, 2, 700, 64, generator=gen) * 0.01).to(torch.bfloat16)
    check_train(q, k, v, g, True, "bf16", label="scales x3/x50/x0.01")


def test_query_rows_the_forward_rescales():
    # Rows whose largest feature is below -8 or above 65535 are scaled by a
    # power of two in the forward; the saved 1/den is the unscaled row's.
    # All rows stay inside the backward's documented range [-60, 2^30].
    gen = torch.Generator().manual_seed(7066)
    N = 300
    q = torch.randn(1, 2, N, 64, generator=gen)
    k = torch.randn(1, 2, N, 64, generator=gen)
    v = torch.randn(1, 2, N, 64, generator=gen)
    g = torch.randn(1, 2, N, 64, generator=gen)
    q[:, :, 5] = -40.0 - 10.0 * torch.rand(1, 2, 64, generator=gen)
    q[:, :, 70] = -9.0 - torch.rand(1, 2, 64, generator=gen)
    q[:, :, 130, 7] = 1.0e5
    q[:, :, 201, 3] = 65536.0
    q[:, :, N - 1] = -20.0 - torch.rand(1, 2, 64, generator=gen)
    q, k, v, g = (x.to(torch.bfloat16) for x in (q, k, v, g))
    check_train(q, k, v, g, True, "bf16", label="rescaled query rows")


def test_zero_queries_and_keys_closed_form_for_dv():
    # phi(0) = 1: o_i is the mean of the visible values, so dv_j is the sum of
    # g_i / (i + 1) over the rows i >= j (bf16 inputs, exact small integers
    # as values would hide nothing here, so compare at the bf16 bar).
    N = 333
    gen = torch.Generator().manual_seed(7008)
    v = torch.randn(1, 1, N, 64, generator=gen).to(torch.bfloat16)
    g = torch.randn(1, 1, N, 64, generator=gen).to(torch.bfloat16)
    z = torch.zeros_like(v)
    note("[train] zero q, k closed form")
    _, (dq, dk, dv) = gpu_train(z, z, v, g, True)
    G = g[0, 0].double().numpy()
    want = np.cumsum((G / np.arange(1, N + 1)[:, None])[::-1], axis=0)[::-1]
    scale = np.cumsum((np.abs(G) / np.arange(1, N + 1)[:, None])[::-1], axis=0)[::-1]
    err = float(np.max(np.abs(dv[0, 0].float().cpu().double().numpy() - want) / scale))
    note(f"[train] closed form dv err={err:.3e}")
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("causal", [True, False])
def test_forward_train_output_is_forward_output(dtype, causal):
    B, H, N = 2, 3, 64 * 13 + 5
    q, k, v = (t.cuda() for t in draw_qkv(B, H, N, 64, 64, dtype, seed=7606))
    note(f"[train] forward_train output {dtype} causal={causal}")
    ref = la.forward(q, k, v, causal=causal)
    got, _ = la.forward_train(q, k, v, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)


@pytest.mark.parametrize("dtype,causal", [("f32", True), ("f32", False), ("bf16", False)])
@pytest.mark.parametrize("segments", [0, 5, 12])
def test_other_forms_equal_backward_after_forward(dtype, causal, segments):
    B, H, N = 1, 3, 64 * 21 + 9
    q, k, v = (t.cuda() for t in draw_qkv(B, H, N, 64, 64, dtype, seed=7707))
    g = draw_grad_output(B, H, N, 64, dtype, 7707).cuda()
    la.set_segments(segments)
    note(f"[train] fallback {dtype} causal={causal} segments={la.plan_segments(B, H, N, q.dtype, causal)}")
    ref = la.backward(q, k, v, g, causal=causal)
    o, ws = la.forward_train(q, k, v, causal=causal)
    got = la.backward_train(q, k, v, o, g, ws, causal=causal)
    torch.cuda.synchronize()
    for x, y in zip(got, ref):
        assert torch.equal(x, y)


def test_run_to_run_bitwise_determinism_and_repeatable_backward():
    q, k, v = (t.cuda() for t in draw_qkv(2, 2, 2900, 64, 64, "bf16", seed=7803))
    g = draw_grad_output(2, 2, 2900, 64, "bf16", 7803).cuda()
    la.set_segments(12)
    note("[train] determinism")
    o, ws = la.forward_train(q, k, v, causal=True)
    a = la.backward_train(q, k, v, o, g, ws, causal=True)
    b = la.backward_train(q, k, v, o, g, ws, causal=True)  # the workspace's saved part is only read
    o2, ws2 = la.forward_train(q, k, v, causal=True)
    c = la.backward_train(q, k, v, o2, g, ws2, causal=True)
    torch.cuda.synchronize()
    for x, y, z in zip(a, b, c):
        assert torch.equal(x, y) and torch.equal(x, z)


@pytest.mark.parametrize("B,H,N", [(1, 1, 32), (1, 64, 32), (1, 64, 64), (2, 48, 17)])
def test_short_walk_segments_repeated_with_lds_traffic_between(B, H, N):
    """Walk segments of one or two 32-token chunks, where a segment's last
    chunk follows its first at once: the dK waves must read that chunk's D
    tiles only after the dQ waves wrote them.  Between repeats a forward on
    other data leaves different LDS contents behind; every repeat must equal
    the first bit for bit, and the first must meet the oracle's bar."""
    q, k, v = draw_qkv(B, H, N, 64, 64, "bf16", seed=7900 + N)
    g = draw_grad_output(B, H, N, 64, "bf16", 7900 + N)
    check_train(q, k, v, g, True, "bf16", label="short segments")
    qd, kd, vd, gd = (t.cuda() for t in (q, k, v, g))
    o, ws = la.forward_train(qd, kd, vd, causal=True)
    first = la.backward_train(qd, kd, vd, o, gd, ws, causal=True)
    other = [t.cuda() for t in draw_qkv(4, 8, 3000, 64, 64, "bf16", seed=7999)]
    for rep in range(12):
        la.forward(*other, causal=rep % 2 == 0)
        again = la.backward_train(qd, kd, vd, o, gd, ws, causal=True)
        torch.cuda.synchronize()
        for x, y in zip(first, again):
            assert torch.equal(x, y), f"repeat {rep} differs"


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_gradients_linear_in_grad_output_exactly(dtype, causal):
    """dQ, dK and dV are linear in dL/dO ("[Paper Review] Transformers are
    RNNs", §3.5: a_i and b_i are linear in g_i, and every gradient is a sum of
    products with exactly one of them).  Scaling dL/dO by 4 scales every such
    product and sum by 4 and commutes with rounding, so both backward paths
    must return exactly 4 times their gradients."""
    B, H, N = 2, 3, 64 * 9 + 21
    q, k, v = (t.cuda() for t in draw_qkv(B, H, N, 64, 64, dtype, seed=8100))
    g = draw_grad_output(B, H, N, 64, dtype, 8100).cuda()
    note(f"[train] linearity in dO {dtype} causal={causal}")
    o, ws = la.forward_train(q, k, v, causal=causal)
    for run in (lambda gg: la.backward_train(q, k, v, o, gg, ws, causal=causal),
                lambda gg: la.backward(q, k, v, gg, causal=causal)):
        one = run(g)
        four = run(g * 4)
        torch.cuda.synchronize()
        for a, b in zip(one, four):
            assert torch.equal(a * 4, b)


@pytest.mark.parametrize("causal", [True, False])
def test_dq_of_a_token_depends_only_on_its_own_grad_output(causal):
    """dphi(q_i) = S_i a_i + b_i z_i ("[Paper Review] Transformers are RNNs",
    §3.5): of dL/dO it reads row i alone.  Changing dL/dO on a few rows must
    change dQ on those rows only, bit for bit elsewhere, in both backward
    paths (a mixed-up token or tile index would leak into other rows)."""
    B, H, N = 1, 4, 64 * 11 + 5
    q, k, v = (t.cuda() for t in draw_qkv(B, H, N, 64, 64, "bf16", seed=8200))
    g = draw_grad_output(B, H, N, 64, "bf16", 8200).cuda()
    rows = torch.tensor([0, 31, 32, 63, 64, 400, N - 1], device="cuda")
    g2 = g.clone()
    g2[:, :, rows] = -g2[:, :, rows] + 0.5
    note(f"[train] dQ locality causal={causal}")
    o, ws = la.forward_train(q, k, v, causal=causal)
    for run in (lambda gg: la.backward_train(q, k, v, o, gg, ws, causal=causal),
                lambda gg: la.backward(q, k, v, gg, causal=causal)):
        dq1 = run(g)[0]
        dq2 = run(g2)[0]
        torch.cuda.synchronize()
        keep = torch.ones(N, dtype=torch.bool, device="cuda")
        keep[rows] = False
        assert torch.equal(dq1[:, :, keep], dq2[:, :, keep])
        assert not torch.equal(dq1[:, :, rows], dq2[:, :, rows])


@pytest.mark.parametrize("name", ["causal_bf16_b16h8n3072", "causal_bf16_b2h8n131072"])
def test_named_workload_train_full_size(name):
    w = WORKLOADS[name]
    q, k, v, g = backward_inputs(w)
    check_train(q, k, v, g, w.causal, w.dtype, label=name)
