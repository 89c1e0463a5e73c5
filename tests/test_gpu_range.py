"""The normaliser's range on the GPU, and structural invariances (GPU tests).

The denominator phi(q_i)^T z_i is positive in exact arithmetic ("Why Replace
Attention?", §5.4), but fp32 has a finite range, which the "Transformers Are
RNNs: Linear Attention" knowledge note raises under "Where It Breaks".  The
library keeps each query row in range by an exact power-of-two scale of
phi(q_i) (o_i is unchanged by any positive scale of phi(q_i)), so any finite
query row matches the oracle.  Key features are the caller's range: with
every key feature a query sees below -104, e^x is 0 in fp32, the denominator
is 0 and o_i is NaN (the documented result; the fp64 oracle still has a
weighted mean there).  Each test prints its case before the GPU work starts.
"""
import numpy as np
import pytest
import torch

import linear_attention_02_amd as la
import oracle
from tests.gpu_util import TOL, check_forward, gpu_forward, note, oracle_forward
from workloads import DTYPES, draw_decode_step, draw_qkv, to_oracle_array

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _reset_segments():
    la.set_segments(0)
    yield
    la.set_segments(0)


def _with_extreme_query_rows(q32: torch.Tensor, g: torch.Generator) -> torch.Tensor:
    """q [B,H,N,64] float32 with rows at the edges of the scaling rule."""
    q = q32.clone()
    N = q.shape[2]
    u = lambda lo, hi: lo + (hi - lo) * torch.rand(q.shape[0], q.shape[1], 64, generator=g)
    rows = {
        0: u(-130.0, -110.0),   # e^x is 0 in fp32: scaled by 2^-e, e ~ -170
        5: u(-95.0, -88.0),     # e^x subnormal in fp32
        70: u(-9.0, -8.5),      # just below the scaling threshold
        130: q[:, :, 130] + 0.0,
        131: u(2.0e37, 3.0e37),  # phi near fp32's largest values
        200: q[:, :, 200] + 0.0,
        201: q[:, :, 201] + 0.0,
    }
    rows[130][..., 7] = 1.0e20    # one huge feature
    rows[200][..., 3] = 65535.0   # exactly at the upper threshold: not scaled
    rows[201][..., 3] = 65536.0   # just above: scaled by 2^-16
    for t, r in rows.items():
        if t < N:
            q[:, :, t] = r
    q[:, :, 71] = -8.0 - torch.rand(q.shape[0], q.shape[1], 64, generator=g)
    q[:, :, 71, 9] = -8.0                      # largest feature exactly at the lower threshold
    q[:, :, N - 1] = u(-210.0, -200.0)         # the ragged tail's last row
    return q


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("causal", [True, False])
def test_extreme_query_rows_match_oracle(causal, dtype):
    g = torch.Generator().manual_seed(8101)
    N = 300  # four full chunks and a ragged tail
    q32 = torch.randn(1, 2, N, 64, generator=g)
    k32 = torch.randn(1, 2, N, 64, generator=g)
    v32 = torch.randn(1, 2, N, 64, generator=g)
    q = _with_extreme_query_rows(q32, g).to(DTYPES[dtype])
    k, v = k32.to(DTYPES[dtype]), v32.to(DTYPES[dtype])
    check_forward(q, k, v, causal, dtype, label=f"extreme query rows causal={causal}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("causal", [True, False])
def test_large_keys_and_queries_near_1e20(causal, dtype):
    # q and k features near 1e20 on some tokens: phi(q) phi(k) ~ 1e40 would
    # overflow fp32 without the query scale; the sums stay within range.
    g = torch.Generator().manual_seed(8102)
    N = 700
    q = torch.randn(1, 2, N, 64, generator=g)
    k = torch.randn(1, 2, N, 64, generator=g)
    v = torch.randn(1, 2, N, 64, generator=g)
    for t in (3, 64, 65, 400, 699):
        k[:, :, t, (t % 64)] = 1.0e20
        q[:, :, t + 1 if t + 1 < N else 0, :] = 0.9e20 + 1.0e19 * torch.rand(1, 2, 64, generator=g)
    q, k, v = (x.to(DTYPES[dtype]) for x in (q, k, v))
    check_forward(q, k, v, causal, dtype, label=f"q, k near 1e20 causal={causal}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_all_keys_underflowing_gives_nan(dtype):
    # Outside the supported range: every key feature below -104, so phi(k) = 0
    # in fp32 and every denominator is 0; the documented result is NaN.
    g = torch.Generator().manual_seed(8103)
    N = 200
    q = torch.randn(1, 2, N, 64, generator=g).to(DTYPES[dtype])
    k = (-110.0 - 20.0 * torch.rand(1, 2, N, 64, generator=g)).to(DTYPES[dtype])
    v = torch.randn(1, 2, N, 64, generator=g).to(DTYPES[dtype])
    for causal in (True, False):
        note(f"[range] all keys below -110 {dtype} causal={causal}")
        out = la.forward(q.cuda(), k.cuda(), v.cuda(), causal=causal)
        torch.cuda.synchronize()
        assert torch.isnan(out.float()).all()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_leading_underflowing_keys(dtype):
    # Keys 0..99 below -110, the rest N(0, 1): causal rows 0..99 see only
    # underflowing keys (NaN, documented); every later row, and every
    # non-causal row, matches the oracle (the lost terms are below e^-110 of
    # the kept ones).
    g = torch.Generator().manual_seed(8104)
    N, n0 = 333, 100
    q = torch.randn(1, 2, N, 64, generator=g)
    k = torch.randn(1, 2, N, 64, generator=g)
    v = torch.randn(1, 2, N, 64, generator=g)
    k[:, :, :n0] = -110.0 - 20.0 * torch.rand(1, 2, n0, 64, generator=g)
    q, k, v = (x.to(DTYPES[dtype]) for x in (q, k, v))
    note(f"[range] leading underflowing keys {dtype}")
    got = gpu_forward(q, k, v, True)
    assert np.isnan(got[:, :, :n0]).all()
    ref, mag = oracle_forward(q, k, v, True)
    err, stats = oracle.parity_error(got[:, :, n0:], ref[:, :, n0:], mag[:, :, n0:])
    note(f"[range] rows >= {n0} err={err:.3e} {stats}")
    assert err <= TOL[dtype]
    check_forward(q, k, v, False, dtype, label="leading underflowing keys, non-causal")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_extreme_queries_and_underflowing_first_key(dtype):
    heads = 8
    S = torch.zeros(heads, 64, 64, device="cuda")
    z = torch.zeros(heads, 64, device="cuda")
    S_ref, z_ref = np.zeros((heads, 64, 64)), np.zeros((heads, 64))
    S_mag, z_mag = np.zeros((heads, 64, 64)), np.zeros((heads, 64))
    g = torch.Generator().manual_seed(8105)
    worst = 0.0
    for t in range(12):
        q, k, v = (x.float() for x in draw_decode_step(heads, 64, 64, "f32", seed=8200 + t))
        if t == 0:
            k = -110.0 - 20.0 * torch.rand(heads, 64, generator=g)  # z = 0 after the step: NaN
        if t == 3:
            q = -130.0 + 20.0 * torch.rand(heads, 64, generator=g)
        if t == 4:
            q = -95.0 + 7.0 * torch.rand(heads, 64, generator=g)
        if t == 5:
            q[:, 11] = 1.0e20
        if t == 6:
            q = 2.0e37 + 1.0e37 * torch.rand(heads, 64, generator=g)
        if t == 7:
            k[:, 5] = 1.0e20
        q, k, v = (x.to(DTYPES[dtype]) for x in (q, k, v))
        note(f"[range] decode step {t} {dtype}")
        o = la.decode_step(S, z, q.cuda(), k.cuda(), v.cuda()).cpu().double().numpy()
        arrs = [to_oracle_array(x) for x in (q, k, v)]
        ref = oracle.decode_step(S_ref, z_ref, *arrs)
        mag = oracle.decode_step(S_mag, z_mag, *arrs, absv=True)
        if t == 0:
            assert np.isnan(o).all()
            continue
        err, _ = oracle.parity_error(o, ref, mag)
        worst = max(worst, err)
    note(f"[range] decode {dtype} worst={worst:.3e}")
    assert worst <= TOL[dtype]


# ---------------------------------------------------------------------------
# Structural invariances.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_noncausal_invariant_under_joint_key_value_permutation(dtype):
    # Non-causal o_i sums over every (k_j, v_j) pair, so reordering the pairs
    # jointly changes only the summation order ("Why Replace Attention?", §6.2).
    q, k, v = draw_qkv(2, 2, 1000, 64, 64, dtype, seed=8106)
    perm = torch.randperm(1000, generator=torch.Generator().manual_seed(8107))
    note(f"[invariance] joint K, V permutation {dtype}")
    a = gpu_forward(q, k, v, False)
    b = gpu_forward(q, k[:, :, perm].contiguous(), v[:, :, perm].contiguous(), False)
    _, mag = oracle_forward(q, k, v, False)
    err = float(np.max(np.abs(a - b) / mag))
    note(f"[invariance] permutation err={err:.3e}")
    assert err <= TOL[dtype]
    check_forward(q, k[:, :, perm].contiguous(), v[:, :, perm].contiguous(), False, dtype, label="permuted")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("causal", [True, False])
def test_output_is_linear_in_values(causal, dtype):
    # o_i = sum_j w_ij v_j / sum_j w_ij is linear in V for fixed Q, K.  V1 and
    # V2 live on disjoint token sets, so V1 + V2 and 2 V1 are exact in bf16.
    q, k, v = draw_qkv(1, 3, 900, 64, 64, dtype, seed=8108)
    mask = (torch.rand(900, generator=torch.Generator().manual_seed(8109)) < 0.5)[None, None, :, None]
    v1 = torch.where(mask, v, torch.zeros_like(v))
    v2 = torch.where(mask, torch.zeros_like(v), v)
    note(f"[invariance] linearity in V {dtype} causal={causal}")
    o1 = gpu_forward(q, k, v1, causal)
    o2 = gpu_forward(q, k, v2, causal)
    o12 = gpu_forward(q, k, v1 + v2, causal)
    o1x2 = gpu_forward(q, k, v1 * 2, causal)
    _, mag = oracle_forward(q, k, v, causal)
    # Sum: each output is rounded once on each side (bf16: 2^-8 relative).
    tol = 1e-5 if dtype == "f32" else 1.2e-2
    err = float(np.max(np.abs(o12 - (o1 + o2)) / mag))
    note(f"[invariance] additivity err={err:.3e}")
    assert err <= tol
    # Scaling by two is exact in every step, so it is bitwise.
    assert np.array_equal(o1x2, 2 * o1)
