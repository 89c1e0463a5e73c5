"""Property tests of the oracle on random tiny shapes (CPU, Hypothesis).

The identities the pages state, checked on shapes and values Hypothesis
chooses (any C and M, ragged N, both phi branches):
  * the quadratic definition and the recurrent / reassociated forms are the
    same function ("Why Replace Attention?", §6.2 and §7.2, associativity);
  * the last causal row equals the non-causal row (§7.3 remark);
  * the first causal output is v_1 (§7.3);
  * every output lies within the range of the values it averages, since the
    weights are positive (§5.4);
  * the definition's gradients (G1) equal the cumulative-sum gradients (G2).
"""
import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle

SETTINGS = settings(max_examples=60, deadline=None, suppress_health_check=[HealthCheck.too_slow])


@st.composite
def qkv(draw, with_grad=False):
    B = draw(st.integers(1, 2))
    H = draw(st.integers(1, 2))
    N = draw(st.integers(1, 12))
    C = draw(st.integers(1, 6))
    M = draw(st.integers(1, 6))
    seed = draw(st.integers(0, 2**31 - 1))
    scale = draw(st.sampled_from([0.25, 1.0, 3.0]))
    rng = np.random.default_rng(seed)
    arrs = [rng.standard_normal((B, H, N, d)) * scale for d in (C, C, M)]
    if with_grad:
        arrs.append(rng.standard_normal((B, H, N, M)))
    return arrs


@SETTINGS
@given(qkv(), st.booleans())
def test_quadratic_equals_recurrent(arrs, causal):
    q, k, v = arrs
    a = oracle.forward_quadratic(q, k, v, causal=causal)
    b = oracle.forward_recurrent(q, k, v, causal=causal)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


@SETTINGS
@given(qkv())
def test_last_causal_row_is_noncausal_and_first_is_v1(arrs):
    q, k, v = arrs
    c = oracle.forward_recurrent(q, k, v, causal=True)
    n = oracle.forward_recurrent(q, k, v, causal=False)
    np.testing.assert_allclose(c[:, :, -1], n[:, :, -1], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(c[:, :, 0], v[:, :, 0], rtol=1e-12, atol=1e-12)


@SETTINGS
@given(qkv(), st.booleans())
def test_outputs_within_value_range(arrs, causal):
    q, k, v = arrs
    o = oracle.forward_recurrent(q, k, v, causal=causal)
    N = v.shape[2]
    for i in range(N):
        seen = v[:, :, : i + 1] if causal else v
        lo, hi = seen.min(axis=2), seen.max(axis=2)
        assert np.all(o[:, :, i] >= lo - 1e-12) and np.all(o[:, :, i] <= hi + 1e-12)


@SETTINGS
@given(qkv(with_grad=True), st.booleans())
def test_gradient_forms_agree(arrs, causal):
    q, k, v, g = arrs
    g1 = oracle.backward_quadratic(q, k, v, g, causal=causal)
    g2 = oracle.backward_recurrent(q, k, v, g, causal=causal)
    for a, b in zip(g1, g2):
        scale = max(1.0, float(np.max(np.abs(a))))
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-10 * scale)
