"""Pins for the fp64 oracle, against facts fixed outside the oracle itself.

Pins used (none of them re-types the oracle's own code):
  * the pages' hand-traced example (tests/golden/worked_example.json),
  * exact rational brute force with ``fractions`` on small integer inputs,
  * library routines: torch's bf16 -> float conversion, torch's ELU,
  * textbook reductions (Q = K = 0 gives the cumulative / column mean of V),
  * invariants the pages state (last causal row = non-causal row, causal o_1 =
    v_1, positive weights so outputs lie in the convex hull of the values),
  * equality of the quadratic, recurrent and decode forms.
The mutation tests at the end plant plausible mistakes in a copy of oracle.c
and check that the pins above catch every one of them.
"""
import json
import math
import os
import shutil
import subprocess
import tempfile
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = json.load(open(os.path.join(HERE, "golden", "worked_example.json")))


def _ex():
    g = GOLDEN["inputs"]
    Q = np.array(g["Q"], dtype=np.float64)[None, None]
    K = np.array(g["K"], dtype=np.float64)[None, None]
    V = np.array(g["V"], dtype=np.float64)[None, None]
    return Q, K, V


def _frac(s):
    return float(Fraction(s))


# ---------------------------------------------------------------------------
# The pages' worked example ("Why Replace Attention?", §5.5, §6.5, §7.3)
# ---------------------------------------------------------------------------

def test_worked_example_phi():
    Q, K, _ = _ex()
    phiQ = np.vectorize(oracle.phi)(Q[0, 0])
    phiK = np.vectorize(oracle.phi)(K[0, 0])
    assert np.array_equal(phiQ, np.array(GOLDEN["phi"]["phiQ"], float))
    assert np.array_equal(phiK, np.array(GOLDEN["phi"]["phiK"], float))


@pytest.mark.parametrize("causal", [False, True])
def test_worked_example_similarity_rows(causal):
    # With V = identity (value j is the j-th unit vector), o_i is row i of the
    # (masked) similarity matrix divided by its sum.
    Q, K, _ = _ex()
    Vid = np.eye(4)[None, None]
    W = np.array(GOLDEN["similarity"]["W"], dtype=np.float64)
    if causal:
        W = np.tril(W)
    expect = W / W.sum(axis=1, keepdims=True)
    for fn in (oracle.forward_quadratic, oracle.forward_recurrent):
        got = fn(Q, K, Vid, causal=causal)[0, 0]
        np.testing.assert_allclose(got, expect, rtol=0, atol=1e-15)


def test_worked_example_noncausal():
    Q, K, V = _ex()
    o1 = [_frac(s) for s in GOLDEN["noncausal"]["o1"]]
    for fn in (oracle.forward_quadratic, oracle.forward_recurrent):
        O = fn(Q, K, V, causal=False)[0, 0]
        np.testing.assert_allclose(O[0], o1, rtol=0, atol=1e-15)
    np.testing.assert_allclose(O[0], GOLDEN["noncausal"]["o1_printed"], atol=5e-3)
    _, S, z = oracle.forward_recurrent(Q, K, V, causal=False, return_state=True)
    assert np.array_equal(S[0, 0], np.array(GOLDEN["noncausal"]["S"], float))
    assert np.array_equal(z[0, 0], np.array(GOLDEN["noncausal"]["z"], float))


def test_worked_example_causal_outputs():
    Q, K, V = _ex()
    expect = np.array([[_frac(s) for s in row] for row in GOLDEN["causal"]["o"]])
    for fn in (oracle.forward_quadratic, oracle.forward_recurrent):
        O = fn(Q, K, V, causal=True)[0, 0]
        np.testing.assert_allclose(O, expect, rtol=0, atol=1e-15)
    np.testing.assert_allclose(O, np.array(GOLDEN["causal"]["o_printed"]), atol=5e-4)


def test_worked_example_causal_states_via_decode():
    Q, K, V = _ex()
    S = np.zeros((1, 2, 2))
    z = np.zeros((1, 2))
    expect_o = [[_frac(s) for s in row] for row in GOLDEN["causal"]["o"]]
    for i in range(4):
        o = oracle.decode_step(S, z, Q[0, 0, i][None], K[0, 0, i][None], V[0, 0, i][None])
        assert np.array_equal(S[0], np.array(GOLDEN["causal"]["S"][i], float)), i
        assert np.array_equal(z[0], np.array(GOLDEN["causal"]["z"][i], float)), i
        np.testing.assert_allclose(o[0], expect_o[i], rtol=0, atol=1e-15)
    # S_4 equals the unmasked S of §6.5.
    assert np.array_equal(S[0], np.array(GOLDEN["noncausal"]["S"], float))


def test_worked_example_final_state_of_causal_forward():
    Q, K, V = _ex()
    _, S, z = oracle.forward_recurrent(Q, K, V, causal=True, return_state=True)
    assert np.array_equal(S[0, 0], np.array(GOLDEN["causal"]["S"][-1], float))
    assert np.array_equal(z[0, 0], np.array(GOLDEN["causal"]["z"][-1], float))


# ---------------------------------------------------------------------------
# Exact brute force with rationals: non-negative integer inputs make
# phi(x) = x + 1 an integer, so every output is an exact fraction.
# ---------------------------------------------------------------------------

def _brute_fraction(Q, K, V, causal):
    N, C = Q.shape
    M = V.shape[1]
    out = []
    for i in range(N):
        js = range(i + 1) if causal else range(N)
        w = {j: sum(Fraction(int(Q[i, c]) + 1) * Fraction(int(K[j, c]) + 1) for c in range(C)) for j in js}
        den = sum(w.values())
        out.append([sum(w[j] * Fraction(int(V[j, m])) for j in js) / den for m in range(M)])
    return out


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("causal", [False, True])
def test_exact_fraction_brute_force(seed, causal):
    rng = np.random.default_rng(100 + seed)
    N, C, M = int(rng.integers(1, 9)), int(rng.integers(1, 4)), int(rng.integers(1, 4))
    Q = rng.integers(0, 4, size=(N, C)).astype(np.float64)
    K = rng.integers(0, 4, size=(N, C)).astype(np.float64)
    V = rng.integers(-5, 6, size=(N, M)).astype(np.float64)
    exact = _brute_fraction(Q, K, V, causal)
    exp = np.array([[float(x) for x in row] for row in exact])
    for fn in (oracle.forward_quadratic, oracle.forward_recurrent):
        got = fn(Q[None, None], K[None, None], V[None, None], causal=causal)[0, 0]
        np.testing.assert_allclose(got, exp, rtol=1e-14, atol=1e-14)


def _brute_float(Q, K, V, causal):
    # Independent pure-Python evaluation of the definition, with math.exp for
    # the negative branch of elu(x) + 1.
    def phi(x):
        return x + 1.0 if x > 0 else math.exp(x)
    N = Q.shape[0]
    out = np.zeros((N, V.shape[1]))
    for i in range(N):
        js = range(i + 1) if causal else range(N)
        w = [math.fsum(phi(Q[i, c]) * phi(K[j, c]) for c in range(Q.shape[1])) for j in js]
        den = math.fsum(w)
        for m in range(V.shape[1]):
            out[i, m] = math.fsum(wj * V[j, m] for wj, j in zip(w, js)) / den
    return out


@pytest.mark.parametrize("causal", [False, True])
def test_float_brute_force_with_negative_inputs(causal):
    rng = np.random.default_rng(7)
    Q = rng.standard_normal((11, 5))
    K = rng.standard_normal((11, 5))
    V = rng.standard_normal((11, 3))
    exp = _brute_float(Q, K, V, causal)
    for fn in (oracle.forward_quadratic, oracle.forward_recurrent):
        got = fn(Q[None, None], K[None, None], V[None, None], causal=causal)[0, 0]
        np.testing.assert_allclose(got, exp, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------
# Library routines.
# ---------------------------------------------------------------------------

def test_bf16_widening_matches_torch_for_every_pattern():
    bits = np.arange(1 << 16, dtype=np.uint16)
    t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    lib = oracle.lib()
    got = np.array([lib.oracle_bf16_to_double(int(b)) for b in bits])
    finite = np.isfinite(t)
    assert np.array_equal(got[finite], t[finite])
    assert np.array_equal(np.isnan(got), np.isnan(t))
    assert np.array_equal(got[np.isinf(t)], t[np.isinf(t)])


def test_bf16_inputs_read_exactly():
    # The same values given as bf16 bits and as float64 give identical results.
    q, k, v = [torch.randn(1, 2, 9, 4, generator=torch.Generator().manual_seed(s)).to(torch.bfloat16)
               for s in (1, 2, 3)]
    as_bits = [x.view(torch.int16).numpy().view(np.uint16) for x in (q, k, v)]
    as_f64 = [x.to(torch.float64).numpy() for x in (q, k, v)]
    a = oracle.forward_recurrent(*as_bits, causal=True)
    b = oracle.forward_recurrent(*as_f64, causal=True)
    assert np.array_equal(a, b)


def test_phi_matches_torch_elu_plus_one():
    x = np.concatenate([np.linspace(-30, 30, 2001), [0.0, -0.0, 1e-300, -1e-300, 700.0, -700.0]])
    ref = (torch.nn.functional.elu(torch.from_numpy(x), alpha=1.0) + 1.0).numpy()
    got = np.array([oracle.phi(v) for v in x])
    # elu(x) + 1 computed as (e^x - 1) + 1 loses absolute precision ~1e-16 by
    # cancellation; compare on that absolute scale, then compare the negative
    # branch to exp itself on a relative scale.
    np.testing.assert_allclose(got, ref, rtol=1e-15, atol=4e-16)
    neg = x <= 0
    np.testing.assert_allclose(got[neg], torch.exp(torch.from_numpy(x[neg])).numpy(), rtol=1e-15, atol=0)
    assert oracle.phi(0.0) == 1.0
    assert all(oracle.phi(v) > 0 for v in (-700.0, -50.0, -1.0, 0.0, 1.0))


# ---------------------------------------------------------------------------
# Identities and textbook reductions.
# ---------------------------------------------------------------------------

def _rand(B, H, N, C, M, seed, scale=1.0):
    g = np.random.default_rng(seed)
    return (g.standard_normal((B, H, N, C)) * scale, g.standard_normal((B, H, N, C)) * scale,
            g.standard_normal((B, H, N, M)))


@pytest.mark.parametrize("shape", [(1, 1, 1, 3, 2), (2, 3, 17, 4, 5), (1, 2, 40, 8, 8)])
def test_quadratic_equals_recurrent(shape):
    q, k, v = _rand(*shape, seed=sum(shape))
    for causal in (False, True):
        a = oracle.forward_quadratic(q, k, v, causal=causal)
        b = oracle.forward_recurrent(q, k, v, causal=causal)
        np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-12)


def test_last_causal_row_equals_noncausal_row():
    q, k, v = _rand(2, 2, 33, 6, 7, seed=5)
    c = oracle.forward_recurrent(q, k, v, causal=True)
    n = oracle.forward_recurrent(q, k, v, causal=False)
    np.testing.assert_allclose(c[:, :, -1], n[:, :, -1], rtol=1e-12, atol=1e-13)


def test_first_causal_row_is_first_value():
    q, k, v = _rand(2, 3, 9, 5, 4, seed=9)
    for fn in (oracle.forward_quadratic, oracle.forward_recurrent):
        o = fn(q, k, v, causal=True)
        np.testing.assert_allclose(o[:, :, 0], v[:, :, 0], rtol=1e-14, atol=1e-15)


def test_zero_queries_and_keys_give_cumulative_and_column_means():
    _, _, v = _rand(1, 2, 25, 4, 3, seed=11)
    z = np.zeros((1, 2, 25, 4))
    cum = np.cumsum(v, axis=2) / np.arange(1, 26)[None, None, :, None]
    col = np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape)
    for fn in (oracle.forward_quadratic, oracle.forward_recurrent):
        np.testing.assert_allclose(fn(z, z, v, causal=True), cum, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(fn(z, z, v, causal=False), col, rtol=1e-13, atol=1e-14)


def test_outputs_lie_in_convex_hull_of_values():
    q, k, v = _rand(1, 2, 30, 6, 5, seed=13, scale=2.0)
    for causal in (False, True):
        o = oracle.forward_recurrent(q, k, v, causal=causal)
        for i in range(30):
            vv = v[:, :, : i + 1] if causal else v
            assert np.all(o[:, :, i] <= vv.max(axis=2) + 1e-12)
            assert np.all(o[:, :, i] >= vv.min(axis=2) - 1e-12)


def test_magnitude_companion_bounds_outputs():
    q, k, v = _rand(2, 2, 20, 4, 4, seed=17)
    for causal in (False, True):
        o = oracle.forward_recurrent(q, k, v, causal=causal)
        mag = oracle.forward_recurrent(q, k, v, causal=causal, absv=True)
        np.testing.assert_allclose(mag, oracle.forward_recurrent(q, k, np.abs(v), causal=causal), rtol=1e-14)
        assert np.all(np.abs(o) <= mag * (1 + 1e-12))


def test_decode_steps_reproduce_causal_forward():
    q, k, v = _rand(2, 3, 14, 5, 6, seed=19)
    ref = oracle.forward_recurrent(q, k, v, causal=True)
    S = np.zeros((6, 5, 6))
    z = np.zeros((6, 5))
    for t in range(14):
        o = oracle.decode_step(S, z, q[:, :, t].reshape(6, 5), k[:, :, t].reshape(6, 5), v[:, :, t].reshape(6, 6))
        np.testing.assert_allclose(o.reshape(2, 3, 6), ref[:, :, t], rtol=1e-12, atol=1e-13)


def test_initial_state_resumes_a_split_sequence():
    q, k, v = _rand(1, 2, 21, 4, 3, seed=23)
    full, S_full, z_full = oracle.forward_recurrent(q, k, v, causal=True, return_state=True)
    a, S1, z1 = oracle.forward_recurrent(q[:, :, :8], k[:, :, :8], v[:, :, :8], causal=True, return_state=True)
    b, S2, z2 = oracle.forward_recurrent(q[:, :, 8:], k[:, :, 8:], v[:, :, 8:], causal=True, S0=S1, z0=z1,
                                         return_state=True)
    np.testing.assert_allclose(np.concatenate([a, b], axis=2), full, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S2, S_full, rtol=1e-12)
    np.testing.assert_allclose(z2, z_full, rtol=1e-12)


def test_nonpositive_denominator_is_reported():
    # exp underflows to 0 in fp64 below about -745, so every feature and every
    # weight is 0: the oracle must report it instead of dividing silently.
    q = np.full((1, 1, 3, 2), -1000.0)
    k = np.full((1, 1, 3, 2), -1000.0)
    v = np.ones((1, 1, 3, 2))
    with pytest.raises(oracle.OracleError):
        oracle.forward_recurrent(q, k, v, causal=True)
    assert oracle.lib().oracle_forward_recurrent(
        q.ctypes.data, k.ctypes.data, v.ctypes.data, 0, 1, 3, 2, 2, 1, 0, None, None,
        np.empty((1, 1, 3, 2)).ctypes.data_as(oracle.ctypes.POINTER(oracle.ctypes.c_double)),
        None, None, 1) == oracle.NONPOSITIVE_DEN


def test_empty_sequence_and_threads_agree():
    q, k, v = _rand(3, 2, 0, 4, 4, seed=1)
    assert oracle.forward_recurrent(q, k, v, causal=True).shape == (3, 2, 0, 4)
    q, k, v = _rand(3, 5, 12, 4, 4, seed=2)
    a = oracle.forward_recurrent(q, k, v, causal=True, threads=1)
    b = oracle.forward_recurrent(q, k, v, causal=True, threads=7)
    assert np.array_equal(a, b)


def test_parity_error_metric():
    ref = np.array([1.0, -0.5, 0.0])
    mag = np.array([2.0, 1.0, 0.0])
    err, _ = oracle.parity_error(ref + np.array([0.02, -0.01, 0.0]), ref, mag)
    assert err == pytest.approx(0.01)
    err, _ = oracle.parity_error(ref + np.array([0, 0, 1e-30]), ref, mag)
    assert err == float("inf")
    err, _ = oracle.parity_error(np.array([np.nan, 0, 0]), ref, mag)
    assert err == float("inf")


# ---------------------------------------------------------------------------
# Mutation checks: each planted mistake must make at least one pin fail.
# ---------------------------------------------------------------------------

MUTATIONS = {
    "phi_dropped_plus_one": ("return x > 0.0 ? x + 1.0 : exp(x);", "return x > 0.0 ? x : exp(x);"),
    "phi_elu_without_plus_one_on_negative_branch": ("return x > 0.0 ? x + 1.0 : exp(x);",
                                                    "return x > 0.0 ? x + 1.0 : exp(x) - 1.0;"),
    "strict_causal_mask": ("const long jmax = x->causal ? i : N - 1;",
                           "const long jmax = x->causal ? i - 1 : N - 1;"),
    "normaliser_counts_tokens": ("den += w;", "den += 1.0;"),
    "transposed_state_read": ("num += pq[c] * S[c * M + m];", "num += pq[c] * S[m * C + c];"),
    "read_before_update": ("        for (long c = 0; c < C; ++c) pq[c] = oracle_phi(elem(x->Q, x->dtype, qk0 + (size_t)i * C + c));\n",
                           "        for (long c = 0; c < C; ++c) pq[c] = oracle_phi(elem(x->Q, x->dtype, qk0 + (size_t)(i > 0 ? i - 1 : 0) * C + c));\n"),
    "bf16_wrong_shift": ("(uint32_t)bits << 16", "(uint32_t)bits << 15"),
    "decode_z_not_updated": ("        z[c] += pk;\n", "        (void)pk;\n"),
}


def _pins_pass() -> bool:
    tests = [test_worked_example_phi, test_worked_example_noncausal, test_worked_example_causal_outputs,
             test_worked_example_causal_states_via_decode, test_bf16_widening_matches_torch_for_every_pattern,
             lambda: test_worked_example_similarity_rows(True),
             lambda: test_exact_fraction_brute_force(0, True), test_first_causal_row_is_first_value,
             test_last_causal_row_equals_noncausal_row,
             lambda: test_float_brute_force_with_negative_inputs(True)]
    for t in tests:
        try:
            t()
        except (AssertionError, oracle.OracleError):
            return False
    return True


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name):
    before, after = MUTATIONS[name]
    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")).read()
    assert src.count(before) >= 1, f"mutation anchor for {name} not found"
    mutated = src.replace(before, after)
    with tempfile.TemporaryDirectory() as d:
        c_path = os.path.join(d, "m.c")
        so_path = os.path.join(d, "m.so")
        open(c_path, "w").write(mutated)
        subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-pthread", "-o", so_path, c_path, "-lm"],
                       check=True)
        with oracle.using_library(so_path):
            caught = not _pins_pass()
    assert caught, f"planted mistake {name} passed every pin"
    # The real oracle still passes the same pins.
    assert _pins_pass()
