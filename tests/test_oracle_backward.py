"""Pins of the oracle's gradients (CPU only).

The pages state that the gradients of causal linear attention are themselves
cumulative sums ("[Paper Review] Transformers are RNNs", §3.5 "Gradient
Computation") but print no formula, so the oracle's gradient code is a
derivation.  It is pinned here to things that do not share that derivation:

  * exact gradients of the forward definition ("Why Replace Attention?", §5.7,
    §7.1), by forward-mode differentiation with rational dual numbers on
    non-negative integer inputs (where phi(x) = x + 1 and e^0 = 1 keep every
    value rational);
  * central finite differences of the fp64 forward oracle, with inputs on both
    branches of phi;
  * torch's fp64 autograd through an independently written forward;
  * closed forms when Q = K = 0 (uniform weights: cumulative and column means);
  * linearity in dL/dO, and the magnitude companion bounding |gradient|.

The planted-mistake tests at the end change one line of a copy of oracle.c and
check that these pins catch it.
"""
import os
import shutil
import subprocess
import tempfile
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _both_forms(q, k, v, g, causal, companion=False):
    return (oracle.backward_quadratic(q, k, v, g, causal, companion=companion),
            oracle.backward_recurrent(q, k, v, g, causal, companion=companion))


# ---------------------------------------------------------------------------
# Exact gradients by rational dual numbers.
# ---------------------------------------------------------------------------
class Dual:
    """a + b*eps with eps^2 = 0, over Fractions: one directional derivative."""

    __slots__ = ("a", "b")

    def __init__(self, a, b=Fraction(0)):
        self.a, self.b = Fraction(a), Fraction(b)

    def __add__(self, o):
        o = o if isinstance(o, Dual) else Dual(o)
        return Dual(self.a + o.a, self.b + o.b)

    __radd__ = __add__

    def __mul__(self, o):
        o = o if isinstance(o, Dual) else Dual(o)
        return Dual(self.a * o.a, self.a * o.b + self.b * o.a)

    __rmul__ = __mul__

    def __truediv__(self, o):
        o = o if isinstance(o, Dual) else Dual(o)
        return Dual(self.a / o.a, (self.b * o.a - self.a * o.b) / (o.a * o.a))


def _phi_dual(x: Dual) -> Dual:
    # elu(x) + 1 on the integers used here: x + 1 for x > 0; at x = 0 the
    # e^x branch gives e^0 = 1 with derivative e^0 = 1, also rational.
    if x.a > 0:
        return x + 1
    assert x.a == 0, "dual-number pin uses non-negative integer inputs only"
    return Dual(1, x.b)


def _loss_dual(Q, K, V, G, causal):
    """L = sum_i g_i . o_i with o_i from the definition, one head, Dual entries."""
    N, C, M = len(Q), len(Q[0]), len(V[0])
    pq = [[_phi_dual(Q[i][c]) for c in range(C)] for i in range(N)]
    pk = [[_phi_dual(K[j][c]) for c in range(C)] for j in range(N)]
    L = Dual(0)
    for i in range(N):
        js = range(i + 1) if causal else range(N)
        den = Dual(0)
        num = [Dual(0) for _ in range(M)]
        for j in js:
            w = Dual(0)
            for c in range(C):
                w = w + pq[i][c] * pk[j][c]
            den = den + w
            for m in range(M):
                num[m] = num[m] + w * V[j][m]
        for m in range(M):
            L = L + G[i][m] * (num[m] / den)
    return L


def _exact_gradients(q, k, v, g, causal):
    N, C = q.shape
    M = v.shape[1]
    base = {name: [[Dual(int(x)) for x in row] for row in arr] for name, arr in (("q", q), ("k", k), ("v", v))}
    G = [[Fraction(int(x)) for x in row] for row in g]
    out = {"q": np.zeros((N, C)), "k": np.zeros((N, C)), "v": np.zeros((N, M))}
    for name in ("q", "k", "v"):
        arr = base[name]
        for r in range(len(arr)):
            for c in range(len(arr[0])):
                arr[r][c] = Dual(arr[r][c].a, 1)
                L = _loss_dual(base["q"], base["k"], base["v"], G, causal)
                arr[r][c] = Dual(arr[r][c].a, 0)
                out[name][r, c] = float(L.b)
    return out["q"], out["k"], out["v"]


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("seed", [0, 1])
def test_exact_dual_number_gradients(seed, causal):
    rng = np.random.default_rng(100 + seed)
    N, C, M = 5, 3, 2
    q = rng.integers(0, 4, (N, C)).astype(np.float64)
    k = rng.integers(0, 4, (N, C)).astype(np.float64)
    v = rng.integers(-3, 4, (N, M)).astype(np.float64)
    g = rng.integers(-3, 4, (N, M)).astype(np.float64)
    q[0, 0] = 0.0  # the e^x branch at its rational point
    exact = _exact_gradients(q, k, v, g, causal)
    for form in _both_forms(q[None, None], k[None, None], v[None, None], g[None, None], causal):
        for got, want in zip(form, exact):
            np.testing.assert_allclose(got[0, 0], want, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# Finite differences and autograd.
# ---------------------------------------------------------------------------
def _loss_oracle(q, k, v, g, causal):
    return float(np.sum(g * oracle.forward_quadratic(q, k, v, causal)))


@pytest.mark.parametrize("causal", [True, False])
def test_central_finite_differences(causal):
    B, H, N, C, M = 1, 2, 6, 3, 4
    q, k = _rand((B, H, N, C), 7), _rand((B, H, N, C), 8)
    v, g = _rand((B, H, N, M), 9), _rand((B, H, N, M), 10)
    grads = _both_forms(q, k, v, g, causal)
    comp = oracle.backward_recurrent(q, k, v, g, causal, companion=True)
    h = 1e-6
    for t, (name, x) in enumerate((("q", q), ("k", k), ("v", v))):
        fd = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[t], args_m[t] = xp, xm
            fd[idx] = (_loss_oracle(*args_p, g, causal) - _loss_oracle(*args_m, g, causal)) / (2 * h)
        for form in grads:
            err = np.max(np.abs(form[t] - fd) / comp[t])
            assert err < 1e-6, (name, err)


def _torch_forward(q, k, v, causal):
    pq = torch.nn.functional.elu(q) + 1.0
    pk = torch.nn.functional.elu(k) + 1.0
    w = pq @ pk.transpose(-1, -2)
    if causal:
        n = q.shape[-2]
        w = w * torch.tril(torch.ones(n, n, dtype=w.dtype))
    return (w @ v) / w.sum(-1, keepdim=True)


@pytest.mark.parametrize("causal", [True, False])
def test_torch_autograd_of_independent_forward(causal):
    B, H, N, C, M = 2, 2, 37, 5, 3
    arrs = [_rand((B, H, N, C), 21), _rand((B, H, N, C), 22), _rand((B, H, N, M), 23), _rand((B, H, N, M), 24)]
    q, k, v = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in arrs[:3])
    g = torch.tensor(arrs[3], dtype=torch.float64)
    (torch.sum(_torch_forward(q, k, v, causal) * g)).backward()
    ref = (q.grad.numpy(), k.grad.numpy(), v.grad.numpy())
    comp = oracle.backward_recurrent(*arrs, causal, companion=True)
    for form in _both_forms(*arrs, causal):
        for got, want, c in zip(form, ref, comp):
            assert np.max(np.abs(got - want) / c) < 1e-12


# ---------------------------------------------------------------------------
# Closed forms and structural properties.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [True, False])
def test_zero_queries_and_keys_closed_forms(causal):
    # phi(0) = 1: every weight is w = C and den_i = C |J(i)|, so o_i is the mean
    # of the visible values.  Then dv_j = sum_{i sees j} g_i / |J(i)|,
    # dphi(k_j) = sum_{i sees j} g_i . (v_j - o_i) / (C |J(i)|) for every feature,
    # and dphi(q_i) = sum_{j in J(i)} g_i . (v_j - o_i) / (C |J(i)|) = 0.
    N, C, M = 9, 4, 3
    q = np.zeros((1, 1, N, C))
    k = np.zeros((1, 1, N, C))
    v, g = _rand((1, 1, N, M), 31), _rand((1, 1, N, M), 32)
    V, G = v[0, 0], g[0, 0]
    cnt = np.arange(1, N + 1, dtype=np.float64) if causal else np.full(N, float(N))
    O = np.cumsum(V, axis=0) / cnt[:, None] if causal else np.tile(V.mean(0), (N, 1))
    dv = np.zeros((N, M))
    dk = np.zeros(N)
    for j in range(N):
        for i in range(N):
            if causal and i < j:
                continue
            dv[j] += G[i] / cnt[i]
            dk[j] += G[i] @ (V[j] - O[i]) / (C * cnt[i])
    comp = oracle.backward_recurrent(q, k, v, g, causal, companion=True)
    for dQ, dK, dV in _both_forms(q, k, v, g, causal):
        np.testing.assert_allclose(dV[0, 0], dv, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(dK[0, 0], np.tile(dk[:, None], (1, C)), rtol=1e-11, atol=1e-13)
        assert np.max(np.abs(dQ) / comp[0]) < 1e-13


def test_gradients_are_linear_in_dO():
    shape = (1, 3, 20, 4)
    q, k, v = _rand(shape, 41), _rand(shape, 42), _rand(shape, 43)
    g1, g2 = _rand(shape, 44), _rand(shape, 45)
    a = oracle.backward_recurrent(q, k, v, g1, True)
    b = oracle.backward_recurrent(q, k, v, g2, True)
    c = oracle.backward_recurrent(q, k, v, g1 + 2.0 * g2, True)
    for x, y, z in zip(a, b, c):
        np.testing.assert_allclose(z, x + 2.0 * y, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_companion_bounds_gradient_magnitudes(causal):
    shape = (2, 2, 50, 8)
    q, k, v, g = (_rand(shape, s) for s in (51, 52, 53, 54))
    grads = oracle.backward_recurrent(q, k, v, g, causal)
    comps = _both_forms(q, k, v, g, causal, companion=True)
    for comp in comps:
        for x, c in zip(grads, comp):
            assert np.all(np.abs(x) <= c * (1 + 1e-12) + 1e-300)
    for x, y in zip(*comps):
        np.testing.assert_allclose(x, y, rtol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_bf16_inputs_are_read_exactly(causal):
    # Raw bf16 patterns give the same gradients as their values widened by
    # torch (an independent bf16 -> fp64 conversion).
    shape = (1, 2, 33, 8)
    raw, widened = [], []
    for s in (61, 62, 63, 64):
        t = torch.tensor(_rand(shape, s), dtype=torch.float32).to(torch.bfloat16)
        raw.append(t.view(torch.int16).numpy().view(np.uint16))
        widened.append(t.to(torch.float64).numpy())
    a = oracle.backward_recurrent(*raw, causal)
    b = oracle.backward_recurrent(*widened, causal)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_empty_sequence_and_thread_counts_agree():
    z = np.zeros((2, 3, 0, 4))
    for x in oracle.backward_recurrent(z, z, z, z, True):
        assert x.shape == (2, 3, 0, 4)
    shape = (2, 3, 40, 4)
    q, k, v, g = (_rand(shape, s) for s in (71, 72, 73, 74))
    one = oracle.backward_recurrent(q, k, v, g, True, threads=1)
    many = oracle.backward_recurrent(q, k, v, g, True, threads=5)
    for x, y in zip(one, many):
        np.testing.assert_array_equal(x, y)


def test_phi_prime_branches():
    assert oracle.phi_prime(2.5) == 1.0
    assert oracle.phi_prime(0.0) == 1.0
    assert oracle.phi_prime(-1.5) == np.exp(-1.5)


# ---------------------------------------------------------------------------
# Planted mistakes: each must make at least one pin fail.
# ---------------------------------------------------------------------------
MUTATIONS = {
    "b_sign_flipped": ("w.b[i] = x->mode ? go / den : -go / den;", "w.b[i] = go / den;"),
    "a_not_normalised": ("w.a[i * M + m] = w.g[i * M + m] / den;", "w.a[i * M + m] = w.g[i * M + m];"),
    "phi_prime_constant": ("return x > 0.0 ? 1.0 : exp(x);", "return 1.0;"),
    "phi_prime_of_positive_is_phi": ("return x > 0.0 ? 1.0 : exp(x);", "return x > 0.0 ? x + 1.0 : exp(x);"),
    "dv_uses_unnormalised_g": ("dv[j * M + m] += wij * w.a[i * M + m];", "dv[j * M + m] += wij * w.g[i * M + m];"),
    "dk_misses_constant_term": ("            double s = z[c];\n", "            double s = 0.0;\n"),
    "dq_misses_normaliser_term": ("            double s = w.b[i] * z[c];\n", "            double s = 0.0;\n"),
    "suffix_is_strict": ("""    for (long j = N - 1; j >= 0; --j) {
        if (x->causal)""", """    for (long j = N - 1; j >= 0; --j) {
        if (x->causal && j < 0)"""),
    "quadratic_dk_uses_phik": ("dk[j * C + c] += coef * w.pq[i * C + c];", "dk[j * C + c] += coef * w.pk[i * C + c];"),
}


def _pins_pass() -> bool:
    tests = [lambda: test_exact_dual_number_gradients(0, True), lambda: test_exact_dual_number_gradients(0, False),
             lambda: test_central_finite_differences(True), test_phi_prime_branches]
    for t in tests:
        try:
            t()
        except (AssertionError, oracle.OracleError):
            return False
    return True


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_gradient_mistake_is_caught(name):
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
    assert _pins_pass()
