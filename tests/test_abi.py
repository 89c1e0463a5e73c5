"""CPU tests of the C ABI: the library loads, exports every declared symbol,
and rejects bad arguments on the host before touching the GPU.

Only argument combinations that fail validation are passed with fake
pointers here; a call that passes validation would enqueue kernels.
"""
import ctypes
import os
import shutil
import subprocess
import tempfile

import pytest

import linear_attention_02_amd as la

OK, NULL, SHAPE, DTYPE, ALIGN, ALIAS, WORKSPACE, HIP, ARG = range(9)


@pytest.fixture(scope="module")
def L():
    return la.lib()


def test_library_exports_every_declared_function(L):
    names = la.declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), f"{n} declared in linattn.h but not exported"


def test_version_and_status_strings(L):
    assert L.linattn_version() == 10000
    for code, name in la.STATUS.items():
        assert L.linattn_status_string(code).decode() == name
    assert L.linattn_status_string(99).decode() == "LINATTN_UNKNOWN_STATUS"


def _fwd(L, Q=16, K=32, V=48, O=64, B=1, H=1, N=64, C=64, M=64, dt=1, causal=1, ws=None, wsb=0):
    return L.linattn_forward(Q, K, V, O, B, H, N, C, M, dt, causal, ws, wsb, None)


def test_forward_rejects_bad_arguments(L):
    assert _fwd(L, Q=None) == NULL
    assert _fwd(L, O=None) == NULL
    assert _fwd(L, C=32) == SHAPE
    assert _fwd(L, M=128) == SHAPE
    assert _fwd(L, N=-1) == SHAPE
    assert _fwd(L, B=-3) == SHAPE
    assert _fwd(L, dt=7) == DTYPE
    assert _fwd(L, Q=17) == ALIGN
    # O overlaps V: 64 tokens x 64 x 2 bytes = 8 KiB tensors.
    assert _fwd(L, Q=0x10000, K=0x20000, V=0x30000, O=0x30000 + 4096) == ALIAS
    assert _fwd(L, Q=0x10000, K=0x20000, V=0x30000, O=0x10000) == ALIAS
    assert "overlaps" in L.linattn_last_error().decode()


def test_forward_requires_workspace_when_the_plan_needs_one(L):
    need = L.linattn_forward_workspace_bytes(1, 1, 1 << 16, 64, 64, 1, 1)
    assert need > 0  # one head, many chunks: the planner splits the sequence
    big = 1 << 30
    args = dict(Q=big, K=2 * big, V=3 * big, O=4 * big, N=1 << 16)
    assert _fwd(L, **args) == WORKSPACE
    assert _fwd(L, ws=5 * big, wsb=need - 1, **args) == WORKSPACE
    assert _fwd(L, ws=big + 64, wsb=need, **args) == ALIAS  # workspace inside Q
    assert _fwd(L, ws=5 * big + 8, wsb=need, **args) == ALIGN


def test_empty_inputs_are_accepted_without_launch(L):
    for B, H, N in ((0, 8, 100), (2, 0, 100), (2, 8, 0)):
        assert _fwd(L, Q=None, K=None, V=None, O=None, B=B, H=H, N=N) == OK
    assert L.linattn_decode_step(None, None, None, None, None, None, 0, 64, 64, 0, None) == OK
    assert L.linattn_last_error().decode() == ""


def test_forward_state_argument_rules(L):
    f = L.linattn_forward_state
    base = (0x100000, 0x200000, 0x300000, 0x400000, 1, 1, 64, 64, 64, 1)
    # S0 without z0
    assert f(*base, 0x500000, None, None, None, None, 0, None) == ARG
    # S_out without z_out
    assert f(*base, None, None, 0x500000, None, None, 0, None) == ARG
    # S_out overlapping O
    assert f(*base, None, None, 0x400000, 0x600000, None, 0, None) == ALIAS
    # S_out partially overlapping S0
    assert f(*base, 0x500000, 0x600000, 0x500000 + 256, 0x700000, None, 0, None) == ALIAS
    # misaligned state
    assert f(*base, 0x500004, 0x600000, None, None, None, 0, None) == ALIGN


def test_decode_rejects_bad_arguments(L):
    d = L.linattn_decode_step
    S, z, q, k, v, o = 0x100000, 0x200000, 0x300000, 0x400000, 0x500000, 0x600000
    assert d(None, z, q, k, v, o, 4, 64, 64, 0, None) == NULL
    assert d(S, z, q, k, v, o, 4, 64, 32, 0, None) == SHAPE
    assert d(S, z, q, k, v, o, -1, 64, 64, 0, None) == SHAPE
    assert d(S, z, q, k, v, o, 4, 64, 64, 5, None) == DTYPE
    assert d(S + 4, z, q, k, v, o, 4, 64, 64, 0, None) == ALIGN
    assert d(S, S + 1024, q, k, v, o, 4, 64, 64, 0, None) == ALIAS   # z inside S
    assert d(S, z, q, k, v, z, 4, 64, 64, 0, None) == ALIAS          # o == z
    assert d(S, z, S, k, v, o, 4, 64, 64, 0, None) == ALIAS          # q inside S


def test_strided_decode_rejects_bad_arguments(L):
    d = L.linattn_decode_step_strided
    S, z, q, o = 0x100000, 0x200000, 0x300000, 0x600000
    assert d(S, z, q, q + 128, q + 256, o, 4, 64, 64, 1, 32, None) == SHAPE      # stride < 64
    assert d(S, z, q, q + 128, q + 256, o, 4, 64, 64, 1, 100, None) == ALIGN     # 200 bytes, not 16-aligned
    assert d(S, z, None, q + 128, q + 256, o, 4, 64, 64, 1, 192, None) == NULL
    # rows of head 3 reach 3 * 192 * 2 + 128 bytes past q: S placed there overlaps
    assert d(q + 1088, z, q, q + 128, q + 256, o, 4, 64, 64, 1, 192, None) == ALIAS
    assert d(S, z, q, q + 128, q + 256, o, 0, 64, 64, 1, 192, None) == OK


def test_planner_segments(L):
    # Few heads, long sequences: split so the grid covers the device.
    assert L.linattn_plan_segments(2, 8, 131072, 1, 1) > 1
    # Many short heads: few segments.
    assert L.linattn_plan_segments(16, 8, 3072, 1, 1) >= 1
    # A single chunk can not be split.
    assert L.linattn_plan_segments(1, 1, 64, 1, 1) == 1
    prev = L.linattn_set_segments(3)
    try:
        assert L.linattn_plan_segments(1, 1, 64 * 10, 1, 1) == 3
        assert L.linattn_plan_segments(1, 1, 64 * 2, 1, 1) == 2  # capped at the chunk count
    finally:
        L.linattn_set_segments(prev)
    # Causal plans with one segment need no workspace.
    assert L.linattn_forward_workspace_bytes(1, 1, 64, 64, 64, 1, 1) == 0
    # Non-causal plans always keep a total record.
    assert L.linattn_forward_workspace_bytes(1, 1, 64, 64, 64, 1, 0) == 2 * 4160 * 4


def _bwd(L, Q=0x100000, K=0x200000, V=0x300000, G=0x400000, dQ=0x500000, dK=0x600000, dV=0x700000, B=1, H=1,
         N=64, C=64, M=64, dt=1, causal=1, ws=None, wsb=0):
    return L.linattn_backward(Q, K, V, G, dQ, dK, dV, B, H, N, C, M, dt, causal, ws, wsb, None)


def test_backward_rejects_bad_arguments(L):
    assert _bwd(L, G=None) == NULL
    assert _bwd(L, dV=None) == NULL
    assert _bwd(L, C=32) == SHAPE
    assert _bwd(L, N=-5) == SHAPE
    assert _bwd(L, dt=9) == DTYPE
    assert _bwd(L, dK=0x600008) == ALIGN
    assert _bwd(L, dQ=0x100000 + 4096) == ALIAS   # dQ inside Q (8 KiB tensors)
    assert _bwd(L, dK=0x400000) == ALIAS          # dK is dO
    assert _bwd(L, dV=0x500000 + 4096) == ALIAS   # dV inside dQ
    assert "overlap" in L.linattn_last_error().decode()
    for B, H, N in ((0, 8, 100), (2, 0, 100), (2, 8, 0)):
        assert L.linattn_backward(None, None, None, None, None, None, None, B, H, N, 64, 64, 1, 1, None, 0,
                                  None) == OK


def test_backward_workspace_rules(L):
    # One head of 2^16 tokens: several segments, so both record sets and the
    # per-token pairs are needed.
    N = 1 << 16
    need = L.linattn_backward_workspace_bytes(1, 1, N, 64, 64, 1, 1)
    P = L.linattn_plan_segments(1, 1, N, 1, 1)
    assert P > 1
    assert need >= 2 * P * 4160 * 4 + N * 8
    # A single-chunk causal head still needs the pairs.
    assert L.linattn_backward_workspace_bytes(1, 1, 64, 64, 64, 1, 1) == 64 * 8
    big = 1 << 30
    args = dict(Q=big, K=2 * big, V=3 * big, G=4 * big, dQ=5 * big, dK=6 * big, dV=7 * big, N=N)
    assert _bwd(L, **args) == WORKSPACE
    assert _bwd(L, ws=8 * big, wsb=need - 1, **args) == WORKSPACE
    assert _bwd(L, ws=6 * big + 4096, wsb=need, **args) == ALIAS   # workspace inside dK
    assert _bwd(L, ws=8 * big + 8, wsb=need, **args) == ALIGN


def test_timer_without_launches(L):
    la.timer.reset()
    assert la.timer.names() == []
    assert la.timer.read("causal_walk_bf16") == (0.0, 0)


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_validation_under_sanitizers():
    from linear_attention_02_amd import build
    with tempfile.TemporaryDirectory() as d:
        try:
            exe = build.build_host_check(d, sanitize=True)
        except subprocess.CalledProcessError:
            exe = build.build_host_check(d, sanitize=False)
        r = subprocess.run([exe], capture_output=True, text=True, timeout=120,
                           env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1"))
        assert r.returncode == 0, r.stdout + r.stderr
        assert "all host validation checks passed" in r.stdout


def test_noalloc_forward_rejects_on_the_host(L):
    # Validation before any device work: bad arguments as linattn_forward,
    # and a plan that needs more than the static scratch.
    nf = lambda **kw: L.linattn_forward_noalloc(*(kw.get(a, d) for a, d in (
        ("Q", 16), ("K", 32), ("V", 48), ("O", 64), ("B", 1), ("H", 1), ("N", 64), ("C", 64), ("M", 64),
        ("dt", 1), ("causal", 1))), None)
    assert nf(Q=None) == NULL
    assert nf(C=32) == SHAPE
    assert nf(dt=5) == DTYPE
    assert nf(Q=17) == ALIGN
    # 4096 heads, non-causal: two 16,640-byte records per head, 136 MB.
    need = L.linattn_forward_workspace_bytes(64, 64, 64, 64, 64, 1, 0)
    assert need > (32 << 20)
    assert nf(B=64, H=64, N=64, causal=0) == WORKSPACE
    assert "static scratch" in L.linattn_last_error().decode()
    assert nf(B=0) == OK


def _ftrain(L, Q=0x100000, K=0x200000, V=0x300000, O=0x400000, B=1, H=1, N=64, C=64, M=64, dt=1, causal=1, ws=None,
            wsb=0):
    return L.linattn_forward_train(Q, K, V, O, B, H, N, C, M, dt, causal, ws, wsb, None)


def _btrain(L, Q=0x100000, K=0x200000, V=0x300000, O=0x800000, G=0x400000, dQ=0x500000, dK=0x600000, dV=0x700000,
            B=1, H=1, N=64, C=64, M=64, dt=1, causal=1, ws=None, wsb=0):
    return L.linattn_backward_train(Q, K, V, O, G, dQ, dK, dV, B, H, N, C, M, dt, causal, ws, wsb, None)


def test_training_pair_rejects_bad_arguments(L):
    # A workspace of the right size, so that each case fails on its own argument.
    need = L.linattn_train_workspace_bytes(1, 1, 64, 64, 64, 1, 1)
    ws = dict(ws=0x900000, wsb=need)
    assert _ftrain(L, O=None, **ws) == NULL
    assert _ftrain(L, C=32, **ws) == SHAPE
    assert _ftrain(L, N=-1, **ws) == SHAPE
    assert _ftrain(L, dt=7, **ws) == DTYPE
    assert _ftrain(L, Q=0x100008, **ws) == ALIGN
    assert _ftrain(L, O=0x300000 + 4096, **ws) == ALIAS  # O inside V (8 KiB tensors)
    assert _btrain(L, O=None, **ws) == NULL
    assert _btrain(L, G=None, **ws) == NULL
    assert _btrain(L, C=32, **ws) == SHAPE
    assert _btrain(L, dt=7, **ws) == DTYPE
    assert _btrain(L, O=0x800008, **ws) == ALIGN
    assert _btrain(L, O=0x500000, **ws) == ALIAS  # O is dQ
    assert _btrain(L, dV=0x100000 + 4096, **ws) == ALIAS  # dV inside Q


def test_training_pair_workspace_rules(L):
    # bf16 causal: even one chunk needs the saved 1/den and the pairs.
    need = L.linattn_train_workspace_bytes(1, 1, 64, 64, 64, 1, 1)
    assert need > 0
    assert _ftrain(L) == WORKSPACE
    assert _btrain(L) == WORKSPACE
    assert _ftrain(L, ws=0x900000, wsb=need - 1) == WORKSPACE
    assert _btrain(L, ws=0x900000, wsb=need - 1) == WORKSPACE
    assert _btrain(L, ws=0x600000 + 64, wsb=need) == ALIAS  # workspace inside dK
    assert _btrain(L, ws=0x900008, wsb=need) == ALIGN
    # The pair's workspace holds the backward's, plus 1/den per token for bf16 causal calls.
    for dt in (0, 1):
        for causal in (0, 1):
            for B, H, N in ((1, 1, 64), (2, 3, 1000), (1, 8, 1 << 16)):
                t = L.linattn_train_workspace_bytes(B, H, N, 64, 64, dt, causal)
                b = L.linattn_backward_workspace_bytes(B, H, N, 64, 64, dt, causal)
                assert t >= b > 0 or (t >= b and not causal)
                if dt == 1 and causal:
                    assert t >= b + B * H * N * 4
    assert L.linattn_train_workspace_bytes(0, 1, 64, 64, 64, 1, 1) == 0
    assert L.linattn_train_workspace_bytes(1, 1, 64, 32, 64, 1, 1) == 0
    assert L.linattn_train_workspace_bytes(1, 1, 64, 64, 64, 7, 1) == 0


def test_training_pair_and_after_forward_accept_empty_inputs(L):
    for B, H, N in ((0, 8, 100), (2, 0, 100), (2, 8, 0)):
        assert L.linattn_forward_train(None, None, None, None, B, H, N, 64, 64, 1, 1, None, 0, None) == OK
        assert L.linattn_backward_train(None, None, None, None, None, None, None, None, B, H, N, 64, 64, 1, 1, None,
                                        0, None) == OK
        assert L.linattn_backward_after_forward(None, None, None, None, None, None, None, B, H, N, 64, 64, 1, 1,
                                                None, 0, None) == OK
    assert L.linattn_last_error().decode() == ""


def test_stream_probe_library_exports_and_host_checks():
    """libstreamprobes.so (bench.py --probes) loads, exports its probes, and
    rejects arguments it cannot take before any launch."""
    from linear_attention_02_amd import build as hip_build
    assert os.path.exists(hip_build.PROBES_LIB), "libstreamprobes.so not built (run __graft_entry__.build())"
    P = ctypes.CDLL(hip_build.PROBES_LIB)
    for n in ("probe_read_lds", "probe_copy", "probe_write", "probe_mix31", "probe_mix31_lds"):
        assert hasattr(P, n), n
    vp, ll, ci = ctypes.c_void_p, ctypes.c_longlong, ctypes.c_int
    P.probe_read_lds.argtypes = [vp, ll, ci, vp, vp]
    P.probe_copy.argtypes = [vp, vp, ll, ci, ci, vp]
    P.probe_write.argtypes = [vp, ll, ci, ci, vp]
    P.probe_mix31.argtypes = [vp, vp, vp, vp, ll, ci, ci, vp]
    P.probe_mix31_lds.argtypes = [vp, vp, vp, vp, ll, ci, vp]
    fake = 1 << 20
    assert P.probe_read_lds(None, 1 << 14, 0, fake, None) == -1
    assert P.probe_read_lds(fake, (1 << 14) + 16, 0, fake, None) == -1      # not whole 16 KB chunks
    assert P.probe_copy(fake, fake, 24, 0, 512, None) == -1                 # not whole 16-byte vectors
    assert P.probe_copy(fake, fake, 1 << 20, 4, 512, None) == -1            # no such policy
    assert P.probe_write(fake, 1 << 20, 0, 0, None) == -1                   # no workgroups
    assert P.probe_write(fake, 1 << 20, 0, 65537, None) == -1               # too many workgroups
    assert P.probe_mix31(fake, None, fake, fake, 1 << 20, 0, 512, None) == -1
    assert P.probe_mix31_lds(fake, fake, fake, fake, 4096, 1024, None) == -1  # not whole 8 KB chunks
    assert P.probe_mix31_lds(fake, fake, fake, fake, 1 << 20, 0, None) == -1
