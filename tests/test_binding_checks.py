"""The Python binding rejects mismatched caller-supplied buffers on the host.

The C library sizes every device access from the inputs' shape and element
type, so an output, gradient or state buffer of another shape or dtype would
be read or written out of bounds.  The binding checks them before it touches
the device, which these CPU tests exercise with CPU tensors.
"""
import pytest
import torch

import linear_attention_02_amd as la


def _qkv(dtype=torch.bfloat16, B=1, H=2, N=10):
    return (torch.zeros(B, H, N, 64, dtype=dtype) for _ in range(3))


@pytest.mark.parametrize("bad, status", [
    (torch.zeros(1, 2, 10, 64, dtype=torch.float32), 3),   # fp32 out for bf16 inputs
    (torch.zeros(1, 2, 9, 64, dtype=torch.bfloat16), 2),    # one token short
    (torch.zeros(2, 10, 64, dtype=torch.bfloat16), 2),      # same numel, other rank
])
def test_forward_out_must_match_v(bad, status):
    q, k, v = _qkv()
    with pytest.raises(la.LinattnError) as e:
        la.forward(q, k, v, causal=True, out=bad)
    assert e.value.status == status


@pytest.mark.parametrize("name, bad, status", [
    ("S0", torch.zeros(2, 64, 63), 2),
    ("z0", torch.zeros(2, 65), 2),
    ("S_out", torch.zeros(1, 64, 64), 2),
    ("z_out", torch.zeros(2, 64, dtype=torch.float64), 3),
    ("S0", torch.zeros(2, 64, 64, dtype=torch.bfloat16), 3),
])
def test_forward_state_buffers_are_checked(name, bad, status):
    q, k, v = _qkv()
    good = {"S0": torch.zeros(2, 64, 64), "z0": torch.zeros(2, 64), "S_out": torch.zeros(2, 64, 64),
            "z_out": torch.zeros(2, 64)}
    good[name] = bad
    with pytest.raises(la.LinattnError) as e:
        la.forward_state(q, k, v, **good)
    assert e.value.status == status


def test_forward_state_accepts_four_dimensional_states_before_the_device_check():
    q, k, v = _qkv()
    # [B, H, C, M] states have the right numel: only the device check remains.
    with pytest.raises(la.LinattnError) as e:
        la.forward_state(q, k, v, S0=torch.zeros(1, 2, 64, 64), z0=torch.zeros(1, 2, 64))
    assert e.value.status == 8


@pytest.mark.parametrize("which", ["dq", "dk", "dv"])
@pytest.mark.parametrize("bad, status", [
    (torch.zeros(1, 2, 10, 64, dtype=torch.float32), 3),
    (torch.zeros(1, 2, 11, 64, dtype=torch.bfloat16), 2),
])
def test_backward_gradient_buffers_must_match_inputs(which, bad, status):
    q, k, v = _qkv()
    g = torch.zeros_like(v)
    with pytest.raises(la.LinattnError) as e:
        la.backward(q, k, v, g, causal=True, **{which: bad})
    assert e.value.status == status


@pytest.mark.parametrize("strided", [False, True])
@pytest.mark.parametrize("name, bad, status", [
    ("S", torch.zeros(4, 64, 32), 2),
    ("S", torch.zeros(4, 64, 64, dtype=torch.bfloat16), 3),
    ("z", torch.zeros(3, 64), 2),
    ("out", torch.zeros(4, 64, dtype=torch.bfloat16), 3),
    ("out", torch.zeros(4, 32), 2),
])
def test_decode_buffers_are_checked(strided, name, bad, status):
    args = {"S": torch.zeros(4, 64, 64), "z": torch.zeros(4, 64), "out": torch.zeros(4, 64)}
    args[name] = bad
    q = k = v = torch.zeros(4, 64)
    fn = la.decode_step_strided if strided else la.decode_step
    with pytest.raises(la.LinattnError) as e:
        fn(args["S"], args["z"], q, k, v, out=args["out"])
    assert e.value.status == status


def test_decode_rejects_three_dimensional_rows():
    with pytest.raises(la.LinattnError) as e:
        la.decode_step(torch.zeros(4, 64, 64), torch.zeros(4, 64), torch.zeros(4, 1, 64), torch.zeros(4, 1, 64),
                       torch.zeros(4, 1, 64))
    assert e.value.status == 2


def test_matching_buffers_reach_the_device_check():
    # Well-formed CPU tensors pass every host check and stop at the device
    # check: no CPU fallback exists.
    q, k, v = _qkv()
    with pytest.raises(la.LinattnError) as e:
        la.forward(q, k, v, causal=True, out=torch.zeros_like(v))
    assert e.value.status == 8


@pytest.mark.parametrize("bad, status", [
    (torch.zeros(1, 2, 10, 64, dtype=torch.float32), 3),
    (torch.zeros(1, 2, 9, 64, dtype=torch.bfloat16), 2),
])
def test_forward_train_out_must_match_v(bad, status):
    q, k, v = _qkv()
    with pytest.raises(la.LinattnError) as e:
        la.forward_train(q, k, v, causal=True, out=bad)
    assert e.value.status == status


@pytest.mark.parametrize("name, bad, status", [
    ("o", torch.zeros(1, 2, 10, 64, dtype=torch.float32), 3),   # fp32 o for bf16 inputs
    ("o", torch.zeros(1, 2, 11, 64, dtype=torch.bfloat16), 2),
    ("o", None, 1),
    ("grad_out", torch.zeros(1, 2, 9, 64, dtype=torch.bfloat16), 2),
    ("dq", torch.zeros(1, 2, 10, 64, dtype=torch.float32), 3),
    ("dv", torch.zeros(1, 2, 11, 64, dtype=torch.bfloat16), 2),
    ("workspace", None, 8),                                     # forward_train's workspace is required
])
def test_backward_train_buffers_are_checked(name, bad, status):
    q, k, v = _qkv()
    nbytes = la.train_workspace_bytes(1, 2, 10, q.dtype, True)
    args = {"o": torch.zeros_like(v), "grad_out": torch.zeros_like(v),
            "workspace": torch.zeros(nbytes, dtype=torch.uint8)}
    args[name] = bad
    extra = {name: bad} if name in ("dq", "dk", "dv") else {}
    with pytest.raises(la.LinattnError) as e:
        la.backward_train(q, k, v, args["o"], args["grad_out"], args["workspace"], causal=True, **extra)
    assert e.value.status == status


def test_training_pair_well_formed_cpu_tensors_reach_the_device_check():
    q, k, v = _qkv()
    with pytest.raises(la.LinattnError) as e:
        la.forward_train(q, k, v, causal=True)
    assert e.value.status == 8
