"""The autograd binding (GPU tests): gradients through linear_attention equal
the training pair's (linattn_forward_train, linattn_backward_train) bit for
bit, on the scan and in-walk prefix paths, and a retained graph can be
back-propagated twice.  Where the pair falls back to the backward that
reuses the forward's records (fp32, non-causal), they also equal
linattn_backward's bit for bit."""
import pytest
import torch

import linear_attention_02_amd as la
from linear_attention_02_amd.autograd import linear_attention
from tests.gpu_util import note
from workloads import draw_grad_output, draw_qkv

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _reset_segments():
    la.set_segments(0)
    yield
    la.set_segments(0)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("segments", [0, 5])  # 0: 14 one-chunk segments (scans); 5: in-walk prefixes
def test_autograd_matches_library_backward(segments, causal, dtype):
    la.set_segments(segments)
    B, H, N = 1, 2, 64 * 13 + 7
    q, k, v = (t.cuda().requires_grad_() for t in draw_qkv(B, H, N, 64, 64, dtype, seed=31))
    w = draw_grad_output(B, H, N, 64, "f32", 31).cuda()
    note(f"[autograd] {dtype} causal={causal} segments={la.plan_segments(B, H, N, q.dtype, causal)}")
    o = linear_attention(q, k, v, causal)
    assert torch.equal(o, la.forward(q.detach(), k.detach(), v.detach(), causal=causal))
    (o.float() * w).sum().backward(retain_graph=True)
    qd, kd, vd = q.detach(), k.detach(), v.detach()
    o2, ws = la.forward_train(qd, kd, vd, causal=causal)
    ref = la.backward_train(qd, kd, vd, o2, w.to(q.dtype), ws, causal=causal)
    torch.cuda.synchronize()
    for t, r in zip((q, k, v), ref):
        assert torch.equal(t.grad, r)
    if not (causal and dtype == "bf16"):
        for t, r in zip((q, k, v), la.backward(qd, kd, vd, w.to(q.dtype), causal=causal)):
            assert torch.equal(t.grad, r)
    first = [t.grad.clone() for t in (q, k, v)]
    (o.float() * w).sum().backward()  # second pass through the retained graph accumulates
    torch.cuda.synchronize()
    for t, f in zip((q, k, v), first):
        assert torch.equal(t.grad, f + f)


def test_autograd_detects_inputs_changed_after_forward():
    q, k, v = (t.cuda().requires_grad_() for t in draw_qkv(1, 1, 200, 64, 64, "f32", seed=32))
    o = linear_attention(q, k, v, True)
    with torch.no_grad():
        k.add_(1.0)  # the saved k no longer matches what the forward read
    with pytest.raises(RuntimeError):
        o.sum().backward()
