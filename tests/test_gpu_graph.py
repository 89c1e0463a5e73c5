"""HIP-graph capture of the library's calls (GPU tests).

The entry points allocate nothing, write no memset nodes and take every
buffer from the caller, so a forward plus backward step can be captured once
and replayed with new input contents.  Each replay is checked bit for bit
against eager calls on the same inputs, with eager work and synchronisation
between the replays; a stale or partially recorded launch would show as a
mismatch on the second or third replay.
"""
import pytest
import torch

import linear_attention_02_amd as la
from tests.gpu_util import note
from workloads import draw_grad_output, draw_qkv

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _reset_segments():
    la.set_segments(0)
    yield
    la.set_segments(0)


# segments: 0 = the library's plan (here 14 one-chunk segments: prefix and
# suffix scans), 5 = three-chunk segments whose walks sum their own prefixes.
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("segments", [0, 5])
def test_forward_backward_graph_replays_match_eager(segments, causal, dtype):
    la.set_segments(segments)
    B, H, N = 2, 3, 64 * 13 + 7
    draws = [draw_qkv(B, H, N, 64, 64, dtype, seed=900 + r) for r in range(3)]
    grads = [draw_grad_output(B, H, N, 64, dtype, 900 + r) for r in range(3)]
    q, k, v = (t.cuda() for t in draws[0])
    g = grads[0].cuda()
    note(f"[graph] {dtype} causal={causal} segments={la.plan_segments(B, H, N, q.dtype, causal)}")
    ws = torch.empty(la.backward_workspace_bytes(B, H, N, q.dtype, causal), dtype=torch.uint8, device="cuda")
    out, dq, dk, dv = (torch.empty_like(t) for t in (v, q, k, v))

    def step():
        la.forward(q, k, v, causal=causal, out=out, workspace=ws)
        la.backward(q, k, v, g, causal=causal, dq=dq, dk=dk, dv=dv, workspace=ws, after_forward=True)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        step()
    torch.cuda.synchronize()

    for rep in (1, 2, 0):
        for dst, src in zip((q, k, v, g), draws[rep] + (grads[rep],)):
            dst.copy_(src.cuda())
        out.zero_(), dq.zero_(), dk.zero_(), dv.zero_()
        graph.replay()
        torch.cuda.synchronize()
        ref_o = la.forward(q, k, v, causal=causal)
        ref = la.backward(q, k, v, g, causal=causal)
        torch.cuda.synchronize()
        note(f"[graph] replay with inputs {rep}")
        assert torch.equal(out, ref_o)
        for got, want in zip((dq, dk, dv), ref):
            assert torch.equal(got, want)


# The training pair as the autograd node runs it: forward_train, then
# backward_train on its output and workspace (bf16 causal: the saved-forward
# backward; segments 0 = the plan, 3 = walks that sum their own prefixes and
# suffixes, 20 = the scans).
@pytest.mark.parametrize("segments", [0, 3, 20])
def test_training_pair_graph_replays_match_eager(segments):
    la.set_segments(segments)
    B, H, N = 2, 3, 64 * 25 + 9
    draws = [draw_qkv(B, H, N, 64, 64, "bf16", seed=950 + r) for r in range(3)]
    grads = [draw_grad_output(B, H, N, 64, "bf16", 950 + r) for r in range(3)]
    q, k, v = (t.cuda() for t in draws[0])
    g = grads[0].cuda()
    note(f"[graph] training pair segments={la.plan_segments(B, H, N, q.dtype, True)}")
    ws = torch.empty(la.train_workspace_bytes(B, H, N, q.dtype, True), dtype=torch.uint8, device="cuda")
    out, dq, dk, dv = (torch.empty_like(t) for t in (v, q, k, v))

    def step():
        la.forward_train(q, k, v, causal=True, out=out, workspace=ws)
        la.backward_train(q, k, v, out, g, ws, causal=True, dq=dq, dk=dk, dv=dv)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        step()
    torch.cuda.synchronize()

    for rep in (1, 2, 0):
        for dst, src in zip((q, k, v, g), draws[rep] + (grads[rep],)):
            dst.copy_(src.cuda())
        out.zero_(), dq.zero_(), dk.zero_(), dv.zero_()
        graph.replay()
        torch.cuda.synchronize()
        ref_o, ref_ws = la.forward_train(q, k, v, causal=True)
        ref = la.backward_train(q, k, v, ref_o, g, ref_ws, causal=True)
        torch.cuda.synchronize()
        note(f"[graph] training pair replay with inputs {rep}")
        assert torch.equal(out, ref_o)
        for got, want in zip((dq, dk, dv), ref):
            assert torch.equal(got, want)
