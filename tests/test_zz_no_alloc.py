"""linattn_forward_noalloc (GPU): the forward with its segment records in the
library's static device scratch instead of a caller's workspace.

Its output must equal linattn_forward's bit for bit (same kernels, same
plan), also when the scratch still holds a larger earlier call's records.
Each case is printed before its GPU work starts.
"""
import pytest
import torch

import linear_attention_02_amd as la
from tests.gpu_util import TOL, note, oracle_forward
import oracle
from workloads import WORKLOADS, draw_qkv, forward_inputs

pytestmark = pytest.mark.gpu

SCRATCH = 32 << 20


def _check(q, k, v, causal, label, vs_oracle=False):
    dtype = "bf16" if q.dtype == torch.bfloat16 else "f32"
    B, H, N, _ = q.shape
    need = la.workspace_bytes(B, H, N, q.dtype, causal)
    note(f"[noalloc] {label} {tuple(q.shape)} {dtype} causal={causal} scratch={need} bytes")
    assert need <= SCRATCH
    dq, dk, dv = q.cuda(), k.cuda(), v.cuda()
    ref = la.forward(dq, dk, dv, causal=causal)
    got = la.forward_noalloc(dq, dk, dv, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(got, ref), label
    if vs_oracle:
        r, mag = oracle_forward(q, k, v, causal)
        err, _ = oracle.parity_error(got.float().cpu().double().numpy(), r, mag)
        note(f"[noalloc] {label} err={err:.3e}")
        assert err <= TOL[dtype]


def test_noalloc_matches_forward_on_consecutive_calls():
    # The largest named plan first (1,024 records, 17 MB), then smaller and
    # ragged calls that find the earlier records still in the scratch.
    w = WORKLOADS["causal_bf16_b2h8n131072"]
    _check(*forward_inputs(w), True, w.name)
    _check(*draw_qkv(1, 3, 1000, 64, 64, "bf16", seed=9101), True, "small causal", vs_oracle=True)
    w = WORKLOADS["noncausal_bf16_b8h8n4096"]
    _check(*forward_inputs(w), False, w.name)
    _check(*draw_qkv(1, 2, 300, 64, 64, "f32", seed=9102), False, "small non-causal", vs_oracle=True)
    _check(*draw_qkv(2, 1, 5000, 64, 64, "f32", seed=9103), True, "fp32 causal", vs_oracle=True)


def test_noalloc_rejects_a_plan_beyond_the_scratch_and_writes_nothing():
    q, k, v = (torch.zeros(64, 64, 64, 64, dtype=torch.bfloat16, device="cuda") for _ in range(3))
    out = torch.full_like(v, 3.0)
    assert la.workspace_bytes(64, 64, 64, torch.bfloat16, False) > SCRATCH
    note("[noalloc] 4096 heads non-causal: beyond the scratch")
    with pytest.raises(la.LinattnError) as e:
        la.forward_noalloc(q, k, v, causal=False, out=out)
    assert e.value.status == 6
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())
