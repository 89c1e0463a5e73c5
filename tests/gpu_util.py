"""Helpers shared by the GPU tests: run the HIP path and the fp64 oracle on the
same seeded inputs and measure the error on the scale the method fixes.

Error metric: err = max |O - O_ref| / O_mag, where O_mag is the oracle run on
|v|.  Each output is a positively weighted mean of values, so |O_ref| <= O_mag,
and O_mag is the scale of that mean.
"""
import sys

import numpy as np
import torch

import linear_attention_02_amd as la
import oracle
from workloads import to_oracle_array

# Bars from the parity contract: fp32 inputs 1e-4, bf16 inputs with fp32
# accumulation 2e-2 (max error relative to the weighted-mean scale).
TOL = {"f32": 1e-4, "bf16": 2e-2}


def note(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def oracle_forward(q, k, v, causal, S0=None, z0=None, return_state=False):
    """Oracle O (and its |v| companion) on CPU tensors."""
    qa, ka, va = (to_oracle_array(t) for t in (q, k, v))
    S0a = None if S0 is None else S0.detach().cpu().double().numpy()
    z0a = None if z0 is None else z0.detach().cpu().double().numpy()
    res = oracle.forward_recurrent(qa, ka, va, causal=causal, S0=S0a, z0=z0a, return_state=return_state)
    mag = oracle.forward_recurrent(qa, ka, va, causal=causal, absv=True,
                                   S0=None if S0a is None else np.abs(S0a), z0=z0a)
    return res, mag


def gpu_forward(q, k, v, causal):
    out = la.forward(q.cuda(), k.cuda(), v.cuda(), causal=causal)
    torch.cuda.synchronize()
    return out.float().cpu().double().numpy()


def check_forward(q, k, v, causal, dtype, label=""):
    note(f"[parity] {label} q{tuple(q.shape)} {dtype} causal={causal}")
    got = gpu_forward(q, k, v, causal)
    ref, mag = oracle_forward(q, k, v, causal)
    err, stats = oracle.parity_error(got, ref, mag)
    note(f"[parity] {label} err={err:.3e} stats={stats}")
    assert err <= TOL[dtype], f"{label}: err {err:.3e} > {TOL[dtype]:.0e} ({stats})"
    return err
