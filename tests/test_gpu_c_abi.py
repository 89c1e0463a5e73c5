"""The C ABI used with no Python in between (GPU test): tests/c_abi_check, a
C++ program built by __graft_entry__.build(), allocates device memory with
hipMalloc, calls linattn_forward, linattn_backward, the training pair
(linattn_forward_train, linattn_backward_train), linattn_backward_after_forward,
linattn_forward_state (a prefill split in two calls that carry the state),
linattn_decode_step and linattn_decode_step_strided on a stream of its own, and
compares the results with the fp64 oracle element by element (bounds 1e-4 for
fp32 inputs, 2e-2 for bf16 inputs)."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi_check")


def test_c_abi_program_matches_oracle():
    assert os.path.exists(EXE), "tests/c_abi_check is missing: run __graft_entry__.build()"
    run = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(run.stdout, flush=True)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "ALL PASS" in run.stdout
