"""GPU: the C ABI used from plain C (tests/c_abi_check.c), with no Python binding
and no torch: device memory from the HIP runtime, solves (fp32 with an annealed
eps, bf16) checked against the fp64 C oracle within the fp32 and bf16 bounds
(1e-3 eps + 1e-5 max|pot|; 2e-2 eps_final), and the host-side error paths.
The program is built by __graft_entry__.build()."""

import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
EXE = os.path.join(HERE, "c_abi_check")


def test_c_program_solves_and_validates():
    try:
        import torch

        if not torch.cuda.is_available():
            pytest.skip("no GPU")
    except ImportError:
        pass
    assert os.path.exists(EXE), f"{EXE} is missing: run __graft_entry__.build()"
    res = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(res.stdout)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "C ABI check passed" in res.stdout
