"""The C ABI from C: tests/c_abi/solve_poisson (built by __graft_entry__.build() with
gcc against include/sla.h and libsla.so) solves and differentiates a Poisson system
with no Python in the process and checks the result on the host."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "solve_poisson")


@pytest.mark.parametrize("N", [1, 96, 300])
def test_c_program_solves_and_differentiates(N):
    if not os.path.exists(EXE):
        pytest.skip("tests/c_abi/solve_poisson not built (python __graft_entry__.py build)")
    print(f"[c abi] N={N}", flush=True)
    r = subprocess.run([EXE, str(N)], capture_output=True, text=True, timeout=120)
    sys.stdout.write(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
