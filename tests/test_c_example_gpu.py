"""The plain-C example (examples/c_abi_decode.c) on the GPU: it drives the
C-ABI with buffers from the HIP runtime, no Python in the process, and checks
two decode calls against closed forms of the update (a zero initial state;
g = 0, beta = 1 and q = k), the padded sequence and the slots outside the
batch.  It is built with the library."""
import os
import subprocess
import sys

import pytest

from gpu_helpers import announce

pytestmark = pytest.mark.gpu


def test_c_example_runs():
    from linear_attention_recurrent_gating_amd import build
    assert os.path.exists(build.C_EXAMPLE), "build the package first"
    announce("c example")
    r = subprocess.run([build.C_EXAMPLE], capture_output=True, text=True, timeout=120)
    sys.stdout.write(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith("ok")
