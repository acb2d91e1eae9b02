"""The C ABI from a plain C program on the GPU (tests/c/forward_c.c, built
next to libmoe.so by the package's build): device memory through the HIP
runtime's C API, moe_forward twice (same bits), the staged entry points
(same bits as moe_forward), finite and non-zero output."""
import os
import subprocess

import pytest

from sparse_mixture_experts_03_amd import build as lib_build

pytestmark = pytest.mark.gpu


def test_c_client_runs_the_layer():
    exe = lib_build.C_CLIENT
    assert os.path.exists(exe), f"{exe} is not built (run the package build)"
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stderr
    assert r.stdout.startswith("ok ")
