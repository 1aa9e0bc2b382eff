"""The fused activation kernel's evaluation method, checked on the CPU: a C
mirror of its fp32 operations (tests/numerics/activation_sweep.c), with the
hardware reciprocal, exp2 and expf each off by up to one ulp, stays within
2^-19 relative (+ 2^-140) of the fp64 definitions of GELU and SiLU for every
finite bf16 input.  The GPU test test_activation_every_bf16_input applies the
same bound to the device results themselves."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "numerics", "activation_sweep.c")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs a C compiler")
def test_activation_method_within_bound_for_every_bf16_input(tmp_path):
    exe = str(tmp_path / "activation_sweep")
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", exe, SRC, "-lm"], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.count("max relative error") == 27 + 3
