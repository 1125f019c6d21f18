"""The comparison build with VALU products (Q.K^T and P.V as VALU bf16 dot
products instead of MFMA) meets the same oracle tolerances as the library: its
timing is only evidence for the MFMA choice if it computes the same thing. One
library build per process, so the check runs in a child process."""

import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
VALU_LIB = os.path.join(os.path.dirname(HERE), "load_balanced_split_amd", "libhpa_valu.so")


@pytest.mark.gpu
@pytest.mark.timeout(600)
def test_valu_product_build_matches_oracle():
    if not os.path.exists(VALU_LIB):
        pytest.skip("libhpa_valu.so not built")
    env = dict(os.environ, HPA_PRODUCTS="valu", HPA_TRACE="0")
    print("valu parity: child process", flush=True)
    r = subprocess.run([sys.executable, "-u", os.path.join(HERE, "valu_parity_main.py")], env=env,
                       capture_output=True, text=True, timeout=540)
    print(r.stdout[-6000:])
    assert r.returncode == 0, r.stderr[-6000:]
    assert "valu parity ok" in r.stdout
