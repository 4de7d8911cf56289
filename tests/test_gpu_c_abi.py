"""The library driven through its C ABI alone: a C++ program (built with the
library, linked against it, no Python or torch inside) runs one layer and
checks it against exact properties of the method.  It runs as a child
process of the test, on the same GPU."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROGRAM = os.path.join(ROOT, "tests", "c_abi", "moe_c_abi_check")

pytestmark = pytest.mark.gpu


def test_c_abi_program():
    assert os.path.exists(PROGRAM), "build the library first (it builds this program too)"
    print("c-abi program", flush=True)
    r = subprocess.run([PROGRAM], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=120)
    print(r.stdout, flush=True)
    assert r.returncode == 0, r.stdout
    assert "c-abi check: ok" in r.stdout
