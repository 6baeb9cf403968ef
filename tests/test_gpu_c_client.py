"""The C ABI from a plain C program (tests/c_abi/zs_c_client.c): HIP-runtime
memory; the flat step, a list plan, the one-shot list call, the clipped
two-pass step, the device loss scaler and the offload step, each checked bit
for bit against the oracle's C entry points; plus argument errors."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

CLIENT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "zs_c_client")


def test_plain_c_client_matches_the_oracle():
    assert os.path.exists(CLIENT), f"{CLIENT} is missing: build it with __graft_entry__.build()"
    print(f"running {CLIENT}", flush=True)
    sys.stdout.flush()
    r = subprocess.run([CLIENT], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=120)
    assert r.returncode == 0, r.stdout
    assert "zs_c_client ok" in r.stdout
