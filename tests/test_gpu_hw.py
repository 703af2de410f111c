"""GPU check of the gfx950 instructions behind the kernels' fast paths
(reciprocal, square root, FP8 and scaled FP8/FP4 converts of bf16, fp16 and
fp32 inputs, the FP4 convert of any fp32 quotient up to 6.0625, the fp16 decode,
the fast division for fp16 numerators and the fp32 -> fp16 / bf16 roundings) over every input the kernels can
give them; see hw_check.hip.  The binary is built by
__graft_entry__.build() (kv_cache_epilog_amd.build.build_hw_check)."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hw_check")


def test_hardware_instructions_match_reference():
    assert os.path.exists(BIN), "tests/hw_check is not built (run __graft_entry__.build())"
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=100)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    lines = [l for l in r.stdout.splitlines() if "mismatches" in l]
    assert len(lines) == 13 and all(l.split(":")[1].strip().startswith("0 ") for l in lines), r.stdout
