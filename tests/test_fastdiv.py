"""Host check of the division shortcuts of the kernel's fast paths: the
Markstein quotient for x / rms, the double-reciprocal quotient for the mode-0
codes v / scale and the double-constant quotients for amax / 448 and
amax / 6 (see
fastdiv_check.c for what is checked and over which inputs)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def test_fast_divisions_match_ieee(tmp_path):
    exe = str(tmp_path / "fastdiv_check")
    subprocess.run(["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-o", exe,
                    os.path.join(HERE, "fastdiv_check.c"), "-lm"], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    print(r.stdout)
    assert r.returncode == 0, r.stdout
    assert r.stdout.count(" 0 of ") == 5
