"""CPU pin of the references tests/hw_check.hip compares the gfx950 FP8 and FP4
converts with: its nearest-value searches over the decoded E4M3 and E2M1 code
tables (e4m3_by_search, e2m1_by_search) are cut out of the .hip source,
compiled for the host and compared with the oracle's encoders (OCP E4M3FN and
E2M1, round to nearest even, saturating) on every bf16 value, on every fp32
value within 4 ulps of each rounding midpoint of either format, and on a
strided sample of the fp32 range the GPU check covers."""
import os
import subprocess

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ORACLE_DIR = os.path.dirname(os.path.abspath(oracle.__file__))

SHIM = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
#include "kvepi_oracle.h"
static inline float __uint_as_float(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static inline uint32_t __float_as_uint(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
#define __builtin_inff() INFINITY
"""

MAIN = r"""
static unsigned long long checked = 0, bad = 0;
static void check(float q) {
  if (!(fabsf(q) <= 456.0f)) return;
  checked++;
  if (e4m3_by_search(q) != kvo_enc_e4m3(q)) bad++;
  if (fabsf(q) <= 6.0625f && e2m1_by_search(q) != kvo_enc_e2m1(q)) bad++;
}
static void around(float m) {
  uint32_t b = __float_as_uint(m);
  for (int d = -4; d <= 4; ++d) {
    if (d < 0 && b < (uint32_t)-d) continue;
    check(__uint_as_float(b + d));
    check(-__uint_as_float(b + d));
  }
}
int main(void) {
  for (uint32_t h = 0; h < 65536; ++h) check(__uint_as_float(h << 16));
  /* midpoints of adjacent E4M3 magnitudes, and 464 */
  for (uint32_t c = 0; c < 126; ++c) {
    float lo = c < 8 ? c * 0x1p-9f : __uint_as_float(((c >> 3) + 120u) << 23 | (c & 7u) << 20);
    uint32_t d = c + 1;
    float hi = d < 8 ? d * 0x1p-9f : __uint_as_float(((d >> 3) + 120u) << 23 | (d & 7u) << 20);
    around(0.5f * (lo + hi));
  }
  around(464.0f);
  {
    static const float e2m1[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
    for (int c = 0; c < 7; ++c) around(0.5f * (e2m1[c] + e2m1[c + 1]));
  }
  for (uint32_t u = 0; u <= 0x43E40000u; u += 997u) {
    check(__uint_as_float(u));
    check(-__uint_as_float(u));
  }
  printf("%llu checked, %llu mismatches\n", checked, bad);
  return bad != 0 || checked < 1000000;
}
"""


def _search_source():
    src = open(os.path.join(HERE, "hw_check.hip")).read()
    a = src.index("// E4M3FN magnitude of code c")
    b = src.index("__global__ void k_fp8")
    return src[a:b].replace("__device__ ", "static ")


def test_hw_check_search_references_match_oracle(tmp_path):
    oracle.build(force=False)
    c_file = tmp_path / "refs.c"
    c_file.write_text(SHIM + _search_source() + MAIN)
    exe = str(tmp_path / "refs")
    subprocess.run(["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math",
                    "-I", ORACLE_DIR, "-o", exe, str(c_file), "-L", ORACLE_DIR,
                    "-lkvepi_oracle", "-Wl,-rpath," + ORACLE_DIR, "-lm"], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert " 0 mismatches" in r.stdout
