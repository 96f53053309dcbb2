"""The value encoder computes the group step (max - min) / (2^b - 1) without a
division: q0 = a * RN(1/L), r = fma(-q0, L, a), q = fma(r, RN(1/L), q0).  This
file checks, exhaustively on the host, that q is the correctly rounded IEEE
binary32 quotient for every finite a >= 0 and both divisors the encoder uses
(L = 3 for 2-bit and 15 for 4-bit groups).  It checks the arithmetic fact the
kernel relies on, in C with fmaf, independently of the kernel and the GPU.
"""
import os
import shutil
import subprocess

import pytest

SRC = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
int main(int argc, char** argv) {
  volatile float lv = (float)atof(argv[1]);
  const float L = lv, y = 1.0f / L;
  unsigned long long bad = 0;
  for (uint32_t u = 0; u < 0x7F800000u; ++u) {   /* +0 .. largest finite */
    float a;
    memcpy(&a, &u, 4);
    const float ref = a / L;
    const float q0 = a * y;
    const float r = fmaf(-q0, L, a);
    const float q = fmaf(r, y, q0);
    uint32_t qb, rb;
    memcpy(&qb, &q, 4);
    memcpy(&rb, &ref, 4);
    bad += qb != rb;
  }
  printf("%llu\n", bad);
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_group_step_division_is_correctly_rounded(tmp_path):
    src = tmp_path / "divchk.c"
    exe = tmp_path / "divchk"
    src.write_text(SRC)
    flags = ["-O2", "-ffp-contract=off"]
    # hardware fma where the host has it (glibc's fmaf is correctly rounded either way)
    if "fma" in open("/proc/cpuinfo").read() if os.path.exists("/proc/cpuinfo") else False:
        flags.append("-mfma")
    subprocess.run(["gcc", *flags, "-o", str(exe), str(src), "-lm"], check=True)
    procs = {L: subprocess.Popen([str(exe), L], stdout=subprocess.PIPE, text=True) for L in ("3", "15")}
    for L, p in procs.items():
        out, _ = p.communicate(timeout=600)
        assert p.returncode == 0
        assert int(out.strip()) == 0, "divisor %s: %s mismatches" % (L, out.strip())
