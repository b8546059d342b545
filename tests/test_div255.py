"""The quantizer forms its scale (hi - lo) / 255 as x * RN(1/255) plus one FMA
correction instead of an IEEE division.  This test recompiles that sequence
on the host and checks it against the IEEE quotient for every non-negative
finite fp32 x (2^31 - 2^23 values, denormals included), so the scales stay
bit-identical to the oracle's division.  About half a minute of CPU.
"""
import os
import shutil
import subprocess

import pytest

SRC = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
int main(void) {
  const float r = 1.0f / 255.0f;
  unsigned long long bad = 0;
  for (uint32_t u = 0; u < 0x7F800000u; ++u) {
    float x; memcpy(&x, &u, 4);
    volatile float d = 255.0f;
    const float ref = x / d;
    const float q0 = x * r;
    const float e = fmaf(-q0, 255.0f, x);
    const float q1 = fmaf(e, r, q0);
    uint32_t a, b; memcpy(&a, &q1, 4); memcpy(&b, &ref, 4);
    bad += a != b;
  }
  printf("%llu\n", bad);
  return 0;
}
"""


@pytest.mark.slow
@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_scale_division_by_255_is_exact_for_every_float(tmp_path):
    c, exe = tmp_path / "div255.c", tmp_path / "div255"
    c.write_text(SRC)
    # -ffp-contract=off: the product and the FMAs exactly as written
    subprocess.run(["gcc", "-O2", "-mfma", "-ffp-contract=off", "-o", str(exe), str(c), "-lm"], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True, timeout=600).stdout
    assert out.strip() == "0"
