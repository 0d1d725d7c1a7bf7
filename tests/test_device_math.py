"""Host checks of device helpers that are plain arithmetic: the float64
sin/cos of a reduced angle used for the rotary phases (device_common.h) is
compiled for the CPU from its source text and compared with the C library
on a dense grid of [-pi, pi]."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "gqa_attention_kv_amd", "csrc", "device_common.h")

DRIVER = r"""
#include <cmath>
#include <cstdio>
using std::fma; using std::rint;
%s
int main() {
  double worst = 0.0;
  const long n = 1000000;
  for (long i = -n; i <= n; ++i) {
    const double x = M_PI * (double)i / (double)n;
    double s, c;
    sincos_pi_f64(x, &s, &c);
    worst = std::fmax(worst, std::fabs(s - std::sin(x)));
    worst = std::fmax(worst, std::fabs(c - std::cos(x)));
  }
  // the quadrant ends and the reduction boundaries exactly
  const double pts[] = {0.0, M_PI / 4, M_PI / 2, 3 * M_PI / 4, M_PI, -M_PI / 4, -M_PI / 2, -M_PI};
  for (double x : pts) {
    double s, c;
    sincos_pi_f64(x, &s, &c);
    worst = std::fmax(worst, std::fabs(s - std::sin(x)));
    worst = std::fmax(worst, std::fabs(c - std::cos(x)));
  }
  std::printf("%%.3e\n", worst);
  return 0;
}
"""


def test_sincos_pi_f64_matches_libm(tmp_path):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    src = open(HDR).read()
    m = re.search(r"__device__ __forceinline__ void sincos_pi_f64\(.*?\n}\n", src, re.S)
    assert m, "sincos_pi_f64 not found"
    body = m.group(0).replace("__device__ __forceinline__ ", "")
    c = tmp_path / "t.cpp"
    c.write_text(DRIVER % body)
    exe = tmp_path / "t"
    subprocess.run([cxx, "-O2", "-o", str(exe), str(c)], check=True)
    worst = float(subprocess.run([str(exe)], check=True, capture_output=True,
                                 text=True).stdout)
    assert worst <= 2.5e-16, worst
