"""The kernels split item and row indices by a multiply-high with constants
from the host's make_fastdiv (csrc/bc_internal.h; Granlund and Montgomery
1994, division by invariant integers using multiplication).  A host program
built against that header takes its constants for every divisor from 1 to
4096 and applies the kernels' 32-bit arithmetic, (umulhi(n, mul) + n) >>
shift with the sum kept in 32 bits, and compares with integer division:
every n below 65536, the multiples of d and their neighbours across the
whole range the kernels use (0 <= n < 2^31), and the top of that range.
Runs on the CPU (the device function's arithmetic is mirrored; the
constants are the library's own)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_causal_attention_gqa_amd", "csrc")

PROGRAM = r"""
#include "bc_internal.h"
#include <cstdio>
#include <cstdint>

static inline uint32_t kernel_div(uint32_t n, bc::FastDiv f) {
  const uint32_t hi = (uint32_t)(((uint64_t)n * f.mul) >> 32);
  return (uint32_t)(hi + n) >> f.shift;   // 32-bit sum, as on the device
}

int main() {
  long long checked = 0;
  for (uint32_t d = 1; d <= 4096; ++d) {
    const bc::FastDiv f = bc::make_fastdiv(d);
    auto check = [&](uint32_t n) -> bool {
      ++checked;
      if (kernel_div(n, f) != n / d) {
        std::printf("MISMATCH d=%u n=%u got=%u want=%u\n", d, n, kernel_div(n, f), n / d);
        return false;
      }
      return true;
    };
    for (uint32_t n = 0; n < 65536; ++n)
      if (!check(n)) return 1;
    const uint32_t top = 0x7fffffffu;
    const uint32_t kmax = top / d;
    const uint32_t stride = kmax / 4000 + 1;
    for (uint32_t k = 1; k <= kmax; k += stride) {
      const uint32_t m = k * d;
      if (!check(m - 1) || !check(m) || (m + 1 <= top && !check(m + 1))) return 1;
    }
    for (uint32_t j = 0; j < 64; ++j)
      if (!check(top - j)) return 1;
    if (!check(kmax * d) || !check(kmax * d - 1)) return 1;
  }
  std::printf("ok %lld\n", checked);
  return 0;
}
"""


def test_fastdiv_constants_divide_exactly(tmp_path):
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    if not os.path.exists(hipcc):
        hipcc = shutil.which("hipcc")
    if hipcc is None:
        pytest.skip("hipcc unavailable")
    src = tmp_path / "fastdiv.cpp"
    src.write_text(PROGRAM)
    exe = tmp_path / "fastdiv"
    r = subprocess.run([hipcc, "-std=c++17", "-O2", "--offload-arch=gfx950", "-x", "hip",
                        "-I", os.path.join(ROOT, "include"), "-I", CSRC, str(src), "-o", str(exe)],
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout
    r = subprocess.run([str(exe)], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=300)
    assert r.returncode == 0, r.stdout
    assert r.stdout.startswith("ok ")
