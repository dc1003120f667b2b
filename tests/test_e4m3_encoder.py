"""The library's FP8 E4M3 encoder (rowquant.h, compiled for the host) against
the oracle's moe_oracle_f32_to_e4m3 on every one of the 2^32 fp32 bit
patterns: the codes of the FP4-weight variant's quantisers are then the
oracle's for any input the quantisers can meet (the GPU tests check the
same codes on the device, where the encoder is the same source)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

HARNESS = r"""
#include "rowquant.h"
#include <cstdio>
#include <cstring>
#include <thread>
#include <vector>
extern "C" uint8_t moe_oracle_f32_to_e4m3(float f);
int main() {
  const int nt = 8;
  std::vector<unsigned long long> bad(nt, 0);
  std::vector<uint32_t> first(nt, 0);
  std::vector<std::thread> th;
  for (int t = 0; t < nt; ++t)
    th.emplace_back([&, t] {
      for (uint64_t b = t; b < (1ull << 32); b += nt) {
        const uint32_t u = static_cast<uint32_t>(b);
        float f;
        memcpy(&f, &u, 4);
        if (moe::e4m3_code(f) != moe_oracle_f32_to_e4m3(f)) {
          if (!bad[t]) first[t] = u;
          ++bad[t];
        }
      }
    });
  for (auto &x : th) x.join();
  unsigned long long total = 0;
  for (int t = 0; t < nt; ++t) {
    total += bad[t];
    if (bad[t]) printf("mismatch at fp32 bits %08x\n", first[t]);
  }
  printf("mismatches %llu\n", total);
  return total != 0;
}
"""


@pytest.mark.skipif(not os.path.exists(HIPCC) or shutil.which("gcc") is None, reason="needs hipcc and gcc")
def test_device_e4m3_encoder_matches_oracle_on_every_fp32(tmp_path):
    src = tmp_path / "e4m3_all.hip"
    src.write_text(HARNESS)
    o1, o2, exe = tmp_path / "oracle.o", tmp_path / "h.o", tmp_path / "e4m3_all"
    subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-c",
                           os.path.join(ROOT, "oracle", "moe_oracle.c"), "-o", str(o1)])
    subprocess.check_call([HIPCC, "-O2", "-std=c++17", "-ffp-contract=off", "-I",
                           os.path.join(ROOT, "moe_expert_ffn_route_amd", "csrc"), "-I",
                           os.path.join(ROOT, "include"), "-c", str(src), "-o", str(o2)],
                          stderr=subprocess.DEVNULL)
    subprocess.check_call([HIPCC, str(o2), str(o1), "-o", str(exe), "-lpthread", "-lm"])
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout
