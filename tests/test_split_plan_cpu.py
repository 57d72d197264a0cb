"""Host logic of the split plan's chunking (csrc/split_plan.h), compiled with g++ and run on
the CPU over a grid of shapes (forward and the backward's dual pass 1): every pass covers each slice's tokens with whole blocks and no
empty chunk, the backward's token pass never has more chunks than pass 1 (its dS^T Q
partials live in a buffer sized for pass 1's), and the workspace sections hold what the
kernels write."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "efficient_vision_transformer_amd", "csrc")

DRIVER = r"""
#include <cstdio>
#include "split_plan.h"
using namespace aa;
static int fail(const char* what, int n, long long slices, int at, int d, int bf16, int cus) {
  std::printf("FAIL %s n=%d slices=%lld at=%d d=%d bf16=%d cus=%d\n", what, n, slices, at, d, bf16, cus);
  return 1;
}
static bool covers(int n, int chunks, int len, int blk) {
  return chunks >= 1 && len % blk == 0 && len > 0 && (long long)chunks * len >= n &&
         (long long)(chunks - 1) * len < n;
}
int main() {
  const int ns[] = {1, 2, 31, 64, 127, 128, 129, 196, 255, 256, 577, 1000, 2051, 4096, 4099,
                    16384, 16385, 65536, 100003};
  const long long slicess[] = {1, 2, 3, 7, 32, 64, 100, 255, 256, 257, 384, 600, 1000, 4096};
  const int ats[] = {2, 4, 6, 8, 12, 16, 24, 32};
  const int ds[] = {32, 64, 128};
  const int cuss[] = {1, 80, 256, 304};
  long long checked = 0;
  for (int n : ns) for (long long sl : slicess) for (int at : ats) for (int d : ds)
  for (int bf16 = 0; bf16 < 2; ++bf16) for (int cus : cuss) for (int dual = 0; dual < 2; ++dual) {
    Geometry g{};
    g.n = n; g.d = d; g.at = at; g.m_pad = 16 * at; g.m = g.m_pad; g.slices = sl;
    g.B = (int)sl; g.h = 1;
    const SplitPlan p = split_plan(g, bf16 != 0, cus, dual != 0);
    if (!covers(n, p.chunks1, p.chunk_len1, kPass1Block)) return fail("pass 1 chunks", n, sl, at, d, bf16, cus);
    if (!covers(n, p.chunks2, p.chunk_len2, kPass2Block)) return fail("pass 2 chunks", n, sl, at, d, bf16, cus);
    if (sl * p.chunks1 > 0x7fffffffLL || sl * p.chunks2 > 0x7fffffffLL) return fail("grid", n, sl, at, d, bf16, cus);
    const size_t part = (size_t)sl * p.chunks1 * g.m_pad * d * sizeof(float);
    const size_t dpart = (size_t)sl * p.chunks1 * g.m_pad * sizeof(float);
    const size_t w = (size_t)sl * g.m_pad * d * (bf16 ? 2 : 4);
    if (p.part_bytes < part || p.dpart_bytes < dpart || p.w_bytes < w) return fail("workspace", n, sl, at, d, bf16, cus);
    if (p.part_bytes % 256 || p.dpart_bytes % 256 || p.w_bytes % 256 || p.lse_bytes % 256)
      return fail("alignment", n, sl, at, d, bf16, cus);
    const bool lse = bf16 && at > 8;
    if (lse != (p.lse_bytes > 0) || (lse && p.lse_bytes < (size_t)sl * n * sizeof(float)))
      return fail("lse", n, sl, at, d, bf16, cus);
    if (p.workspace_bytes() != p.part_bytes + p.dpart_bytes + p.w_bytes + p.lse_bytes)
      return fail("workspace sum", n, sl, at, d, bf16, cus);
    int ct = 0, lt = 0;
    token_pass_chunks(g, p, cus, &ct, &lt);
    if (!covers(n, ct, lt, kPass1Block) || ct > p.chunks1) return fail("token pass chunks", n, sl, at, d, bf16, cus);
    ++checked;
  }
  std::printf("OK %lld\n", checked);
  return 0;
}
"""


def test_split_plan_chunking_invariants(tmp_path):
    src = tmp_path / "plan_check.cpp"
    src.write_text(DRIVER)
    exe = tmp_path / "plan_check"
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-Werror", "-I", CSRC, str(src), "-o", str(exe)],
                   check=True, capture_output=True, text=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    print(out.stdout)
    assert out.returncode == 0 and out.stdout.startswith("OK"), out.stdout + out.stderr
