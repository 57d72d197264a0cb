// split_plan.h -- how the split plan cuts each slice's tokens into chunks for its passes
// (and the backward's token pass), and the workspace that follows from it.  The chunking
// decides the partials' traffic, so it is part of what the measured HBM bytes of the split
// workloads were taken for.
#pragma once
#include <algorithm>
#include <stddef.h>

#include "geometry.h"

namespace aa {

// The split plan of one call (bf16 or fp32) on num_cus compute units.  dual: the
// backward's pass 1 on V and dH in one launch, which fits one workgroup per CU.
inline SplitPlan split_plan(const Geometry& g, bool bf16, int num_cus, bool dual = false) {
  SplitPlan p{};
  const int n = g.n;
  // Pass 1: chunks a multiple of the 128-token block; about one workgroup per CU for the
  // token-split bf16 pass 1 (up to 128 anchors: fewer, longer chunks halve the partials
  // and measured faster) and for the eight-wave anchor-split one above 256 anchors (one
  // fits a CU), about two for the four-wave anchor-split one and for fp32 (one was slower
  // for both: long bf16 147.6 -> 165.9 us, long fp32 716 -> 755 us).
  const bool one_per_cu = bf16 && (g.at <= 8 || g.at >= 24 || dual);
  const long long want1 = (one_per_cu ? 1LL : 2LL) * num_cus;
  int max_chunks1 = (n + kPass1Block - 1) / kPass1Block;
  int c1 = (int)std::min<long long>(max_chunks1, std::max<long long>(1, (want1 + g.slices - 1) / g.slices));
  int len1 = (n + c1 - 1) / c1;
  len1 = (len1 + kPass1Block - 1) / kPass1Block * kPass1Block;
  p.chunk_len1 = len1;
  p.chunks1 = (n + len1 - 1) / len1;
  // Pass 2: chunks a multiple of the 64-token block; about four workgroups per CU, two for
  // the bf16 pass 2 with two 16-token tiles per step (129 to 256 anchors; long step 141.9
  // -> 139.5 us, while two made the dense step slower, 52.7 -> 53.9 us, and eight were
  // slower at both), one for the eight-wave passes 2 whose U and W fill the LDS (one fits a
  // CU): bf16 above 256 anchors, fp32 with more than 80 KB of them (long fp32 708 -> 695
  // us).
  const bool two_tile_pass2 = bf16 && g.d <= 64 && g.at > 8 && g.at <= 16;
  const bool wide_pass2 = bf16 ? g.at >= 24 : (long long)g.at * g.d * 128 > 80 * 1024;
  const long long want2 = (wide_pass2 ? 1LL : two_tile_pass2 ? 2LL : 4LL) * num_cus;
  int max_chunks2 = (n + kPass2Block - 1) / kPass2Block;
  int c2 = (int)std::min<long long>(max_chunks2, std::max<long long>(1, (want2 + g.slices - 1) / g.slices));
  int len2 = (n + c2 - 1) / c2;
  len2 = (len2 + kPass2Block - 1) / kPass2Block * kPass2Block;
  p.chunk_len2 = len2;
  p.chunks2 = (n + len2 - 1) / len2;
  const size_t es = bf16 ? 2 : 4;
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  p.part_bytes = al((size_t)g.slices * p.chunks1 * g.m_pad * g.d * sizeof(float));
  p.dpart_bytes = al((size_t)g.slices * p.chunks1 * g.m_pad * sizeof(float));
  p.w_bytes = al((size_t)g.slices * g.m_pad * g.d * es);
  // each token's log-sum-exp, passed from pass 1 to pass 2 above 128 anchors (bf16)
  p.lse_bytes = (bf16 && g.at > 8) ? al((size_t)g.slices * n * sizeof(float)) : 0;
  return p;
}

// The backward's token pass fits one workgroup per CU (its U and dP blocks, ~400
// registers): its chunks aim at one per CU and never outnumber pass 1's, for which the
// dS^T Q partials are sized.  Chunks are whole 128-token blocks.
inline void token_pass_chunks(const Geometry& g, const SplitPlan& p, int num_cus, int* chunks,
                              int* chunk_len) {
  const int maxc = (g.n + kPass1Block - 1) / kPass1Block;
  const int c = (int)std::min<long long>(
      std::min<long long>(maxc, p.chunks1),
      std::max<long long>(1, ((long long)num_cus + g.slices - 1) / g.slices));
  int len = (g.n + c - 1) / c;
  len = (len + kPass1Block - 1) / kPass1Block * kPass1Block;
  *chunk_len = len;
  *chunks = (g.n + len - 1) / len;
}

}  // namespace aa
