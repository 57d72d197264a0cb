// tile_ops.h -- bf16 tile building blocks shared by the fused kernel and the split pass 1:
// selection operands, the transposed-logits softmax of one 16-token tile, and streaming
// row loads in MFMA operand layout.
#pragma once
#include "device_common.h"

namespace aa {

// bf16 0/1 selection operands (8 slots, two per dword; bf16 1.0 = 0x3F80), built in
// registers.  A transpose, output anchor half `half`: slot s is 1 iff it holds anchor c,
// i.e. s - 4*half == c - 4g.  V transpose, output dim group p: slot c&7 is 1 iff
// g == 2p + (c >> 3).  (Same matrices as asel_operand / vsel_operand.)
__device__ __forceinline__ bf16x8 sel_slot(bool hit, int slot) {
  const unsigned val = (slot & 1) ? 0x3F800000u : 0x00003F80u;
  const int dw = slot >> 1;
  u32x4 r;
#pragma unroll
  for (int k = 0; k < 4; ++k) r[k] = (hit && dw == k) ? val : 0u;
  return as_bf16x8(r);
}
__device__ __forceinline__ bf16x8 sel_a(int half, int c, int g) {
  const int idx = c - 4 * g;
  return sel_slot((unsigned)idx < 4u, 4 * half + (idx & 3));
}
__device__ __forceinline__ bf16x8 sel_v(int p, int c, int g) {
  return sel_slot(g == 2 * p + (c >> 3), c & 7);
}

// Logits and softmax for one 16-token tile, transposed: returns A as the right operand
// of H^T = W^T A^T, ab[jj] = anchors {32jj + 4g + s, 32jj + 16 + 4g + s - 4} of token c.
template <int D, int MP>
__device__ __forceinline__ void tile_softmax(const u32x4 (*u_lds)[D / 32][kWave], const u32x4* q,
                                             int lane, int g, int m, bool token_ok, float c2,
                                             bf16x8* ab) {
  constexpr int KS = D / 32, AT = 2 * MP;
  f32x4 s[AT];
#pragma unroll
  for (int j = 0; j < AT; ++j) {
    f32x4 acc = zero4();
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) acc = mfma_bf16(as_bf16x8(u_lds[j][kk][lane]), as_bf16x8(q[kk]), acc);
    // padded anchors (>= m) exist only in the last 32 when m is not a multiple of 32
    if (j >= AT - 2 && m < 32 * MP) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (16 * j + 4 * g + r >= m) acc[r] = -INFINITY;
    }
    s[j] = acc;
  }
  float mx = s[0][0];
#pragma unroll
  for (int j = 0; j < AT; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[j][r]);
  mx = xor32_max(xor16_max(mx));
  const float mneg = -mx * c2;
  float z = 0.f;
#pragma unroll
  for (int j = 0; j < AT; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float e = exp2_fast(fmaf(s[j][r], c2, mneg));
      s[j][r] = e;
      z += e;
    }
  z = xor32_sum(xor16_sum(z));
  const float inv = token_ok ? 1.f / z : 0.f;
#pragma unroll
  for (int jj = 0; jj < MP; ++jj) ab[jj] = pack_bf16(s[2 * jj] * inv, s[2 * jj + 1] * inv);
}

// Loads rows of Q or V in operand layout (lane (c,g): dims 8*KS*g ..), streaming (each
// byte is read once, so the loads are marked non-temporal).  Rows past the
// slice's end read its last row instead; their softmax weights are zeroed, so they add
// nothing (and a non-finite value there belongs to the same slice anyway).
template <int D>
__device__ __forceinline__ void load_rows(const __bf16* __restrict__ X, size_t base, int row, int n,
                                          int g, u32x4* out) {
  constexpr int KS = D / 32;
  const size_t off = base + (size_t)min(row, n - 1) * D + 8 * KS * g;
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) out[kk] = __builtin_nontemporal_load((const u32x4*)(X + off + 8 * kk));
}

}  // namespace aa
