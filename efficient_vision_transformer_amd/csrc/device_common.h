// device_common.h -- CDNA4 (gfx950) building blocks shared by the anchor-attention kernels.
//
// MFMA lane layouts used throughout (wave64, lane = 16*g + c, c in [0,16), g in [0,4)):
//   v_mfma_f32_16x16x32_bf16:  X operand (A-matrix, M x K): lane holds X[M=c][K=8g+s], s<8
//                              Y operand (B-matrix, K x N): lane holds Y[K=8g+s][N=c]
//                              accumulator:                 lane holds D[M=4g+r][N=c], r<4
//   v_mfma_f32_16x16x4_f32:    X: X[M=c][K=g]; Y: Y[K=g][N=c]; accumulator as above.
// Because K is a contraction index, any fixed relabelling of K that both operands share
// leaves the product unchanged; the kernels use that freedom to keep contiguous memory
// per lane.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace aa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(unsigned)))) unsigned u32x2;

constexpr int kWave = 64;

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 x, bf16x8 y, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, y, acc, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32(float x, float y, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(x, y, acc, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ u32x4 as_u32x4(bf16x8 v) { return __builtin_bit_cast(u32x4, v); }

// Round-to-nearest-even conversion of two accumulators into one 8 x bf16 operand.
__device__ __forceinline__ bf16x8 pack_bf16(f32x4 lo, f32x4 hi) {
  bf16x8 r;
  r[0] = (__bf16)lo[0]; r[1] = (__bf16)lo[1]; r[2] = (__bf16)lo[2]; r[3] = (__bf16)lo[3];
  r[4] = (__bf16)hi[0]; r[5] = (__bf16)hi[1]; r[6] = (__bf16)hi[2]; r[7] = (__bf16)hi[3];
  return r;
}

// Round-to-nearest-even conversion of one accumulator into four packed bf16.
__device__ __forceinline__ u32x2 pack4_bf16(f32x4 a) {
  typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
  const bf16x4 r = {(__bf16)a[0], (__bf16)a[1], (__bf16)a[2], (__bf16)a[3]};
  return __builtin_bit_cast(u32x2, r);
}

__device__ __forceinline__ bf16x8 splat_bf16(float v) {
  const __bf16 b = (__bf16)v;
  return bf16x8{b, b, b, b, b, b, b, b};
}

// ---- staging global memory into LDS ----------------------------------------------------
// A loop "for (i = tid; i < N; i += T) lds[i] = src(i)" waits for each pass's load before
// its LDS write: one memory round trip per pass.  Stage holds a thread's share of N
// 16-byte chunks so that every load is issued first (stage_load) and LDS is written
// afterwards (stage_store).  The block must have exactly T threads.
template <int N, int T>
struct Stage {
  static constexpr int kPer = (N + T - 1) / T;
  u32x4 r[kPer];
};

template <int N, int T, typename F>
__device__ __forceinline__ void stage_load(Stage<N, T>& s, F src) {
#pragma unroll
  for (int i = 0; i < Stage<N, T>::kPer; ++i) {
    const int idx = (int)threadIdx.x + i * T;
    if (N % T == 0 || idx < N) s.r[i] = src(idx);
  }
}

template <int N, int T>
__device__ __forceinline__ void stage_store(const Stage<N, T>& s, u32x4* dst) {
#pragma unroll
  for (int i = 0; i < Stage<N, T>::kPer; ++i) {
    const int idx = (int)threadIdx.x + i * T;
    if (N % T == 0 || idx < N) dst[idx] = s.r[i];
  }
}

// ---- cross-lane reductions ------------------------------------------------------------
// Over the 16 lanes of one DPP row (lanes with the same g): butterfly with quad
// permutations and the two row mirrors; every lane of the row ends with the same value.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp_f<0xB1>(x));   // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp_f<0x4E>(x));   // quad_perm [2,3,0,1]
  x = fmaxf(x, dpp_f<0x141>(x));  // row_half_mirror
  x = fmaxf(x, dpp_f<0x140>(x));  // row_mirror
  return x;
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_f<0xB1>(x);
  x += dpp_f<0x4E>(x);
  x += dpp_f<0x141>(x);
  x += dpp_f<0x140>(x);
  return x;
}

// Across the four lane groups g (lanes c, c+16, c+32, c+48) with the gfx950 permlane
// swaps: permlane16_swap(v, v) hands each lane {v[l], v[l^16]}, permlane32_swap
// {v[l], v[l^32]} (in some order), so a commutative op of the pair is symmetric.
__device__ __forceinline__ float xor16_max(float v) {
  auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float xor32_max(float v) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float xor16_sum(float v) {
  auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float xor32_sum(float v) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- tensor views (View: element strides of a [B, h, n, d] view, see kernels.h) ---------
__device__ __forceinline__ size_t view_base(const View& w, int slice, int h) {
  const int b = slice / h, hd = slice - b * h;
  return (size_t)((long long)b * w.sb + (long long)hd * w.sh);
}
__device__ __forceinline__ size_t view_row(const View& w, int row) {
  return (size_t)((long long)row * w.st);
}

// ---- padded anchors ----------------------------------------------------------------------
// m is rounded up to a multiple of 32 (m <= 128) or 64 (m > 128), so padded anchors (index
// >= m) occupy at most the last pad_tiles(AT) 16-anchor tiles.
__host__ __device__ constexpr int pad_tiles(int at) { return at > 8 ? 4 : 2; }

// mask[hh] is the initial logits accumulator of anchor tile AT - NPAD + hh, accumulator rows
// 4g + r: -inf on padded anchors, 0 elsewhere.  The padded U rows are finite, so those
// logits stay -inf and drop out of the softmax without any per-element select.
template <int AT, int NPAD>
__device__ __forceinline__ void pad_mask_tiles(int g, int m, f32x4* mask) {
#pragma unroll
  for (int hh = 0; hh < NPAD; ++hh)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      mask[hh][r] = (16 * (AT - NPAD + hh) + 4 * g + r < m) ? 0.f : -INFINITY;
}

}  // namespace aa
