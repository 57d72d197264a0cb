// linear_bf16.hip -- ReLU kernel linear attention (L2ViT page, the decomposable kernel
// identity of its Eq. (4) with phi = ReLU and the denominator clamped below at Cmin), bf16
// in and out, fp32 accumulation:
//   S = phi(K)^T V (d x d),  z = phi(K)^T 1,
//   out_i = phi(q_i) S / max(phi(q_i) . z, cmin)
// (the caller's query scale a > 0 enters as cmin / a, since phi(a q) = a phi(q)).
// One workgroup per (batch, head) slice reads Q, K and V once and writes the output once;
// with few slices a split plan spreads each slice over workgroups (pass 1: partial S and z
// per token chunk; finalize: chunk sums in chunk order as operands; pass 2: phase 3 per
// chunk).
//   Phase 1 (rounds of one 32-token pair per wave): rows of phi(K) and V go to LDS as
//     they are; each wave accumulates its (16-dim, 16-dim) tiles of S, and z with its dim
//     tile 0, through transposing LDS reads (the same tile accumulation as A^T V).
//   Phase 2: S rounded to bf16 as the left operands of out^T = S^T phi(Q)^T, z in LDS.
//   Phase 3 (rounds again): phi(Q) in operand layout, the products on the MFMA, the
//     denominator on the VALU plus two permlane swaps, the clamp, 64-byte row stores.
#include <algorithm>

#include "device_common.h"
#include "kernels.h"
#include "tile_ops.h"

namespace aa {

// LDS of one workgroup that handles the DW output dims from d0 of a slice (DW = D, or
// D / 2 when two workgroups share the slice).
template <int D, int NW, int DW = D>
struct LinLds {
  static constexpr int KS = D / 32, DTW = DW / 16;
  static constexpr int KSTR = tr_stride<D>(), VS = tr_stride<DW>();
  __attribute__((aligned(16))) __bf16 k[NW * 32 * KSTR];  // rows of phi(K), this round
  __attribute__((aligned(16))) __bf16 v[NW * 32 * VS];    // rows of V (DW dims), this round
  u32x4 s[DTW][KS][kWave];                                // S^T left operands
  __attribute__((aligned(16))) float z[D];
};

// ReLU of eight packed bf16: clears every half-word whose sign bit is set.
__device__ __forceinline__ u32x4 relu_bf16x8(u32x4 x) {
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] &= ~(((x[i] >> 15) & 0x00010001u) * 0xFFFFu);
  return x;
}

// Phase 1 over tokens [t0, t1) of a slice: S and z tiles of this wave accumulated in
// pacc / dacc (tile t = w*TPW + k: input-dim tile t / DTW, rows 16ja + 4g + r; output-dim
// tile t % DTW, dim d0 + 16dt + c; z of an input tile with its output tile 0).
template <int D, int NW, int DW>
__device__ __forceinline__ void lin_reduce(LinLds<D, NW, DW>& L, const __bf16* __restrict__ K,
                                           const __bf16* __restrict__ V, size_t kb, long long ks,
                                           size_t vb, long long vs, int t0, int t1, int n,
                                           int d0, f32x4* pacc, f32x4* dacc) {
  constexpr int DT = D / 16, KS = D / 32, KV = DW / 32, DTW = DW / 16;
  constexpr int KSTR = LinLds<D, NW, DW>::KSTR, VS = LinLds<D, NW, DW>::VS;
  constexpr int TPW = DT * DTW / NW;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, g = lane >> 4;
  const int npairs = (t1 - t0 + 31) >> 5;
  const int rounds = (npairs + NW - 1) / NW;
  const bf16x8 ones = splat_bf16(1.f);
  u32x4 kc[2][KS], vc[2][KV];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    load_rows_c<D, D>(K, kb, ks, t0 + 32 * w + 16 * tt + c, n, g, 0, kc[tt]);
    load_rows_c<D, DW>(V, vb, vs, t0 + 32 * w + 16 * tt + c, n, g, d0, vc[tt]);
  }
  for (int r = 0; r < rounds; ++r) {
    const int pairs_here = min(NW, npairs - r * NW);  // uniform over the workgroup
    const int p = r * NW + w;
    // the next round's rows, requested unconditionally (rows past the range read its last
    // row and are never used): a load under a branch would turn the wait for this round's
    // rows at the join into a wait for everything
    u32x4 kn[2][KS], vn[2][KV];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int row = min(t0 + 32 * (p + NW) + 16 * tt + c, t1 - 1);
      load_rows_c<D, D>(K, kb, ks, row, n, g, 0, kn[tt]);
      load_rows_c<D, DW>(V, vb, vs, row, n, g, d0, vn[tt]);
    }
    if (p < npairs) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        // Rows past the range hold other tokens (or the last row again): their keys are
        // zeroed, so they add nothing to S or z.
        const bool ok = t0 + 32 * p + 16 * tt + c < t1;
        __bf16* krow = L.k + (32 * w + 16 * tt + c) * KSTR + 8 * g;
        __bf16* vrow = L.v + (32 * w + 16 * tt + c) * VS + 8 * g;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
          *(u32x4*)(krow + 32 * kk) = ok ? relu_bf16x8(kc[tt][kk]) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int kk = 0; kk < KV; ++kk) *(u32x4*)(vrow + 32 * kk) = vc[tt][kk];
      }
    }
    __syncthreads();
    accumulate_tiles<TPW, DTW, KSTR, VS, true>(L.k, L.v, w * TPW, pairs_here, c, g, ones, pacc, dacc);
    __syncthreads();
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) kc[tt][kk] = kn[tt][kk];
#pragma unroll
      for (int kk = 0; kk < KV; ++kk) vc[tt][kk] = vn[tt][kk];
    }
  }
}

// Element of the S^T operand block [DT][KS][lane][8] holding S[in][out]: lane (c', g') of
// [dt2][kk] holds output dim out_dim_c(dt2, c') and input dims 32kk + 8g' .. + 7 (the
// layout of phi(Q)'s chunks).
template <int D>
__device__ __forceinline__ int sop_pos(int in, int out) {
  constexpr int KS = D / 32;
  const int q = out & 31, dt2 = 2 * (out >> 5) + ((q & 7) >> 2), cc = 4 * (q >> 3) + (q & 3);
  return (((dt2 * KS + (in >> 5)) * kWave) + 16 * ((in >> 3) & 3) + cc) * 8 + (in & 7);
}

// Phase 3 over tokens [t0, t1): out = phi(Q) S / max(phi(Q) z, cmin) with S^T operands and
// z in LDS.  Waves work independently (no barrier).
// Output dims d0 .. d0 + DW - 1.  q_first, when given, holds this wave's first pair of Q
// rows, loaded by the caller.
template <int D, int NW, int DW = D>
__device__ __forceinline__ void lin_apply(const u32x4 (*sop)[D / 32][kWave], const float* zl,
                                          const __bf16* __restrict__ Q, size_t qb, long long qs,
                                          __bf16* __restrict__ O, size_t ob, const View& ow,
                                          int t0, int t1, int n, float cmin,
                                          const u32x4 (*q_first)[D / 32] = nullptr, int d0 = 0) {
  constexpr int DT = DW / 16, KS = D / 32;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, g = lane >> 4;
  const int npairs = (t1 - t0 + 31) >> 5;
  float zr[KS][8];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk)
#pragma unroll
    for (int s = 0; s < 8; ++s) zr[kk][s] = zl[32 * kk + 8 * g + s];
  u32x4 qc[2][KS];
  if (q_first) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) qc[tt][kk] = q_first[tt][kk];
  } else {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) load_rows_c<D, D>(Q, qb, qs, t0 + 32 * w + 16 * tt + c, n, g, 0, qc[tt]);
  }
  for (int p = w; p < npairs; p += NW) {
    u32x4 qn[2][KS];   // next pair's rows, unconditionally (see lin_reduce)
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
      load_rows_c<D, D>(Q, qb, qs, min(t0 + 32 * (p + NW) + 16 * tt + c, t1 - 1), n, g, 0, qn[tt]);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int row = t0 + 32 * p + 16 * tt + c;
      bf16x8 pq[KS];
      float part = 0.f;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        pq[kk] = as_bf16x8(relu_bf16x8(qc[tt][kk]));
#pragma unroll
        for (int s = 0; s < 8; ++s) part = fmaf((float)pq[kk][s], zr[kk][s], part);
      }
      const float den = xor32_sum(xor16_sum(part));
      const float inv = 1.f / fmaxf(den, cmin);
      f32x4 acc[DT];
#pragma unroll
      for (int dt2 = 0; dt2 < DT; ++dt2) {
        f32x4 a = zero4();
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) a = mfma_bf16(as_bf16x8(sop[dt2][kk][lane]), pq[kk], a);
        acc[dt2] = a * inv;
      }
      if (row < t1) {
        __bf16* dst = O + ob + view_row(ow, row) + d0 + 8 * g;
#pragma unroll
        for (int hh = 0; hh < DT / 2; ++hh)
          __builtin_nontemporal_store(as_u32x4(pack_bf16(acc[2 * hh], acc[2 * hh + 1])),
                                      (u32x4*)(dst + 32 * hh));
      }
    }
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) qc[tt][kk] = qn[tt][kk];
  }
}

// One workgroup's share of a slice: all tokens, output dims d0 .. d0 + DW - 1.  Reduce
// over all tokens, S to operands, apply to all tokens.
template <int D, int NW, int DW>
__device__ __forceinline__ void lin_fused_part(LinLds<D, NW, DW>& L, const __bf16* __restrict__ Q,
                                               const __bf16* __restrict__ K,
                                               const __bf16* __restrict__ V, __bf16* __restrict__ O,
                                               const View& qw, const View& kw, const View& vw,
                                               const View& ow, int slice, int d0, int h, int n,
                                               float cmin) {
  constexpr int DT = D / 16, DTW = DW / 16, KS = D / 32;
  constexpr int TILES = DT * DTW, TPW = TILES / NW;
  static_assert(TILES % NW == 0 && TPW >= 1, "tiles split evenly over the waves");
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, g = lane >> 4;
  // The first Q rows go out together with K and V, so their latency is hidden behind the
  // reduction.
  const size_t qb = view_base(qw, slice, h);
  u32x4 q0[2][KS];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) load_rows_c<D, D>(Q, qb, qw.st, 32 * w + 16 * tt + c, n, g, 0, q0[tt]);
  f32x4 pacc[TPW], dacc[TPW];
#pragma unroll
  for (int k = 0; k < TPW; ++k) { pacc[k] = zero4(); dacc[k] = zero4(); }
  lin_reduce<D, NW, DW>(L, K, V, view_base(kw, slice, h), kw.st, view_base(vw, slice, h), vw.st,
                        0, n, n, d0, pacc, dacc);
  __bf16* so = (__bf16*)&L.s[0][0][0];
#pragma unroll
  for (int k = 0; k < TPW; ++k) {
    const int t = w * TPW + k, ja = t / DTW, dt = t - (t / DTW) * DTW;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int in = 16 * ja + 4 * g + r;
      so[sop_pos<D>(in, 16 * dt + c)] = (__bf16)pacc[k][r];
      if (dt == 0 && c == 0) L.z[in] = dacc[k / DTW][r];
    }
  }
  __syncthreads();
  lin_apply<D, NW, DW>(L.s, L.z, Q, qb, qw.st, O, view_base(ow, slice, h), ow, 0, n, n, cmin,
                       q0, d0);
}

// Workgroups 0 .. full - 1 take slices 0 .. full - 1 whole; with d = 64 the remaining
// slices are shared by two workgroups, one per half of the output dims (both compute z
// and read all of Q and K; each reads half of V and writes half of the output), so that a
// grid with between one and two slices per CU gives every CU about the same work.  At
// d = 128 every slice is shared (full == 0): a whole slice's S tiles, V rows and S
// operands would take more registers and LDS than one workgroup has.  Ids i and i + 8 of
// each run of 16 shared workgroups take the two halves of one slice (the same XCD, so the
// second reads of Q and K can hit its L2).
template <int D, int NW>
__global__ __launch_bounds__(NW * kWave, 2)
void relu_linear_bf16(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                      const __bf16* __restrict__ V, __bf16* __restrict__ O, View qw, View kw,
                      View vw, View ow, int h, int n, float cmin, int full) {
  __shared__ LinLds<D, NW, D == 128 ? D / 2 : D> L;
  const int b = blockIdx.x;
  if (b < full) {
    if constexpr (D != 128) lin_fused_part<D, NW, D>(L, Q, K, V, O, qw, kw, vw, ow, b, 0, h, n, cmin);
  } else if constexpr (D >= 64) {
    const int k = b - full;
    const int nsh = (int)(gridDim.x - full);
    int sl, hf;
    if ((k | 15) < (nsh & ~15)) {
      sl = ((k >> 4) << 3) + (k & 7);
      hf = (k >> 3) & 1;
    } else {
      sl = k >> 1;
      hf = k & 1;
    }
    static_assert(sizeof(LinLds<D, NW, D / 2>) <= sizeof(L), "half fits");
    lin_fused_part<D, NW, D / 2>(*reinterpret_cast<LinLds<D, NW, D / 2>*>(&L), Q, K, V, O, qw, kw,
                                 vw, ow, full + sl, hf * (D / 2), h, n, cmin);
  }
}

// Split plan, pass 1: per (slice, chunk) partial S tiles [slice][chunk][t][4][64] (tile t:
// input-dim tile t / DT, output-dim tile t % DT) and z [slice][chunk][D].  At d = 128 two
// workgroups take each chunk, one per half of the output dims (a whole chunk's tiles would
// take more registers and LDS than one workgroup has); the first of them writes z.
template <int D, int NW>
__global__ __launch_bounds__(NW * kWave, 2)
void relu_linear_pass1(const __bf16* __restrict__ K, const __bf16* __restrict__ V, View kw,
                       View vw, float* __restrict__ part, float* __restrict__ zpart, int h,
                       int n, int chunks, int chunk_len) {
  constexpr int HALVES = D == 128 ? 2 : 1, DW = D / HALVES;
  using L_t = LinLds<D, NW, DW>;
  constexpr int DT = D / 16, DTW = DW / 16, TILES = DT * DT, TPW = DT * DTW / NW;
  __shared__ L_t L;
  const int hf = blockIdx.x % HALVES, bc = blockIdx.x / HALVES;
  const int slice = bc / chunks, chunk = bc - slice * chunks;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, g = lane >> 4;
  const int t0 = chunk * chunk_len, t1 = min(n, t0 + chunk_len);
  f32x4 pacc[TPW], dacc[TPW];
#pragma unroll
  for (int k = 0; k < TPW; ++k) { pacc[k] = zero4(); dacc[k] = zero4(); }
  lin_reduce<D, NW, DW>(L, K, V, view_base(kw, slice, h), kw.st, view_base(vw, slice, h), vw.st,
                        t0, t1, n, hf * DW, pacc, dacc);
  const size_t sc = (size_t)slice * chunks + chunk;
#pragma unroll
  for (int k = 0; k < TPW; ++k) {
    const int tl = w * TPW + k, ja = tl / DTW, dt = hf * DTW + tl - (tl / DTW) * DTW;
    const int t = ja * DT + dt;
    float* dst = part + (sc * TILES + t) * 256;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      dst[r * 64 + lane] = pacc[k][r];
      if (dt == 0 && c == 0) zpart[sc * D + 16 * ja + 4 * g + r] = dacc[k / DTW][r];
    }
  }
}

// Split plan, finalize: chunk sums in chunk order, S as bf16 operands
// [slice][DT][KS][64] x 16 B and z [slice][D].  Workgroup (slice, group): wave w sums
// tile 4 * group + w; group 0 also sums z.
template <int D>
__global__ __launch_bounds__(256)
void relu_linear_finalize(const float* __restrict__ part, const float* __restrict__ zpart,
                          __bf16* __restrict__ sops, float* __restrict__ zs, int chunks) {
  constexpr int DT = D / 16, TILES = DT * DT, GROUPS = (TILES + 3) / 4;
  const int slice = blockIdx.x / GROUPS, grp = blockIdx.x - slice * GROUPS;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int t = 4 * grp + w;
  if (t < TILES) {
    const int ja = t / DT, dt = t - (t / DT) * DT;
    f32x4 acc = zero4();
    constexpr int U = 8;   // loads of U chunks in flight, then the adds in chunk order
    for (int ch0 = 0; ch0 < chunks; ch0 += U) {
      f32x4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int ch = min(ch0 + u, chunks - 1);
        const float* src = part + (((size_t)slice * chunks + ch) * TILES + t) * 256 + lane;
        v[u] = f32x4{src[0], src[64], src[128], src[192]};
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (ch0 + u < chunks) acc += v[u];
    }
    __bf16* so = sops + (size_t)slice * D * D;
#pragma unroll
    for (int r = 0; r < 4; ++r) so[sop_pos<D>(16 * ja + 4 * g + r, 16 * dt + c)] = (__bf16)acc[r];
  }
  if (grp == 0) {
    for (int i = threadIdx.x; i < D; i += 256) {
      float z = 0.f;
      for (int ch = 0; ch < chunks; ++ch) z += zpart[((size_t)slice * chunks + ch) * D + i];
      zs[(size_t)slice * D + i] = z;
    }
  }
}

// Split plan, pass 2: per (slice, chunk), the slice's operands to LDS, then phase 3.  At
// d = 128 two workgroups take each chunk, one per half of the output dims (operand blocks
// dt2 of that half; the whole would spill registers).
template <int D, int NW>
__global__ __launch_bounds__(NW * kWave, D == 128 ? 2 : 4)
void relu_linear_pass2(const __bf16* __restrict__ Q, __bf16* __restrict__ O, View qw, View ow,
                       const u32x4* __restrict__ sops, const float* __restrict__ zs, int h, int n,
                       int chunks, int chunk_len, float cmin) {
  constexpr int HALVES = D == 128 ? 2 : 1, DW = D / HALVES;
  constexpr int DT = D / 16, DTW = DW / 16, KS = D / 32;
  __shared__ u32x4 s_lds[DTW][KS][kWave];
  __shared__ __attribute__((aligned(16))) float z_lds[D];
  const int hf = blockIdx.x % HALVES, bc = blockIdx.x / HALVES;
  const int slice = bc / chunks, chunk = bc - slice * chunks;
  const u32x4* src = sops + ((size_t)slice * DT + hf * DTW) * KS * kWave;
  for (int i = threadIdx.x; i < DTW * KS * kWave; i += NW * kWave) (&s_lds[0][0][0])[i] = src[i];
  for (int i = threadIdx.x; i < D; i += NW * kWave) z_lds[i] = zs[(size_t)slice * D + i];
  __syncthreads();
  const int t0 = chunk * chunk_len, t1 = min(n, t0 + chunk_len);
  lin_apply<D, NW, DW>(s_lds, z_lds, Q, view_base(qw, slice, h), qw.st, O, view_base(ow, slice, h),
                       ow, t0, t1, n, cmin, nullptr, hf * DW);
}

hipError_t launch_relu_linear_bf16(const Geometry& g, const void* Q, const View& qw, const void* K,
                                   const View& kw, const void* V, const View& vw, void* O,
                                   const View& ow, float cmin, int num_cus, hipStream_t s) {
  constexpr int NW = 4;
  const long long shared =
      (g.d == 128) ? g.slices
      : (g.d == 64) ? std::min<long long>(g.slices, std::max<long long>(0, 2LL * num_cus - g.slices))
                    : 0;
  const long long full = g.slices - shared, grid = full + 2 * shared;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 gr((unsigned)grid), block(NW * kWave);
  if (g.d == 64)
    relu_linear_bf16<64, NW><<<gr, block, 0, s>>>((const __bf16*)Q, (const __bf16*)K,
                                                  (const __bf16*)V, (__bf16*)O, qw, kw, vw, ow,
                                                  g.h, g.n, cmin, (int)full);
  else if (g.d == 128)
    relu_linear_bf16<128, NW><<<gr, block, 0, s>>>((const __bf16*)Q, (const __bf16*)K,
                                                   (const __bf16*)V, (__bf16*)O, qw, kw, vw, ow,
                                                   g.h, g.n, cmin, (int)full);
  else if (g.d == 32)
    relu_linear_bf16<32, NW><<<gr, block, 0, s>>>((const __bf16*)Q, (const __bf16*)K,
                                                  (const __bf16*)V, (__bf16*)O, qw, kw, vw, ow,
                                                  g.h, g.n, cmin, (int)full);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

template <int D>
static hipError_t lin_split_t(const Geometry& g, const LinearSplitPlan& p, const void* Q,
                              const View& qw, const void* K, const View& kw, const void* V,
                              const View& vw, void* O, const View& ow, float cmin, void* ws,
                              hipStream_t s) {
  constexpr int NW = 4;
  char* w = (char*)ws;
  float* part = (float*)w;
  float* zpart = (float*)(w + p.part_bytes);
  __bf16* sops = (__bf16*)(w + p.part_bytes + p.zpart_bytes);
  float* zs = (float*)(w + p.part_bytes + p.zpart_bytes + p.sop_bytes);
  const long long g1 = g.slices * p.chunks1, g2 = g.slices * p.chunks2;
  if (2 * g1 > 0x7fffffffLL || 2 * g2 > 0x7fffffffLL) return hipErrorInvalidValue;
  relu_linear_pass1<D, NW><<<dim3((unsigned)(g1 * (D == 128 ? 2 : 1))), dim3(NW * kWave), 0, s>>>(
      (const __bf16*)K, (const __bf16*)V, kw, vw, part, zpart, g.h, g.n, p.chunks1, p.chunk_len1);
  constexpr int GROUPS = ((D / 16) * (D / 16) + 3) / 4;
  relu_linear_finalize<D><<<dim3((unsigned)(g.slices * GROUPS)), dim3(256), 0, s>>>(
      part, zpart, sops, zs, p.chunks1);
  relu_linear_pass2<D, NW><<<dim3((unsigned)(g2 * (D == 128 ? 2 : 1))), dim3(NW * kWave), 0, s>>>(
      (const __bf16*)Q, (__bf16*)O, qw, ow, (const u32x4*)sops, zs, g.h, g.n, p.chunks2,
      p.chunk_len2, cmin);
  return hipGetLastError();
}

hipError_t launch_relu_linear_split_bf16(const Geometry& g, const LinearSplitPlan& p, const void* Q,
                                         const View& qw, const void* K, const View& kw,
                                         const void* V, const View& vw, void* O, const View& ow,
                                         float cmin, void* ws, hipStream_t s) {
  if (g.d == 64) return lin_split_t<64>(g, p, Q, qw, K, kw, V, vw, O, ow, cmin, ws, s);
  if (g.d == 32) return lin_split_t<32>(g, p, Q, qw, K, kw, V, vw, O, ow, cmin, ws, s);
  if (g.d == 128) return lin_split_t<128>(g, p, Q, qw, K, kw, V, vw, O, ow, cmin, ws, s);
  return hipErrorInvalidValue;
}

}  // namespace aa
