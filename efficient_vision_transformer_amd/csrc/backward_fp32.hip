// backward_fp32.hip -- gradients of anchor attention with fp32 inputs, fp32 accumulation
// and fp32 results; every product runs on v_mfma_f32_16x16x4_f32 (full fp32 products).
//
// Same function as the bf16 backward (AnchorFormer abstract: the anchors are learnable;
// Pith verdict page: the forward is Eq. (11) in the Eq. (12) order), c = 1/sqrt(d),
// G = dL/dH:
//   dW = A^T G,   dP = dW / Delta,   dDelta = -rowsum(dW * W) / Delta   (0 where Delta = 0)
//   dA = G W^T + V dP^T + 1 dDelta^T,   dS = A * (dA - rowsum(A * dA))
//   dQ = c dS U,   dV = A dP,   dU = c sum over the batch of dS^T Q.
// Kernels (on top of the fp32 split pass 1, run on (Q, U, V) and on (Q, U, G)):
//   bwd_finalize_fp32 (per slice x 16 anchors): chunk sums in chunk order; W and dP as
//     row-major [anchor][dim] blocks, dDelta per anchor;
//   bwd_tokens_fp32 (per slice x token chunk, one 16-token tile per wave at a time, lanes
//     = tokens): A recomputed; dA^T = dDelta + W G^T + dP V^T; dS in registers;
//     dQ^T = c U^T dS^T and dV^T = dP^T A^T written out; dS written to the workspace.
//     U and dP sit in LDS as row-major blocks, which give both the logits-side operands
//     (lane (c,g): anchor 16j + c, four consecutive dims) and the output-side ones (one
//     anchor row per K step, output dims across the lanes); W's operands are read from
//     its row-major block in global memory (L2), since U, W and dP together exceed the
//     LDS at 256 anchors;
//   bwd_dsq_fp32 (per slice x token chunk): per-chunk partial tiles of dS^T Q;
//   du_reduce_fp32 (per head x 16 anchors x 16 dims): dU = c x (partials summed over
//     batch and chunks in a fixed order).
#include <algorithm>

#include "device_common.h"
#include "kernels.h"
#include "pass2_layout.h"

namespace aa {

// ---------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256)
void bwd_finalize_fp32(const float* __restrict__ partP, const float* __restrict__ partG,
                       const float* __restrict__ dpart, float* __restrict__ wrm,
                       float* __restrict__ dprm, float* __restrict__ dd, int chunks, int AT) {
  constexpr int DT = D / 16;
  const int slice = blockIdx.x / AT;
  const int jt = blockIdx.x - slice * AT;
  const int r = (threadIdx.x >> 6) & 3, lane = threadIdx.x & 63;
  const int c = lane & 15, g = lane >> 4;
  const int anchor = 16 * jt + 4 * g + r;
  float p[DT], q[DT], delta = 0.f;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) { p[dt] = 0.f; q[dt] = 0.f; }
  constexpr int U = 4;   // loads of U chunks in flight, then the adds in chunk order
  for (int ch0 = 0; ch0 < chunks; ch0 += U) {
    float dv[U], pv[U][DT], qv[U][DT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t sc = (size_t)slice * chunks + min(ch0 + u, chunks - 1);
      dv[u] = dpart[sc * (16 * AT) + anchor];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const size_t e = ((sc * AT + jt) * DT + dt) * 256 + r * 64 + lane;
        pv[u][dt] = partP[e];
        qv[u][dt] = partG[e];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (ch0 + u < chunks) {
        delta += dv[u];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          p[dt] += pv[u][dt];
          q[dt] += qv[u][dt];
        }
      }
    }
  }
  const bool live = delta > 0.f;
  float dot = 0.f;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    p[dt] = live ? p[dt] / delta : 0.f;   // W
    dot += q[dt] * p[dt];                  // dW . W over this lane's dims
    q[dt] = live ? q[dt] / delta : 0.f;   // dP
  }
  dot = row16_sum(dot);                    // over the 16 lanes c: all D dims of the anchor
  if (c == 0) dd[(size_t)slice * (16 * AT) + anchor] = live ? -dot / delta : 0.f;
  const size_t row = ((size_t)slice * 16 * AT + anchor) * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    wrm[row + 16 * dt + c] = p[dt];
    dprm[row + 16 * dt + c] = q[dt];
  }
}

// ---------------------------------------------------------------------------------------
// Row loads in the fp32 token layout: lane (c,g) holds token row, dims (D/4)g + 4kq ..
// + 3 in chunk kq.  Rows past the slice's end read its last row (their weights are zeroed).
template <int D>
__device__ __forceinline__ void load_rows_f32(const float* __restrict__ X, size_t base,
                                              long long st, int row, int n, int g, f32x4* out) {
  constexpr int KQ = D / 16;
  const size_t off = base + (size_t)((long long)min(row, n - 1) * st) + (D / 4) * g;
#pragma unroll
  for (int kq = 0; kq < KQ; ++kq) out[kq] = __builtin_nontemporal_load((const f32x4*)(X + off + 4 * kq));
}

template <int D, int AT>
__global__ __launch_bounds__(4 * kWave, 1)
void bwd_tokens_fp32(const float* __restrict__ Q, const float* __restrict__ U,
                     const float* __restrict__ V, const float* __restrict__ G,
                     const float* __restrict__ wrm, const float* __restrict__ dprm,
                     const float* __restrict__ dd, float* __restrict__ dQ,
                     float* __restrict__ dV, float* __restrict__ dS, BwdViews bv, int h, int n,
                     int m, int chunks, int chunk_len, float c2, float cs) {
  constexpr int NW = 4, KQ = D / 16, DT = D / 16, NPAD = pad_tiles(AT);
  constexpr int RS = D + 4;        // row stride (floats) of the U and dP blocks
  constexpr int MPAD = 16 * AT;
  int slice, chunk;
  slice_chunk_of(blockIdx.x, chunks, slice, chunk);   // a slice's chunks on one XCD
  const int head = slice % h;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, g = lane >> 4;
  const size_t qb = view_base(bv.q, slice, h), vb = view_base(bv.v, slice, h);
  const size_t gb = view_base(bv.g, slice, h);
  const size_t dqb = view_base(bv.dq, slice, h), dvb = view_base(bv.dv, slice, h);
  const int t_begin = chunk * chunk_len;
  const int t_end = min(n, t_begin + chunk_len);

  __shared__ __attribute__((aligned(16))) float u_rm[MPAD * RS];
  __shared__ __attribute__((aligned(16))) float dp_rm[MPAD * RS];
  __shared__ __attribute__((aligned(16))) float dd_lds[MPAD];

  // Stage U (padded anchors zero) and dP: every load issued before the first LDS write.
  constexpr int T = NW * kWave, RCH = MPAD * D / 4;
  const float* Uh = U + (size_t)head * m * D;
  const float* dph = dprm + (size_t)slice * MPAD * D;
  const float* wh = wrm + (size_t)slice * MPAD * D;
  Stage<RCH, T> ust, dpst;
  stage_load(ust, [&](int idx) {
    const int a = idx / (D / 4), k = 4 * (idx - a * (D / 4));
    u32x4 v = {0u, 0u, 0u, 0u};
    if (a < m) v = *(const u32x4*)(Uh + (size_t)a * D + k);
    return v;
  });
  stage_load(dpst, [&](int idx) { return *(const u32x4*)(dph + 4 * (size_t)idx); });
  const float ddv = ((int)threadIdx.x < MPAD) ? dd[(size_t)slice * MPAD + threadIdx.x] : 0.f;
#pragma unroll
  for (int i = 0; i < Stage<RCH, T>::kPer; ++i) {
    const int idx = (int)threadIdx.x + i * T;
    if (RCH % T == 0 || idx < RCH) {
      const int a = idx / (D / 4), k = 4 * (idx - a * (D / 4));
      *(u32x4*)(u_rm + a * RS + k) = ust.r[i];
      *(u32x4*)(dp_rm + a * RS + k) = dpst.r[i];
    }
  }
  if ((int)threadIdx.x < MPAD) dd_lds[threadIdx.x] = ddv;
  f32x4 mask[NPAD];
  pad_mask_tiles<AT, NPAD>(g, m, mask);
  __syncthreads();

  for (int t0 = t_begin + 16 * w; t0 < t_end; t0 += 16 * NW) {
    const int row = t0 + c;
    const bool ok = row < t_end;
    f32x4 qv[KQ], vv[KQ], gv[KQ];
    load_rows_f32<D>(Q, qb, bv.q.st, row, n, g, qv);
    load_rows_f32<D>(V, vb, bv.v.st, row, n, g, vv);
    load_rows_f32<D>(G, gb, bv.g.st, row, n, g, gv);
    // S^T = U Q^T (lane (c,g): token c, anchors 16j + 4g + r), softmax over the anchors
    f32x4 a[AT];
#pragma unroll
    for (int j = 0; j < AT; ++j) {
      if (j % 4 == 0) asm volatile("" ::: "memory");   // LDS reads stay in the loop
      f32x4 acc = (j >= AT - NPAD) ? mask[j - (AT - NPAD)] : zero4();
#pragma unroll
      for (int kq = 0; kq < KQ; ++kq) {
        const f32x4 uu = *(const f32x4*)(u_rm + (16 * j + c) * RS + (D / 4) * g + 4 * kq);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = mfma_f32(uu[e], qv[kq][e], acc);
      }
      a[j] = acc;
    }
    float mx = a[0][0];
#pragma unroll
    for (int j = 0; j < AT; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, a[j][r]);
    mx = xor32_max(xor16_max(mx));
    const float mneg = -mx * c2;
    float z = 0.f;
#pragma unroll
    for (int j = 0; j < AT; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float e = exp2_fast(fmaf(a[j][r], c2, mneg));
        a[j][r] = e;
        z += e;
      }
    z = xor32_sum(xor16_sum(z));
    const float inv = ok ? 1.f / z : 0.f;
#pragma unroll
    for (int j = 0; j < AT; ++j) a[j] *= inv;
    // dA^T = dDelta + W G^T + dP V^T, rs = rowsum(A * dA), dS = A * (dA - rs)
    f32x4 ds[AT];
    float rs = 0.f;
#pragma unroll
    for (int j = 0; j < AT; ++j) {
      if (j % 4 == 0) asm volatile("" ::: "memory");
      f32x4 acc = *(const f32x4*)&dd_lds[16 * j + 4 * g];
#pragma unroll
      for (int kq = 0; kq < KQ; ++kq) {
        const f32x4 ww = *(const f32x4*)(wh + (size_t)(16 * j + c) * D + (D / 4) * g + 4 * kq);
        const f32x4 pp = *(const f32x4*)(dp_rm + (16 * j + c) * RS + (D / 4) * g + 4 * kq);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc = mfma_f32(ww[e], gv[kq][e], acc);
          acc = mfma_f32(pp[e], vv[kq][e], acc);
        }
      }
      ds[j] = acc;
#pragma unroll
      for (int r = 0; r < 4; ++r) rs = fmaf(a[j][r], acc[r], rs);
    }
    rs = xor32_sum(xor16_sum(rs));
#pragma unroll
    for (int j = 0; j < AT; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) ds[j][r] = a[j][r] * (ds[j][r] - rs);
    // dQ^T = c U^T dS^T and dV^T = dP^T A^T: K step (j, r) contracts anchor 16j + 4g + r;
    // the left operand of output tile dt2 gives lane c dim (D/4)(c/4) + 4dt2 + c % 4, so
    // lane group g ends with the dims (D/4)g .. + D/4 - 1 of token c (16-byte stores).
    f32x4 qa[DT], va[DT];
#pragma unroll
    for (int dt2 = 0; dt2 < DT; ++dt2) { qa[dt2] = zero4(); va[dt2] = zero4(); }
    const int ocol = (D / 4) * (c >> 2) + (c & 3);
#pragma unroll
    for (int j = 0; j < AT; ++j) {
      if (j % 2 == 0) asm volatile("" ::: "memory");
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float* ur = u_rm + (16 * j + 4 * g + r) * RS + ocol;
        const float* pr = dp_rm + (16 * j + 4 * g + r) * RS + ocol;
#pragma unroll
        for (int dt2 = 0; dt2 < DT; ++dt2) {
          qa[dt2] = mfma_f32(ur[4 * dt2], ds[j][r], qa[dt2]);
          va[dt2] = mfma_f32(pr[4 * dt2], a[j][r], va[dt2]);
        }
      }
    }
    if (ok) {
      float* oq = dQ + dqb + view_row(bv.dq, row) + (D / 4) * g;
      float* ov = dV + dvb + view_row(bv.dv, row) + (D / 4) * g;
#pragma unroll
      for (int dt2 = 0; dt2 < DT; ++dt2) {
        __builtin_nontemporal_store(qa[dt2] * cs, (f32x4*)(oq + 4 * dt2));
        __builtin_nontemporal_store(va[dt2], (f32x4*)(ov + 4 * dt2));
      }
      // dS rows [slice][token][anchor] for the dU pass
      float* os = dS + ((size_t)slice * n + row) * MPAD + 4 * g;
#pragma unroll
      for (int j = 0; j < AT; ++j) *(f32x4*)(os + 16 * j) = ds[j];
    }
  }
}

// ---------------------------------------------------------------------------------------
// Per-chunk partial tiles of dS^T Q: the (16-anchor, 16-dim) tiles are dealt to the four
// waves in turn; K step k contracts tokens 4k .. 4k + 3 (lane (c,g): anchor or dim c of
// token 4k + g), read straight from dS rows and Q rows.  Tokens past the chunk add zero.
template <int D, int AT>
__global__ __launch_bounds__(4 * kWave)
void bwd_dsq_fp32(const float* __restrict__ dS, const float* __restrict__ Q,
                  float* __restrict__ partU, View qw, int h, int n, int chunks, int chunk_len) {
  constexpr int NW = 4, DT = D / 16, TILES = AT * DT, TPW = (TILES + NW - 1) / NW;
  constexpr int MPAD = 16 * AT, KU = 4;   // K steps per batch of loads
  int slice, chunk;
  slice_chunk_of(blockIdx.x, chunks, slice, chunk);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, g = lane >> 4;
  const size_t qb = view_base(qw, slice, h);
  const int t_begin = chunk * chunk_len;
  const int t_end = min(n, t_begin + chunk_len);
  const float* ds = dS + (size_t)slice * n * MPAD;

  f32x4 acc[TPW];
#pragma unroll
  for (int k = 0; k < TPW; ++k) acc[k] = zero4();
  for (int t0 = t_begin; t0 < t_end; t0 += 4 * KU) {
    float xs[KU][TPW], ys[KU][TPW];
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const int tok = t0 + 4 * u + g;
      const int tc = min(tok, t_end - 1);
      const bool ok = tok < t_end;
#pragma unroll
      for (int k = 0; k < TPW; ++k) {
        const int t = w + NW * k;
        const int tt = (TILES % NW == 0 || t < TILES) ? t : 0;
        const int ja = tt / DT, dt = tt - ja * DT;
        const float xv = ds[(size_t)tc * MPAD + 16 * ja + c];
        const float yv = Q[qb + view_row(qw, tc) + 16 * dt + c];
        xs[u][k] = ok ? xv : 0.f;
        ys[u][k] = yv;
      }
    }
#pragma unroll
    for (int u = 0; u < KU; ++u)
#pragma unroll
      for (int k = 0; k < TPW; ++k) acc[k] = mfma_f32(xs[u][k], ys[u][k], acc[k]);
  }
  const size_t sc = (size_t)slice * chunks + chunk;
#pragma unroll
  for (int k = 0; k < TPW; ++k) {
    const int t = w + NW * k;
    if (TILES % NW != 0 && t >= TILES) break;
    const int ja = t / DT, dt = t - ja * DT;
    float* dst = partU + ((sc * AT + ja) * DT + dt) * 256;
#pragma unroll
    for (int r = 0; r < 4; ++r) dst[r * 64 + lane] = acc[k][r];
  }
}

// dU[head][16jt + 4g + r][16dt + c] = cs x the sum of the partial tiles over batch and
// chunk, in the fixed order of du_reduce (wave q takes entries e = q mod 8 in increasing
// e, then the wave sums are added in wave order).
template <int D>
__global__ __launch_bounds__(512)
void du_reduce_fp32(const float* __restrict__ partU, float* __restrict__ dU, int B, int h, int m,
                    int chunks, int AT, float cs) {
  constexpr int DT = D / 16, NWR = 8;
  __shared__ f32x4 red[NWR][kWave];
  const int tile = blockIdx.x;
  const int dt = tile % DT, jt = (tile / DT) % AT, head = tile / (DT * AT);
  const int lane = threadIdx.x & 63, q = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  f32x4 acc = zero4();
  const long long total = (long long)B * chunks;
  constexpr int U = 8;
  for (long long e0 = q; e0 < total; e0 += (long long)U * NWR) {
    f32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const long long e = min(e0 + (long long)u * NWR, total - 1);
      const long long b = e / chunks, ch = e - b * chunks;
      const size_t sc = ((size_t)b * h + head) * chunks + ch;
      const float* src = partU + ((sc * AT + jt) * DT + dt) * 256 + lane;
      v[u] = f32x4{src[0], src[64], src[128], src[192]};
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (e0 + (long long)u * NWR < total) acc += v[u];
  }
  red[q][lane] = acc;
  __syncthreads();
  if (q == 0) {
    f32x4 s = red[0][lane];
#pragma unroll
    for (int i = 1; i < NWR; ++i) s += red[i][lane];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int anchor = 16 * jt + 4 * g + r;
      if (anchor < m) dU[((size_t)head * m + anchor) * D + 16 * dt + c] = s[r] * cs;
    }
  }
}

// ---------------------------------------------------------------------------------------
template <int D, int AT>
static hipError_t go_bwd_fp32(const Geometry& g, const SplitPlan& p, const BackwardBuffersF32& wb,
                              const BwdViews& bv, const void* Q, const void* U, const void* V,
                              const void* G, void* dQ, void* dU, void* dV, hipStream_t s) {
  const float cs = 1.0f / sqrtf((float)D);
  Geometry gv = g, gg = g;
  gv.vw.q = gg.vw.q = bv.q;
  gv.vw.v = bv.v;
  gg.vw.v = bv.g;
  hipError_t e;
  if constexpr (D <= 64) {
    // one pass 1 for both: Q read and A formed once (at d = 128 its LDS would not fit)
    e = launch_pass1_dual_fp32(gv, p, Q, U, V, bv.v, G, bv.g, wb.partP, wb.partG, wb.dpart, s);
  } else {
    e = launch_pass1_fp32(gv, p, Q, U, V, wb.partP, wb.dpart, s);
    if (e != hipSuccess) return e;
    e = launch_pass1_fp32(gg, p, Q, U, G, wb.partG, wb.dpart, s);
  }
  if (e != hipSuccess) return e;
  const long long grid = g.slices * p.chunks1;
  bwd_finalize_fp32<D><<<dim3((unsigned)(g.slices * AT)), dim3(256), 0, s>>>(
      wb.partP, wb.partG, wb.dpart, wb.wrm, wb.dprm, wb.dd, p.chunks1, AT);
  bwd_tokens_fp32<D, AT><<<dim3((unsigned)grid), dim3(4 * kWave), 0, s>>>(
      (const float*)Q, (const float*)U, (const float*)V, (const float*)G, wb.wrm, wb.dprm,
      wb.dd, (float*)dQ, (float*)dV, wb.ds, bv, g.h, g.n, g.m, p.chunks1, p.chunk_len1, g.c2, cs);
  bwd_dsq_fp32<D, AT><<<dim3((unsigned)grid), dim3(4 * kWave), 0, s>>>(
      wb.ds, (const float*)Q, wb.partU, bv.q, g.h, g.n, p.chunks1, p.chunk_len1);
  const long long rgrid = (long long)g.h * AT * (D / 16);
  du_reduce_fp32<D><<<dim3((unsigned)rgrid), dim3(512), 0, s>>>(wb.partU, (float*)dU, g.B, g.h,
                                                               g.m, p.chunks1, AT, cs);
  return hipGetLastError();
}

template <int D>
static hipError_t dispatch_bwd_fp32(const Geometry& g, const SplitPlan& p,
                                    const BackwardBuffersF32& wb, const BwdViews& bv,
                                    const void* Q, const void* U, const void* V, const void* G,
                                    void* dQ, void* dU, void* dV, hipStream_t s) {
  switch (g.at) {
    case 2: return go_bwd_fp32<D, 2>(g, p, wb, bv, Q, U, V, G, dQ, dU, dV, s);
    case 4: return go_bwd_fp32<D, 4>(g, p, wb, bv, Q, U, V, G, dQ, dU, dV, s);
    case 6: return go_bwd_fp32<D, 6>(g, p, wb, bv, Q, U, V, G, dQ, dU, dV, s);
    case 8: return go_bwd_fp32<D, 8>(g, p, wb, bv, Q, U, V, G, dQ, dU, dV, s);
    // at d = 128 the U and dP blocks of the token pass take the LDS up to 128 anchors
    case 12: if constexpr (D <= 64) return go_bwd_fp32<D, 12>(g, p, wb, bv, Q, U, V, G, dQ, dU, dV, s);
             return hipErrorInvalidValue;
    case 16: if constexpr (D <= 64) return go_bwd_fp32<D, 16>(g, p, wb, bv, Q, U, V, G, dQ, dU, dV, s);
             return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

bool bwd_fp32_supported(const Geometry& g) {
  return ((g.d == 32 || g.d == 64) && g.at <= 16) || (g.d == 128 && g.at <= 8);
}

hipError_t launch_backward_fp32(const Geometry& g, const SplitPlan& p,
                                const BackwardBuffersF32& wb, const BwdViews& bv, const void* Q,
                                const void* U, const void* V, const void* G, void* dQ, void* dU,
                                void* dV, hipStream_t s) {
  if (!bwd_fp32_supported(g)) return hipErrorInvalidValue;
  if (g.d == 64) return dispatch_bwd_fp32<64>(g, p, wb, bv, Q, U, V, G, dQ, dU, dV, s);
  if (g.d == 128) return dispatch_bwd_fp32<128>(g, p, wb, bv, Q, U, V, G, dQ, dU, dV, s);
  return dispatch_bwd_fp32<32>(g, p, wb, bv, Q, U, V, G, dQ, dU, dV, s);
}

}  // namespace aa
