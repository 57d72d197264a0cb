// backward_bf16.hip -- gradients of anchor attention, bf16 in / bf16 out, fp32 accumulate.
//
// For each slice (AnchorFormer abstract: the anchors are learnable, so the layer is
// trained through; Pith verdict page: the forward is Eq. (11) in the Eq. (12) order),
// with c = 1/sqrt(d), given G = dL/dH (chain rule through the forward steps in reverse):
//   dW = A^T G,   dP = dW / Delta,   dDelta = -rowsum(dW * W) / Delta   (0 where Delta = 0)
//   dA = G W^T + V dP^T + 1 dDelta^T,   dS = A * (dA - rowsum(A * dA))
//   dQ = c dS U,   dV = A dP,   dU = c sum over the batch of dS^T Q.
// Kernels (on top of the split plan's pass 1, run on (Q, U, V) and on (Q, U, G)):
//   bwd_finalize (per slice x 16 anchors): chunk sums of P, dW and Delta in chunk order;
//     W as logits-layout MFMA operands, dP as a row-major [anchor][dim] block, dDelta;
//   bwd_tokens_rm (per slice x token chunk, one 16-token tile per wave per round): A
//     recomputed; dA^T = dDelta + W G^T + dP V^T on the MFMA (lanes = tokens); dS in
//     registers; dQ^T = c U^T dS^T and dV^T = dP^T A^T written out; the round's rows of dS
//     and Q go to LDS and every wave accumulates its tiles of dS^T Q (transposing LDS
//     reads) into per-chunk partials of dU;
//   du_reduce (per head x 16 anchors x 16 dims): dU = c x (partials summed over batch and
//     chunks in a fixed order).
#include <algorithm>

#include "device_common.h"
#include "kernels.h"
#include "pass2_layout.h"
#include "tile_ops.h"

namespace aa {

// Anchor a, dim k of an m_pad x D matrix -> position in the "U layout" left operand of a
// logits-like product (lane (c,g) of (tile j, chunk kk): anchor 16j + c, dims
// 8*KS*g + 8kk .. + 7).
template <int D>
__device__ __forceinline__ size_t u_layout_index(int AT, int a, int k) {
  constexpr int KS = D / 32;
  const int j = a >> 4, cc = a & 15, gg = k / (8 * KS), rem = k % (8 * KS);
  return ((((size_t)j * KS + (rem >> 3)) * kWave) + 16 * gg + cc) * 8 + (rem & 7);
}

// ---------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256)
void bwd_finalize(const float* __restrict__ partP, const float* __restrict__ partG,
                  const float* __restrict__ dpart, __bf16* __restrict__ wu,
                  __bf16* __restrict__ dprm, float* __restrict__ dd, int chunks, int AT) {
  constexpr int DT = D / 16, KS = D / 32;
  const int MP = AT / 2;
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
  const float rinv = (delta > 0.f) ? 1.f / delta : 0.f;
  float dot = 0.f;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    p[dt] *= rinv;                 // W
    dot += q[dt] * p[dt];          // dW . W over this lane's dims
    q[dt] *= rinv;                 // dP
  }
  dot = row16_sum(dot);            // over the 16 lanes c: all D dims of the anchor
  if (c == 0) dd[(size_t)slice * (16 * AT) + anchor] = -dot * rinv;
  const size_t su = (size_t)slice * AT * KS * kWave * 8;
  const size_t sr = (size_t)slice * 16 * AT * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    const int k = 16 * dt + c;
    wu[su + u_layout_index<D>(AT, anchor, k)] = (__bf16)p[dt];
    dprm[sr + (size_t)anchor * D + k] = (__bf16)q[dt];   // row-major [anchor][dim]
  }
}

// ---------------------------------------------------------------------------------------
// Output-layout operand of a product whose contraction runs over anchors (dQ^T = U^T dS^T,
// dV^T = dP^T A^T), read with the transposing LDS read from a row-major [anchor][dim]
// block: lane (c, g) gets dim out_dim_c(dt2, c) of anchors 4g + s (s < 4) and
// 16 + 4g + s - 4 (s >= 4) counted from blk.  Reading lane 4k + q of group g points at
// anchor 4g + k, dims out_dim_c(dt2, 4q) .. + 3 (four consecutive dims).
__device__ __forceinline__ bf16x8 rows_operand_out(const __bf16* blk, int stride, int dt2, int c,
                                                   int g) {
  const __bf16* p = blk + (4 * g + (c >> 2)) * stride + out_dim_c(dt2, 4 * (c & 3));
  const s16x4 lo = lds_read_tr(p);
  const s16x4 hi = lds_read_tr(p + 16 * stride);
  const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// Token pass: up to 256 anchors at d = 32 or 64, up to 128 at d = 128.  U and dP are kept
// once in LDS, as row-major [anchor][dim] blocks, and serve both as the logits-layout left
// operands (16-byte row reads) and as the output-layout ones (transposing reads); W stays
// in its logits layout.  (An earlier pass kept five operand blocks, U, W and dP in the
// logits layout and U^T, dP^T in the output layout, which could not grow past 128 anchors
// and, without the row prefetch, was slower at every size.)  Each of the four waves takes
// one 16-token tile per round, so a
// round's rows of dS and Q for the dU tiles cover 64 tokens.  The next round's rows of Q,
// V and dH are requested before the current round is computed.
// LSE: A comes from each token's base-2 log-sum-exp written by pass 1 ([slice][n]), one
// FMA and one exponential per entry, instead of the softmax formed again.
template <int D, int AT, bool LSE = false>
__global__ __launch_bounds__(4 * kWave, 1)
void bwd_tokens_rm(const __bf16* __restrict__ Q, const __bf16* __restrict__ U,
                   const __bf16* __restrict__ V, const __bf16* __restrict__ G,
                   const u32x4* __restrict__ wu, const __bf16* __restrict__ dprm,
                   const float* __restrict__ dd, __bf16* __restrict__ dQ, __bf16* __restrict__ dV,
                   float* __restrict__ partU, BwdViews bv, int h, int n, int m, int chunks,
                   int chunk_len, float c2, float cs, const float* __restrict__ lse = nullptr) {
  constexpr int NW = 4, KS = D / 32, DT = D / 16, MP = AT / 2, NPAD = pad_tiles(AT);
  constexpr int TILES = AT * DT, TPW = TILES / NW;
  constexpr int RS = D + 16;                      // row stride of U, dP and Q rows
  constexpr int AS = tr_stride<16 * AT>();        // row stride of dS rows
  constexpr int TOK = 16 * NW;                    // tokens per round
  static_assert(TILES % NW == 0, "tiles split evenly over the waves");
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

  __shared__ __attribute__((aligned(16))) __bf16 u_rm[16 * AT * RS];    // U rows
  __shared__ __attribute__((aligned(16))) __bf16 dp_rm[16 * AT * RS];   // dP rows
  __shared__ u32x4 wu_lds[AT][KS][kWave];                               // W, logits layout
  __shared__ __attribute__((aligned(16))) float dd_lds[16 * AT];
  __shared__ __attribute__((aligned(16))) __bf16 s_rows[TOK * AS];      // rows of dS
  __shared__ __attribute__((aligned(16))) __bf16 q_rows[TOK * RS];      // rows of Q

  // Stage the slice's operands: every load is issued before the first LDS write.
  constexpr int T = NW * kWave, RCH = 16 * AT * D / 8, WCH = AT * KS * kWave;
  const __bf16* Uh = U + (size_t)head * m * D;
  const __bf16* dph = dprm + (size_t)slice * 16 * AT * D;
  Stage<RCH, T> ust, dpst;
  stage_load(ust, [&](int idx) {
    const int a = idx / (D / 8), k = 8 * (idx - a * (D / 8));
    u32x4 v = {0u, 0u, 0u, 0u};
    if (a < m) v = *(const u32x4*)(Uh + (size_t)a * D + k);
    return v;
  });
  stage_load(dpst, [&](int idx) { return *(const u32x4*)(dph + 8 * (size_t)idx); });
  Stage<WCH, T> wst;
  stage_load(wst, [&](int idx) { return wu[(size_t)slice * WCH + idx]; });
  const float ddv = ((int)threadIdx.x < 16 * AT) ? dd[(size_t)slice * 16 * AT + threadIdx.x] : 0.f;
#pragma unroll
  for (int i = 0; i < Stage<RCH, T>::kPer; ++i) {
    const int idx = (int)threadIdx.x + i * T;
    if (RCH % T == 0 || idx < RCH) {
      const int a = idx / (D / 8), k = 8 * (idx - a * (D / 8));
      *(u32x4*)(u_rm + a * RS + k) = ust.r[i];
      *(u32x4*)(dp_rm + a * RS + k) = dpst.r[i];
    }
  }
  stage_store(wst, &wu_lds[0][0][0]);
  if ((int)threadIdx.x < 16 * AT) dd_lds[threadIdx.x] = ddv;
  f32x4 mask[NPAD];
  pad_mask_tiles<AT, NPAD>(g, m, mask);
  const bf16x8 ones = splat_bf16(1.f);

  f32x4 pacc[TPW], dummy[1];
#pragma unroll
  for (int k = 0; k < TPW; ++k) pacc[k] = zero4();
  dummy[0] = zero4();

  const int rounds = (t_end - t_begin + TOK - 1) / TOK;
  u32x4 qv[KS], vv[KS], gv[KS];
  const float* lse_s = LSE ? lse + (size_t)slice * n : nullptr;
  float lv = 0.f;
  {
    const int row = min(t_begin + 16 * w + c, t_end - 1);
    if constexpr (LSE) lv = lse_s[row];
    load_rows<D>(Q, qb, bv.q.st, row, n, g, qv);
    load_rows<D>(V, vb, bv.v.st, row, n, g, vv);
    load_rows<D>(G, gb, bv.g.st, row, n, g, gv);
  }
  __syncthreads();

  for (int r = 0; r < rounds; ++r) {
    const int row = t_begin + TOK * r + 16 * w + c;
    const bool ok = row < t_end;
    // next round's rows (past the chunk: its last row, which is cached, rather than the
    // next chunk's rows)
    u32x4 nq[KS], nv[KS], ng[KS];
    const int nrow = min(row + TOK, t_end - 1);
    float nlv = 0.f;
    if constexpr (LSE) nlv = lse_s[nrow];
    load_rows<D>(Q, qb, bv.q.st, nrow, n, g, nq);
    load_rows<D>(V, vb, bv.v.st, nrow, n, g, nv);
    load_rows<D>(G, gb, bv.g.st, nrow, n, g, ng);
    asm volatile("" ::: "memory");   // LDS operands are re-read each round, not hoisted
    // A (normalised, bf16): ab[jj] lane (c,g) holds token c, anchors 32jj + 4g .. + 3
    // (slots 0-3) and 32jj + 16 + 4g .. + 3 (slots 4-7).
    bf16x8 ab[MP];
    {
      f32x4 sc[AT];
#pragma unroll
      for (int j = 0; j < AT; ++j) {
        f32x4 acc = (j >= AT - NPAD) ? mask[j - (AT - NPAD)] : zero4();
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
          const bf16x8 uo = as_bf16x8(*(const u32x4*)(u_rm + (16 * j + c) * RS + 8 * KS * g + 8 * kk));
          acc = mfma_bf16(uo, as_bf16x8(qv[kk]), acc);
        }
        sc[j] = acc;
      }
      if constexpr (LSE) {
        // already normalised; tokens past the end get exp2(-inf) = 0 (and so do padded
        // anchors, whose logits start from -inf)
        const float nl = ok ? -lv : -INFINITY;
#pragma unroll
        for (int j = 0; j < AT; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) sc[j][q] = exp2_fast(fmaf(sc[j][q], c2, nl));
#pragma unroll
        for (int jj = 0; jj < MP; ++jj) ab[jj] = pack_bf16(sc[2 * jj], sc[2 * jj + 1]);
      } else {
        float mx = sc[0][0];
#pragma unroll
        for (int j = 0; j < AT; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) mx = fmaxf(mx, sc[j][q]);
        mx = xor32_max(xor16_max(mx));
        const float mneg = -mx * c2;
        f32x4 zt = zero4();
#pragma unroll
        for (int j = 0; j < AT; ++j) {
#pragma unroll
          for (int q = 0; q < 4; ++q) sc[j][q] = exp2_fast(fmaf(sc[j][q], c2, mneg));
          zt += sc[j];
        }
        const float z = xor32_sum(xor16_sum((zt[0] + zt[1]) + (zt[2] + zt[3])));
        const float inv = ok ? 1.f / z : 0.f;
#pragma unroll
        for (int jj = 0; jj < MP; ++jj) ab[jj] = pack_bf16(sc[2 * jj] * inv, sc[2 * jj + 1] * inv);
      }
    }
    // this tile's rows of Q ([token][dim]) for the dU tiles
    {
      __bf16* qrow = q_rows + (16 * w + c) * RS + 8 * KS * g;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) *(u32x4*)(qrow + 8 * kk) = qv[kk];
    }
    // dA^T = dDelta + W G^T + dP V^T and dS = A * (dA - rowsum(A * dA))
    bf16x8 dsb[MP];
    {
      f32x4 da[AT];
      float rs = 0.f;
#pragma unroll
      for (int j = 0; j < AT; ++j) {
        f32x4 acc = *(const f32x4*)&dd_lds[16 * j + 4 * g];
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
          const bf16x8 po = as_bf16x8(*(const u32x4*)(dp_rm + (16 * j + c) * RS + 8 * KS * g + 8 * kk));
          acc = mfma_bf16(as_bf16x8(wu_lds[j][kk][lane]), as_bf16x8(gv[kk]), acc);
          acc = mfma_bf16(po, as_bf16x8(vv[kk]), acc);
        }
        da[j] = acc;
#pragma unroll
        for (int q = 0; q < 4; ++q) rs = fmaf((float)ab[j >> 1][4 * (j & 1) + q], acc[q], rs);
      }
      rs = xor32_sum(xor16_sum(rs));
#pragma unroll
      for (int jj = 0; jj < MP; ++jj) {
        f32x4 d0, d1;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          d0[q] = (float)ab[jj][q] * (da[2 * jj][q] - rs);
          d1[q] = (float)ab[jj][4 + q] * (da[2 * jj + 1][q] - rs);
        }
        dsb[jj] = pack_bf16(d0, d1);
      }
    }
    // dQ^T = c U^T dS^T and dV^T = dP^T A^T, two dim tiles at a time (64-byte row runs)
    const size_t oq = dqb + view_row(bv.dq, row) + 8 * g;
    const size_t ov = dvb + view_row(bv.dv, row) + 8 * g;
#pragma unroll
    for (int hh = 0; hh < DT / 2; ++hh) {
      f32x4 q0 = zero4(), q1 = zero4(), v0 = zero4(), v1 = zero4();
#pragma unroll
      for (int jj = 0; jj < MP; ++jj) {
        q0 = mfma_bf16(rows_operand_out(u_rm + 32 * jj * RS, RS, 2 * hh, c, g), dsb[jj], q0);
        q1 = mfma_bf16(rows_operand_out(u_rm + 32 * jj * RS, RS, 2 * hh + 1, c, g), dsb[jj], q1);
      }
      if (ok) __builtin_nontemporal_store(as_u32x4(pack_bf16(q0 * cs, q1 * cs)), (u32x4*)(dQ + oq + 32 * hh));
#pragma unroll
      for (int jj = 0; jj < MP; ++jj) {
        v0 = mfma_bf16(rows_operand_out(dp_rm + 32 * jj * RS, RS, 2 * hh, c, g), ab[jj], v0);
        v1 = mfma_bf16(rows_operand_out(dp_rm + 32 * jj * RS, RS, 2 * hh + 1, c, g), ab[jj], v1);
      }
      if (ok) __builtin_nontemporal_store(as_u32x4(pack_bf16(v0, v1)), (u32x4*)(dV + ov + 32 * hh));
    }
    // this tile's rows of dS ([token][anchor]); zero for tokens past the end
    {
      __bf16* srow = s_rows + (16 * w + c) * AS + 4 * g;
#pragma unroll
      for (int jj = 0; jj < MP; ++jj) {
        const u32x4 v = as_u32x4(dsb[jj]);
        *(u32x2*)(srow + 32 * jj) = u32x2{v[0], v[1]};
        *(u32x2*)(srow + 32 * jj + 16) = u32x2{v[2], v[3]};
      }
    }
    __syncthreads();
    // dS^T Q over the round's 32-token blocks that hold tokens, this wave's tiles
    const int blocks = min(TOK / 32, (t_end - (t_begin + TOK * r) + 31) / 32);
    accumulate_tiles<TPW, DT, AS, RS, false>(s_rows, q_rows, w * TPW, blocks, c, g, ones, pacc,
                                             dummy);
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      qv[kk] = nq[kk];
      vv[kk] = nv[kk];
      gv[kk] = ng[kk];
    }
    if constexpr (LSE) lv = nlv;
  }

  // dU partials: [slice][chunk][jt][dt][r][lane] holds the sum over the chunk's tokens of
  // dS[token][16jt + 4g + r] Q[token][16dt + c] (the layout du_reduce reads)
  const size_t sc = (size_t)slice * chunks + chunk;
#pragma unroll
  for (int k = 0; k < TPW; ++k) {
    const int t = w * TPW + k;
    const int ja = t / DT, dt = t - (t / DT) * DT;
    float* dst = partU + ((sc * AT + ja) * DT + dt) * 256;
#pragma unroll
    for (int q = 0; q < 4; ++q) dst[q * 64 + lane] = pacc[k][q];
  }
}

// ---------------------------------------------------------------------------------------
// dU[head][16jt + 4g + r][16dt + c] = cs x the sum of the partial tiles over batch and
// chunk.  One workgroup per (head, anchor tile, dim tile); wave q sums the entries
// e = b * chunks + ch with e = q (mod 8) in increasing e, and the eight wave sums are then
// added in wave order, so the result does not depend on scheduling.
template <int D>
__global__ __launch_bounds__(512)
void du_reduce(const float* __restrict__ partU, __bf16* __restrict__ dU, int B, int h, int m,
               int chunks, int AT, float cs) {
  constexpr int DT = D / 16, NWR = 8;
  __shared__ f32x4 red[NWR][kWave];
  const int tile = blockIdx.x;
  const int dt = tile % DT, jt = (tile / DT) % AT, head = tile / (DT * AT);
  const int lane = threadIdx.x & 63, q = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  f32x4 acc = zero4();
  const long long total = (long long)B * chunks;
  constexpr int U = 8;   // loads of U entries in flight, then the adds in entry order
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
      if (anchor < m) dU[((size_t)head * m + anchor) * D + 16 * dt + c] = (__bf16)(s[r] * cs);
    }
  }
}

hipError_t launch_du_reduce_bf16(const Geometry& g, const float* partU, int chunks, void* dU,
                                 hipStream_t s) {
  const long long grid = (long long)g.h * g.at * (g.d / 16);
  if (grid <= 0 || grid > 0x7fffffffLL) return hipErrorInvalidValue;
  const float cs = 1.0f / sqrtf((float)g.d);
  if (g.d == 64)
    du_reduce<64><<<dim3((unsigned)grid), dim3(512), 0, s>>>(partU, (__bf16*)dU, g.B, g.h, g.m,
                                                            chunks, g.at, cs);
  else if (g.d == 32)
    du_reduce<32><<<dim3((unsigned)grid), dim3(512), 0, s>>>(partU, (__bf16*)dU, g.B, g.h, g.m,
                                                            chunks, g.at, cs);
  else if (g.d == 128)
    du_reduce<128><<<dim3((unsigned)grid), dim3(512), 0, s>>>(partU, (__bf16*)dU, g.B, g.h, g.m,
                                                             chunks, g.at, cs);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
template <int D, int AT>
static hipError_t go_bwd(const Geometry& g, const SplitPlan& p, const BackwardBuffers& wb,
                         const BwdViews& bv, const void* Q, const void* U, const void* V,
                         const void* G, void* dQ, void* dU, void* dV, hipStream_t s) {
  constexpr int MP = AT / 2;
  const float cs = 1.0f / sqrtf((float)D);
  // pass 1 reads Q through the first view of its geometry and X through the second
  Geometry gv = g, gg = g;
  gv.vw.q = gg.vw.q = bv.q;
  gv.vw.v = bv.v;
  gg.vw.v = bv.g;
  hipError_t e;
  if constexpr (D <= 64 || AT <= 6) {
    // one pass 1 for both: Q read and A formed once (at d = 128 with 128 anchors its
    // registers would spill)
    e = launch_pass1_dual_bf16(gv, p, Q, U, V, bv.v, G, bv.g, wb.partP, wb.partG, wb.dpart,
                               AT > 8 ? wb.lse : nullptr, s);
  } else {
    e = launch_pass1_bf16(gv, p, Q, U, V, wb.partP, wb.dpart, s);
    if (e != hipSuccess) return e;
    e = launch_pass1_bf16(gg, p, Q, U, G, wb.partG, wb.dpart, s);
  }
  if (e != hipSuccess) return e;
  bwd_finalize<D><<<dim3((unsigned)(g.slices * AT)), dim3(256), 0, s>>>(
      wb.partP, wb.partG, wb.dpart, (__bf16*)wb.wu, (__bf16*)wb.dprm, wb.dd, p.chunks1, AT);
  // above 128 anchors A comes from pass 1's log-sum-exp
  constexpr bool kLse = (D <= 64 || AT <= 6) && AT > 8;
  if (kLse && !wb.lse) return hipErrorInvalidValue;
  bwd_tokens_rm<D, AT, kLse><<<dim3((unsigned)(g.slices * wb.chunks_t)), dim3(4 * kWave), 0, s>>>(
      (const __bf16*)Q, (const __bf16*)U, (const __bf16*)V, (const __bf16*)G,
      (const u32x4*)wb.wu, (const __bf16*)wb.dprm, wb.dd, (__bf16*)dQ, (__bf16*)dV, wb.partU,
      bv, g.h, g.n, g.m, wb.chunks_t, wb.chunk_len_t, g.c2, cs, wb.lse);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_du_reduce_bf16(g, wb.partU, wb.chunks_t, dU, s);
}

template <int D>
static hipError_t dispatch_bwd(const Geometry& g, const SplitPlan& p, const BackwardBuffers& wb,
                               const BwdViews& bv, const void* Q, const void* U, const void* V,
                               const void* G, void* dQ, void* dU, void* dV, hipStream_t s) {
  switch (g.at) {
    case 2: return go_bwd<D, 2>(g, p, wb, bv, Q, U, V, G, dQ, dU, dV, s);
    case 4: return go_bwd<D, 4>(g, p, wb, bv, Q, U, V, G, dQ, dU, dV, s);
    case 6: return go_bwd<D, 6>(g, p, wb, bv, Q, U, V, G, dQ, dU, dV, s);
    case 8: return go_bwd<D, 8>(g, p, wb, bv, Q, U, V, G, dQ, dU, dV, s);
    case 12:
      if constexpr (D <= 64) return go_bwd<D, 12>(g, p, wb, bv, Q, U, V, G, dQ, dU, dV, s);
      return hipErrorInvalidValue;
    case 16:
      if constexpr (D <= 64) return go_bwd<D, 16>(g, p, wb, bv, Q, U, V, G, dQ, dU, dV, s);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

bool bwd_split_supported(const Geometry& g) {
  return (g.d == 32 || g.d == 64) ? g.at <= 16 : (g.d == 128 && g.at <= 8);
}

__global__ __launch_bounds__(256) void fill_zero_u32(unsigned* __restrict__ p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = 0u;
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s) {
  const size_t n = bytes / 4;   // callers pass 16-byte aligned buffers of bf16 pairs
  if (n == 0) return hipSuccess;
  const unsigned blocks = (unsigned)std::min<size_t>(1024, (n + 255) / 256);
  fill_zero_u32<<<dim3(blocks), dim3(256), 0, s>>>((unsigned*)p, n);
  return hipGetLastError();
}

hipError_t launch_backward_bf16(const Geometry& g, const SplitPlan& p, const BackwardBuffers& wb,
                                const BwdViews& bv, const void* Q, const void* U, const void* V,
                                const void* G, void* dQ, void* dU, void* dV, hipStream_t s) {
  if (!bwd_split_supported(g)) return hipErrorInvalidValue;
  if (g.d == 64) return dispatch_bwd<64>(g, p, wb, bv, Q, U, V, G, dQ, dU, dV, s);
  if (g.d == 32) return dispatch_bwd<32>(g, p, wb, bv, Q, U, V, G, dQ, dU, dV, s);
  if (g.d == 128) return dispatch_bwd<128>(g, p, wb, bv, Q, U, V, G, dQ, dU, dV, s);
  return hipErrorInvalidValue;
}

}  // namespace aa
