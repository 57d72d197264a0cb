// split_bf16.hip -- anchor attention for long token sequences, bf16 in / bf16 out.
//
// Per (batch, head) slice (AnchorFormer, Pith verdict page: referee summary, Eq. (11)
// evaluated in the Eq. (12) order; desk-editor letter: A row-stochastic, Delta its
// column sums):
//   A = rowsoftmax(Q U^T / sqrt(d)),  Delta = 1^T A,  W = Delta^-1 (A^T V),  H = A W.
// The tokens of a slice are split into chunks so that the whole chip is busy:
//   pass 1  (one workgroup per chunk): logits, softmax, column sums and A^T V of the
//           chunk -> fp32 partials in the workspace;
//   finalize (one workgroup per 16 anchors of a slice): sums the partials over chunks
//           in chunk order (deterministic), W = P / Delta (0 where Delta == 0), written
//           as bf16 MFMA operands;
//   pass 2  (one workgroup per chunk): recomputes A from Q and writes H = A W.
// All products run on v_mfma_f32_16x16x32_bf16 with fp32 accumulation.
#include "device_common.h"
#include "kernels.h"

namespace aa {

// ---------------------------------------------------------------------------------------
// Pass 1.  Four waves split the anchors (NA groups) and, when there are few anchor tiles,
// the dims of A^T V (4/NA groups).  Each block of 128 tokens is staged through LDS: every
// wave loads one 32-token pair of Q (kept in its MFMA operand layout) and of V (moved to
// the token-in-register layout by a selection MFMA).  Logits are formed as S = Q U^T
// (lanes = anchors, registers = tokens), so the softmax over anchors is a 16-lane DPP
// reduction plus an exchange of per-token maxima and sums between anchor groups, and the
// normalised A is directly the left operand of A^T V.
template <int D, int AT, int NA>
__global__ __launch_bounds__(kPass1Waves * kWave)
void pass1_bf16(const __bf16* __restrict__ Q, const __bf16* __restrict__ U,
                const __bf16* __restrict__ V, float* __restrict__ part,
                float* __restrict__ dpart, int h, int n, int m, int chunks, int chunk_len,
                float c2) {
  constexpr int NW = kPass1Waves, ND = NW / NA, KS = D / 32, DT = D / 16;
  constexpr int J = AT / NA, DTW = DT / ND;
  static_assert(AT % NA == 0 && DT % ND == 0, "wave split must tile the anchors and dims");
  const int slice = blockIdx.x / chunks;
  const int chunk = blockIdx.x - slice * chunks;
  const int head = slice % h;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int ag = w % NA, dg = w / NA;
  const size_t base = (size_t)slice * (size_t)n * D;
  const int t_begin = chunk * chunk_len;
  const int t_end = min(n, t_begin + chunk_len);

  __shared__ u32x4 q_lds[NW][2][KS][kWave];
  __shared__ u32x4 v_lds[NW][DT][kWave];
  __shared__ float st_max[NA][32];
  __shared__ float st_sum[NA][32];

  // This wave's anchors as right operands of S = Q U^T: lane (c,g) holds anchor 16j + c,
  // dims 8*KS*g + 8*kk + s.  Padded anchors (>= m) are zero and masked below.
  bf16x8 uop[J][KS];
  const __bf16* Uh = U + (size_t)head * m * D;
#pragma unroll
  for (int jl = 0; jl < J; ++jl) {
    const int a = 16 * (ag * J + jl) + c;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (a < m) v = *(const u32x4*)(Uh + (size_t)a * D + 8 * KS * g + 8 * kk);
      uop[jl][kk] = as_bf16x8(v);
    }
  }
  const bf16x8 vsel0 = vsel_operand(0, c, g), vsel1 = vsel_operand(1, c, g);
  const bf16x8 ones = splat_bf16(1.f);
  f32x4 pacc[J][DTW];
  f32x4 dacc[J];
#pragma unroll
  for (int jl = 0; jl < J; ++jl) {
    dacc[jl] = zero4();
#pragma unroll
    for (int dl = 0; dl < DTW; ++dl) pacc[jl][dl] = zero4();
  }

  for (int blk = t_begin; blk < t_end; blk += 32 * NW) {
    {  // stage pair w of this block
      const int p0 = blk + 32 * w;
      f32x4 vt[2][DT];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int row = p0 + 16 * tt + c;
        const bool ok = row < t_end;
        const size_t off = base + (size_t)(ok ? row : 0) * D + 8 * KS * g;
        u32x4 qv[KS], vv[KS];
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
          qv[kk] = ok ? *(const u32x4*)(Q + off + 8 * kk) : u32x4{0u, 0u, 0u, 0u};
          vv[kk] = ok ? *(const u32x4*)(V + off + 8 * kk) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) q_lds[w][tt][kk][lane] = qv[kk];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          vt[tt][dt] = mfma_bf16(as_bf16x8(vv[dt >> 1]), (dt & 1) ? vsel1 : vsel0, zero4());
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) v_lds[w][dt][lane] = as_u32x4(pack_bf16(vt[0][dt], vt[1][dt]));
    }
    __syncthreads();

    for (int ps = 0; ps < NW; ++ps) {
      const int p0 = blk + 32 * ps;
      if (p0 >= t_end) break;  // uniform over the workgroup
      // a1: logits in base-2 units later; s[tt][jl] lane (c,g): anchor 16j+c, token 4g+r.
      f32x4 s[2][J];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int jl = 0; jl < J; ++jl) {
          f32x4 acc = zero4();
#pragma unroll
          for (int kk = 0; kk < KS; ++kk)
            acc = mfma_bf16(as_bf16x8(q_lds[ps][tt][kk][lane]), uop[jl][kk], acc);
          if (16 * (ag * J + jl) + c >= m) acc = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
          s[tt][jl] = acc;
        }
      // a2: softmax over the anchors of each token.
      float mx[2][4];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float v = s[tt][0][r];
#pragma unroll
          for (int jl = 1; jl < J; ++jl) v = fmaxf(v, s[tt][jl][r]);
          mx[tt][r] = row16_max(v);
        }
      if (c == 0) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int r = 0; r < 4; ++r) st_max[ag][16 * tt + 4 * g + r] = mx[tt][r];
      }
      __syncthreads();
      float z[2][4];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int tok = 16 * tt + 4 * g + r;
          float M = st_max[0][tok];
#pragma unroll
          for (int a2 = 1; a2 < NA; ++a2) M = fmaxf(M, st_max[a2][tok]);
          const float mneg = -M * c2;
          float zz = 0.f;
#pragma unroll
          for (int jl = 0; jl < J; ++jl) {
            const float e = exp2_fast(fmaf(s[tt][jl][r], c2, mneg));
            s[tt][jl][r] = e;
            zz += e;
          }
          z[tt][r] = row16_sum(zz);
        }
      if (c == 0) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int r = 0; r < 4; ++r) st_sum[ag][16 * tt + 4 * g + r] = z[tt][r];
      }
      __syncthreads();
      f32x4 inv[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int tok = 16 * tt + 4 * g + r;
          float Z = st_sum[0][tok];
#pragma unroll
          for (int a2 = 1; a2 < NA; ++a2) Z += st_sum[a2][tok];
          inv[tt][r] = (p0 + tok < t_end) ? 1.f / Z : 0.f;
        }
      // a3: Delta and A^T V.  The left operand holds anchor c and tokens
      // {4g+s of tile 0, 4g+s-4 of tile 1}; the staged V^T uses the same token order.
#pragma unroll
      for (int jl = 0; jl < J; ++jl) {
        const bf16x8 ax = pack_bf16(s[0][jl] * inv[0], s[1][jl] * inv[1]);
#pragma unroll
        for (int dl = 0; dl < DTW; ++dl)
          pacc[jl][dl] = mfma_bf16(ax, as_bf16x8(v_lds[ps][dg * DTW + dl][lane]), pacc[jl][dl]);
        if (dg == 0) dacc[jl] = mfma_bf16(ax, ones, dacc[jl]);
      }
    }
    __syncthreads();
  }

  // Partials in accumulator layout: [slice][chunk][jt][dt][r][lane] holds
  // P[16jt + 4g + r][vt_dim(dt, c)]; Delta as [slice][chunk][anchor].
  const size_t sc = (size_t)slice * chunks + chunk;
#pragma unroll
  for (int jl = 0; jl < J; ++jl) {
    const int jt = ag * J + jl;
#pragma unroll
    for (int dl = 0; dl < DTW; ++dl) {
      const int dt = dg * DTW + dl;
      float* dst = part + ((sc * AT + jt) * DT + dt) * 256;
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[r * 64 + lane] = pacc[jl][dl][r];
    }
    if (dg == 0 && c == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) dpart[sc * (16 * AT) + 16 * jt + 4 * g + r] = dacc[jl][r];
    }
  }
}

// ---------------------------------------------------------------------------------------
// Finalize: W = Delta^-1 (sum over chunks of P), chunk order fixed.  One workgroup per
// (slice, 16-anchor tile).  Output layout = the left operand of pass 2's H^T = W^T A^T:
// [slice][dt2][jj][lane'][slot] with lane' (c',g') holding dim out_dim(dt2, c') and
// anchors {32jj + 4g' + slot (slot<4), 32jj + 16 + 4g' + slot - 4 (slot>=4)}.
template <int D>
__global__ __launch_bounds__(256)
void finalize_bf16(const float* __restrict__ part, const float* __restrict__ dpart,
                   __bf16* __restrict__ Wop, int chunks, int AT) {
  constexpr int DT = D / 16;
  const int MP = AT / 2;
  const int slice = blockIdx.x / AT;
  const int jt = blockIdx.x - slice * AT;
  for (int e = threadIdx.x; e < DT * 256; e += 256) {
    const int dt = e >> 8, r = (e >> 6) & 3, lane = e & 63;
    const int c = lane & 15, g = lane >> 4;
    const int anchor = 16 * jt + 4 * g + r;
    const int dim = vt_dim<D>(dt, c);
    float p = 0.f, delta = 0.f;
    for (int ch = 0; ch < chunks; ++ch) {
      const size_t sc = (size_t)slice * chunks + ch;
      p += part[((sc * AT + jt) * DT + dt) * 256 + r * 64 + lane];
      delta += dpart[sc * (16 * AT) + anchor];
    }
    const float wv = (delta > 0.f) ? p / delta : 0.f;
    const int rem = dim % (D / 4);
    const int dt2 = rem >> 2;
    const int cc = 4 * (dim / (D / 4)) + (rem & 3);
    const int jj = anchor >> 5, half = (anchor >> 4) & 1, gg = (anchor >> 2) & 3;
    const int slot = 4 * half + (anchor & 3);
    Wop[((((size_t)slice * DT + dt2) * MP + jj) * 64 + 16 * gg + cc) * 8 + slot] = (__bf16)wv;
  }
}

// ---------------------------------------------------------------------------------------
// Pass 2.  Each wave takes 16-token tiles.  Logits are formed transposed, S^T = U Q^T
// (lanes = tokens, registers = anchors), so the softmax is an in-register reduction plus
// two permlane swaps and the normalised A is directly the right operand of
// H^T = W^T A^T.  U and W stay in LDS for the whole chunk.
template <int D, int AT>
__global__ __launch_bounds__(kPass2Waves * kWave)
void pass2_bf16(const __bf16* __restrict__ Q, const __bf16* __restrict__ U,
                const u32x4* __restrict__ Wop, __bf16* __restrict__ H, int h, int n, int m,
                int chunks, int chunk_len, float c2) {
  constexpr int NW = kPass2Waves, KS = D / 32, DT = D / 16, MP = AT / 2;
  const int slice = blockIdx.x / chunks;
  const int chunk = blockIdx.x - slice * chunks;
  const int head = slice % h;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const size_t base = (size_t)slice * (size_t)n * D;
  const int t_begin = chunk * chunk_len;
  const int t_end = min(n, t_begin + chunk_len);

  __shared__ u32x4 u_lds[AT][KS][kWave];
  __shared__ u32x4 w_lds[DT][MP][kWave];
  const __bf16* Uh = U + (size_t)head * m * D;
  for (int idx = threadIdx.x; idx < AT * KS * kWave; idx += NW * kWave) {
    const int j = idx / (KS * kWave), kk = (idx / kWave) % KS, l = idx & 63;
    const int a = 16 * j + (l & 15);
    u32x4 v = {0u, 0u, 0u, 0u};
    if (a < m) v = *(const u32x4*)(Uh + (size_t)a * D + 8 * KS * (l >> 4) + 8 * kk);
    u_lds[j][kk][l] = v;
  }
  const u32x4* Ws = Wop + (size_t)slice * DT * MP * kWave;
  for (int idx = threadIdx.x; idx < DT * MP * kWave; idx += NW * kWave)
    (&w_lds[0][0][0])[idx] = Ws[idx];
  __syncthreads();

  for (int t0 = t_begin + 16 * w; t0 < t_end; t0 += 16 * NW) {
    const int row = t0 + c;
    const bool ok = row < t_end;
    const size_t off = base + (size_t)(ok ? row : 0) * D + 8 * KS * g;
    u32x4 q[KS];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) q[kk] = ok ? *(const u32x4*)(Q + off + 8 * kk) : u32x4{0u, 0u, 0u, 0u};
    // a1 (transposed): s[j] lane (c,g): token c, anchors 16j + 4g + r.
    f32x4 s[AT];
#pragma unroll
    for (int j = 0; j < AT; ++j) {
      f32x4 acc = zero4();
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) acc = mfma_bf16(as_bf16x8(u_lds[j][kk][lane]), as_bf16x8(q[kk]), acc);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (16 * j + 4 * g + r >= m) acc[r] = -INFINITY;
      s[j] = acc;
    }
    // a2
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
    const float inv = 1.f / z;
    bf16x8 abf[MP];
#pragma unroll
    for (int jj = 0; jj < MP; ++jj) abf[jj] = pack_bf16(s[2 * jj] * inv, s[2 * jj + 1] * inv);
    // a5: H^T = W^T A^T; lane (c,g) ends with token c, dims (D/4)g + 4dt2 + r.
    f32x4 hacc[DT];
#pragma unroll
    for (int dt2 = 0; dt2 < DT; ++dt2) {
      f32x4 acc = zero4();
#pragma unroll
      for (int jj = 0; jj < MP; ++jj) acc = mfma_bf16(as_bf16x8(w_lds[dt2][jj][lane]), abf[jj], acc);
      hacc[dt2] = acc;
    }
    if (ok) {
      __bf16* dst = H + base + (size_t)row * D + (D / 4) * g;
#pragma unroll
      for (int half = 0; half < DT / 2; ++half)
        *(u32x4*)(dst + 8 * half) = as_u32x4(pack_bf16(hacc[2 * half], hacc[2 * half + 1]));
    }
  }
}

// ---------------------------------------------------------------------------------------
template <int D, int AT>
static hipError_t launch_split_bf16_t(const Geometry& geo, const SplitPlan& p, const void* Q,
                                      const void* U, const void* V, void* H, void* ws,
                                      hipStream_t stream) {
  constexpr int NA = (AT % 4 == 0) ? 4 : 2;
  char* wsb = (char*)ws;
  float* part = (float*)wsb;
  float* dpart = (float*)(wsb + p.part_bytes);
  void* Wop = (void*)(wsb + p.part_bytes + p.dpart_bytes);
  const long long g1 = geo.slices * p.chunks1;
  pass1_bf16<D, AT, NA><<<dim3((unsigned)g1), dim3(kPass1Waves * kWave), 0, stream>>>(
      (const __bf16*)Q, (const __bf16*)U, (const __bf16*)V, part, dpart, geo.h, geo.n, geo.m,
      p.chunks1, p.chunk_len1, geo.c2);
  finalize_bf16<D><<<dim3((unsigned)(geo.slices * AT)), dim3(256), 0, stream>>>(
      part, dpart, (__bf16*)Wop, p.chunks1, AT);
  const long long g2 = geo.slices * p.chunks2;
  pass2_bf16<D, AT><<<dim3((unsigned)g2), dim3(kPass2Waves * kWave), 0, stream>>>(
      (const __bf16*)Q, (const __bf16*)U, (const u32x4*)Wop, (__bf16*)H, geo.h, geo.n, geo.m,
      p.chunks2, p.chunk_len2, geo.c2);
  return hipGetLastError();
}

template <int D>
static hipError_t dispatch_at(const Geometry& g, const SplitPlan& p, const void* Q, const void* U,
                              const void* V, void* H, void* ws, hipStream_t s) {
  switch (g.at) {
    case 2: return launch_split_bf16_t<D, 2>(g, p, Q, U, V, H, ws, s);
    case 4: return launch_split_bf16_t<D, 4>(g, p, Q, U, V, H, ws, s);
    case 6: return launch_split_bf16_t<D, 6>(g, p, Q, U, V, H, ws, s);
    case 8: return launch_split_bf16_t<D, 8>(g, p, Q, U, V, H, ws, s);
    case 10: return launch_split_bf16_t<D, 10>(g, p, Q, U, V, H, ws, s);
    case 12: return launch_split_bf16_t<D, 12>(g, p, Q, U, V, H, ws, s);
    case 14: return launch_split_bf16_t<D, 14>(g, p, Q, U, V, H, ws, s);
    case 16: return launch_split_bf16_t<D, 16>(g, p, Q, U, V, H, ws, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_split_bf16(const Geometry& g, const SplitPlan& p, const void* Q, const void* U,
                             const void* V, void* H, void* ws, hipStream_t stream) {
  if (g.d == 64) return dispatch_at<64>(g, p, Q, U, V, H, ws, stream);
  if (g.d == 32) return dispatch_at<32>(g, p, Q, U, V, H, ws, stream);
  return hipErrorInvalidValue;
}

}  // namespace aa
