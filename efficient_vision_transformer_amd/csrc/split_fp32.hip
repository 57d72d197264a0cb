// split_fp32.hip -- anchor attention with fp32 inputs, fp32 accumulation and output.
//
// Same three-kernel structure as the bf16 path (pass 1 partials, ordered finalize,
// pass 2 recompute-and-apply), computing per (batch, head) slice
//   A = rowsoftmax(Q U^T / sqrt(d)),  W = Delta^-1 (A^T V) with Delta = 1^T A,  H = A W
// (AnchorFormer, Pith verdict page: referee summary, Eq. (11) in the Eq. (12) order).
// Every product runs on v_mfma_f32_16x16x4_f32 (full fp32 products, fp32 accumulate);
// there is no reduced-precision step anywhere on this path.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace aa {

// Pass 1 (fp32).  Logits S = Q U^T with lanes = anchors, registers = tokens, so the
// normalised A (one token per K step) feeds A^T V directly, and V's right operand
// (one token row per K step, 16 consecutive dims across lanes) is read from a plain
// row-major LDS copy.  DUAL (the backward): a second operand G (view gw) is staged beside
// V and A^T G accumulated into partG from the same A (no Delta).
template <int D, int AT, int NA, bool DUAL = false>
__global__ __launch_bounds__(kPass1Waves * kWave, DUAL ? 1 : 2)
void pass1_fp32(const float* __restrict__ Q, const float* __restrict__ U,
                const float* __restrict__ V, float* __restrict__ part,
                float* __restrict__ dpart, View qw, View vw, int h, int n, int m, int chunks,
                int chunk_len, float c2, const float* __restrict__ G = nullptr,
                View gw = View{0, 0, 0}, float* __restrict__ partG = nullptr) {
  constexpr int NW = kPass1Waves, ND = NW / NA, DT = D / 16, KQ = D / 16;
  constexpr int J = AT / NA, DTW = DT / ND, VS = D + 4;
  static_assert(AT % NA == 0 && DT % ND == 0, "wave split must tile the anchors and dims");
  const int slice = blockIdx.x / chunks;
  const int chunk = blockIdx.x - slice * chunks;
  const int head = slice % h;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int ag = w % NA, dg = w / NA;
  const size_t qb = view_base(qw, slice, h), vb = view_base(vw, slice, h);
  const size_t gb = DUAL ? view_base(gw, slice, h) : 0;
  const int t_begin = chunk * chunk_len;
  const int t_end = min(n, t_begin + chunk_len);

  // Q as left operands: lane (c,g) of tile tt holds token c, dims (D/4)g + 4kq + e.
  __shared__ f32x4 q_lds[NW][2][KQ][kWave];
  __shared__ __attribute__((aligned(16))) float v_lds[NW][32][VS];
  __shared__ __attribute__((aligned(16))) float g_lds[DUAL ? NW : 1][DUAL ? 32 : 1][DUAL ? VS : 4];
  __shared__ float st_max[NA][32];
  __shared__ float st_sum[NA][32];

  // Right operands of S = Q U^T: lane (c,g) holds anchor 16j + c, dims (D/4)g + kk.
  f32x4 uop[J][KQ];
  const float* Uh = U + (size_t)head * m * D;
#pragma unroll
  for (int jl = 0; jl < J; ++jl) {
    const int a = 16 * (ag * J + jl) + c;
#pragma unroll
    for (int kq = 0; kq < KQ; ++kq)
      uop[jl][kq] = (a < m) ? *(const f32x4*)(Uh + (size_t)a * D + (D / 4) * g + 4 * kq) : zero4();
  }
  f32x4 pacc[J][DTW], gacc[DUAL ? J : 1][DTW];
  f32x4 dacc[J];
#pragma unroll
  for (int jl = 0; jl < J; ++jl) {
    dacc[jl] = zero4();
#pragma unroll
    for (int dl = 0; dl < DTW; ++dl) pacc[jl][dl] = zero4();
  }
#pragma unroll
  for (int jl = 0; jl < (DUAL ? J : 1); ++jl)
#pragma unroll
    for (int dl = 0; dl < DTW; ++dl) gacc[jl][dl] = zero4();

  for (int blk = t_begin; blk < t_end; blk += 32 * NW) {
    {  // stage pair w
      const int p0 = blk + 32 * w;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int row = p0 + 16 * tt + c;
        const bool ok = row < t_end;
        const size_t qo = qb + view_row(qw, ok ? row : 0) + (D / 4) * g;
        const size_t vo = vb + view_row(vw, ok ? row : 0) + (D / 4) * g;
        const size_t go = DUAL ? gb + view_row(gw, ok ? row : 0) + (D / 4) * g : 0;
#pragma unroll
        for (int kq = 0; kq < KQ; ++kq) {
          const f32x4 qv = ok ? *(const f32x4*)(Q + qo + 4 * kq) : zero4();
          const f32x4 vv = ok ? *(const f32x4*)(V + vo + 4 * kq) : zero4();
          q_lds[w][tt][kq][lane] = qv;
          *(f32x4*)&v_lds[w][16 * tt + c][(D / 4) * g + 4 * kq] = vv;
          if constexpr (DUAL) {
            const f32x4 gv = ok ? *(const f32x4*)(G + go + 4 * kq) : zero4();
            *(f32x4*)&g_lds[w][16 * tt + c][(D / 4) * g + 4 * kq] = gv;
          }
        }
      }
    }
    __syncthreads();

    for (int ps = 0; ps < NW; ++ps) {
      const int p0 = blk + 32 * ps;
      if (p0 >= t_end) break;  // uniform over the workgroup
      f32x4 s[2][J];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int jl = 0; jl < J; ++jl) {
          f32x4 acc = zero4();
#pragma unroll
          for (int kq = 0; kq < KQ; ++kq) {
            const f32x4 qq = q_lds[ps][tt][kq][lane];
#pragma unroll
            for (int e = 0; e < 4; ++e) acc = mfma_f32(qq[e], uop[jl][kq][e], acc);
          }
          if (16 * (ag * J + jl) + c >= m) acc = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
          s[tt][jl] = acc;
        }
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
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int tok = 16 * tt + 4 * g + r;
          float Z = st_sum[0][tok];
#pragma unroll
          for (int a2 = 1; a2 < NA; ++a2) Z += st_sum[a2][tok];
          const float inv = (p0 + tok < t_end) ? 1.f / Z : 0.f;
#pragma unroll
          for (int jl = 0; jl < J; ++jl) s[tt][jl][r] *= inv;
        }
      // a3: K step (tt, r) contracts token 4g + r of tile tt.
#pragma unroll
      for (int jl = 0; jl < J; ++jl) {
#pragma unroll
        for (int dl = 0; dl < DTW; ++dl) {
          f32x4 acc = pacc[jl][dl];
          const int col = 16 * (dg * DTW + dl) + c;
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              acc = mfma_f32(s[tt][jl][r], v_lds[ps][16 * tt + 4 * g + r][col], acc);
          pacc[jl][dl] = acc;
        }
        if (dg == 0) {
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int r = 0; r < 4; ++r) dacc[jl] = mfma_f32(s[tt][jl][r], 1.f, dacc[jl]);
        }
        if constexpr (DUAL) {
#pragma unroll
          for (int dl = 0; dl < DTW; ++dl) {
            f32x4 acc = gacc[jl][dl];
            const int col = 16 * (dg * DTW + dl) + c;
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
              for (int r = 0; r < 4; ++r)
                acc = mfma_f32(s[tt][jl][r], g_lds[ps][16 * tt + 4 * g + r][col], acc);
            gacc[jl][dl] = acc;
          }
        }
      }
    }
    __syncthreads();
  }

  // Partials: [slice][chunk][jt][dt][r][lane] holds P[16jt + 4g + r][16dt + c].
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
      if constexpr (DUAL) {
        float* dgp = partG + ((sc * AT + jt) * DT + dt) * 256;
#pragma unroll
        for (int r = 0; r < 4; ++r) dgp[r * 64 + lane] = gacc[jl][dl][r];
      }
    }
    if (dg == 0 && c == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) dpart[sc * (16 * AT) + 16 * jt + 4 * g + r] = dacc[jl][r];
    }
  }
}

// Finalize (fp32): W = Delta^-1 sum_chunks P in chunk order; output is the left operand
// of pass 2's H^T = W^T A^T per K step (j, r): [slice][dt2][j][r][lane'] with lane'
// (c', g') holding W[16j + 4g' + r][(D/4)(c' / 4) + 4dt2 + c' % 4] (lane group g of the
// output then holds the contiguous dims (D/4)g .. (D/4)g + D/4 - 1 of its token).
template <int D>
__global__ __launch_bounds__(256)
void finalize_fp32(const float* __restrict__ part, const float* __restrict__ dpart,
                   float* __restrict__ Wop, int chunks, int AT) {
  constexpr int DT = D / 16, U = 8;
  const int slice = blockIdx.x / AT;
  const int jt = blockIdx.x - slice * AT;
  // Thread t owns accumulator slot (r, lane) of every dim tile: element dt*256 + t.
  const int r = (threadIdx.x >> 6) & 3, lane = threadIdx.x & 63;
  const int c = lane & 15, g = lane >> 4;
  const int anchor = 16 * jt + 4 * g + r;
  float p[DT], delta = 0.f;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) p[dt] = 0.f;
  for (int ch0 = 0; ch0 < chunks; ch0 += U) {
    // all loads of U chunks first, then the adds in chunk order
    float pv[U][DT], dv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ch = min(ch0 + u, chunks - 1);
      const size_t sc = (size_t)slice * chunks + ch;
      dv[u] = dpart[sc * (16 * AT) + anchor];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) pv[u][dt] = part[((sc * AT + jt) * DT + dt) * 256 + r * 64 + lane];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (ch0 + u < chunks) {
        delta += dv[u];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) p[dt] += pv[u][dt];
      }
    }
  }
  const int j = anchor >> 4, gg = (anchor >> 2) & 3, rr = anchor & 3;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    const float wv = (delta > 0.f) ? p[dt] / delta : 0.f;
    const int dim = 16 * dt + c;
    const int rem = dim % (D / 4);
    const int dt2 = rem >> 2;
    const int cc = 4 * (dim / (D / 4)) + (rem & 3);
    Wop[((((size_t)slice * DT + dt2) * AT + j) * 4 + rr) * 64 + 16 * gg + cc] = wv;
  }
}

// Pass 2 (fp32): transposed logits S^T = U Q^T (lanes = tokens), softmax in registers
// plus two permlane swaps, then H^T = W^T A^T with A feeding the right operand one
// anchor per K step.  U and W in fp32 take AT * D * 128 bytes of LDS; when that leaves
// room for one workgroup per CU, the workgroup has eight waves (two per SIMD).
template <int D, int AT>
constexpr int pass2_fp32_waves() { return AT * D * 128 > 80 * 1024 ? 8 : kPass2Waves; }

template <int D, int AT>
__global__ __launch_bounds__((pass2_fp32_waves<D, AT>() * kWave))
void pass2_fp32(const float* __restrict__ Q, const float* __restrict__ U,
                const float* __restrict__ Wop, float* __restrict__ H, View qw, View ow, int h,
                int n, int m, int chunks, int chunk_len, float c2) {
  constexpr int NW = pass2_fp32_waves<D, AT>(), DT = D / 16, KQ = D / 16;
  const int slice = blockIdx.x / chunks;
  const int chunk = blockIdx.x - slice * chunks;
  const int head = slice % h;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const size_t qb = view_base(qw, slice, h), ob = view_base(ow, slice, h);
  const int t_begin = chunk * chunk_len;
  const int t_end = min(n, t_begin + chunk_len);

  __shared__ f32x4 u_lds[AT][KQ][kWave];      // lane (c,g): anchor 16j + c, dims (D/4)g + 4kq..
  __shared__ float w_lds[DT][AT][4][kWave];
  // U, then W, each with all of its loads issued before the first LDS write.
  const float* Uh = U + (size_t)head * m * D;
  {
    Stage<AT * KQ * kWave, NW * kWave> ust;
    stage_load(ust, [&](int idx) {
      const int j = idx / (KQ * kWave), kq = (idx / kWave) % KQ, l = idx & 63;
      const int a = 16 * j + (l & 15);
      u32x4 v = {0u, 0u, 0u, 0u};
      if (a < m) v = *(const u32x4*)(Uh + (size_t)a * D + (D / 4) * (l >> 4) + 4 * kq);
      return v;
    });
    stage_store(ust, (u32x4*)&u_lds[0][0][0]);
  }
  {
    // W: DT * AT * 4 * kWave floats, copied as 16-byte chunks
    const u32x4* Ws = (const u32x4*)(Wop + (size_t)slice * DT * AT * 4 * kWave);
    Stage<DT * AT * kWave, NW * kWave> wst;
    stage_load(wst, [&](int idx) { return Ws[idx]; });
    stage_store(wst, (u32x4*)&w_lds[0][0][0][0]);
  }
  constexpr int NPAD = pad_tiles(AT);
  f32x4 mask[NPAD];
  pad_mask_tiles<AT, NPAD>(g, m, mask);
  __syncthreads();

  // Software pipeline: the next tile's Q rows are requested before this tile is computed.
  // Rows past the chunk read its last row (clamped) and are not stored.
  auto load_q = [&](int t0, f32x4* q) {
    const size_t off = qb + view_row(qw, min(t0 + c, t_end - 1)) + (D / 4) * g;
#pragma unroll
    for (int kq = 0; kq < KQ; ++kq) q[kq] = __builtin_nontemporal_load((const f32x4*)(Q + off + 4 * kq));
  };
  f32x4 q[KQ];
  if (t_begin + 16 * w < t_end) load_q(t_begin + 16 * w, q);
  for (int t0 = t_begin + 16 * w; t0 < t_end; t0 += 16 * NW) {
    const int row = t0 + c;
    const bool ok = row < t_end;
    f32x4 qn[KQ];   // the next tile's rows, unconditionally (clamped; unused past the end)
    load_q(t0 + 16 * NW, qn);
    f32x4 s[AT];
#pragma unroll
    for (int j = 0; j < AT; ++j) {
      // keeps the LDS operand loads of later tiles from being hoisted (register budget)
      if (j % 4 == 0) asm volatile("" ::: "memory");
      // padded anchors (>= m) lie in the last NPAD tiles and start from -inf
      f32x4 acc = (j >= AT - NPAD) ? mask[j - (AT - NPAD)] : zero4();
#pragma unroll
      for (int kq = 0; kq < KQ; ++kq) {
        const f32x4 uu = u_lds[j][kq][lane];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = mfma_f32(uu[e], q[kq][e], acc);
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
    const float inv = 1.f / z;
    f32x4 hacc[DT];
#pragma unroll
    for (int dt2 = 0; dt2 < DT; ++dt2) hacc[dt2] = zero4();
#pragma unroll
    for (int j = 0; j < AT; ++j) {
      if (j % 2 == 0) asm volatile("" ::: "memory");
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float a = s[j][r] * inv;
#pragma unroll
        for (int dt2 = 0; dt2 < DT; ++dt2) hacc[dt2] = mfma_f32(w_lds[dt2][j][r][lane], a, hacc[dt2]);
      }
    }
    if (ok) {
      float* dst = H + ob + view_row(ow, row) + (D / 4) * g;
#pragma unroll
      for (int dt2 = 0; dt2 < DT; ++dt2) __builtin_nontemporal_store(hacc[dt2], (f32x4*)(dst + 4 * dt2));
    }
#pragma unroll
    for (int kq = 0; kq < KQ; ++kq) q[kq] = qn[kq];
  }
}

template <int D, int AT>
static hipError_t launch_split_fp32_t(const Geometry& geo, const SplitPlan& p, const void* Q,
                                      const void* U, const void* V, void* H, void* ws,
                                      hipStream_t stream) {
  constexpr int NA = (AT % 4 == 0) ? 4 : 2;
  char* wsb = (char*)ws;
  float* part = (float*)wsb;
  float* dpart = (float*)(wsb + p.part_bytes);
  float* Wop = (float*)(wsb + p.part_bytes + p.dpart_bytes);
  const long long g1 = geo.slices * p.chunks1;
  pass1_fp32<D, AT, NA><<<dim3((unsigned)g1), dim3(kPass1Waves * kWave), 0, stream>>>(
      (const float*)Q, (const float*)U, (const float*)V, part, dpart, geo.vw.q, geo.vw.v, geo.h,
      geo.n, geo.m, p.chunks1, p.chunk_len1, geo.c2);
  finalize_fp32<D><<<dim3((unsigned)(geo.slices * AT)), dim3(256), 0, stream>>>(
      part, dpart, Wop, p.chunks1, AT);
  const long long g2 = geo.slices * p.chunks2;
  pass2_fp32<D, AT><<<dim3((unsigned)g2), dim3(pass2_fp32_waves<D, AT>() * kWave), 0, stream>>>(
      (const float*)Q, (const float*)U, Wop, (float*)H, geo.vw.q, geo.vw.o, geo.h, geo.n, geo.m,
      p.chunks2, p.chunk_len2, geo.c2);
  return hipGetLastError();
}

template <int D>
static hipError_t dispatch_at(const Geometry& g, const SplitPlan& p, const void* Q, const void* U,
                              const void* V, void* H, void* ws, hipStream_t s) {
  switch (g.at) {
    case 2: return launch_split_fp32_t<D, 2>(g, p, Q, U, V, H, ws, s);
    case 4: return launch_split_fp32_t<D, 4>(g, p, Q, U, V, H, ws, s);
    case 6: return launch_split_fp32_t<D, 6>(g, p, Q, U, V, H, ws, s);
    case 8: return launch_split_fp32_t<D, 8>(g, p, Q, U, V, H, ws, s);
    // at d = 128, U and W in fp32 outgrow pass 2's LDS above 128 anchors
    case 12: if constexpr (D <= 64) return launch_split_fp32_t<D, 12>(g, p, Q, U, V, H, ws, s);
             return hipErrorInvalidValue;
    case 16: if constexpr (D <= 64) return launch_split_fp32_t<D, 16>(g, p, Q, U, V, H, ws, s);
             return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_split_fp32(const Geometry& g, const SplitPlan& p, const void* Q, const void* U,
                             const void* V, void* H, void* ws, hipStream_t stream) {
  if (g.d == 64) return dispatch_at<64>(g, p, Q, U, V, H, ws, stream);
  if (g.d == 32) return dispatch_at<32>(g, p, Q, U, V, H, ws, stream);
  if (g.d == 128) return dispatch_at<128>(g, p, Q, U, V, H, ws, stream);   // m <= 128
  return hipErrorInvalidValue;
}

hipError_t launch_pass1_dual_fp32(const Geometry& g, const SplitPlan& p, const void* Q,
                                  const void* U, const void* V, const View& vw, const void* G,
                                  const View& gw, float* part, float* partG, float* dpart,
                                  hipStream_t s) {
  const long long g1 = g.slices * p.chunks1;
  auto at = [&](auto D) -> hipError_t {
    constexpr int d = decltype(D)::value;
#define AA_P1FD(AT)                                                                          \
  pass1_fp32<d, AT, (AT % 4 == 0) ? 4 : 2, true><<<dim3((unsigned)g1), dim3(kPass1Waves * kWave), 0, s>>>( \
      (const float*)Q, (const float*)U, (const float*)V, part, dpart, g.vw.q, vw, g.h, g.n, \
      g.m, p.chunks1, p.chunk_len1, g.c2, (const float*)G, gw, partG)
    switch (g.at) {
      case 2: AA_P1FD(2); break;
      case 4: AA_P1FD(4); break;
      case 6: AA_P1FD(6); break;
      case 8: AA_P1FD(8); break;
      case 12: AA_P1FD(12); break;
      case 16: AA_P1FD(16); break;
      default: return hipErrorInvalidValue;
    }
#undef AA_P1FD
    return hipGetLastError();
  };
  if (g.d == 64) return at(std::integral_constant<int, 64>{});
  if (g.d == 32) return at(std::integral_constant<int, 32>{});
  return hipErrorInvalidValue;
}

hipError_t launch_pass1_fp32(const Geometry& g, const SplitPlan& p, const void* Q, const void* U,
                             const void* X, float* part, float* dpart, hipStream_t s) {
  const long long g1 = g.slices * p.chunks1;
  auto at = [&](auto D) -> hipError_t {
    constexpr int d = decltype(D)::value;
#define AA_P1F(AT)                                                                           \
  pass1_fp32<d, AT, (AT % 4 == 0) ? 4 : 2><<<dim3((unsigned)g1), dim3(kPass1Waves * kWave), 0, s>>>( \
      (const float*)Q, (const float*)U, (const float*)X, part, dpart, g.vw.q, g.vw.v, g.h, g.n, \
      g.m, p.chunks1, p.chunk_len1, g.c2)
    switch (g.at) {
      case 2: AA_P1F(2); break;
      case 4: AA_P1F(4); break;
      case 6: AA_P1F(6); break;
      case 8: AA_P1F(8); break;
      case 12:
        if constexpr (d <= 64) { AA_P1F(12); break; }
        return hipErrorInvalidValue;
      case 16:
        if constexpr (d <= 64) { AA_P1F(16); break; }
        return hipErrorInvalidValue;
      default: return hipErrorInvalidValue;
    }
#undef AA_P1F
    return hipGetLastError();
  };
  if (g.d == 64) return at(std::integral_constant<int, 64>{});
  if (g.d == 32) return at(std::integral_constant<int, 32>{});
  if (g.d == 128) return at(std::integral_constant<int, 128>{});   // up to 128 anchors
  return hipErrorInvalidValue;
}

}  // namespace aa
