// nystrom_bf16.hip -- Nystrom attention with given landmark tokens (bf16 in and out, fp32
// accumulation).
//
// Fast Nystrom Attention page (key machinery): the attention matrix is approximated by three
// row softmaxes through s landmark rows q = Q[idx], k = K[idx], the middle one inverted.  Per
// (batch, head) slice, with c = 1/sqrt(d):
//   F1 = rowsoftmax(Q k^T c) (n x s),  F2 = rowsoftmax(q k^T c) (s x s),
//   F3 = rowsoftmax(q K^T c) (s x n),  H = F1 (F2^-1 (F3 V)).
// Five launches:
//   nys_gather  per slice: the landmark rows of Q and K (token indices per batch element).
//   nys_max     per (slice, token chunk): each landmark's largest logit q_a . k_t over the
//               chunk (MFMA, tokens in lanes).
//   pass 1      (split plan, landmark mode): exp(c q_a . k_t - c M_a) with M_a the maximum
//               over all chunks, accumulated against V and against ones: F3 V and F3's row
//               sums, unnormalised, per chunk.
//   nys_solve   per slice: chunk sums -> F3 V; F2 in fp32 from the landmark rows; Z = F2^-1
//               (F3 V) by Gauss-Jordan elimination with partial pivoting in LDS; Z stored as
//               pass 2's W operands.
//   pass 2      (split plan, per-slice anchors = the landmark keys): H = rowsoftmax(Q k^T c) Z.
#include <algorithm>

#include "device_common.h"
#include "kernels.h"
#include "tile_ops.h"

namespace aa {

// Landmark rows of one slice: qt[slice][a] = Q[b, head, idx[b][a]], kt likewise (token
// indices clamped to [0, n)).  Q and K contiguous [B, h, n, d].
template <int D>
__global__ __launch_bounds__(256)
void nys_gather(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                const int* __restrict__ idx, __bf16* __restrict__ qt, __bf16* __restrict__ kt,
                int h, int n, int s) {
  constexpr int CH = D / 8;   // 16-byte chunks per row
  constexpr int U = 4;
  const int slice = blockIdx.x, b = slice / h;
  const size_t ib = (size_t)slice * n * D, ob = (size_t)slice * s * D;
  const int total = s * CH;
  for (int i0 = 0; i0 < total; i0 += 256 * U) {
    u32x4 vq[U], vk[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + (int)threadIdx.x + 256 * u;
      if (i < total) {
        const int a = i / CH, ch = i - a * CH;
        const int t = min(max(idx[(size_t)b * s + a], 0), n - 1);
        vq[u] = *(const u32x4*)(Q + ib + (size_t)t * D + 8 * ch);
        vk[u] = *(const u32x4*)(K + ib + (size_t)t * D + 8 * ch);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + (int)threadIdx.x + 256 * u;
      if (i < total) {
        const int a = i / CH, ch = i - a * CH;
        *(u32x4*)(qt + ob + (size_t)a * D + 8 * ch) = vq[u];
        *(u32x4*)(kt + ob + (size_t)a * D + 8 * ch) = vk[u];
      }
    }
  }
}

// Per (slice, chunk): cmax[slice][chunk][a] = max over the chunk's tokens t of q_a . k_t
// (raw logits, fp32 accumulation of bf16 products in the same MFMA order as pass 1's, so
// pass 1's exponents are never positive).  Four waves; each takes 16-token tiles with the
// next tile's rows in flight.  Entries of padded landmarks (a >= m) repeat landmark m - 1.
template <int D, int AT>
__global__ __launch_bounds__(256)
void nys_max(const __bf16* __restrict__ K, const __bf16* __restrict__ qt,
             float* __restrict__ cmax, View kw, int h, int n, int m, int chunks, int chunk_len) {
  constexpr int KS = D / 32, NW = 4;
  const int slice = blockIdx.x / chunks;
  const int chunk = blockIdx.x - slice * chunks;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, g = lane >> 4;
  const size_t kb = view_base(kw, slice, h);
  const int t_begin = chunk * chunk_len;
  const int t_end = min(n, t_begin + chunk_len);

  __shared__ u32x4 u_lds[AT][KS][kWave];
  __shared__ float red[NW][16 * AT];
  const __bf16* Uh = qt + (size_t)slice * m * D;
  Stage<AT * KS * kWave, NW * kWave> ust;
  stage_load(ust, [&](int idx) {
    const int j = idx / (KS * kWave), kk = (idx / kWave) % KS, l = idx & 63;
    const int a = min(16 * j + (l & 15), m - 1);
    return *(const u32x4*)(Uh + (size_t)a * D + 8 * KS * (l >> 4) + 8 * kk);
  });
  u32x4 kr[KS];
  load_rows<D>(K, kb, kw.st, t_begin + 16 * w + c, n, g, kr);
  stage_store(ust, &u_lds[0][0][0]);
  __syncthreads();

  float mx[AT][4];
#pragma unroll
  for (int j = 0; j < AT; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) mx[j][r] = -INFINITY;
  for (int t0 = t_begin + 16 * w; t0 < t_end; t0 += 16 * NW) {
    u32x4 kn[KS];
    load_rows<D>(K, kb, kw.st, t0 + 16 * NW + c, n, g, kn);   // rows clamped to the slice
    const bool ok = t0 + c < t_end;
#pragma unroll
    for (int j = 0; j < AT; ++j) {
      f32x4 acc = zero4();
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) acc = mfma_bf16(as_bf16x8(u_lds[j][kk][lane]), as_bf16x8(kr[kk]), acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) mx[j][r] = ok ? fmaxf(mx[j][r], acc[r]) : mx[j][r];
    }
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) kr[kk] = kn[kk];
  }
  // lane (c, g) holds landmarks 16j + 4g + r over its tokens; reduce over the 16 lanes c
#pragma unroll
  for (int j = 0; j < AT; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float v = row16_max(mx[j][r]);
      if (c == 0) red[w][16 * j + 4 * g + r] = v;
    }
  __syncthreads();
  if ((int)threadIdx.x < 16 * AT) {
    float M = red[0][threadIdx.x];
#pragma unroll
    for (int ww = 1; ww < NW; ++ww) M = fmaxf(M, red[ww][threadIdx.x]);
    cmax[((size_t)slice * chunks + chunk) * 16 * AT + threadIdx.x] = M;
  }
}

// Per slice: F3 V from the chunk partials, F2 from the landmark rows, Z = F2^-1 (F3 V) by
// Gauss-Jordan elimination with partial pivoting on the augmented matrix [F2 | F3 V] in LDS
// (fp32), Z written as pass 2's W operands (rows of padded landmarks zero).
// Partials: part[slice][chunk][jt][dt][r][lane] = sum_t e_(16jt+4g+r, t) v_(t, 16dt+c) and
// dpart[slice][chunk][a] = sum_t e_(a, t), as pass 1 leaves them.
template <int D, int AT>
__global__ __launch_bounds__(256, 1)
void nys_solve(const float* __restrict__ part, const float* __restrict__ dpart,
               const __bf16* __restrict__ qt, const __bf16* __restrict__ kt,
               __bf16* __restrict__ Wop, int m, int chunks, float c2) {
  constexpr int MPAD = 16 * AT, DT = D / 16, MP = AT / 2, LD = MPAD + D + 1, T = 256;
  const int slice = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  __shared__ float Mx[MPAD * LD];                         // [F2 | F3 V], row stride LD
  __shared__ __attribute__((aligned(16))) __bf16 ql[MPAD * D], kl[MPAD * D];
  __shared__ float zl[MPAD], fcol[MPAD];
  __shared__ int piv_s;

  // landmark rows (rows >= m zero; they are never read)
  {
    const u32x4* qs = (const u32x4*)(qt + (size_t)slice * m * D);
    const u32x4* ks = (const u32x4*)(kt + (size_t)slice * m * D);
    Stage<MPAD * D / 8, T> qst, kst;
    stage_load(qst, [&](int i) { return (i < m * D / 8) ? qs[i] : u32x4{0u, 0u, 0u, 0u}; });
    stage_load(kst, [&](int i) { return (i < m * D / 8) ? ks[i] : u32x4{0u, 0u, 0u, 0u}; });
    stage_store(qst, (u32x4*)ql);
    stage_store(kst, (u32x4*)kl);
  }
  // chunk sums in chunk order: thread (r, lane) = tid owns slot r*64 + lane of every tile
  {
    const int r = tid >> 6, g = lane >> 4, cc = lane & 15;
    float p[AT][DT];
#pragma unroll
    for (int ja = 0; ja < AT; ++ja)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) p[ja][dt] = 0.f;
    float z = 0.f;
    for (int ch = 0; ch < chunks; ++ch) {
      const size_t sc = (size_t)slice * chunks + ch;
      float v[AT][DT];
#pragma unroll
      for (int ja = 0; ja < AT; ++ja)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) v[ja][dt] = part[((sc * AT + ja) * DT + dt) * 256 + tid];
      const float dz = (tid < MPAD) ? dpart[sc * MPAD + tid] : 0.f;
#pragma unroll
      for (int ja = 0; ja < AT; ++ja)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) p[ja][dt] += v[ja][dt];
      z += dz;
    }
#pragma unroll
    for (int ja = 0; ja < AT; ++ja)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        Mx[(16 * ja + 4 * g + r) * LD + MPAD + 16 * dt + cc] = p[ja][dt];
    if (tid < MPAD) zl[tid] = z;
  }
  __syncthreads();
  // F3 V = P / z (z >= 1: each landmark's largest weight is exp(0)); F2 logits
  for (int e = tid; e < m * D; e += T) {
    const int a = e / D, k = e - a * D;
    Mx[a * LD + MPAD + k] /= zl[a];
  }
  for (int e = tid; e < m * m; e += T) {
    const int a = e / m, l = e - a * m;
    float acc = 0.f;
#pragma unroll 8
    for (int k = 0; k < D; ++k) acc = fmaf((float)ql[a * D + k], (float)kl[l * D + k], acc);
    Mx[a * LD + l] = acc;
  }
  __syncthreads();
  // row softmax of F2 over the m landmark keys (one thread per row)
  if (tid < m) {
    float* row = Mx + tid * LD;
    float mx = row[0];
    for (int l = 1; l < m; ++l) mx = fmaxf(mx, row[l]);
    float z = 0.f;
    for (int l = 0; l < m; ++l) {
      const float e = exp2_fast((row[l] - mx) * c2);
      row[l] = e;
      z += e;
    }
    const float iz = 1.f / z;
    for (int l = 0; l < m; ++l) row[l] *= iz;
  }
  __syncthreads();

  // Gauss-Jordan: pivot column col, updated columns (col, m) and the D right-hand sides.
  for (int col = 0; col < m; ++col) {
    const int nl = m - col - 1, ncols = nl + D;
    if (w == 0) {
      float best = -1.f;
      int bi = col;
      for (int r = col + lane; r < m; r += 64) {
        const float v = fabsf(Mx[r * LD + col]);
        if (v > best) { best = v; bi = r; }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const float ob = __shfl_xor(best, o);
        const int oi = __shfl_xor(bi, o);
        if (ob > best || (ob == best && oi < bi)) { best = ob; bi = oi; }
      }
      // multipliers of the rows after the swap of rows col and bi (row col: the pivot row)
      for (int r = lane; r < m; r += 64) {
        const float v = (r == bi) ? Mx[col * LD + col] : Mx[r * LD + col];
        fcol[r] = (r == col) ? 0.f : v;
      }
      if (lane == 0) piv_s = bi;
    }
    __syncthreads();
    // the swap below never writes column col, so the pivot stays readable
    const int p = piv_s;
    const float ipv = 1.f / Mx[p * LD + col];
    for (int jj = tid; jj < ncols; jj += T) {
      const int j = (jj < nl) ? col + 1 + jj : MPAD + (jj - nl);
      const float a = Mx[col * LD + j], b = Mx[p * LD + j];
      Mx[p * LD + j] = a;
      Mx[col * LD + j] = b * ipv;
    }
    __syncthreads();
    for (int e = tid; e < m * ncols; e += T) {
      const int r = e / ncols, jj = e - r * ncols;
      if (r == col) continue;
      const int j = (jj < nl) ? col + 1 + jj : MPAD + (jj - nl);
      Mx[r * LD + j] = fmaf(-fcol[r], Mx[col * LD + j], Mx[r * LD + j]);
    }
    __syncthreads();
  }
  // Z as W operands (anchor a = landmark, dim k)
  __bf16* dst = Wop + (size_t)slice * MPAD * D;
  for (int e = tid; e < MPAD * D; e += T) {
    const int a = e / D, k = e - a * D;
    dst[wt_layout_index<D>(MP, a, k)] = (__bf16)((a < m) ? Mx[a * LD + MPAD + k] : 0.f);
  }
}

// ---------------------------------------------------------------------------------------
template <int D, int AT>
static void launch_nys_kernels_t(const Geometry& g, const SplitPlan& p, const NystromBuffers& nb,
                                 const void* K, hipStream_t s, bool solve) {
  if (!solve) {
    nys_max<D, AT><<<dim3((unsigned)(g.slices * p.chunks1)), dim3(256), 0, s>>>(
        (const __bf16*)K, nb.qt, nb.cmax, g.vw.q, g.h, g.n, g.m, p.chunks1, p.chunk_len1);
  } else {
    nys_solve<D, AT><<<dim3((unsigned)g.slices), dim3(256), 0, s>>>(
        nb.part, nb.dpart, nb.qt, nb.kt, nb.wop, g.m, p.chunks1, g.c2);
  }
}

template <int D>
static hipError_t launch_nys_t(const Geometry& g, const SplitPlan& p, const NystromBuffers& nb,
                               const void* K, hipStream_t s, bool solve) {
  switch (g.at) {
    case 2: launch_nys_kernels_t<D, 2>(g, p, nb, K, s, solve); break;
    case 4: launch_nys_kernels_t<D, 4>(g, p, nb, K, s, solve); break;
    case 6: launch_nys_kernels_t<D, 6>(g, p, nb, K, s, solve); break;
    case 8: launch_nys_kernels_t<D, 8>(g, p, nb, K, s, solve); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_nystrom_bf16(const Geometry& g, const SplitPlan& p, const void* Q, const void* K,
                               const void* V, const int* idx, void* H, const NystromBuffers& nb,
                               hipStream_t stream) {
  if (g.d != 32 && g.d != 64) return hipErrorInvalidValue;
  auto step = [&](bool solve) {
    return g.d == 64 ? launch_nys_t<64>(g, p, nb, K, stream, solve)
                     : launch_nys_t<32>(g, p, nb, K, stream, solve);
  };
  if (g.d == 64)
    nys_gather<64><<<dim3((unsigned)g.slices), dim3(256), 0, stream>>>(
        (const __bf16*)Q, (const __bf16*)K, idx, nb.qt, nb.kt, g.h, g.n, g.m);
  else
    nys_gather<32><<<dim3((unsigned)g.slices), dim3(256), 0, stream>>>(
        (const __bf16*)Q, (const __bf16*)K, idx, nb.qt, nb.kt, g.h, g.n, g.m);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if ((e = step(false)) != hipSuccess) return e;
  e = launch_nystrom_pass1_bf16(g, p, K, g.vw.q, nb.qt, V, g.vw.v, nb.part, nb.dpart, nb.cmax,
                                stream);
  if (e != hipSuccess) return e;
  if ((e = step(true)) != hipSuccess) return e;
  return launch_nystrom_pass2_bf16(g, p, Q, g.vw.q, nb.kt, nb.wop, H, g.vw.o, stream);
}

}  // namespace aa
