// nystrom_bf16.hip -- Nystrom attention with given landmark tokens (bf16 in and out, fp32
// accumulation).
//
// Fast Nystrom Attention page (key machinery): the attention matrix is approximated by three
// row softmaxes through s landmark rows q = Q[idx], k = K[idx], the middle one inverted.  Per
// (batch, head) slice, with c = 1/sqrt(d):
//   F1 = rowsoftmax(Q k^T c) (n x s),  F2 = rowsoftmax(q k^T c) (s x s),
//   F3 = rowsoftmax(q K^T c) (s x n),  H = F1 (F2^-1 (F3 V)).
// Three launches:
//   pass 1      (split plan, landmark mode): the landmark query rows (gathered from Q
//               through the indices) as anchors, the keys K streamed as the tokens; per
//               chunk, each landmark's largest logit q_a . k_t over the chunk (a first
//               sweep), then exp(c q_a . k_t - c M_a) accumulated against V and against
//               ones: F3 V and F3's row sums, unnormalised, with the chunk maxima M_a.
//   nys_solve   per slice: the chunks rescaled to each landmark's overall maximum and
//               summed -> F3 V; F2 in fp32 from the landmark rows (gathered through the
//               indices; the key rows are also written out for pass 2); Z = F2^-1 (F3 V) by
//               Gauss-Jordan elimination with partial pivoting; Z stored as pass 2's W
//               operands.
//   pass 2      (split plan, per-slice anchors = the landmark keys): H = rowsoftmax(Q k^T c) Z.
#include <algorithm>

#include "device_common.h"
#include "kernels.h"
#include "pass2_layout.h"
#include "tile_ops.h"

namespace aa {

// A double from lane `lane` of the wave (two 32-bit lane reads), and the double of lane
// l ^ 32.  permlane32_swap(v, v) hands each lane its own word and its partner's, in an
// order that depends on the lane's half, so the partner's word is whichever of the two
// is not the lane's own (when both are equal, either is).
__device__ __forceinline__ double readlane_f64(double v, int lane) {
  const long long b = __double_as_longlong(v);
  const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)b, lane);
  const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(b >> 32), lane);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}
__device__ __forceinline__ double swap32_f64(double v) {
  const unsigned long long b = (unsigned long long)__double_as_longlong(v);
  const unsigned bl = (unsigned)b, bh = (unsigned)(b >> 32);
  const auto lo = __builtin_amdgcn_permlane32_swap(bl, bl, false, false);
  const auto hi = __builtin_amdgcn_permlane32_swap(bh, bh, false, false);
  const unsigned pl = lo[0] == bl ? lo[1] : lo[0];
  const unsigned ph = hi[0] == bh ? hi[1] : hi[0];
  return __longlong_as_double((long long)(((unsigned long long)ph << 32) | pl));
}

// Landmark rows of Q and K for one slice into LDS (row stride RS, rows >= m zero), the
// key rows also to kt ([slice][m][d], pass 2's anchors).  T threads; Q and K contiguous
// [B, h, n, d] (view vw); indices clamped to [0, n).
template <int D, int MPAD, int T, int RS>
__device__ __forceinline__ void nys_landmark_rows(const __bf16* __restrict__ Q,
                                                  const __bf16* __restrict__ K, const View& vw,
                                                  const int* __restrict__ idx, int slice, int h,
                                                  int n, int m, int tid, __bf16* ql, __bf16* kl,
                                                  __bf16* __restrict__ kt) {
  constexpr int CH = D / 8, N = MPAD * CH;
  const size_t base = view_base(vw, slice, h);
  const int* ib = idx + (size_t)(slice / h) * m;
  auto src = [&](int i) {
    const int a = i / CH, k8 = i - a * CH;
    const int tok = min(max(ib[min(a, m - 1)], 0), n - 1);
    return base + (size_t)((long long)tok * vw.st) + 8 * k8;
  };
  Stage<N, T> qst, kst;
  stage_load(qst, [&](int i) { return (i < m * CH) ? *(const u32x4*)(Q + src(i)) : u32x4{0u, 0u, 0u, 0u}; });
  stage_load(kst, [&](int i) { return (i < m * CH) ? *(const u32x4*)(K + src(i)) : u32x4{0u, 0u, 0u, 0u}; });
#pragma unroll
  for (int i = 0; i < Stage<N, T>::kPer; ++i) {
    const int e = tid + i * T;
    if (N % T == 0 || e < N) {
      const int a = e / CH, k8 = e - a * CH;
      *(u32x4*)(ql + a * RS + 8 * k8) = qst.r[i];
      *(u32x4*)(kl + a * RS + 8 * k8) = kst.r[i];
      if (a < m) *(u32x4*)(kt + ((size_t)slice * m + a) * D + 8 * k8) = kst.r[i];
    }
  }
}

// F3 V (unnormalised) and F3's row sums from the chunk partials: chunk c's weights are
// relative to its own maxima M_c (cmax), so each chunk is scaled by exp(c (M_c - M)) with M
// the landmark's overall maximum, and the chunks are added in chunk order.  Partial
// element f of a chunk: tile f / 256 = (jt, dt), slot r * 64 + l, i.e. landmark
// 16 jt + 4 (l / 16) + r, dim 16 dt + l % 16.  Results go to Mx[a * LD + MPAD + k] and
// zl[a].  T threads; Ml and facl are LDS scratch (MPAD and 2 x MPAD floats).
template <int D, int AT, int T, int LD>
__device__ __forceinline__ void nys_rhs(const float* __restrict__ part,
                                        const float* __restrict__ dpart,
                                        const float* __restrict__ cmax, int slice, int chunks,
                                        int m, float c2, int tid, float* Mx, float* zl,
                                        float* Ml, float (*facl)[16 * AT]) {
  constexpr int MPAD = 16 * AT, DT = D / 16, EPT = (MPAD * D + T - 1) / T;
  const float* cm = cmax + (size_t)slice * chunks * MPAD;
  // a chunk's partials (indices clamped, so the loads are unconditional)
  const int tc = min(tid, MPAD - 1);
  auto load_chunk = [&](int ch, float* v, float& dz, float& cmv) {
    const size_t sc = (size_t)slice * chunks + min(ch, chunks - 1);
    const float* src = part + sc * MPAD * D;
#pragma unroll
    for (int e = 0; e < EPT; ++e) v[e] = src[min(tid + e * T, MPAD * D - 1)];
    dz = dpart[sc * MPAD + tc];
    cmv = cm[(sc - (size_t)slice * chunks) * MPAD + tc];
  };
  float v[EPT], dz, cmv;
  load_chunk(0, v, dz, cmv);
  {  // each landmark's overall maximum, four chunks' maxima in flight at a time
    float M = -INFINITY;
    for (int ch = 0; ch < chunks; ch += 4) {
      float mc[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) mc[i] = cm[(size_t)min(ch + i, chunks - 1) * MPAD + tc];
#pragma unroll
      for (int i = 0; i < 4; ++i) M = fmaxf(M, mc[i]);
    }
    if (tid < MPAD) Ml[tid] = M;
  }
  float acc[EPT], z = 0.f;
#pragma unroll
  for (int e = 0; e < EPT; ++e) acc[e] = 0.f;
  for (int ch = 0; ch < chunks; ++ch) {
    // the next chunk's partials are requested before this chunk is used
    float vn[EPT], dzn, cmvn;
    load_chunk(ch + 1, vn, dzn, cmvn);
    __syncthreads();   // Ml written; the previous use of this facl buffer is over
    if (tid < MPAD) facl[ch & 1][tid] = (tid < m) ? exp2_fast((cmv - Ml[tid]) * c2) : 0.f;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const int f = tid + e * T, slot = f & 255, l = slot & 63;
      const int a = 16 * ((f >> 8) / DT) + 4 * (l >> 4) + (slot >> 6);
      if (f < MPAD * D) acc[e] = fmaf(facl[ch & 1][a], v[e], acc[e]);
    }
    if (tid < MPAD) z = fmaf(facl[ch & 1][tid], dz, z);
#pragma unroll
    for (int e = 0; e < EPT; ++e) v[e] = vn[e];
    dz = dzn;
    cmv = cmvn;
  }
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int f = tid + e * T;
    if (f < MPAD * D) {
      const int tile = f >> 8, slot = f & 255, jt = tile / DT, dt = tile - jt * DT;
      const int l = slot & 63, a = 16 * jt + 4 * (l >> 4) + (slot >> 6), k = 16 * dt + (l & 15);
      Mx[a * LD + MPAD + k] = acc[e];
    }
  }
  if (tid < MPAD) zl[tid] = z;
}

// Per slice: F3 V from the chunk partials, F2 from the landmark rows, Z = F2^-1 (F3 V) by
// Gauss-Jordan elimination with partial pivoting (fp32), Z written as pass 2's W operands.
// Partials: part[slice][chunk][jt][dt][r][lane] = sum_t e_(16jt+4g+r, t) v_(t, 16dt+c) and
// dpart[slice][chunk][a] = sum_t e_(a, t), as pass 1 leaves them.
//
// The system is padded to MPAD = 16 AT unknowns with identity rows (zero right-hand
// sides), so the elimination runs a compile-time number of steps.  The augmented matrix
// [F2 | F3 V] (MPAD x (MPAD + D)) lives in registers: wave w owns CW consecutive columns
// (32 up to 64 unknowns, else 16), lane l rows l and l + 64.  Rows are never swapped: the
// row chosen as pivot at step col ends holding unknown col (see the elimination loop).
template <int D, int AT>
constexpr int nys_solve_cw() { return 16 * AT <= 64 ? 32 : 16; }   // columns per wave
template <int D, int AT>
constexpr int nys_solve_waves() { return (16 * AT + D) / nys_solve_cw<D, AT>(); }

template <int D, int AT>
__global__ __launch_bounds__((nys_solve_waves<D, AT>() * kWave), 1)
void nys_solve(const float* __restrict__ part, const float* __restrict__ dpart,
               const float* __restrict__ cmax, const __bf16* __restrict__ Q,
               const __bf16* __restrict__ K, View vw, const int* __restrict__ idx,
               __bf16* __restrict__ kt, __bf16* __restrict__ Wop, int h, int n, int m,
               int chunks, float c2) {
  constexpr int MPAD = 16 * AT, MP = AT / 2, NC = MPAD + D, LD = NC + 1;
  constexpr int NG = nys_solve_waves<D, AT>(), T = NG * kWave, RPL = (MPAD + 63) / 64;
  constexpr int CW = nys_solve_cw<D, AT>();
  static_assert(MPAD % CW == 0 && D % CW == 0, "column groups of CW");
  const int slice = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  __shared__ float Mx[MPAD * LD];                         // set-up only
  // landmark rows with a row stride of D + 8 bf16 (144 or 80 bytes), so that the rows read
  // together by neighbouring threads fall on different LDS banks
  constexpr int RS = D + 8;
  __shared__ __attribute__((aligned(16))) __bf16 ql[MPAD * RS], kl[MPAD * RS];
  __shared__ float zl[MPAD];
  __shared__ double fbuf[2][MPAD];
  __shared__ int pbuf[2];
  __shared__ double pvbuf[2];

  __shared__ float Ml[MPAD], facl[2][MPAD];
  nys_landmark_rows<D, MPAD, T, RS>(Q, K, vw, idx, slice, h, n, m, tid, ql, kl, kt);
  nys_rhs<D, AT, T, LD>(part, dpart, cmax, slice, chunks, m, c2, tid, Mx, zl, Ml, facl);
  // F2 logits (fp32 sums of the bf16 products), identity rows and zero columns for padding
  for (int e = tid; e < MPAD * MPAD; e += T) {
    const int a = e / MPAD, l = e - a * MPAD;
    float v;
    if (a < m && l < m) {
      const u32x4* qa = (const u32x4*)(ql + a * RS);
      const u32x4* kb = (const u32x4*)(kl + l * RS);
      v = 0.f;
#pragma unroll
      for (int k8 = 0; k8 < D / 8; ++k8) {
        const bf16x8 x = as_bf16x8(qa[k8]), y = as_bf16x8(kb[k8]);
#pragma unroll
        for (int u = 0; u < 8; ++u) v = fmaf((float)x[u], (float)y[u], v);
      }
    } else {
      v = (a == l && a >= m) ? 1.f : 0.f;
    }
    Mx[a * LD + l] = v;
  }
  __syncthreads();
  // F3 V = P / z (z >= 1: each landmark's largest weight is exp(0)); zero rows for padding
  for (int e = tid; e < MPAD * D; e += T) {
    const int a = e / D, k = e - a * D;
    Mx[a * LD + MPAD + k] = (a < m) ? Mx[a * LD + MPAD + k] / zl[a] : 0.f;
  }
  // row softmax of F2 over the m landmark keys: one wave per row, lanes over the keys
  for (int a = w; a < m; a += NG) {
    float* row = Mx + a * LD;
    float e[RPL], mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
      const int l = lane + 64 * i;
      e[i] = (l < m) ? row[l] : -INFINITY;
      mx = fmaxf(mx, e[i]);
    }
    mx = xor32_max(xor16_max(row16_max(mx)));
    float z = 0.f;
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
      e[i] = exp2_fast((e[i] - mx) * c2);   // 0 for l >= m
      z += e[i];
    }
    z = xor32_sum(xor16_sum(row16_sum(z)));
    const float iz = 1.f / z;
#pragma unroll
    for (int i = 0; i < RPL; ++i)
      if (lane + 64 * i < m) row[lane + 64 * i] = e[i] * iz;
  }
  __syncthreads();

  // the elimination in fp64: with a sink token among the landmarks F2's condition number
  // reaches 1e14, beyond what fp32 can invert, while H (in which Z's huge components
  // cancel) stays well defined
  double x[RPL][CW];
  bool used[RPL];
  int var[RPL];
#pragma unroll
  for (int i = 0; i < RPL; ++i) {
    const int r = lane + 64 * i;
    used[i] = r >= MPAD;   // lanes past the padded system never pivot
    var[i] = 0;
#pragma unroll
    for (int jj = 0; jj < CW; ++jj) x[i][jj] = (r < MPAD) ? (double)Mx[r * LD + CW * w + jj] : 0.0;
  }

  // Step col: the wave owning column col picks the pivot among the unused rows (largest
  // |value| as a float, smallest row on ties: wave maximum with DPP and permlane swaps, the
  // row from a ballot; a column holding NaN takes its first unused row) and publishes the
  // column, the pivot row and its value through LDS; after one barrier every wave still
  // holding columns >= col takes the pivot row from that lane of its own registers
  // (readlane) and subtracts (x_r[col] / pivot) times it from every other row.  The pivot
  // row is left unscaled (its own factor is zero); unknown col is its right-hand side over
  // the pivot, divided out at the end.  Steps run in groups of CW (the column group W,
  // uniform), unrolled within a group so that register indices are static.
  double pvr[RPL];
#pragma unroll
  for (int i = 0; i < RPL; ++i) pvr[i] = 1.0;
  for (int W = 0; W < MPAD / CW; ++W) {
#pragma unroll
  for (int jc = 0; jc < CW; ++jc) {
    const int col = CW * W + jc, b = jc & 1;
    if (w == W) {
      float v[RPL], best = -1.f;
#pragma unroll
      for (int i = 0; i < RPL; ++i) {
        v[i] = used[i] ? -1.f : (float)fabs(x[i][jc]);
        best = fmaxf(best, v[i]);
      }
      best = xor32_max(xor16_max(row16_max(best)));
      int bi = MPAD, bu = MPAD;
#pragma unroll
      for (int i = RPL - 1; i >= 0; --i) {
        const unsigned long long bal = __ballot(!used[i] && v[i] == best);
        const unsigned long long un = __ballot(!used[i]);
        if (bal) bi = 64 * i + __builtin_ctzll(bal);
        if (un) bu = 64 * i + __builtin_ctzll(un);
      }
      if (bi == MPAD) bi = bu;
#pragma unroll
      for (int i = 0; i < RPL; ++i) {
        const int r = lane + 64 * i;
        if (r < MPAD) fbuf[b][r] = x[i][jc];
        if (r == bi) pvbuf[b] = x[i][jc];
      }
      if (lane == 0) pbuf[b] = bi;
    }
    __syncthreads();
    if (CW * w + CW - 1 < col) continue;   // this wave's columns are all eliminated
    const int p = __builtin_amdgcn_readfirstlane(pbuf[b]);
    const double pv = pvbuf[b];
    // 1 / pv: the hardware reciprocal refined by one Newton step
    double ipv = __builtin_amdgcn_rcp(pv);
    ipv = fma(ipv, fma(-pv, ipv, 1.0), ipv);
    const int ip = p >> 6, lp = p & 63;
    double f[RPL];
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
      const int r = lane + 64 * i;
      const bool piv = (r == p);
      if (piv) { used[i] = true; var[i] = col; pvr[i] = pv; }
      f[i] = (piv || r >= MPAD) ? 0.0 : fbuf[b][r] * ipv;
    }
#pragma unroll
    for (int jj = 0; jj < CW; ++jj) {
      double xv = x[0][jj];
#pragma unroll
      for (int i = 1; i < RPL; ++i) xv = (ip == i) ? x[i][jj] : xv;
      const double pr = readlane_f64(xv, lp);
#pragma unroll
      for (int i = 0; i < RPL; ++i) x[i][jj] = fma(-f[i], pr, x[i][jj]);
    }
  }
  }
  // Z[var][k]: the right-hand-side waves hold unknown var[i] in row lane + 64 i
  if (CW * w >= MPAD) {
    __bf16* dst = Wop + (size_t)slice * MPAD * D;
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
      if (lane + 64 * i >= MPAD) continue;
      const int a = var[i];
#pragma unroll
      for (int jj = 0; jj < CW; ++jj) {
        const int k = CW * w - MPAD + jj;
        dst[w2_layout_index(MP, a, k)] = (__bf16)(float)((a < m) ? x[i][jj] / pvr[i] : 0.0);
      }
    }
  }
}

// The same solve for up to 32 landmarks with F2's part of the elimination in one wave.
// Wave 0 holds F2 (lane l: row l % MPAD; column group l / MPAD holds the interleaved
// columns 2j + group, so that the columns already eliminated die in both groups at once
// and are no longer updated), finds each step's pivot and the rows' multipliers, and
// hands them to the other waves through LDS; wave 1 + r holds right-hand-side columns
// 2RC r .. 2RC r + 2RC - 1 (RC per column group) and applies each step one barrier later.
//   set-up: landmark rows of Q and K into LDS; F3 V from the chunk partials in chunk
//           order (all waves); F2's logits on the MFMA (fp32 sums of the bf16 products)
//           and its row softmax (wave 0); the matrix into the lanes' registers;
//   step k: wave 0: the largest |x[k]| among unused rows (smallest row on ties), its
//           pivot value by readlane, the multipliers x[k] / pivot (0 on the pivot row)
//           and the pivot row published, and x -= multiplier * pivot row on its F2
//           columns; the right-hand-side waves apply step k - 1 the same way, their own
//           pivot row exchanged through LDS inside each wave.  Unknown k ends in the
//           pivot row's right-hand side over its pivot.
template <int D, int RC>
constexpr int nys_solve1_waves() { return 1 + D / (2 * RC); }
// right-hand-side columns per lane in the solve up to 32 landmarks
constexpr int kNysRhsCols = 8;

template <int D, int AT, int RC>
__global__ __launch_bounds__((nys_solve1_waves<D, RC>() * kWave), 1)
void nys_solve1(const float* __restrict__ part, const float* __restrict__ dpart,
                const float* __restrict__ cmax, const __bf16* __restrict__ Q,
                const __bf16* __restrict__ K, View vw, const int* __restrict__ idx,
                __bf16* __restrict__ kt, __bf16* __restrict__ Wop, int h, int n, int m,
                int chunks, float c2) {
  constexpr int MPAD = 16 * AT, NC = MPAD + D, NW = nys_solve1_waves<D, RC>(), T = NW * kWave;
  constexpr int G = 2, CPL = 16;   // two column groups of 16 registers in every wave
  constexpr int KS = D / 32, MP = AT / 2, LD = NC + 1, RS = D + 8;
  static_assert(MPAD == 32 && G * MPAD == kWave && G * CPL == MPAD, "32 rows, two groups");
  static_assert(RC <= CPL && (NW - 1) * G * RC == D, "2 RC right-hand-side columns per wave");
  const int slice = blockIdx.x;
  const int tid = threadIdx.x, w = tid / kWave, lane = tid % kWave;
  const int c = lane & 15, g = lane >> 4;
  const int row = lane % MPAD, grp = lane / MPAD;
  __shared__ float Mx[MPAD * LD];
  __shared__ __attribute__((aligned(16))) __bf16 ql[MPAD * RS], kl[MPAD * RS];
  __shared__ float zl[MPAD];
  __shared__ __attribute__((aligned(16))) double prow[NW][2][G][CPL];   // by step parity
  __shared__ double fkl[2][MPAD];   // a step's multipliers, by step parity
  __shared__ int pkl[2];            // a step's pivot row
  __shared__ double pvl[MPAD];      // each row's pivot
  __shared__ int varl[MPAD];        // the unknown each row ends with
  __shared__ float Ml[MPAD], facl[2][MPAD];
  nys_landmark_rows<D, MPAD, T, RS>(Q, K, vw, idx, slice, h, n, m, tid, ql, kl, kt);
  nys_rhs<D, AT, T, LD>(part, dpart, cmax, slice, chunks, m, c2, tid, Mx, zl, Ml, facl);
  __syncthreads();
  // F2 = rowsoftmax(q k^T c) (wave 0): logits q_a . k_l on the MFMA, tile (ti, tj), lane
  // (c,g) ends with a = 16ti + 4g + r, l = 16tj + c; each row's maximum and sum over its m
  // columns across the 16 lanes c (DPP); padded rows become identity rows
  if (w == 0) {
    f32x4 f2[AT][AT];
#pragma unroll
    for (int ti = 0; ti < AT; ++ti)
#pragma unroll
      for (int tj = 0; tj < AT; ++tj) {
        f32x4 acc = zero4();
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
          const bf16x8 x = as_bf16x8(*(const u32x4*)(ql + (16 * ti + c) * RS + 8 * KS * g + 8 * kk));
          const bf16x8 y = as_bf16x8(*(const u32x4*)(kl + (16 * tj + c) * RS + 8 * KS * g + 8 * kk));
          acc = mfma_bf16(x, y, acc);
        }
        f2[ti][tj] = acc;
      }
#pragma unroll
    for (int ti = 0; ti < AT; ++ti)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int a = 16 * ti + 4 * g + r;
        float mx = -INFINITY;
#pragma unroll
        for (int tj = 0; tj < AT; ++tj) mx = (16 * tj + c < m) ? fmaxf(mx, f2[ti][tj][r]) : mx;
        mx = row16_max(mx);
        float e[AT], z = 0.f;
#pragma unroll
        for (int tj = 0; tj < AT; ++tj) {
          e[tj] = (16 * tj + c < m) ? exp2_fast((f2[ti][tj][r] - mx) * c2) : 0.f;
          z += e[tj];
        }
        const float iz = 1.f / row16_sum(z);
#pragma unroll
        for (int tj = 0; tj < AT; ++tj) {
          const int l = 16 * tj + c;
          Mx[a * LD + l] = (a < m) ? e[tj] * iz : ((a == l) ? 1.f : 0.f);
        }
      }
  }
  __syncthreads();

  // the elimination in fp64 (see nys_solve); the right-hand side is F3 V over F3's row
  // sums (zero for padded landmark rows)
  const float izl = (row < m) ? 1.f / zl[row] : 0.f;   // zl >= 1: each landmark's largest weight is exp(0)
  // wave 0: register j holds F2 column 2j + grp; wave 1 + r: right-hand-side column
  // 2RC r + RC grp + j (j < RC)
  const int rhs0 = MPAD + 2 * RC * (w - 1) + RC * grp;
  double x[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    if (w == 0) {
      x[j] = (double)Mx[row * LD + G * j + grp];
    } else if (j < RC) {
      x[j] = (double)(Mx[row * LD + rhs0 + j] * izl);
    }
  }
  bool used = false;
  int var = 0;
  double pvr = 1.0;
  // wave 0 applies step k's elimination at the start of step k + 1: first to column
  // k + 1 alone, whose pivot-row value prk comes by readlane, so that step k + 1's pivot
  // search can start at once; then to its other live columns with the pivot row read
  // back from LDS a step earlier
  double fprev = 0.0, prk = 0.0;
  double pr[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) pr[j] = 0.0;
  int lp = 0;
  double f = 0.0;
  // the right-hand-side waves apply step s (multipliers and pivot row published by wave
  // 0 before the barrier that ends step s)
  auto rhs_apply = [&](int s) {
    const int b = s & 1;
    const double fr = fkl[b][row];
    const int p = pkl[b];
    if (row == p) {
#pragma unroll
      for (int j = 0; j < RC; ++j) prow[w][b][grp][j] = x[j];
    }
    // one wave: its LDS writes are done before its reads (a wait and a compiler fence)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int j = 0; j < RC; ++j) x[j] = fma(-fr, prow[w][b][grp][j], x[j]);
  };
  // fully unrolled, so that column k is a fixed register in every step
#pragma clang loop unroll(full)
  for (int k = 0; k < MPAD; ++k) {
    const int gk = k % G, kr = k / G;   // column k: register kr of group gk
    const int b = k & 1;
    if (w == 0) {
      if (grp == gk) x[kr] = fma(-fprev, prk, x[kr]);
      const bool cand = grp == gk && !used;
      const float v = cand ? (float)fabs(x[kr]) : -1.f;
      // maximum over the MPAD lanes of each group (other groups' lanes hold -1)
      float best = row16_max(v);
      best = xor16_max(best);
      // no candidate equals the maximum only when the column holds NaN: then the first
      // unused row (the output is non-finite, and every unknown still gets its row)
      const unsigned long long bal = __ballot(cand && v == best);
      const unsigned long long any = __ballot(cand);
      lp = (int)__builtin_ctzll(bal ? bal : any);
      const int p = lp - gk * MPAD;
      const double pv = readlane_f64(x[kr], lp);
      // this lane's row in column k, from the lane of group gk that holds it (the
      // exchange runs on every lane, outside any branch: a lane exchange under a
      // divergent branch reads inactive lanes)
      const double other = swap32_f64(x[kr]);
      const double xk = grp == gk ? x[kr] : other;
      // 1 / pv: the hardware reciprocal refined by one Newton step
      double ipv = __builtin_amdgcn_rcp(pv);
      ipv = fma(ipv, fma(-pv, ipv, 1.0), ipv);
      const bool piv = row == p;
      f = piv ? 0.0 : xk * ipv;
      if (piv) {
        used = true;
        var = k;
        pvr = pv;
      }
      if (grp == 0) fkl[b][row] = f;
      if (lane == 0) pkl[b] = p;
      // step k - 1 on the columns still live: registers above kr, and register kr of
      // group 1 when it holds column k + 1
#pragma unroll
      for (int j = kr + 1; j < CPL; ++j) x[j] = fma(-fprev, pr[j], x[j]);
      if (gk == 0 && grp == 1) x[kr] = fma(-fprev, pr[kr], x[kr]);
      // step k's pivot row on the columns step k + 1 updates (complete through step k - 1)
      if (piv) {
#pragma unroll
        for (int j = (k + 1) / G; j < CPL; ++j) prow[0][b][grp][j] = x[j];
      }
    } else if (k > 0) {
      rhs_apply(k - 1);
    }
    // publishes step k to every wave, and with the two buffers orders the previous
    // step's reads before the next writes
    __syncthreads();
    if (w == 0) {
#pragma unroll
      for (int j = (k + 1) / G; j < CPL; ++j) pr[j] = prow[0][b][grp][j];
      if (k + 1 < MPAD) {
        const int gk1 = (k + 1) % G, kr1 = (k + 1) / G;
        prk = readlane_f64(x[kr1], lp + (gk1 - gk) * MPAD);
      }
      fprev = f;
    }
  }
  if (w == 0) {
    if (grp == 0) {
      varl[row] = var;
      pvl[row] = pvr;
    }
  } else {
    rhs_apply(MPAD - 1);
  }
  __syncthreads();
  // Z[var][k] = right-hand side over the pivot: through LDS (row var of Mx), then out as
  // pass 2's W operands in 16-byte pieces
  if (w > 0) {
    const int vr = varl[row];
    const double ipr = (vr < m) ? 1.0 / pvl[row] : 0.0;
#pragma unroll
    for (int j = 0; j < RC; ++j) Mx[vr * LD + rhs0 + j] = (float)(x[j] * ipr);
  }
  __syncthreads();
  u32x4* dst = (u32x4*)(Wop + (size_t)slice * MPAD * D);
  constexpr int PIECES = MPAD * D / 8;
#pragma unroll
  for (int i = 0; i < (PIECES + T - 1) / T; ++i) {
    // piece q = tid + T i of [dt2][jj][lane'][8]: lane' (c', g') holds dim
    // out_dim_c(dt2, c') and anchors 32jj + 4g' + s (s < 4), 32jj + 16 + 4g' + s - 4
    const int q = tid + T * i;
    if (PIECES % T == 0 || q < PIECES) {
      const int lq = q & 63, jj = (q >> 6) % MP, dt2 = (q >> 6) / MP;
      const int k = out_dim_c(dt2, lq & 15), a0 = 32 * jj + 4 * (lq >> 4);
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = Mx[(a0 + (e < 4 ? e : 12 + e)) * LD + MPAD + k];
      dst[q] = as_u32x4(pack_bf16(f32x4{v[0], v[1], v[2], v[3]}, f32x4{v[4], v[5], v[6], v[7]}));
    }
  }
}

// ---------------------------------------------------------------------------------------
template <int D, int AT>
static void launch_nys_solve_t(const Geometry& g, const SplitPlan& p, const NystromBuffers& nb,
                               const void* Q, const void* K, const int* idx, hipStream_t s) {
  if constexpr (16 * AT <= 32 && D <= 64) {
    // F2's elimination in one wave up to 32 landmarks (at 64, a one-wave solve over all
    // 128 columns made the ViT-B/16-shape step 153 us against 122 us with the multi-wave one)
    constexpr int RC = kNysRhsCols;
    nys_solve1<D, AT, RC><<<dim3((unsigned)g.slices), dim3(nys_solve1_waves<D, RC>() * kWave), 0, s>>>(
        nb.part, nb.dpart, nb.cmax, (const __bf16*)Q, (const __bf16*)K, g.vw.q, idx, nb.kt,
        nb.wop, g.h, g.n, g.m, p.chunks1, g.c2);
  } else {
    nys_solve<D, AT><<<dim3((unsigned)g.slices), dim3(nys_solve_waves<D, AT>() * kWave), 0, s>>>(
        nb.part, nb.dpart, nb.cmax, (const __bf16*)Q, (const __bf16*)K, g.vw.q, idx, nb.kt,
        nb.wop, g.h, g.n, g.m, p.chunks1, g.c2);
  }
}

template <int D>
static hipError_t launch_nys_solve(const Geometry& g, const SplitPlan& p, const NystromBuffers& nb,
                                   const void* Q, const void* K, const int* idx, hipStream_t s) {
  switch (g.at) {
    case 2: launch_nys_solve_t<D, 2>(g, p, nb, Q, K, idx, s); break;
    case 4: launch_nys_solve_t<D, 4>(g, p, nb, Q, K, idx, s); break;
    case 6: launch_nys_solve_t<D, 6>(g, p, nb, Q, K, idx, s); break;
    case 8:
      if constexpr (D <= 64) { launch_nys_solve_t<D, 8>(g, p, nb, Q, K, idx, s); break; }
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_nystrom_bf16(const Geometry& g, const SplitPlan& p, const void* Q, const void* K,
                               const void* V, const int* idx, void* H, const NystromBuffers& nb,
                               hipStream_t stream) {
  // d = 128 up to 96 landmarks (the solve's set-up matrix would outgrow LDS above)
  if (g.d != 32 && g.d != 64 && !(g.d == 128 && g.at <= 6)) return hipErrorInvalidValue;
  hipError_t e = launch_nystrom_pass1_bf16(g, p, K, g.vw.q, Q, g.vw.q, idx, V, g.vw.v, nb.part,
                                           nb.dpart, nb.cmax, stream);
  if (e != hipSuccess) return e;
  e = g.d == 64    ? launch_nys_solve<64>(g, p, nb, Q, K, idx, stream)
      : g.d == 128 ? launch_nys_solve<128>(g, p, nb, Q, K, idx, stream)
                   : launch_nys_solve<32>(g, p, nb, Q, K, idx, stream);
  if (e != hipSuccess) return e;
  return launch_nystrom_pass2_bf16(g, p, Q, g.vw.q, nb.kt, nb.wop, H, g.vw.o, stream);
}

}  // namespace aa
