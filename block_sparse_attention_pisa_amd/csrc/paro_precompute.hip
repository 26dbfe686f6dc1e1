// Pre-computation stage of PISA ("PISA: Piecewise Sparse Attention Is Wiser
// for Efficient Diffusion Transformers", section 2, "hardware
// implementation", pre-computation; M_j from "covariance-aware routing").
//
// Per (batch, head) and block j of 64 tokens (n_j valid):
//   kbar_j = (1/n_j) sum_n k_n           vsum_j = sum_n v_n
//   H_j    = sum_n (k_n - kbar_j)^T v_n = K_j^T V_j - kbar_j^T vsum_j
//   Hbar   = (1/T) sum_j H_j             M_j = sigma_max(H_j - Hbar)
//
// Three launches on one stream:
//   1. k_block_stats   : streams K and V once; writes kbar, vsum and one
//                        partial sum of H_j per chunk of blocks (workspace).
//                        K_j^T V_j runs on bf16 MFMA 16x16x32 (exact products,
//                        fp32 accumulation) from LDS tiles transposed so that
//                        tokens are contiguous.
//   2. k_hbar_reduce   : fixed-order fp64 sum of the chunk partials -> Hbar.
//   3. k_block_spectral: re-reads K and V, rebuilds H_j in registers, forms
//                        A = H_j - Hbar and finds its largest singular value
//                        by restarted Lanczos on A^T A (fp32 vectors, fp64
//                        scalars); the final ||A x|| / ||x|| is accumulated in
//                        fp64. H_j never reaches memory.
// No float atomics anywhere: results are bitwise reproducible.
#include "paro_common.h"

namespace paro {
namespace {

constexpr int kThreads = 256;
constexpr int kLdT = kBlock + 8;  // row stride (elements) of a transposed tile

template <typename E, int D>
struct TileLds {
  E kt[D][kLdT];  // keys transposed: kt[dim][token]
  E vt[D][kLdT];  // values transposed
  float colred[2][4][D];
  float kbar[D];
  float vsum[D];
};


// H accumulator: entry (mi, nt, r) holds
//   H[16 * (MTW * wave + mi) + 4 * (lane / 16) + r][16 * nt + lane % 16],
// the C layout of the 16x16x32 MFMA. Each lane owns MTW*4 rows and D/16
// columns, so A x reduces over 16 lanes (one DPP row) and A^T y over the
// 16 lane groups of the workgroup.
template <int D>
struct HAcc {
  static constexpr int MTW = D / 64;
  static constexpr int NTT = D / 16;
  f32x4 v[MTW][NTT];
};

template <int D>
__device__ __forceinline__ int acc_row(int mi, int r) {
  const int w = threadIdx.x / 64, l = threadIdx.x % 64;
  return 16 * ((D / 64) * w + mi) + 4 * (l / 16) + r;
}
__device__ __forceinline__ int acc_col(int nt) { return 16 * nt + (threadIdx.x % 16); }

__device__ __forceinline__ uint32_t half16(const uint4& v, int e) {
  const uint32_t w = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
  return (e & 1) ? (w >> 16) : (w & 0xFFFFu);
}

// Stage rows [row0, row0 + nvalid) of a [L, D] bf16 matrix into dst[dim][token],
// zero-filling tokens >= nvalid. Each item moves 4 tokens x 8 dims: four
// 16-byte global loads (coalesced along d), eight 8-byte LDS writes.
template <int D>
__device__ __forceinline__ void stage_transposed(const uint16_t* __restrict__ src, int row0,
                                                 int nvalid, uint16_t (*dst)[kLdT]) {
  constexpr int DG = D / 8;
  for (int item = threadIdx.x; item < 16 * DG; item += kThreads) {
    const int tg = item / DG, dg = item % DG;
    uint4 r[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int tok = 4 * tg + q;
      r[q] = tok < nvalid
                 ? *reinterpret_cast<const uint4*>(src + static_cast<size_t>(row0 + tok) * D + 8 * dg)
                 : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t w0 = half16(r[0], e) | (half16(r[1], e) << 16);
      const uint32_t w1 = half16(r[2], e) | (half16(r[3], e) << 16);
      *reinterpret_cast<uint2*>(&dst[8 * dg + e][4 * tg]) = make_uint2(w0, w1);
    }
  }
}
template <int D>
__device__ __forceinline__ void stage_transposed(const float* __restrict__ src, int row0, int nvalid,
                                                 float (*dst)[kLdT]) {
  for (int e = threadIdx.x; e < kBlock * D; e += kThreads) {
    const int tok = e / D, dim = e % D;
    dst[dim][tok] = tok < nvalid ? src[static_cast<size_t>(row0 + tok) * D + dim] : 0.f;
  }
}

__device__ __forceinline__ float tile_val(uint16_t x) { return bf16_to_f32(x); }
__device__ __forceinline__ float tile_val(float x) { return x; }

// Column sums of the staged tiles; writes s.kbar (mean over nvalid) and s.vsum.
template <typename E, int D>
__device__ __forceinline__ void column_sums(TileLds<E, D>& s, int nvalid) {
  constexpr int P = kThreads / D;
  constexpr int TP = kBlock / P;
  const int a = threadIdx.x % D, part = threadIdx.x / D;
  float ks = 0.f, vs = 0.f;
#pragma unroll 8
  for (int t = 0; t < TP; ++t) {
    ks += tile_val(s.kt[a][part * TP + t]);
    vs += tile_val(s.vt[a][part * TP + t]);
  }
  s.colred[0][part][a] = ks;
  s.colred[1][part][a] = vs;
  __syncthreads();
  if (threadIdx.x < D) {
    float k = 0.f, v = 0.f;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      k += s.colred[0][p][a];
      v += s.colred[1][p][a];
    }
    s.kbar[a] = k / static_cast<float>(nvalid);
    s.vsum[a] = v;
  }
  __syncthreads();
}

// acc += K_j^T V_j from the staged transposed tiles.
template <int D>
__device__ __forceinline__ void accumulate_ktv(const TileLds<uint16_t, D>& s, HAcc<D>& acc) {
  constexpr int MTW = HAcc<D>::MTW, NTT = HAcc<D>::NTT;
  const int w = threadIdx.x / 64, l = threadIdx.x % 64;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    bf16x8 a[MTW];
#pragma unroll
    for (int mi = 0; mi < MTW; ++mi)
      a[mi] = *reinterpret_cast<const bf16x8*>(&s.kt[16 * (MTW * w + mi) + l % 16][32 * ks + 8 * (l / 16)]);
#pragma unroll
    for (int nt = 0; nt < NTT; ++nt) {
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(&s.vt[16 * nt + l % 16][32 * ks + 8 * (l / 16)]);
#pragma unroll
      for (int mi = 0; mi < MTW; ++mi) acc.v[mi][nt] = mfma16x16x32(a[mi], b, acc.v[mi][nt]);
    }
  }
}
template <int D>
__device__ __forceinline__ void accumulate_ktv(const TileLds<float, D>& s, HAcc<D>& acc) {
  constexpr int MTW = HAcc<D>::MTW, NTT = HAcc<D>::NTT;
#pragma unroll
  for (int mi = 0; mi < MTW; ++mi)
#pragma unroll
    for (int nt = 0; nt < NTT; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = acc_row<D>(mi, r), col = acc_col(nt);
        float sum = 0.f;
#pragma unroll 4
        for (int t = 0; t < kBlock; ++t) sum += s.kt[row][t] * s.vt[col][t];
        acc.v[mi][nt][r] += sum;
      }
}

template <typename E, int D>
__device__ __forceinline__ void subtract_rank1(const TileLds<E, D>& s, HAcc<D>& acc) {
#pragma unroll
  for (int mi = 0; mi < HAcc<D>::MTW; ++mi)
#pragma unroll
    for (int nt = 0; nt < HAcc<D>::NTT; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc.v[mi][nt][r] -= s.kbar[acc_row<D>(mi, r)] * s.vsum[acc_col(nt)];
}

// ------------------------------------------------------------ kernel 1
template <typename E, int D>
__global__ __launch_bounds__(kThreads) void k_block_stats(const E* __restrict__ K, const E* __restrict__ V,
                                                          float* __restrict__ kbar, float* __restrict__ vsum,
                                                          float* __restrict__ ws, int L, int T, int G, int nchunk) {
  extern __shared__ __align__(16) unsigned char smem[];
  TileLds<E, D>& s = *reinterpret_cast<TileLds<E, D>*>(smem);
  const int c = blockIdx.x, bh = blockIdx.y;
  const E* Kh = K + static_cast<size_t>(bh) * L * D;
  const E* Vh = V + static_cast<size_t>(bh) * L * D;
  HAcc<D> acc;
#pragma unroll
  for (int mi = 0; mi < HAcc<D>::MTW; ++mi)
#pragma unroll
    for (int nt = 0; nt < HAcc<D>::NTT; ++nt) acc.v[mi][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int j0 = c * G, j1 = min(T, j0 + G);
  for (int j = j0; j < j1; ++j) {
    const int row0 = j * kBlock, nvalid = min(kBlock, L - row0);
    __syncthreads();
    stage_transposed<D>(Kh, row0, nvalid, s.kt);
    stage_transposed<D>(Vh, row0, nvalid, s.vt);
    __syncthreads();
    column_sums(s, nvalid);
    if (threadIdx.x < D) {
      const size_t o = (static_cast<size_t>(bh) * T + j) * D + threadIdx.x;
      kbar[o] = s.kbar[threadIdx.x];
      vsum[o] = s.vsum[threadIdx.x];
    }
    accumulate_ktv<D>(s, acc);
    subtract_rank1(s, acc);
  }
  float* out = ws + (static_cast<size_t>(bh) * nchunk + c) * D * D;
#pragma unroll
  for (int mi = 0; mi < HAcc<D>::MTW; ++mi)
#pragma unroll
    for (int nt = 0; nt < HAcc<D>::NTT; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) out[acc_row<D>(mi, r) * D + acc_col(nt)] = acc.v[mi][nt][r];
}

// ------------------------------------------------------------ kernel 2
__global__ __launch_bounds__(256) void k_hbar_reduce(const float* __restrict__ ws, float* __restrict__ Hbar,
                                                     int D2, int nchunk, int T) {
  const int bh = blockIdx.y;
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= D2) return;
  double sum = 0.0;
  for (int c = 0; c < nchunk; ++c) sum += ws[(static_cast<size_t>(bh) * nchunk + c) * D2 + e];
  Hbar[static_cast<size_t>(bh) * D2 + e] = static_cast<float>(sum / T);
}

// ------------------------------------------------------------ kernel 3
// M_j by restarted Lanczos on B = A^T A (A = H_j - Hbar). Each cycle runs
// kLanczosK steps w = B v_k with classical Gram-Schmidt against the whole
// basis (fp32 vectors, fp64 dot products), finds the top eigenpair of the
// small tridiagonal matrix (64-point Sturm multisection across the lanes of
// one wave, then inverse iteration), restarts from the Ritz vector, and
// stops when the Ritz residual bound res^2 / (gap * theta) is negligible.
// Power iteration alone needs thousands of steps when sigma_2 / sigma_1 is
// close to 1 (blocks of i.i.d. keys); this reaches the fp32 floor in one
// cycle for almost every block. M_j = ||A x|| / ||x|| is then evaluated in
// fp64 from the fp32 Ritz vector, so its error is quadratic in the angle.
constexpr int kLanczosK = 8;
constexpr int kLanczosCycles = 16;
constexpr double kLanczosTol = 1e-10;

__device__ __forceinline__ float start_sign(int row) {
  return ((static_cast<uint32_t>(row + 1) * 2654435761u) >> 16) & 1u ? -1.f : 1.f;
}

template <int D>
struct SpectralLds {
  float xpart[16][D];           // column partials of A^T y (one row per 16-lane group)
  float vk[kLanczosK + 1][D];   // Lanczos basis
  float xs[D];                  // Ritz vector of the last cycle
  double alpha[kLanczosK];
  double beta[kLanczosK];
  double red2[16];
  double x2;
  int flag;                     // 0 running, 1 converged, 2 A == 0
};

// xpart[group][col] = sum over this lane's rows of A[row][col] * y[row].
template <int D>
__device__ __forceinline__ void write_col_partials(const HAcc<D>& A, const float (&y)[D / 64][4],
                                                   SpectralLds<D>& sp) {
  const int grp = threadIdx.x / 16;
#pragma unroll
  for (int nt = 0; nt < HAcc<D>::NTT; ++nt) {
    float p = 0.f;
#pragma unroll
    for (int mi = 0; mi < HAcc<D>::MTW; ++mi)
#pragma unroll
      for (int r = 0; r < 4; ++r) p += A.v[mi][nt][r] * y[mi][r];
    sp.xpart[grp][acc_col(nt)] = p;
  }
}

// xpart <- column partials of A^T (A x) for x = vk[k] (all threads).
template <int D>
__device__ __forceinline__ void apply_ata(const HAcc<D>& A, SpectralLds<D>& sp, int k) {
  constexpr int MTW = HAcc<D>::MTW, NTT = HAcc<D>::NTT;
  float xc[NTT];
#pragma unroll
  for (int nt = 0; nt < NTT; ++nt) xc[nt] = sp.vk[k][acc_col(nt)];
  float y[MTW][4];
#pragma unroll
  for (int mi = 0; mi < MTW; ++mi)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float p = 0.f;
#pragma unroll
      for (int nt = 0; nt < NTT; ++nt) p += A.v[mi][nt][r] * xc[nt];
      y[mi][r] = row_sum16(p);
    }
  write_col_partials<D>(A, y, sp);
}

// One Lanczos step on wave 0 (lane l holds entries l + 64 e).
template <int D>
__device__ __forceinline__ void lanczos_step(SpectralLds<D>& sp, int k, int l) {
  constexpr int E = D / 64;
  float w0[E], w[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < 16; ++q) s += sp.xpart[q][l + 64 * e];
    w0[e] = s;
    w[e] = s;
  }
  double alpha = 0.0;
#pragma unroll
  for (int kk = 0; kk < kLanczosK; ++kk) {
    if (kk <= k) {
      double part = 0.0;
#pragma unroll
      for (int e = 0; e < E; ++e) part += static_cast<double>(w0[e]) * sp.vk[kk][l + 64 * e];
      const double c = wave_sum_f64(part);
      if (kk == k) alpha = c;
      const float cf = static_cast<float>(c);
#pragma unroll
      for (int e = 0; e < E; ++e) w[e] -= cf * sp.vk[kk][l + 64 * e];
    }
  }
  double n = 0.0;
#pragma unroll
  for (int e = 0; e < E; ++e) n += static_cast<double>(w[e]) * w[e];
  const double beta = sqrt(wave_sum_f64(n));
  const float inv = beta > 0.0 ? static_cast<float>(1.0 / beta) : 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) sp.vk[k + 1][l + 64 * e] = w[e] * inv;
  if (l == 0) {
    sp.alpha[k] = alpha;
    sp.beta[k] = beta;
  }
}

// Number of eigenvalues below x of the tridiagonal (al, be): sign changes of
// the Sturm sequence p_i = det(T_i - x I), evaluated without division.
__device__ __forceinline__ int sturm_below(const double (&al)[kLanczosK], const double (&be)[kLanczosK], double x) {
  double p0 = 1.0, p1 = al[0] - x;
  int changes = p1 < 0.0 ? 1 : 0;
#pragma unroll
  for (int i = 1; i < kLanczosK; ++i) {
    const double p2 = (al[i] - x) * p1 - be[i - 1] * be[i - 1] * p0;
    changes += ((p2 < 0.0) != (p1 < 0.0)) ? 1 : 0;
    p0 = p1;
    p1 = p2;
  }
  return changes;
}

// Bracket the m-th largest eigenvalue inside [lo, hi] by 64-point multisection.
__device__ __forceinline__ void multisect(const double (&al)[kLanczosK], const double (&be)[kLanczosK], int m,
                                          int rounds, double& lo, double& hi, int l) {
  for (int r = 0; r < rounds; ++r) {
    const double step = (hi - lo) / 65.0;
    const double x = lo + step * (l + 1);
    const bool above = kLanczosK - sturm_below(al, be, x) >= m;  // x still below theta_m
    const int c = __builtin_popcountll(__ballot(above));
    const double nlo = c > 0 ? lo + step * c : lo;
    const double nhi = c < 64 ? lo + step * (c + 1) : hi;
    lo = nlo;
    hi = nhi;
  }
}

// End of a cycle on wave 0: Ritz pair, convergence test, restart vector.
template <int D>
__device__ __forceinline__ void lanczos_restart(SpectralLds<D>& sp, int l, bool last) {
  constexpr int K = kLanczosK, E = D / 64;
  double al[K], be[K];
#pragma unroll
  for (int i = 0; i < K; ++i) {
    al[i] = sp.alpha[i];
    be[i] = sp.beta[i];
  }
  double lo = al[0], hi = al[0];
#pragma unroll
  for (int i = 0; i < K; ++i) {
    const double r = (i > 0 ? fabs(be[i - 1]) : 0.0) + (i < K - 1 ? fabs(be[i]) : 0.0);
    lo = fmin(lo, al[i] - r);
    hi = fmax(hi, al[i] + r);
  }
  double lo1 = lo, hi1 = hi, lo2 = lo, hi2 = hi;
  multisect(al, be, 1, 9, lo1, hi1, l);
  multisect(al, be, 2, 5, lo2, hi2, l);
  const double theta = 0.5 * (lo1 + hi1);
  // inverse iteration with (mu I - T), mu just above theta: positive definite
  const double mu = theta + fmax(fabs(theta) * 1e-13, 1e-300);
  double s[K];
#pragma unroll
  for (int i = 0; i < K; ++i) s[i] = 1.0;
  for (int pass = 0; pass < 2; ++pass) {
    double cp[K], bp[K];
    double den = mu - al[0];
    den = fmax(den, 1e-300);
    cp[0] = -be[0] / den;
    bp[0] = s[0] / den;
#pragma unroll
    for (int i = 1; i < K; ++i) {
      den = (mu - al[i]) + be[i - 1] * cp[i - 1];
      den = fmax(den, 1e-300);
      cp[i] = -be[i] / den;
      bp[i] = (s[i] + be[i - 1] * bp[i - 1]) / den;
    }
    s[K - 1] = bp[K - 1];
#pragma unroll
    for (int i = K - 2; i >= 0; --i) s[i] = bp[i] - cp[i] * s[i + 1];
    double n = 0.0;
#pragma unroll
    for (int i = 0; i < K; ++i) n += s[i] * s[i];
    const double inv = 1.0 / sqrt(n);
#pragma unroll
    for (int i = 0; i < K; ++i) s[i] *= inv;
  }
  const double res = fabs(be[K - 1] * s[K - 1]);
  const double gap = theta - hi2;
  const bool conv = res == 0.0 || (gap > 0.0 && theta > 0.0 && res * res < kLanczosTol * gap * theta);
  float x[E];
  double n = 0.0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < K; ++i) acc += static_cast<float>(s[i]) * sp.vk[i][l + 64 * e];
    x[e] = acc;
    n += static_cast<double>(acc) * acc;
  }
  n = wave_sum_f64(n);
  const float inv = n > 0.0 ? static_cast<float>(1.0 / sqrt(n)) : 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    sp.xs[l + 64 * e] = x[e];
    sp.vk[0][l + 64 * e] = x[e] * inv;
  }
  if (l == 0) sp.flag = (conv || last) ? 1 : 0;
}

template <typename E, int D>
__global__ __launch_bounds__(kThreads) void k_block_spectral(const E* __restrict__ K, const E* __restrict__ V,
                                                             const float* __restrict__ kbar,
                                                             const float* __restrict__ vsum,
                                                             const float* __restrict__ Hbar,
                                                             double* __restrict__ M, int L, int T, int G2) {
  extern __shared__ __align__(16) unsigned char smem[];
  TileLds<E, D>& s = *reinterpret_cast<TileLds<E, D>*>(smem);
  SpectralLds<D>& sp = *reinterpret_cast<SpectralLds<D>*>(smem + sizeof(TileLds<E, D>));
  constexpr int MTW = HAcc<D>::MTW, NTT = HAcc<D>::NTT, NE = D / 64;
  const int bh = blockIdx.y;
  const int t = threadIdx.x, w = t / 64, l = t % 64;
  const E* Kh = K + static_cast<size_t>(bh) * L * D;
  const E* Vh = V + static_cast<size_t>(bh) * L * D;

  HAcc<D> hb;  // Hbar in the accumulator layout
  const float* Hh = Hbar + static_cast<size_t>(bh) * D * D;
#pragma unroll
  for (int mi = 0; mi < MTW; ++mi)
#pragma unroll
    for (int nt = 0; nt < NTT; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) hb.v[mi][nt][r] = Hh[acc_row<D>(mi, r) * D + acc_col(nt)];

  const int j0 = blockIdx.x * G2, j1 = min(T, j0 + G2);
  for (int j = j0; j < j1; ++j) {
    const int row0 = j * kBlock, nvalid = min(kBlock, L - row0);
    __syncthreads();
    stage_transposed<D>(Kh, row0, nvalid, s.kt);
    stage_transposed<D>(Vh, row0, nvalid, s.vt);
    if (t < D) {
      const size_t o = (static_cast<size_t>(bh) * T + j) * D + t;
      s.kbar[t] = kbar[o];
      s.vsum[t] = vsum[o];
    }
    __syncthreads();
    HAcc<D> A;
#pragma unroll
    for (int mi = 0; mi < MTW; ++mi)
#pragma unroll
      for (int nt = 0; nt < NTT; ++nt) A.v[mi][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    accumulate_ktv<D>(s, A);
    subtract_rank1(s, A);
#pragma unroll
    for (int mi = 0; mi < MTW; ++mi)
#pragma unroll
      for (int nt = 0; nt < NTT; ++nt) A.v[mi][nt] -= hb.v[mi][nt];

    // start vector A^T r with a fixed +-1 pattern r over the rows
    {
      float y[MTW][4];
#pragma unroll
      for (int mi = 0; mi < MTW; ++mi)
#pragma unroll
        for (int r = 0; r < 4; ++r) y[mi][r] = start_sign(acc_row<D>(mi, r));
      write_col_partials<D>(A, y, sp);
    }
    __syncthreads();
    if (w == 0) {
      float x[NE];
      double n = 0.0;
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        float sum = 0.f;
#pragma unroll
        for (int q = 0; q < 16; ++q) sum += sp.xpart[q][l + 64 * e];
        x[e] = sum;
        n += static_cast<double>(sum) * sum;
      }
      n = wave_sum_f64(n);
      const float inv = n > 0.0 ? static_cast<float>(1.0 / sqrt(n)) : 0.f;
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        sp.vk[0][l + 64 * e] = x[e] * inv;
        sp.xs[l + 64 * e] = x[e];
      }
      if (l == 0) sp.flag = n > 0.0 ? 0 : 2;
    }
    __syncthreads();
    const bool zero = sp.flag == 2;
    if (!zero) {
      for (int cyc = 0; cyc < kLanczosCycles; ++cyc) {
        for (int k = 0; k < kLanczosK; ++k) {
          apply_ata<D>(A, sp, k);
          __syncthreads();
          if (w == 0) lanczos_step<D>(sp, k, l);
          __syncthreads();
        }
        if (w == 0) lanczos_restart<D>(sp, l, cyc == kLanczosCycles - 1);
        __syncthreads();
        if (sp.flag == 1) break;
      }
    }
    // M_j = ||A x|| / ||x|| in fp64 from the fp32 Ritz vector.
    double mval = 0.0;
    if (!zero) {
      float xc[NTT];
#pragma unroll
      for (int nt = 0; nt < NTT; ++nt) xc[nt] = sp.xs[acc_col(nt)];
      double ysq = 0.0;
#pragma unroll
      for (int mi = 0; mi < MTW; ++mi)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          double p = 0.0;
#pragma unroll
          for (int nt = 0; nt < NTT; ++nt) p += static_cast<double>(A.v[mi][nt][r]) * xc[nt];
          p = row_sum16(p);
          ysq += p * p;
        }
      if (l % 16 == 0) sp.red2[t / 16] = ysq;
      if (w == 0) {
        double x2 = 0.0;
#pragma unroll
        for (int e = 0; e < NE; ++e) x2 += static_cast<double>(sp.xs[l + 64 * e]) * sp.xs[l + 64 * e];
        x2 = wave_sum_f64(x2);
        if (l == 0) sp.x2 = x2;
      }
      __syncthreads();
      if (t == 0) {
        double ys = 0.0;
        for (int q = 0; q < 16; ++q) ys += sp.red2[q];
        mval = sqrt(ys / sp.x2);
      }
    }
    if (t == 0) M[static_cast<size_t>(bh) * T + j] = mval;
  }
}

template <typename E, int D>
int stats_chunks(const paro_problem& p, int* G) {
  const int T = ceil_div(p.L, kBlock);
  const int bh = p.B * p.H;
  int nchunk = max(1, min(T, ceil_div(1024, bh)));
  *G = ceil_div(T, nchunk);
  return ceil_div(T, *G);
}

template <typename E, int D>
hipError_t launch_typed(const paro_problem& p, const E* K, const E* V, float* kbar, float* vsum,
                        float* Hbar, double* M, void* ws, hipStream_t st) {
  const int T = ceil_div(p.L, kBlock);
  const int bh = p.B * p.H;
  int G = 1;
  const int nchunk = stats_chunks<E, D>(p, &G);
  const size_t lds1 = sizeof(TileLds<E, D>);
  const size_t lds3 = sizeof(TileLds<E, D>) + sizeof(SpectralLds<D>);
  hipError_t e;
  if (lds1 > 65536 && (e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_block_stats<E, D>),
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               static_cast<int>(lds1))) != hipSuccess)
    return e;
  if (lds3 > 65536 && (e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_block_spectral<E, D>),
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               static_cast<int>(lds3))) != hipSuccess)
    return e;
  hipLaunchKernelGGL((k_block_stats<E, D>), dim3(nchunk, bh), dim3(kThreads), lds1, st, K, V, kbar, vsum,
                     static_cast<float*>(ws), p.L, T, G, nchunk);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_hbar_reduce, dim3(ceil_div(D * D, 256), bh), dim3(256), 0, st,
                     static_cast<const float*>(ws), Hbar, D * D, nchunk, T);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int G2 = max(1, min(16, ceil_div(T * bh, 4096)));
  hipLaunchKernelGGL((k_block_spectral<E, D>), dim3(ceil_div(T, G2), bh), dim3(kThreads), lds3, st, K, V, kbar,
                     vsum, Hbar, M, p.L, T, G2);
  return hipGetLastError();
}

}  // namespace

size_t precompute_workspace_bytes(const paro_problem& p) {
  int G = 1;
  const int nchunk = stats_chunks<float, 64>(p, &G);
  return static_cast<size_t>(p.B) * p.H * nchunk * p.d * p.d * sizeof(float);
}

hipError_t launch_precompute(const paro_problem& p, const void* K, const void* V, float* kbar, float* vsum,
                             float* Hbar, double* M, void* ws, hipStream_t s) {
  if (p.dtype == PARO_DTYPE_BF16) {
    const auto* k = static_cast<const uint16_t*>(K);
    const auto* v = static_cast<const uint16_t*>(V);
    return p.d == 128 ? launch_typed<uint16_t, 128>(p, k, v, kbar, vsum, Hbar, M, ws, s)
                      : launch_typed<uint16_t, 64>(p, k, v, kbar, vsum, Hbar, M, ws, s);
  }
  const auto* k = static_cast<const float*>(K);
  const auto* v = static_cast<const float*>(V);
  return p.d == 128 ? launch_typed<float, 128>(p, k, v, kbar, vsum, Hbar, M, ws, s)
                    : launch_typed<float, 64>(p, k, v, kbar, vsum, Hbar, M, ws, s);
}

}  // namespace paro
