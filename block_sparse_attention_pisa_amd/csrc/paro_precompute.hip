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
//                        A = H_j - Hbar and runs fp32 power iteration on A^T A
//                        until the Rayleigh estimate has converged far below
//                        the fp32 rounding of A; the final ||A x|| / ||x|| is
//                        accumulated in fp64. H_j never reaches memory.
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

template <int D>
struct SpectralLds {
  float xpart[16][D];  // column partials of A^T y (one row per 16-lane group)
  float xs[D];         // current iterate (unnormalised)
  double red[4][3];    // per-wave partial sums
  double red2[16];
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
  for (int mi = 0; mi < MTW; ++mi)
    for (int nt = 0; nt < NTT; ++nt)
      for (int r = 0; r < 4; ++r) {
        const int row = acc_row<D>(mi, r), col = acc_col(nt);
        float sum = 0.f;
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
__device__ __forceinline__ float start_sign(int row) {
  return ((static_cast<uint32_t>(row + 1) * 2654435761u) >> 16) & 1u ? -1.f : 1.f;
}

// xpart[group][col] = sum over this lane's rows of A[row][col] * y[row].
template <int D>
__device__ __forceinline__ void write_col_partials(const HAcc<D>& A, const float (&y)[D / 64][4],
                                                   SpectralLds<D>& sp) {
  const int grp = threadIdx.x / 16;  // 16 groups of 16 lanes
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

// Sums over the waves that hold the D entries of the iterate.
template <int D>
__device__ __forceinline__ double red_total(const SpectralLds<D>& sp, int k) {
  double t = sp.red[0][k];
  if (D > 64) t += sp.red[1][k];
  return t;
}

constexpr int kMaxPowerIters = 500;
// Stop when the estimated remaining relative error of the Rayleigh value
// ||A x|| / ||x|| falls below this (far below the fp32 rounding of A).
constexpr double kPowerTol = 1e-10;

template <typename E, int D>
__global__ __launch_bounds__(kThreads) void k_block_spectral(const E* __restrict__ K, const E* __restrict__ V,
                                                             const float* __restrict__ kbar,
                                                             const float* __restrict__ vsum,
                                                             const float* __restrict__ Hbar,
                                                             double* __restrict__ M, int L, int T, int G2) {
  extern __shared__ __align__(16) unsigned char smem[];
  TileLds<E, D>& s = *reinterpret_cast<TileLds<E, D>*>(smem);
  SpectralLds<D>& sp = *reinterpret_cast<SpectralLds<D>*>(smem + sizeof(TileLds<E, D>));
  constexpr int MTW = HAcc<D>::MTW, NTT = HAcc<D>::NTT;
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

    // x0 = A^T r with a fixed +-1 pattern r over the rows.
    float y[MTW][4];
#pragma unroll
    for (int mi = 0; mi < MTW; ++mi)
#pragma unroll
      for (int r = 0; r < 4; ++r) y[mi][r] = start_sign(acc_row<D>(mi, r));
    write_col_partials<D>(A, y, sp);
    __syncthreads();
    if (t < D) {
      float xp = 0.f;
#pragma unroll
      for (int q = 0; q < 16; ++q) xp += sp.xpart[q][t];
      sp.xs[t] = xp;
      const double n2 = wave_sum_f64(static_cast<double>(xp) * xp);
      if (l == 0) sp.red[w][0] = n2;
    }
    __syncthreads();
    double n2 = red_total<D>(sp, 0);
    bool zero = !(n2 > 0.0);
    float inv = zero ? 0.f : static_cast<float>(1.0 / sqrt(n2));
    double delta_prev = 0.0;
    for (int it = 1; it <= kMaxPowerIters && !zero; ++it) {
      // y = A x (x = xs * inv), all-reduced over the 16 lanes sharing rows.
      float xc[NTT];
#pragma unroll
      for (int nt = 0; nt < NTT; ++nt) xc[nt] = sp.xs[acc_col(nt)] * inv;
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
      __syncthreads();
      if (t < D) {
        const float xo = sp.xs[t] * inv;
        float xp = 0.f;
#pragma unroll
        for (int q = 0; q < 16; ++q) xp += sp.xpart[q][t];
        sp.xs[t] = xp;
        const double a = wave_sum_f64(static_cast<double>(xp) * xp);
        const double b = wave_sum_f64(static_cast<double>(xp) * xo);
        const double c = wave_sum_f64(static_cast<double>(xo) * xo);
        if (l == 0) {
          sp.red[w][0] = a;
          sp.red[w][1] = b;
          sp.red[w][2] = c;
        }
      }
      __syncthreads();
      n2 = red_total<D>(sp, 0);
      const double dp = red_total<D>(sp, 1), o2 = red_total<D>(sp, 2);
      if (!(n2 > 0.0)) {
        zero = true;
        break;
      }
      inv = static_cast<float>(1.0 / sqrt(n2));
      const double cosang = dp / sqrt(n2 * o2);
      const double delta2 = fmax(0.0, 2.0 - 2.0 * cosang);
      const double delta = sqrt(delta2);
      if (it >= 2) {
        if (delta == 0.0) break;
        double rho = delta_prev > 0.0 ? delta / delta_prev : 0.999;
        rho = fmin(rho, 0.999);
        if (delta2 * rho * rho / (2.0 * (1.0 - rho)) < kPowerTol) break;
      }
      delta_prev = delta;
    }
    // M_j = ||A x|| / ||x|| evaluated in fp64 from the fp32 iterate.
    double mval = 0.0;
    if (!zero) {
      double ysq = 0.0;
      float xc[NTT];
#pragma unroll
      for (int nt = 0; nt < NTT; ++nt) xc[nt] = sp.xs[acc_col(nt)];
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
      if (t < D) {
        const double x2 = wave_sum_f64(static_cast<double>(sp.xs[t]) * sp.xs[t]);
        if (l == 0) sp.red[w][0] = x2;
      }
      __syncthreads();
      if (t == 0) {
        double ys = 0.0;
        for (int q = 0; q < 16; ++q) ys += sp.red2[q];
        mval = sqrt(ys / red_total<D>(sp, 0));
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
