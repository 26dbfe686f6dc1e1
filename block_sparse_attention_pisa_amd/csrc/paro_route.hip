// Covariance-aware top-k routing ("PISA: Piecewise Sparse Attention Is Wiser
// for Efficient Diffusion Transformers", section 2, "covariance-aware
// routing"): score_ij = scale * qbar_i . kbar_j + lambda * M_j, and S_i is the
// set of the keep_k best-scoring kv-blocks of query block i.
//
// One workgroup (4 waves) handles R consecutive query blocks of one
// (batch, head):
//   1. qbar_i in fp64 from the valid query rows (Q streamed once);
//   2. all T scores of the R rows in fp64 (exact products of fp64 qbar and
//      fp32 kbar), kept in LDS;
//   3. per row, one wave finds the keep_k-th largest score by an MSB-first
//      radix select over order-preserving 64-bit keys (8 passes of 8 bits,
//      LDS histogram), then writes the winners in ascending j with a
//      ballot / mbcnt compaction. Exact ties go to the lower j, so the result
//      is a deterministic integer function of the scores.
#include "paro_common.h"

namespace paro {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxRows = 8;
constexpr size_t kLdsBudget = 152 * 1024;

// Order-preserving map of a double onto uint64 (larger score -> larger key);
// -0.0 is folded onto +0.0 first so equal scores give equal keys.
__device__ __forceinline__ uint64_t score_key(double s) {
  s = s + 0.0;
  const uint64_t u = __builtin_bit_cast(uint64_t, s);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

__device__ __forceinline__ uint64_t ballot64(bool p) { return __ballot(p); }

template <typename E, int D>
__global__ __launch_bounds__(kThreads) void k_route(const E* __restrict__ Q, const float* __restrict__ kbar,
                                                    const double* __restrict__ M, int32_t* __restrict__ idx,
                                                    int L, int T, int R, int keep_k, double scale,
                                                    double lambda) {
  extern __shared__ __align__(16) unsigned char smem[];
  double* qbar = reinterpret_cast<double*>(smem);                      // [D][R]
  double* score = qbar + D * kMaxRows;                                  // [R][T]
  uint32_t* hist = reinterpret_cast<uint32_t*>(score + static_cast<size_t>(R) * T);  // [4][256]
  double* qred = reinterpret_cast<double*>(hist + 4 * 256);             // [4][D] partials

  const int bh = blockIdx.y;
  const int i0 = blockIdx.x * R;
  const int nrows = min(R, T - i0);
  const int t = threadIdx.x, w = t / 64, l = t % 64;
  const E* Qh = Q + static_cast<size_t>(bh) * L * D;
  const float* kb = kbar + static_cast<size_t>(bh) * T * D;
  const double* Mh = M + static_cast<size_t>(bh) * T;

  // 1. qbar (fp64 sums of the valid rows)
  constexpr int P = kThreads / D;
  constexpr int TP = kBlock / P;
  const int a = t % D, part = t / D;
  for (int r = 0; r < nrows; ++r) {
    const int row0 = (i0 + r) * kBlock, nvalid = min(kBlock, L - row0);
    double sum = 0.0;
    for (int q = part * TP; q < min(nvalid, part * TP + TP); ++q)
      sum += load_elem<E>(Qh + static_cast<size_t>(row0 + q) * D + a);
    qred[part * D + a] = sum;
    __syncthreads();
    if (t < D) {
      double s = 0.0;
      for (int p = 0; p < P; ++p) s += qred[p * D + a];
      qbar[a * kMaxRows + r] = s / nvalid;
    }
    __syncthreads();
  }

  // 2. scores
  for (int j = t; j < T; j += kThreads) {
    double acc[kMaxRows];
#pragma unroll
    for (int r = 0; r < kMaxRows; ++r) acc[r] = 0.0;
    const float4* krow = reinterpret_cast<const float4*>(kb + static_cast<size_t>(j) * D);
    for (int a4 = 0; a4 < D / 4; ++a4) {
      const float4 kv = krow[a4];
      const float ke[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const double kd = ke[e];
        const double* qa = qbar + (4 * a4 + e) * kMaxRows;
#pragma unroll
        for (int r = 0; r < kMaxRows; ++r) acc[r] += qa[r] * kd;
      }
    }
    const double lm = lambda * Mh[j];
    for (int r = 0; r < nrows; ++r) score[static_cast<size_t>(r) * T + j] = scale * acc[r] + lm;
  }
  __syncthreads();

  // 3. selection, one wave per row
  uint32_t* h = hist + 256 * w;
  for (int r = w; r < nrows; r += 4) {
    const double* sc = score + static_cast<size_t>(r) * T;
    int32_t* out = idx + (static_cast<size_t>(bh) * T + i0 + r) * keep_k;
    uint64_t prefix = 0, mask = 0;
    int remaining = keep_k;  // how many of the keys matching prefix are still needed
    if (keep_k < T) {
      for (int shift = 56; shift >= 0; shift -= 8) {
        for (int b = l; b < 256; b += 64) h[b] = 0;
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_wave_barrier();
        for (int j = l; j < T; j += 64) {
          const uint64_t key = score_key(sc[j]);
          if ((key & mask) == prefix) atomicAdd(&h[(key >> shift) & 255u], 1u);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_wave_barrier();
        // lane l owns digits 4l..4l+3; count of all digits above this lane's
        uint32_t c[4];
        for (int e = 0; e < 4; ++e) c[e] = h[4 * l + e];
        const uint32_t mine = c[0] + c[1] + c[2] + c[3];
        // exclusive suffix sum over lanes: digits held by lanes above l
        uint32_t incl = mine;
        for (int o = 1; o < 64; o <<= 1) {
          const uint32_t v = __shfl_down(incl, o);
          if (l + o < 64) incl += v;
        }
        const uint32_t above = incl - mine;
        int found = -1;
        uint32_t cum = above;
        int newrem = 0;
        for (int e = 3; e >= 0; --e) {
          if (found < 0 && cum < static_cast<uint32_t>(remaining) && cum + c[e] >= static_cast<uint32_t>(remaining)) {
            found = 4 * l + e;
            newrem = remaining - static_cast<int>(cum);
          }
          cum += c[e];
        }
        const uint64_t bal = ballot64(found >= 0);
        const int src = __builtin_ctzll(bal);
        const int digit = __shfl(found, src);
        remaining = __shfl(newrem, src);
        prefix |= static_cast<uint64_t>(digit) << shift;
        mask |= 255ull << shift;
      }
    }
    // prefix is now the keep_k-th largest key; take every key above it and
    // the first `remaining` keys equal to it, in ascending j.
    int written = 0, eq_seen = 0;
    for (int base = 0; base < T; base += 64) {
      const int j = base + l;
      bool gt = false, eq = false;
      if (j < T) {
        if (keep_k >= T) {
          gt = true;
        } else {
          const uint64_t key = score_key(sc[j]);
          gt = key > prefix;
          eq = key == prefix;
        }
      }
      const uint64_t beq = ballot64(eq);
      const int eq_rank = eq_seen + __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(beq >> 32),
                                                                __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(beq), 0));
      const bool sel = gt || (eq && eq_rank < remaining);
      const uint64_t bsel = ballot64(sel);
      const int pos = written + __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(bsel >> 32),
                                                          __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bsel), 0));
      if (sel && pos < keep_k) out[pos] = j;
      written += __builtin_popcountll(bsel);
      eq_seen += __builtin_popcountll(beq);
    }
  }
}

size_t route_lds_bytes(int T, int d, int R) {
  return sizeof(double) * (static_cast<size_t>(d) * kMaxRows + static_cast<size_t>(R) * T) +
         4 * 256 * sizeof(uint32_t) + sizeof(double) * 4 * d;
}

template <typename E, int D>
hipError_t launch_typed(const paro_problem& p, const E* Q, const float* kbar, const double* M, int keep_k,
                        double lambda, int32_t* idx, hipStream_t s) {
  const int T = ceil_div(p.L, kBlock);
  const int R = route_rows_per_group(T, D);
  const size_t lds = route_lds_bytes(T, D, R);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_route<E, D>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_route<E, D>), dim3(ceil_div(T, R), p.B * p.H), dim3(kThreads), lds, s, Q, kbar, M, idx,
                     p.L, T, R, keep_k, p.scale, lambda);
  return hipGetLastError();
}

}  // namespace

int route_rows_per_group(int T, int d) {
  for (int R = kMaxRows; R >= 1; R /= 2)
    if (route_lds_bytes(T, d, R) <= kLdsBudget) return R;
  return 0;
}

hipError_t launch_route(const paro_problem& p, const void* Q, const float* kbar, const double* M, int keep_k,
                        double lambda, int32_t* idx, hipStream_t s) {
  if (keep_k == 0) return hipSuccess;
  if (p.dtype == PARO_DTYPE_BF16) {
    const auto* q = static_cast<const uint16_t*>(Q);
    return p.d == 128 ? launch_typed<uint16_t, 128>(p, q, kbar, M, keep_k, lambda, idx, s)
                      : launch_typed<uint16_t, 64>(p, q, kbar, M, keep_k, lambda, idx, s);
  }
  const auto* q = static_cast<const float*>(Q);
  return p.d == 128 ? launch_typed<float, 128>(p, q, kbar, M, keep_k, lambda, idx, s)
                    : launch_typed<float, 64>(p, q, kbar, M, keep_k, lambda, idx, s);
}

}  // namespace paro
