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
#include <algorithm>

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
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  const uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), m);
  const uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), m);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

template <typename E, int D>
__global__ __launch_bounds__(kThreads) void k_route(const E* __restrict__ Q, const float* __restrict__ kbar,
                                                    const double* __restrict__ M, int32_t* __restrict__ idx,
                                                    int L, int T, int R, int keep_k, double scale,
                                                    double lambda) {
  extern __shared__ __align__(16) unsigned char smem[];
  double* qbar = reinterpret_cast<double*>(smem);                      // [D][R]
  uint32_t* hist = reinterpret_cast<uint32_t*>(qbar + D * kMaxRows);    // [4][256]
  double* score = reinterpret_cast<double*>(hist + 4 * 256);            // [R][T]
  double* qred = score;  // qbar partials [2 * rows per sweep][D], used before any score exists

  const int bh = blockIdx.y;
  const int i0 = blockIdx.x * R;
  const int nrows = min(R, T - i0);
  const int t = threadIdx.x, w = t / 64, l = t % 64;
  const E* Qh = Q + static_cast<size_t>(bh) * L * D;
  const float* kb = kbar + static_cast<size_t>(bh) * T * D;
  const double* Mh = M + static_cast<size_t>(bh) * T;

  // 1. qbar (fp64 sums of the valid rows). Thread t reads 16-byte pieces of
  //    rows t / G, t / G + 256 / G, ... at dim group t % G (G pieces per row);
  //    the loads of two query blocks are in flight together.
  constexpr int EPL = 16 / sizeof(E);  // elements per 16-byte piece
  constexpr int G = D / EPL;           // pieces per row
  constexpr int RS = kThreads / G;     // rows covered per sweep
  constexpr int SW = kBlock / RS;      // sweeps per block
  const int dg = t % G, ro = t / G;
  for (int r0 = 0; r0 < nrows; r0 += 2) {
    uint4 raw[2][SW];
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int r = r0 + rr;
      const int row0 = (i0 + r) * kBlock, nvalid = r < nrows ? min(kBlock, L - row0) : 0;
#pragma unroll
      for (int sw = 0; sw < SW; ++sw) {
        const int tok = ro + RS * sw;
        raw[rr][sw] = tok < nvalid
                          ? *reinterpret_cast<const uint4*>(Qh + static_cast<size_t>(row0 + tok) * D + EPL * dg)
                          : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      double acc[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = 0.0;
#pragma unroll
      for (int sw = 0; sw < SW; ++sw) {
        const E* x = reinterpret_cast<const E*>(&raw[rr][sw]);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] += load_elem<E>(x + e);
      }
#pragma unroll
      for (int e = 0; e < EPL; ++e) qred[(rr * RS + ro) * D + EPL * dg + e] = acc[e];
    }
    __syncthreads();
    for (int e = t; e < 2 * D; e += kThreads) {
      const int rr = e / D, a = e % D, r = r0 + rr;
      if (r < nrows) {
        const int row0 = (i0 + r) * kBlock, nvalid = min(kBlock, L - row0);
        double sum = 0.0;
        for (int p = 0; p < RS; ++p) sum += qred[(rr * RS + p) * D + a];
        qbar[a * kMaxRows + r] = sum / nvalid;
      }
    }
    __syncthreads();
  }

  // 2. scores: each thread handles centroids j and j + 256 together, with
  //    8 loads of 16 bytes per centroid in flight; qbar is read as LDS broadcasts.
  for (int ja = t; ja < T; ja += 2 * kThreads) {
    const int jb = ja + kThreads;
    const bool okb = jb < T;
    double acc_a[kMaxRows], acc_b[kMaxRows];
#pragma unroll
    for (int r = 0; r < kMaxRows; ++r) {
      acc_a[r] = 0.0;
      acc_b[r] = 0.0;
    }
    const float4* rowa = reinterpret_cast<const float4*>(kb + static_cast<size_t>(ja) * D);
    const float4* rowb = reinterpret_cast<const float4*>(kb + static_cast<size_t>(okb ? jb : ja) * D);
#pragma unroll 1
    for (int a0 = 0; a0 < D / 4; a0 += 8) {
      float4 ka[8], kc[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        ka[u] = rowa[a0 + u];
        kc[u] = rowb[a0 + u];
      }
      __builtin_amdgcn_sched_barrier(0);  // keep the 16 loads in flight together
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float xa[4] = {ka[u].x, ka[u].y, ka[u].z, ka[u].w};
        const float xb[4] = {kc[u].x, kc[u].y, kc[u].z, kc[u].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const double* qa = qbar + (4 * (a0 + u) + e) * kMaxRows;
#pragma unroll
          for (int r = 0; r < kMaxRows; ++r) {
            acc_a[r] += qa[r] * static_cast<double>(xa[e]);
            acc_b[r] += qa[r] * static_cast<double>(xb[e]);
          }
        }
      }
    }
    const double lma = lambda * Mh[ja];
    const double lmb = okb ? lambda * Mh[jb] : 0.0;
#pragma unroll
    for (int r = 0; r < kMaxRows; ++r) {
      if (r < nrows) {
        score[static_cast<size_t>(r) * T + ja] = scale * acc_a[r] + lma;
        if (okb) score[static_cast<size_t>(r) * T + jb] = scale * acc_b[r] + lmb;
      }
    }
  }
  __syncthreads();

  // 3. selection, one wave per row
  uint32_t* h = hist + 256 * w;
  for (int r = w; r < nrows; r += 4) {
    const double* sc = score + static_cast<size_t>(r) * T;
    int32_t* out = idx + (static_cast<size_t>(bh) * T + i0 + r) * keep_k;
    // Radix select over the digits below the common prefix of the row's keys:
    // keys are order-preserving images of the scores, so the first digits of
    // a row usually agree and would all hit one histogram bin.
    uint64_t kmin = ~0ull, kmax = 0ull;
    for (int j = l; j < T; j += 64) {
      const uint64_t key = score_key(sc[j]);
      kmin = key < kmin ? key : kmin;
      kmax = key > kmax ? key : kmax;
    }
    for (int o = 1; o < 64; o <<= 1) {
      const uint64_t a0 = shfl_xor_u64(kmin, o), a1 = shfl_xor_u64(kmax, o);
      kmin = a0 < kmin ? a0 : kmin;
      kmax = a1 > kmax ? a1 : kmax;
    }
    int top = kmin == kmax ? -8 : (63 - __builtin_clzll(kmin ^ kmax)) / 8 * 8;  // digit holding the top differing bit
    uint64_t mask = top + 8 >= 64 ? 0ull : ~((1ull << (top + 8)) - 1);
    uint64_t prefix = kmax & mask;
    int remaining = keep_k;  // how many keys equal to prefix (on the mask bits) are still needed
    if (keep_k < T) {
      for (int shift = top; shift >= 0; shift -= 8) {
        for (int b = l; b < 256; b += 64) h[b] = 0;
        __builtin_amdgcn_wave_barrier();
        for (int j = l; j < T; j += 64) {
          const uint64_t key = score_key(sc[j]);
          if ((key & mask) == prefix) atomicAdd(&h[(key >> shift) & 255u], 1u);
        }
        __builtin_amdgcn_wave_barrier();
        // lane l owns digits 4l..4l+3
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
        uint32_t cum = above, binc = 0;
        int newrem = 0;
        for (int e = 3; e >= 0; --e) {
          if (found < 0 && cum < static_cast<uint32_t>(remaining) && cum + c[e] >= static_cast<uint32_t>(remaining)) {
            found = 4 * l + e;
            newrem = remaining - static_cast<int>(cum);
            binc = c[e];
          }
          cum += c[e];
        }
        const uint64_t bal = ballot64(found >= 0);
        const int src = __builtin_ctzll(bal);
        const int digit = __shfl(found, src);
        remaining = __shfl(newrem, src);
        const int bin_count = __shfl(static_cast<int>(binc), src);
        prefix |= static_cast<uint64_t>(digit) << shift;
        mask |= 255ull << shift;
        if (remaining == bin_count) break;  // the whole bin is taken: no finer digit needed
      }
    }
    // Take every key whose masked bits exceed prefix, and the first
    // `remaining` (in ascending j) whose masked bits equal it.
    int written = 0, eq_seen = 0;
    for (int base = 0; base < T; base += 64) {
      const int j = base + l;
      bool gt = false, eq = false;
      if (j < T) {
        if (keep_k >= T) {
          gt = true;
        } else {
          const uint64_t key = score_key(sc[j]) & mask;
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
  const size_t scores = static_cast<size_t>(R) * T, partials = 2 * (kThreads / (d * 2 / 16)) * static_cast<size_t>(d);
  return sizeof(double) * (static_cast<size_t>(d) * kMaxRows + std::max(scores, partials)) + 4 * 256 * sizeof(uint32_t);
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
