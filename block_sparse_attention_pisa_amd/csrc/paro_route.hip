// Covariance-aware top-k routing ("PISA: Piecewise Sparse Attention Is Wiser
// for Efficient Diffusion Transformers", section 2, "covariance-aware
// routing"): score_ij = scale * qbar_i . kbar_j + lambda * M_j, and S_i is the
// set of the keep_k best-scoring kv-blocks of query block i.
//
// One workgroup (kWaves waves) handles R <= 16 consecutive query blocks of
// one (batch, head):
//   1. qbar_i: each wave sums the valid query rows of its blocks in fp64
//      (one pass over Q, cross-lane reduction by shuffles) and stores qbar in
//      fp32;
//   2. the dot products qbar_i . kbar_j of all R rows and T centroids on fp32
//      MFMA 16x16x4 (R rows are the 16 rows of the MFMA tile), kept in LDS as
//      fp32. Their error (~1e-7) is far below the 1e-5 score gaps that decide
//      routing;
//   3. per row, one wave forms the fp64 scores scale * dot + lambda * M_j,
//      maps them onto order-preserving 64-bit keys held in registers, and
//      finds the keep_k-th largest key bit by bit, from the highest bit where
//      the row's keys differ down: for each bit it counts, with one 64-bit
//      compare per key and wave ballots (no LDS traffic, no atomics), the keys
//      at or above the candidate threshold; it stops as soon as the keys that
//      agree with the prefix found so far are exactly the ones still needed. The winners are
//      written in ascending j with a ballot / mbcnt compaction. Exact ties go
//      to the lower j, so the result is a deterministic integer function of
//      the scores.
#include <algorithm>

#include "paro_common.h"

namespace paro {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxRows = 16;   // query blocks per workgroup = rows of the 16x16 MFMA tile
constexpr int kMaxKeyRegs = 32;  // keys per lane kept in registers: rows of T <= 2048 never re-read LDS
constexpr int kCompactRegs = 4;  // registers per lane of the selection's late bits (up to 256 keys)
constexpr size_t kLdsBudget = 152 * 1024;

// Order-preserving map of a double onto uint64 (larger score -> larger key);
// -0.0 is folded onto +0.0 first so equal scores give equal keys. Finite
// scores never map to 0.
__device__ __forceinline__ uint64_t score_key(double s) {
  s = s + 0.0;
  const uint64_t u = __builtin_bit_cast(uint64_t, s);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

__device__ __forceinline__ double shfl_xor_f64(double v, int m) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = __shfl_xor(static_cast<uint32_t>(u), m);
  const uint32_t hi = __shfl_xor(static_cast<uint32_t>(u >> 32), m);
  return __builtin_bit_cast(double, (static_cast<uint64_t>(hi) << 32) | lo);
}

__device__ __forceinline__ int lanes_below(uint64_t bal) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(bal >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bal), 0));
}

__device__ __forceinline__ int count_lanes(bool p) { return __builtin_popcountll(__ballot(p)); }

// A wave-uniform 64-bit value, moved to scalar registers (so that the
// comparisons against it take a scalar operand).
__device__ __forceinline__ uint64_t uniform64(uint64_t v) {
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(v))));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(v >> 32))));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// acc[e] += element e of a 16-byte piece of a row (8 bf16 or 4 fp32 values)
template <typename E>
__device__ __forceinline__ void add_piece(double* acc, uint4 raw);
template <>
__device__ __forceinline__ void add_piece<uint16_t>(double* acc, uint4 raw) {
  const uint32_t u[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    acc[2 * h] += __uint_as_float(u[h] << 16);
    acc[2 * h + 1] += __uint_as_float(u[h] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void add_piece<float>(double* acc, uint4 raw) {
  acc[0] += __uint_as_float(raw.x);
  acc[1] += __uint_as_float(raw.y);
  acc[2] += __uint_as_float(raw.z);
  acc[3] += __uint_as_float(raw.w);
}

// Modes of k_route: the fixed-k routing; the weights pass of the budgeted
// routing (qbar kept for the select pass, and each row's need w_i = exp of
// the entropy of its zeroth-order block masses, as 2^16 fixed point); the
// select pass of the budgeted routing (qbar read back, row i keeps the
// offsets[i + 1] - offsets[i] best blocks at idx + offsets[i]).
constexpr int kRouteFixed = 0, kRouteWeights = 1, kRouteRagged = 2;

// Rows of more than 1280 blocks (NI >= 24) take over 80 KB of LDS for the
// dots of 16 rows, so only one workgroup fits on a CU: those instantiations
// may use 256 registers (two waves per SIMD) instead of spilling the keys.
template <int NI>
constexpr int route_waves_per_eu() { return NI >= 24 ? 2 : 4; }

template <typename E, int D, int NI, int kMode>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(route_waves_per_eu<NI>()))) void k_route(const E* __restrict__ Q, const float* __restrict__ kbar,
                                                    const double* __restrict__ M, int32_t* __restrict__ idx,
                                                    int L, int T, int R, int keep_k, double scale,
                                                    double lambda, float* __restrict__ qbar_ws,
                                                    int64_t* __restrict__ wq, const int32_t* __restrict__ offsets,
                                                    int kstride) {
  extern __shared__ __align__(16) unsigned char smem[];
  float* qs = reinterpret_cast<float*>(smem);    // qbar [R][D]; dead once the MFMA operands are loaded
  float* dots = reinterpret_cast<float*>(smem);  // [R][T], written after qs is dead

  // XCD-aware order: consecutive workgroup ids go to different XCDs, so each
  // XCD gets a contiguous run of (head, row group) items and a head's kbar,
  // which every row group of the head reads in full, stays in one L2.
  const int nwg = gridDim.x, ngrp = ceil_div(T, R);
  int wg = blockIdx.x;
  const int n8 = (nwg / 8) * 8;
  if (wg < n8) wg = (wg % 8) * (nwg / 8) + wg / 8;
  const int bh = wg / ngrp;
  const int i0 = (wg % ngrp) * R;
  const int nrows = min(R, T - i0);
  const int t = threadIdx.x, w = t / 64, l = t % 64;
  const E* Qh = Q + static_cast<size_t>(bh) * L * D;
  const float* kb = kbar + static_cast<size_t>(bh) * T * D;
  const double* Mh = M + static_cast<size_t>(bh) * T;
  float* qbh = qbar_ws + (static_cast<size_t>(bh) * T + i0) * D;  // this group's rows of the kept qbar

  if (kMode == kRouteRagged) {
    for (int e = t; e < nrows * D; e += kThreads) qs[e] = qbh[e];
  } else {
  // 1. qbar. Lane l reads the 16-byte piece dg = l % G of rows rg, rg + RG,
  //    ... (rg = l / G) of the block, sums them in fp64, and the RG lanes of
  //    one piece are then reduced by shuffles.
  {
    constexpr int EPL = 16 / sizeof(E);  // elements per 16-byte piece
    constexpr int G = D / EPL;           // pieces per row
    constexpr int RG = 64 / G;           // rows read together by one load instruction
    constexpr int NL = kBlock / RG;      // loads per lane per block
    constexpr int CH = NL < 8 ? NL : 8;  // loads kept in flight together
    const int dg = l % G, rg = l / G;
    for (int r = w; r < nrows; r += kWaves) {
      const int row0 = (i0 + r) * kBlock, nvalid = min(kBlock, L - row0);
      const E* base = Qh + static_cast<size_t>(row0) * D + EPL * dg;
      double acc[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = 0.0;
#pragma unroll 1
      for (int s0 = 0; s0 < NL; s0 += CH) {
        uint4 raw[CH];
#pragma unroll
        for (int s = 0; s < CH; ++s) {
          const int tok = rg + RG * (s0 + s);
          raw[s] = tok < nvalid ? *reinterpret_cast<const uint4*>(base + static_cast<size_t>(tok) * D)
                                : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int s = 0; s < CH; ++s) add_piece<E>(acc, raw[s]);
      }
#pragma unroll
      for (int o = G; o < 64; o <<= 1)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] += shfl_xor_f64(acc[e], o);
      if (rg == 0) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          const float x = static_cast<float>(acc[e] / nvalid);
          qs[r * D + EPL * dg + e] = x;
          if (kMode == kRouteWeights) qbh[r * D + EPL * dg + e] = x;
        }
      }
    }
  }
  }
  __syncthreads();

  // 2. dots. Lane l = 16 g + n16 supplies A = qbar[n16][.] and B =
  //    kbar[16 c + n16][.]; k-step 4 q + u of a lane of group g uses dim
  //    16 q + 4 g + u, so every lane reads whole float4s and the four groups
  //    of one row read 64 contiguous bytes per load. The C layout gives lane l
  //    the dots of rows 4 g .. 4 g + 3 with centroid 16 c + n16. Rows
  //    n16 >= nrows are zero. Wave w takes centroid blocks c = w, w + kWaves, ...
  {
    constexpr int NQ = D / 16;
    const int g = l / 16, n16 = l % 16;
    float qa[4 * NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const float4 x = n16 < nrows ? *reinterpret_cast<const float4*>(qs + n16 * D + 16 * q + 4 * g)
                                   : make_float4(0.f, 0.f, 0.f, 0.f);
      qa[4 * q] = x.x;
      qa[4 * q + 1] = x.y;
      qa[4 * q + 2] = x.z;
      qa[4 * q + 3] = x.w;
    }
    __syncthreads();  // qs is overwritten by the dots from here on
    const int nblk = ceil_div(T, 16);
    // the centroids of the next block of 16 are loaded while the current
    // ones are multiplied (one register set in flight)
    auto load_kv = [&](int c, float4 (&kv4)[NQ]) {
      const int n = min(16 * c + n16, T - 1);
      const float4* kr = reinterpret_cast<const float4*>(kb + static_cast<size_t>(n) * D) + g;
#pragma unroll
      for (int q = 0; q < NQ; ++q) kv4[q] = kr[4 * q];
    };
    float4 nxt[NQ];
    if (w < nblk) load_kv(w, nxt);
    for (int c = w; c < nblk; c += kWaves) {
      const int n = 16 * c + n16;
      float kv[4 * NQ];
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        kv[4 * q] = nxt[q].x;
        kv[4 * q + 1] = nxt[q].y;
        kv[4 * q + 2] = nxt[q].z;
        kv[4 * q + 3] = nxt[q].w;
      }
      if (c + kWaves < nblk) load_kv(c + kWaves, nxt);
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4 * NQ; ++ks) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[ks], kv[ks], acc, 0, 0, 0);
      if (n < T) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * g + i;
          if (r < nrows) dots[r * T + n] = acc[i];
        }
      }
    }
  }
  // lambda M_j of the keys each lane holds in registers (blocks 64 i + l):
  // the same for every row of the group, so loaded once per wave, and here,
  // where their latency hides behind the barrier that ends the dots
  // (unconditional loads, the index clamped to the last block, so all of
  // them are in flight together; lanes past T then take 0 as before)
  double lm[NI];
  if constexpr (kMode != kRouteWeights) {
#pragma unroll
    for (int i = 0; i < NI; ++i) lm[i] = Mh[min(64 * i + l, T - 1)];
#pragma unroll
    for (int i = 0; i < NI; ++i) lm[i] = 64 * i + l < T ? lambda * lm[i] : 0.0;
  }
  __syncthreads();

  // 3. selection, one wave per row
  // Lane l keeps the keys of j = l + 64 i, i < NI, in registers (NI * 64 >= T
  // unless T > 64 * kMaxKeyRegs); keys from tail0 on are re-formed from LDS
  // whenever they are needed. Padding keys (j >= T) are 0, which no finite
  // score maps to and no prefix test below matches.
  constexpr int tail0 = 64 * NI;
  if (kMode == kRouteWeights) {
    // w = exp(H), H the entropy of p_j = n_j e^{a_j} / sum, a_j = scale qbar . kbar_j;
    // log n_j - log 64 is 0 except for a partial last block
    const double lnlast = log(static_cast<double>(L - kBlock * (T - 1)) / kBlock);
    for (int r = w; r < nrows; r += kWaves) {
      const float* dr = dots + r * T;
      auto xat = [&](int j) { return scale * static_cast<double>(dr[j]) + (j == T - 1 ? lnlast : 0.0); };
      double mx = -__builtin_huge_val();
      for (int j = l; j < T; j += 64) mx = fmax(mx, xat(j));
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) mx = fmax(mx, shfl_xor_f64(mx, o));
      double z = 0.0, ez = 0.0;
      for (int j = l; j < T; j += 64) {
        const double y = xat(j) - mx, e = exp(y);
        z += e;
        ez += y * e;
      }
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        z += shfl_xor_f64(z, o);
        ez += shfl_xor_f64(ez, o);
      }
      if (l == 0) {
        const double wgt = exp(log(z) - ez / z);
        wq[static_cast<size_t>(bh) * T + i0 + r] = static_cast<int64_t>(floor(wgt * 65536.0 + 0.5));
      }
    }
    return;
  }
  for (int r = w; r < nrows; r += kWaves) {
    const float* dr = dots + r * T;
    int32_t* out;
    if (kMode == kRouteRagged) {
      const int32_t* orow = offsets + static_cast<size_t>(bh) * (T + 1) + i0 + r;
      keep_k = orow[1] - orow[0];
      out = idx + static_cast<size_t>(bh) * kstride + orow[0];
    } else {
      out = idx + (static_cast<size_t>(bh) * T + i0 + r) * keep_k;
    }
    if (keep_k == 0) continue;
    if (keep_k >= T) {
      for (int j = l; j < T; j += 64) out[j] = j;
      continue;
    }
    auto score_at = [&](int j) { return scale * static_cast<double>(dr[j]) + lambda * Mh[j]; };
    uint64_t key[NI];
    double smin = __builtin_huge_val(), smax = -__builtin_huge_val();
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int j = 64 * i + l;
      key[i] = 0;
      if (j < T) {
        const double s = scale * static_cast<double>(dr[j]) + lm[i];  // = score_at(j)
        key[i] = score_key(s);
        smin = fmin(smin, s);
        smax = fmax(smax, s);
      }
    }
    for (int j = tail0 + l; j < T; j += 64) {
      const double s = score_at(j);
      smin = fmin(smin, s);
      smax = fmax(smax, s);
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      smin = fmin(smin, shfl_xor_f64(smin, o));
      smax = fmax(smax, shfl_xor_f64(smax, o));
    }
    const uint64_t kmin = uniform64(score_key(smin)), kmax = uniform64(score_key(smax));
    // Invariants: every key whose bits under `mask` exceed `prefix` is taken
    // (keep_k - rem of them); `match` keys equal prefix under mask and rem of
    // them are still needed, so match >= rem. `mask` covers bits 63 .. b + 1
    // and prefix has no bits below them, so for want = prefix | 2^b a key is
    // >= want exactly when it is above prefix under mask or equal to it with
    // bit b set: the keys with bit b set among those that can still match
    // are the ones >= want, less the keep_k - rem already taken.
    uint64_t mask = ~0ull, prefix = kmax;
    int rem = keep_k;
    if (kmin != kmax) {
      const int top = 63 - __builtin_clzll(kmin ^ kmax);  // highest bit where the row's keys differ
      mask = top == 63 ? 0ull : ~0ull << (top + 1);
      prefix = kmax & mask;
      int match = T;
      // decide bit b from the count c1 of keys (among those equal to prefix
      // under mask, the only ones that can match want) that have it set
      auto decide = [&](int b, int c1) {
        if (rem <= c1) {
          prefix = prefix | (1ull << b);
          match = c1;
        } else {
          rem -= c1;
          match -= c1;
        }
        mask |= 1ull << b;
      };
      int b = top;
      // Once few keys still equal prefix under mask (`match` of them), they
      // are gathered into kCompactRegs registers per lane and the remaining
      // bits are counted over those alone: a key that differs from prefix
      // under mask never matches again (mask only grows), so every count,
      // and with it the result, is the same. The gather goes through this
      // row's slice of `dots`, dead once the keys are in registers (T <=
      // tail0), 8-byte aligned inside it.
      // (dots is 16-byte aligned, so the slice's base is 8-byte aligned when r T is even)
      uint64_t* gathered = reinterpret_cast<uint64_t*>(dots + r * T + ((r * T) & 1));
      const int cap = T <= tail0 ? min(64 * kCompactRegs, (4 * T - 4) / 8) : 0;
      for (; b >= 0 && match != rem && match > cap; --b) {
        const uint64_t want = prefix | (1ull << b);
        int ge = 0;
#pragma unroll
        for (int i = 0; i < NI; ++i) ge += count_lanes(key[i] >= want);
        for (int base = tail0; base < T; base += 64) {
          const int j = base + l;
          ge += count_lanes(j < T && score_key(score_at(j)) >= want);
        }
        decide(b, ge - (keep_k - rem));
      }
      if (b >= 0 && match != rem) {
        // (here T <= tail0: every key is in key[], padding keys are 0)
        int pos = 0;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const bool alive = 64 * i + l < T && (key[i] & mask) == prefix;
          const uint64_t bal = __ballot(alive);
          if (alive) gathered[pos + lanes_below(bal)] = key[i];
          pos += __builtin_popcountll(bal);
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        // pos == match <= cap; lanes past it hold 0, which never equals a
        // want (bit b is set in every want)
        uint64_t ck[kCompactRegs];
#pragma unroll
        for (int c = 0; c < kCompactRegs; ++c) ck[c] = 64 * c + l < pos ? gathered[64 * c + l] : 0ull;
        // the keys taken from here on are all gathered ones (the others are
        // above or below prefix under mask already)
        const int taken0 = keep_k - rem;
        for (; b >= 0 && match != rem; --b) {
          const uint64_t want = prefix | (1ull << b);
          int ge = 0;
#pragma unroll
          for (int c = 0; c < kCompactRegs; ++c) ge += count_lanes(ck[c] >= want);
          decide(b, ge - (keep_k - rem - taken0));
        }
      }
    }
    // Take every key above prefix under mask and the first rem (in ascending
    // j) equal to it: exactly keep_k indices.
    // (above prefix under mask: above its largest completion hi; padding
    // keys are 0 and never above)
    int written = 0, eq_seen = 0;
    const uint64_t hi = prefix | ~mask;
    auto emit = [&](int j, uint64_t k, bool valid) {
      const bool gt = k > hi;
      const bool eq = valid && !gt && k >= prefix;
      const uint64_t beq = __ballot(eq);
      const bool sel = gt || (eq && eq_seen + lanes_below(beq) < rem);
      const uint64_t bsel = __ballot(sel);
      const int pos = written + lanes_below(bsel);
      if (sel && pos < keep_k) out[pos] = j;
      written += __builtin_popcountll(bsel);
      eq_seen += __builtin_popcountll(beq);
    };
#pragma unroll
    for (int i = 0; i < NI; ++i) emit(64 * i + l, key[i], 64 * i + l < T);
    for (int base = tail0; base < T; base += 64) {
      const int j = base + l;
      emit(j, j < T ? score_key(score_at(j)) : 0ull, j < T);
    }
  }
}

size_t route_lds_bytes(int T, int d, int R) {
  return sizeof(float) * static_cast<size_t>(R) * static_cast<size_t>(std::max(T, d));
}

// Arguments of one routing launch beyond the problem (the budgeted modes use
// the workspace qbar, the integer weights and the CSR offsets).
struct RouteArgs {
  int keep_k;
  double lambda;
  int32_t* idx;
  float* qbar_ws;
  int64_t* wq;
  const int32_t* offsets;
  int kstride;
};

template <typename E, int D, int NI, int kMode>
hipError_t launch_ni(const paro_problem& p, const E* Q, const float* kbar, const double* M, const RouteArgs& ra,
                     hipStream_t s) {
  const int T = ceil_div(p.L, kBlock);
  const int R = route_rows_per_group(T, D);
  const size_t lds = route_lds_bytes(T, D, R);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_route<E, D, NI, kMode>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_route<E, D, NI, kMode>), dim3(ceil_div(T, R) * p.B * p.H), dim3(kThreads), lds, s, Q, kbar,
                     M, ra.idx, p.L, T, R, ra.keep_k, p.scale, ra.lambda, ra.qbar_ws, ra.wq, ra.offsets, ra.kstride);
  return hipGetLastError();
}

// Register chunks per lane: ceil(T / 64) rounded up to a multiple of 4.
template <typename E, int D, int kMode>
hipError_t launch_typed(const paro_problem& p, const E* Q, const float* kbar, const double* M, const RouteArgs& ra,
                        hipStream_t s) {
  switch (std::min((ceil_div(ceil_div(p.L, kBlock), 64) + 3) / 4, kMaxKeyRegs / 4)) {
    case 1: return launch_ni<E, D, 4, kMode>(p, Q, kbar, M, ra, s);
    case 2: return launch_ni<E, D, 8, kMode>(p, Q, kbar, M, ra, s);
    case 3: return launch_ni<E, D, 12, kMode>(p, Q, kbar, M, ra, s);
    case 4: return launch_ni<E, D, 16, kMode>(p, Q, kbar, M, ra, s);
    case 5: return launch_ni<E, D, 20, kMode>(p, Q, kbar, M, ra, s);
    case 6: return launch_ni<E, D, 24, kMode>(p, Q, kbar, M, ra, s);
    case 7: return launch_ni<E, D, 28, kMode>(p, Q, kbar, M, ra, s);
    default: return launch_ni<E, D, 32, kMode>(p, Q, kbar, M, ra, s);
  }
}

template <int kMode>
hipError_t launch_mode(const paro_problem& p, const void* Q, const float* kbar, const double* M, const RouteArgs& ra,
                       hipStream_t s) {
  if (p.dtype == PARO_DTYPE_BF16) {
    const auto* q = static_cast<const uint16_t*>(Q);
    return p.d == 128 ? launch_typed<uint16_t, 128, kMode>(p, q, kbar, M, ra, s)
                      : launch_typed<uint16_t, 64, kMode>(p, q, kbar, M, ra, s);
  }
  const auto* q = static_cast<const float*>(Q);
  return p.d == 128 ? launch_typed<float, 128, kMode>(p, q, kbar, M, ra, s)
                    : launch_typed<float, 64, kMode>(p, q, kbar, M, ra, s);
}

// Budget sharing for one head (one workgroup): k_i = k_min + floor(R wq_i / S)
// plus one for the R - sum(floors) rows of largest remainder R wq_i mod S
// (ties to the lower i), where rows whose floor share reaches T - k_min are
// first set to T and R, S are re-formed over the others until none does
// (the total stays k_total); then the CSR offsets (exclusive sums).
// The leftover rows are found as the keys (remainder << 20 | 2^20 - 1 - i),
// all distinct, that are at least the left-th largest one, by a bitwise
// search with block-wide counts.
constexpr int kAllocThreads = 1024;
__global__ __launch_bounds__(kAllocThreads) void k_budget_alloc(const int64_t* __restrict__ wq,
                                                                 int32_t* __restrict__ offsets, int T, int k_total,
                                                                 int k_min) {
  __shared__ long long red[kAllocThreads / 64];
  __shared__ int scan[kAllocThreads / 64];
  __shared__ uint32_t full[PARO_MAX_BLOCKS / 32];  // rows set to T (their excess is shared again)
  const int bh = blockIdx.x, t = threadIdx.x, w = t / 64, l = t % 64;
  const int64_t* wh = wq + static_cast<size_t>(bh) * T;
  int32_t* oh = offsets + static_cast<size_t>(bh) * (T + 1);
  auto block_sum = [&](long long v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    __syncthreads();
    if (l == 0) red[w] = v;
    __syncthreads();
    long long sum = 0;
#pragma unroll
    for (int i = 0; i < kAllocThreads / 64; ++i) sum += red[i];
    return sum;
  };
  for (int e = t; e < (T + 31) / 32; e += kAllocThreads) full[e] = 0u;
  __syncthreads();
  auto is_full = [&](int i) { return ((full[i >> 5] >> (i & 31)) & 1u) != 0u; };
  // Water-filling: a row whose floor share reaches the cap T - k_min is set
  // to T and leaves; the rest of R is shared again among the others, until
  // no share reaches the cap. Each thread tests and sets only its own rows'
  // bits; block_sum's barriers separate the rounds.
  const long long cap = static_cast<long long>(T) - k_min;
  long long Rr = static_cast<long long>(k_total) - static_cast<long long>(T) * k_min;
  long long S = 0;
  for (;;) {
    long long part = 0;
    for (int i = t; i < T; i += kAllocThreads) part += is_full(i) ? 0 : wh[i];
    S = block_sum(part);
    if (S == 0) break;
    long long c = 0;
    for (int i = t; i < T; i += kAllocThreads) c += (!is_full(i) && Rr * wh[i] / S >= cap) ? 1 : 0;
    const long long nf = block_sum(c);
    if (nf == 0) break;
    for (int i = t; i < T; i += kAllocThreads)
      if (!is_full(i) && Rr * wh[i] / S >= cap) atomicOr(&full[i >> 5], 1u << (i & 31));
    __syncthreads();
    Rr -= nf * cap;
  }
  long long part = 0;
  for (int i = t; i < T; i += kAllocThreads) part += (S > 0 && !is_full(i) ? Rr * wh[i] / S : 0);
  const long long left = Rr - block_sum(part);
  // full rows get key 0, which no candidate below reaches
  auto key_of = [&](int i) -> unsigned long long {
    if (S == 0 || is_full(i)) return 0ull;
    const long long rem = Rr * wh[i] % S;
    return (static_cast<unsigned long long>(rem) << 20) | static_cast<unsigned long long>((1 << 20) - 1 - i);
  };
  unsigned long long thr = ~0ull;  // no extra block when left == 0
  if (left > 0) {
    // each thread's keys (rows t, t + kAllocThreads, ...) computed once, not
    // once per bit (a 64-bit division each); rows past T hold 0, below every
    // candidate. The search starts at the highest bit any key has: above it
    // every count is 0 < left and the prefix would not change.
    constexpr int kRows = PARO_MAX_BLOCKS / kAllocThreads;
    unsigned long long kc[kRows];
    unsigned long long any = 0;
#pragma unroll
    for (int u = 0; u < kRows; ++u) {
      const int i = t + u * kAllocThreads;
      kc[u] = i < T ? key_of(i) : 0ull;
      any |= kc[u];
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) any |= __shfl_xor(any, o);
    __syncthreads();
    if (l == 0) red[w] = static_cast<long long>(any);
    __syncthreads();
    any = 0;
#pragma unroll
    for (int i = 0; i < kAllocThreads / 64; ++i) any |= static_cast<unsigned long long>(red[i]);
    unsigned long long prefix = 0;
    for (int b = any ? 63 - __builtin_clzll(any) : -1; b >= 0; --b) {
      const unsigned long long cand = prefix | (1ull << b);
      long long c = 0;
#pragma unroll
      for (int u = 0; u < kRows; ++u) c += kc[u] >= cand ? 1 : 0;
      if (block_sum(c) >= left) prefix = cand;
    }
    thr = prefix;
  }
  // k_i and their exclusive prefix sums, in chunks of kAllocThreads rows
  int base = 0;
  for (int c0 = 0; c0 < T; c0 += kAllocThreads) {
    const int i = c0 + t;
    int k = 0;
    if (i < T) {
      if (is_full(i)) {
        k = T;
      } else {
        const long long q = S > 0 ? Rr * wh[i] / S : 0;
        k = static_cast<int>(min(static_cast<long long>(T), k_min + q + (key_of(i) >= thr ? 1 : 0)));
      }
    }
    int incl = k;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o);
      if (l >= o) incl += v;
    }
    __syncthreads();
    if (l == 63) scan[w] = incl;
    __syncthreads();
    int before = base;
    for (int v = 0; v < w; ++v) before += scan[v];
    if (i < T) oh[i] = before + incl - k;
    int total = 0;
#pragma unroll
    for (int v = 0; v < kAllocThreads / 64; ++v) total += scan[v];
    base += total;
  }
  if (t == 0) oh[T] = base;
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
  const RouteArgs ra{keep_k, lambda, idx, nullptr, nullptr, nullptr, 0};
  return launch_mode<kRouteFixed>(p, Q, kbar, M, ra, s);
}

size_t route_budget_workspace_bytes(const paro_problem& p) {
  return static_cast<size_t>(p.B) * p.H * ceil_div(p.L, kBlock) * p.d * sizeof(float);
}

hipError_t launch_route_budget(const paro_problem& p, const void* Q, const float* kbar, const double* M, int k_total,
                               int k_min, double lambda, int64_t* wq, int32_t* offsets, int32_t* idx, void* ws,
                               hipStream_t s) {
  const int T = ceil_div(p.L, kBlock);
  RouteArgs ra{0, lambda, idx, static_cast<float*>(ws), wq, offsets, k_total};
  hipError_t e = launch_mode<kRouteWeights>(p, Q, kbar, M, ra, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_budget_alloc, dim3(p.B * p.H), dim3(kAllocThreads), 0, s, static_cast<const int64_t*>(wq),
                     offsets, T, k_total, k_min);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return launch_mode<kRouteRagged>(p, Q, kbar, M, ra, s);
}

}  // namespace paro
