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
//   2. k_hbar_reduce   : fixed-order fp64 sum of the chunk partials -> Hbar
//                        (and a register-order copy of it in the workspace).
//   3. k_block_spectral: one workgroup of two waves per block; re-reads K_j
//                        and V_j, rebuilds A = H_j - Hbar in registers on
//                        MFMA and finds its largest singular value by
//                        restarted Lanczos on A^T A (fp32 vectors and
//                        tridiagonal eigenproblem); the final ||A x|| / ||x||
//                        is accumulated in fp64. H_j never reaches memory.
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

// Transposed staging of a 64 x D tile (rows [row0, row0 + nvalid) of a
// [L, D] matrix) into dst[dim][token], tokens >= nvalid zero-filled. Item i
// moves tokens 4 tg .. 4 tg + 3 (tg = i % 16) of dims 8 dg .. 8 dg + 7
// (dg = i / 16): four 16-byte global loads, eight 8-byte LDS writes. The 16
// lanes of a DPP row hold the 16 token groups of one dim group, so each LDS
// write instruction fills whole 128-byte row segments, and the column sums
// of the tile are one 16-lane reduction away.
template <int D>
__device__ __forceinline__ void load_item(const uint16_t* __restrict__ src, int row0, int nvalid, int item,
                                          uint4 (&r)[4]) {
  // a buffer descriptor over the valid rows only: rows past nvalid read as
  // zeros, with no per-row select (so the loads stay unconditional and the
  // compiler can count them across loop iterations)
  const int tg = item % 16, dg = item / 16;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(src + static_cast<size_t>(row0) * D), static_cast<short>(0),
      static_cast<int>(nvalid * D * 2), 0x00020000);
#pragma unroll
  for (int q = 0; q < 4; ++q)
    r[q] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                         rs, static_cast<uint32_t>(((4 * tg + q) * D + 8 * dg) * 2), 0, 0));
}
__device__ __forceinline__ void store_item(uint16_t (*dst)[kLdT], int item, const uint4 (&r)[4]) {
  const int tg = item % 16, dg = item / 16;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t w0 = half16(r[0], e) | (half16(r[1], e) << 16);
    const uint32_t w1 = half16(r[2], e) | (half16(r[3], e) << 16);
    *reinterpret_cast<uint2*>(&dst[8 * dg + e][4 * tg]) = make_uint2(w0, w1);
  }
}
// Sums over the 64 tokens of the item's 8 dims (valid in every lane of the row).
__device__ __forceinline__ void item_colsum(const uint4 (&r)[4], float (&cs)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float s4 = (bf16_to_f32(half16(r[0], e)) + bf16_to_f32(half16(r[1], e))) +
                     (bf16_to_f32(half16(r[2], e)) + bf16_to_f32(half16(r[3], e)));
    cs[e] = row_sum16(s4);
  }
}

template <int D, int NTHR>
__device__ __forceinline__ void stage_transposed(const uint16_t* __restrict__ src, int row0, int nvalid,
                                                 uint16_t (*dst)[kLdT]) {
  for (int item = threadIdx.x; item < 2 * D; item += NTHR) {
    uint4 r[4];
    load_item<D>(src, row0, nvalid, item, r);
    store_item(dst, item, r);
  }
}
template <int D, int NTHR>
__device__ __forceinline__ void stage_transposed(const float* __restrict__ src, int row0, int nvalid,
                                                 float (*dst)[kLdT]) {
  for (int e = threadIdx.x; e < kBlock * D; e += NTHR) {
    const int tok = e / D, dim = e % D;
    dst[dim][tok] = tok < nvalid ? src[static_cast<size_t>(row0 + tok) * D + dim] : 0.f;
  }
}

__device__ __forceinline__ float tile_val(uint16_t x) { return bf16_to_f32(x); }
__device__ __forceinline__ float tile_val(float x) { return x; }

// Column sums of staged fp32 tiles; writes s.kbar (mean over nvalid) and s.vsum.
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
// One workgroup per chunk of G consecutive blocks of one (batch, head). For
// bf16 the next block's K and V sit in registers (one staging item per
// thread) while the current block is reduced, and the column sums come from
// those registers; only LDS barriers separate the steps.
template <typename E, int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void k_block_stats(const E* __restrict__ K, const E* __restrict__ V,
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
  if constexpr (sizeof(E) == 2) {
    static_assert(2 * D <= kThreads, "one staging item per thread");
    const int item = threadIdx.x;
    const bool has_item = item < 2 * D;
    // two blocks in flight: block j is staged from one register set while
    // the loads of block j + 1 are outstanding in the other; after staging,
    // the set is refilled with block j + 2 (the loop is unrolled by two so
    // that both sets stay in registers)
    uint4 rkA[4], rvA[4], rkB[4], rvB[4];
    // (a block past the chunk is fetched as zero rows: its descriptor
    // covers no bytes, so no memory is read, and the loads stay
    // unconditional, which lets the compiler count them exactly instead of
    // waiting for both register sets)
    auto fetch = [&](int j, uint4 (&rk)[4], uint4 (&rv)[4]) {
      // (wave-uniform; said so, so that the descriptors stay scalar)
      const int jj = __builtin_amdgcn_readfirstlane(j < j1 ? j : j0);
      const int nv = __builtin_amdgcn_readfirstlane(j < j1 ? min(kBlock, L - j * kBlock) : 0);
      load_item<D>(Kh, jj * kBlock, nv, item, rk);
      load_item<D>(Vh, jj * kBlock, nv, item, rv);
    };
    if (has_item) {
      fetch(j0, rkA, rvA);
      fetch(j0 + 1, rkB, rvB);
    }
    // Stage block j from its register set, write its column sums, and refill
    // the set with block j + 2. The 16 lanes of a dim group hold the same
    // sums, so all of them write them (same value, same address): no
    // branch and no condition on any memory instruction of the loop, so
    // the compiler counts the outstanding loads exactly and block j + 1
    // stays in flight while block j is waited for.
    auto stage = [&](int j, uint4 (&rk)[4], uint4 (&rv)[4]) {
      const int nvalid = min(kBlock, L - j * kBlock);
      store_item(s.kt, item, rk);
      store_item(s.vt, item, rv);
      float ks[8], vs[8];
      item_colsum(rk, ks);
      item_colsum(rv, vs);
      const int dg = item / 16;
      const size_t o = (static_cast<size_t>(bh) * T + j) * D + 8 * dg;
      const float fn = static_cast<float>(nvalid);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ks[e] = ks[e] / fn;
        s.kbar[8 * dg + e] = ks[e];
        s.vsum[8 * dg + e] = vs[e];
      }
      *reinterpret_cast<f32x4*>(kbar + o) = f32x4{ks[0], ks[1], ks[2], ks[3]};
      *reinterpret_cast<f32x4*>(kbar + o + 4) = f32x4{ks[4], ks[5], ks[6], ks[7]};
      *reinterpret_cast<f32x4*>(vsum + o) = f32x4{vs[0], vs[1], vs[2], vs[3]};
      *reinterpret_cast<f32x4*>(vsum + o + 4) = f32x4{vs[4], vs[5], vs[6], vs[7]};
      fetch(j + 2, rk, rv);
    };
    auto body = [&](int j, uint4 (&rk)[4], uint4 (&rv)[4]) {
      lds_barrier();  // the previous block's tiles have been consumed
      if constexpr (2 * D == kThreads) {
        stage(j, rk, rv);  // every thread has an item
      } else {
        if (has_item) stage(j, rk, rv);
      }
      lds_barrier();
      accumulate_ktv<D>(s, acc);
      subtract_rank1(s, acc);
    };
    // pairs of blocks, both bodies unconditional (so the loads of set B are
    // always the newer ones where set A is waited for), then an odd last one
    int j = j0;
    for (; j + 1 < j1; j += 2) {
      body(j, rkA, rvA);
      body(j + 1, rkB, rvB);
    }
    if (j < j1) body(j, rkA, rvA);
  } else {
    for (int j = j0; j < j1; ++j) {
      const int row0 = j * kBlock, nvalid = min(kBlock, L - row0);
      __syncthreads();
      stage_transposed<D, kThreads>(Kh, row0, nvalid, s.kt);
      stage_transposed<D, kThreads>(Vh, row0, nvalid, s.vt);
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
  }
  float* out = ws + (static_cast<size_t>(bh) * nchunk + c) * D * D;
#pragma unroll
  for (int mi = 0; mi < HAcc<D>::MTW; ++mi)
#pragma unroll
    for (int nt = 0; nt < HAcc<D>::NTT; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) out[acc_row<D>(mi, r) * D + acc_col(nt)] = acc.v[mi][nt][r];
}

// ------------------------------------------------------------ kernel 3 layout
// A = H_j - Hbar is split over the two waves of a k_block_spectral workgroup
// in the C layout of the 16x16 MFMA: wave w, lane l (g = l / 16, c = l % 16)
// holds v[ti][tj][r] = A[16 (MT w + ti) + 4 g + r][16 tj + c].
template <int D>
struct PairA {
  static constexpr int MT = D / 32;  // 16-row tiles per wave
  static constexpr int NT = D / 16;  // 16-column tiles
  f32x4 v[MT][NT];
};

// Position of Hbar[row][col] in the per-lane order of PairA (so that each
// lane loads its share of Hbar with 16-byte loads).
template <int D>
__device__ __forceinline__ int pair_perm_index(int row, int col) {
  constexpr int MT = PairA<D>::MT, NT = PairA<D>::NT;
  const int w = row / (D / 2), rr = row % (D / 2);
  const int ti = rr / 16, g = (rr % 16) / 4, r = rr % 4;
  const int tj = col / 16, c = col % 16;
  return (((w * 64 + 16 * g + c) * MT + ti) * NT + tj) * 4 + r;
}

// ------------------------------------------------------------ kernel 2
// Fixed-order fp64 sum of the chunk partials -> Hbar (row-major), plus a copy
// of Hbar in PairA order for kernel 3.
template <int D>
__global__ __launch_bounds__(256) void k_hbar_reduce(const float* __restrict__ ws, float* __restrict__ Hbar,
                                                     float* __restrict__ hperm, int nchunk, int T) {
  const int bh = blockIdx.y;
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= D * D) return;
  // eight partials in flight at a time (unconditional loads, the index
  // clamped to the last chunk), added in chunk order: the same sum as one
  // load per chunk, without one memory round trip per chunk
  constexpr int kBatch = 8;
  const float* src = ws + static_cast<size_t>(bh) * nchunk * D * D + e;
  double sum = 0.0;
  for (int c0 = 0; c0 < nchunk; c0 += kBatch) {
    float p[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) p[u] = src[static_cast<size_t>(min(c0 + u, nchunk - 1)) * D * D];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) sum = c0 + u < nchunk ? sum + p[u] : sum;
  }
  const float h = static_cast<float>(sum / T);
  Hbar[static_cast<size_t>(bh) * D * D + e] = h;
  hperm[static_cast<size_t>(bh) * D * D + pair_perm_index<D>(e / D, e % D)] = h;
}

// ------------------------------------------------------------ kernel 3
// M_j = sigma_max(A), A = H_j - Hbar, by Lanczos on A^T A. One workgroup of
// two waves per block: each wave keeps half of the rows of A in registers
// (rebuilt from K_j, V_j on MFMA), so y = A x needs no communication and
// A^T y needs one exchange of a D-vector through LDS per step. Everything
// in the column space of A (the Lanczos vectors, their coefficients and the
// small tridiagonal eigenproblem) is computed by both waves on bitwise
// identical data, so the waves take identical decisions without further
// synchronisation.
//   * Vectors: fp32, lane l holds entries 16 tj + c (tj < D / 16); dot
//     products are 16-lane DPP sums.
//   * Three-term recurrence (the basis is kept in LDS only to form the Ritz
//     vector). After steps 5, 6, 7 and 8, then at steps predicted from the
//     decay of the residual bound between the last two checks, the Ritz pair
//     of the tridiagonal is computed (64-point Sturm multisection across the
//     lanes, then inverse iteration); the block stops when the residual
//     bound res^2 / (gap * theta) < kLanczosTol, otherwise the process
//     restarts from the Ritz vector after kLanczosK steps. Almost every block of the video workloads stops within 8 steps;
//     the long cycle is for blocks of i.i.d. keys (the text tokens of the
//     image shape: sigma_2 / sigma_1 about 0.9-0.99), which restarted every 8
//     steps needed up to 37 and with 24-step cycles about 20.
//   * M_j = ||A x|| / ||x|| is then evaluated in fp64 from the fp32 Ritz
//     vector, so its error is quadratic in the angle of x.
// Power iteration alone needs thousands of steps when sigma_2 / sigma_1 is
// close to 1 (blocks of i.i.d. keys); Lanczos converges in 5 to 8 steps for
// almost every block of the video workloads.
constexpr int kLanczosK = 24;        // steps per cycle before a restart
constexpr int kLanczosCheck = 5;     // first step count at which convergence is tested
constexpr int kLanczosCycles = 6;
constexpr double kLanczosTol = 3e-9;
constexpr int kPairThreads = 128;

__device__ __forceinline__ float start_sign(int row) {
  return ((static_cast<uint32_t>(row + 1) * 2654435761u) >> 16) & 1u ? -1.f : 1.f;
}

template <typename E, int D>
struct PairLds {
  union {
    struct {
      E kt[D][kLdT];
      E vt[D][kLdT];
    } tile;
    struct {
      float basis[2][kLanczosK + 1][D];  // per wave; vector entry 16 tj + c stored at c * NT + tj
      float zx[2][2][D];                 // [parity][wave] partial A^T y, same order
    } lz;
  } u;
  float kbar[D];
  float vsum[D];
  float al[2][kLanczosK];
  float be[2][kLanczosK];
  float rz[2][3][kLanczosK];  // per wave: sv, cp, bp of ritz_step_long
  double red[2][4];
};

template <int NT>
__device__ __forceinline__ void load_vec(const float* base, int c, float (&x)[NT]) {
#pragma unroll
  for (int q = 0; q < NT / 4; ++q) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(base + c * NT + 4 * q);
#pragma unroll
    for (int e = 0; e < 4; ++e) x[4 * q + e] = v[e];
  }
}
template <int NT>
__device__ __forceinline__ void store_vec(float* base, int c, const float (&x)[NT]) {
#pragma unroll
  for (int q = 0; q < NT / 4; ++q)
    *reinterpret_cast<f32x4*>(base + c * NT + 4 * q) = f32x4{x[4 * q], x[4 * q + 1], x[4 * q + 2], x[4 * q + 3]};
}
// Dot product of two column-space vectors (bitwise identical in every lane).
template <int NT>
__device__ __forceinline__ float vdot(const float (&a)[NT], const float (&b)[NT]) {
  float p = 0.f;
#pragma unroll
  for (int tj = 0; tj < NT; ++tj) p += a[tj] * b[tj];
  return row_sum16(p);
}

// y = A x for this wave's rows (y[ti][r] is row 16 (MT w + ti) + 4 g + r).
template <int D>
__device__ __forceinline__ void pair_ax(const PairA<D>& A, const float (&x)[D / 16], float (&y)[D / 32][4]) {
#pragma unroll
  for (int ti = 0; ti < PairA<D>::MT; ++ti)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float p = 0.f;
#pragma unroll
      for (int tj = 0; tj < PairA<D>::NT; ++tj) p += A.v[ti][tj][r] * x[tj];
      y[ti][r] = row_sum16(p);
    }
}
// Sum over the four 16-lane rows of a wave (lanes l, l ^ 16, l ^ 32, l ^ 48);
// the two additions are commutative pairs, so all four lanes get bitwise the
// same total. (Not the cross-row swaps of CDNA4: the compiler takes both
// results of its two-result swap builtin from one register.)
__device__ __forceinline__ float sum_over_rows4(float q) {
  q += __shfl_xor(q, 16);
  return q + __shfl_xor(q, 32);
}

// z = (partial over this wave's rows of) A^T y, summed over the 4 lane groups.
template <int D>
__device__ __forceinline__ void pair_aty(const PairA<D>& A, const float (&y)[D / 32][4], float (&z)[D / 16]) {
#pragma unroll
  for (int tj = 0; tj < PairA<D>::NT; ++tj) {
    float q = 0.f;
#pragma unroll
    for (int ti = 0; ti < PairA<D>::MT; ++ti)
#pragma unroll
      for (int r = 0; r < 4; ++r) q += A.v[ti][tj][r] * y[ti][r];
    z[tj] = sum_over_rows4(q);
  }
}

// 64-bit DPP move (both halves with the same control).
template <int CTRL>
__device__ __forceinline__ double dpp64(double v) {
  int2 x = __builtin_bit_cast(int2, v);
  x.x = __builtin_amdgcn_update_dpp(0, x.x, CTRL, 0xF, 0xF, false);
  x.y = __builtin_amdgcn_update_dpp(0, x.y, CTRL, 0xF, 0xF, false);
  return __builtin_bit_cast(double, x);
}
// One level of the reduce-scatter: lanes whose bit `bit` is set keep the
// upper half of `in` and send the lower half, the others the reverse; the
// partner (given by the DPP control, a lane with that bit flipped and the
// same higher bits) sends back the half this lane keeps.
template <int N, int CTRL>
__device__ __forceinline__ void rs_level(const double (&in)[2 * N], double (&out)[N], bool bit) {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const double keep = bit ? in[N + i] : in[i];
    const double send = bit ? in[i] : in[N + i];
    out[i] = keep + dpp64<CTRL>(send);
  }
}
// Sum over the 16 lanes of a DPP row of 16 values per lane; returns, in lane
// c of the row, the total of value c. Partners: row_mirror (c, 15 - c),
// row_half_mirror (c, c ^ 7 within each 8), quad_perm (c ^ 2), quad_perm
// (c ^ 1): each pairs lanes that differ in the level's bit and share the
// bits above it, so after four levels every lane has summed all 16 lanes.
__device__ __forceinline__ double butterfly16(const double (&p)[16], int c) {
  double a[8], b[4], d[2], e[1];
  rs_level<8, 0x140>(p, a, (c & 8) != 0);
  rs_level<4, 0x141>(a, b, (c & 4) != 0);
  rs_level<2, 0x4E>(b, d, (c & 2) != 0);
  rs_level<1, 0xB1>(d, e, (c & 1) != 0);
  return e[0];
}

// Number of eigenvalues below x of the tridiagonal (al, be): sign changes of
// the Sturm sequence p_i = det(T_i - x I), evaluated without division. The
// caller scales T so that its entries are at most 1 in magnitude, which keeps
// every p_i far from the fp32 range limits for m <= 8.
template <int m>
__device__ __forceinline__ int sturm_below(const float (&al)[m], const float (&be)[m], float x) {
  static_assert(m <= 8, "longer tridiagonals go through sturm_below_long");
  float p0 = 1.f, p1 = al[0] - x;
  int changes = p1 < 0.f ? 1 : 0;
#pragma unroll
  for (int i = 1; i < m; ++i) {
    const float p2 = (al[i] - x) * p1 - be[i - 1] * be[i - 1] * p0;
    changes += ((p2 < 0.f) != (p1 < 0.f)) ? 1 : 0;
    p0 = p1;
    p1 = p2;
  }
  return changes;
}
// The same count for a tridiagonal of m <= kLanczosK terms read from LDS
// (al, be unscaled; sc = 1 / ||T||). Past 8 terms the pair (p_{i-1}, p_i) is
// rescaled by 2^64 or 2^-64 whenever it has become tiny or huge: the
// recurrence is linear in the pair, so a common positive factor leaves
// every sign, and so the count, as it is.
__device__ __forceinline__ int sturm_below_long(const float* al, const float* be, int m, float sc, float x) {
  float p0 = 1.f, p1 = al[0] * sc - x;
  int changes = p1 < 0.f ? 1 : 0;
  for (int i = 1; i < m; ++i) {
    const float b = be[i - 1] * sc;
    float p2 = (al[i] * sc - x) * p1 - b * b * p0;
    changes += ((p2 < 0.f) != (p1 < 0.f)) ? 1 : 0;
    const float big = fmaxf(fabsf(p1), fabsf(p2));
    const float f = big < 0x1p-64f ? 0x1p64f : (big > 0x1p64f ? 0x1p-64f : 1.f);
    p0 = p1 * f;
    p1 = p2 * f;
  }
  return changes;
}

// Bracket the q-th largest eigenvalue inside [lo, hi] by 64-point multisection.
template <int m>
__device__ __forceinline__ void multisect(const float (&al)[m], const float (&be)[m], int q, int rounds,
                                          float& lo, float& hi, int l) {
  for (int rd = 0; rd < rounds; ++rd) {
    const float step = (hi - lo) * (1.f / 65.f);
    const float x = lo + step * static_cast<float>(l + 1);
    const bool above = m - sturm_below<m>(al, be, x) >= q;  // x still below theta_q
    const int cnt = __builtin_popcountll(__ballot(above));
    const float nlo = cnt > 0 ? lo + step * static_cast<float>(cnt) : lo;
    const float nhi = cnt < 64 ? lo + step * static_cast<float>(cnt + 1) : hi;
    lo = nlo;
    hi = nhi;
  }
}

// Ritz pair of the m-step tridiagonal of this wave: returns whether the
// residual bound is met, and writes the (unnormalised) Ritz vector to x when
// it is or when `form` is set (a restart needs it). Computed in fp32 on
// T / ||T|| (the Lanczos coefficients are fp32 quantities; M_j itself is
// evaluated afterwards in fp64 from the vector): the top eigenvalue to fp32
// precision by four rounds of 64-point multisection, the second one only to
// a conservative bracket (two rounds; the test uses its upper end, so the
// gap is never overestimated), the eigenvector by two passes of inverse
// iteration just above the top eigenvalue.
template <int m, int D>
__device__ __forceinline__ bool ritz_step(const float* al_s, const float* be_s, const float (*basis)[D], int l,
                                          int c, bool form, float (&x)[D / 16], float& need) {
  constexpr int NT = D / 16;
  float al[m], be[m];
  float lo = 0.f, hi = 0.f;
#pragma unroll
  for (int i = 0; i < m; ++i) {
    al[i] = al_s[i];
    be[i] = be_s[i];
  }
#pragma unroll
  for (int i = 0; i < m; ++i) {
    const float rr = (i > 0 ? fabsf(be[i - 1]) : 0.f) + (i < m - 1 ? fabsf(be[i]) : 0.f);
    lo = i == 0 ? al[0] - rr : fminf(lo, al[i] - rr);
    hi = i == 0 ? al[0] + rr : fmaxf(hi, al[i] + rr);
  }
  const float scale = fmaxf(fabsf(lo), fabsf(hi));
  if (!(scale > 0.f)) {  // T == 0: the start vector is in the null space of A
    load_vec<NT>(basis[0], c, x);
    return true;
  }
  const float inv_scale = 1.f / scale;
#pragma unroll
  for (int i = 0; i < m; ++i) {
    al[i] *= inv_scale;
    be[i] *= inv_scale;
  }
  float lo1 = lo * inv_scale, hi1 = hi * inv_scale;
  multisect<m>(al, be, 1, 4, lo1, hi1, l);
  float lo2 = lo * inv_scale, hi2 = hi1;
  multisect<m>(al, be, 2, 2, lo2, hi2, l);
  const float theta = 0.5f * (lo1 + hi1);
  // inverse iteration with (mu I - T), mu just above theta: positive definite
  const float mu = hi1 + fmaxf(fabsf(theta) * 1e-6f, 1e-30f);
  float sv[m];
#pragma unroll
  for (int i = 0; i < m; ++i) sv[i] = 1.f;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    float cp[m], bp[m];
    float rden = __builtin_amdgcn_rcpf(fmaxf(mu - al[0], 1e-30f));
    cp[0] = -be[0] * rden;
    bp[0] = sv[0] * rden;
#pragma unroll
    for (int i = 1; i < m; ++i) {
      rden = __builtin_amdgcn_rcpf(fmaxf((mu - al[i]) + be[i - 1] * cp[i - 1], 1e-30f));
      cp[i] = -be[i] * rden;
      bp[i] = (sv[i] + be[i - 1] * bp[i - 1]) * rden;
    }
    sv[m - 1] = bp[m - 1];
#pragma unroll
    for (int i = m - 2; i >= 0; --i) sv[i] = bp[i] - cp[i] * sv[i + 1];
    float n = 0.f;
#pragma unroll
    for (int i = 0; i < m; ++i) n += sv[i] * sv[i];
    const float inv = __builtin_amdgcn_rsqf(n);
#pragma unroll
    for (int i = 0; i < m; ++i) sv[i] *= inv;
  }
  // residual ||A^T A x - theta x|| = |beta_m s_m|; everything in units of scale
  const float res = fabsf(be[m - 1] * sv[m - 1]);
  const float gap = theta - hi2;
  const bool conv = res == 0.f || (gap > 0.f && theta > 0.f &&
                                   static_cast<double>(res) * res < kLanczosTol * gap * theta);
  need = gap > 0.f && theta > 0.f ? static_cast<float>(static_cast<double>(res) * res / (kLanczosTol * gap * theta))
                                  : INFINITY;
  if (conv || form) {
#pragma unroll
    for (int tj = 0; tj < NT; ++tj) x[tj] = 0.f;
#pragma unroll
    for (int i = 0; i < m; ++i) {
      float b[NT];
      load_vec<NT>(basis[i], c, b);
#pragma unroll
      for (int tj = 0; tj < NT; ++tj) x[tj] += sv[i] * b[tj];
    }
  }
  return conv;
}

// ritz_step for m > 8 steps, with the tridiagonal (al_s, be_s) and the
// vectors of the inverse iteration (sv, cp, bp: kLanczosK floats each, this
// wave's) kept in LDS and loops left rolled, so that the long, rarely taken
// checks hold no registers beside A. Every lane computes the same values;
// the LDS writes of those values race only with themselves.
template <int D>
__device__ __forceinline__ bool ritz_step_long(const float* al_s, const float* be_s, int m, float* sv, float* cp,
                                               float* bp, const float (*basis)[D], int l, int c, bool form,
                                               float (&x)[D / 16], float& need) {
  constexpr int NT = D / 16;
  float lo = 0.f, hi = 0.f;
  for (int i = 0; i < m; ++i) {
    const float rr = (i > 0 ? fabsf(be_s[i - 1]) : 0.f) + (i < m - 1 ? fabsf(be_s[i]) : 0.f);
    lo = i == 0 ? al_s[0] - rr : fminf(lo, al_s[i] - rr);
    hi = i == 0 ? al_s[0] + rr : fmaxf(hi, al_s[i] + rr);
  }
  const float scale = fmaxf(fabsf(lo), fabsf(hi));
  if (!(scale > 0.f)) {
    load_vec<NT>(basis[0], c, x);
    return true;
  }
  const float sc = 1.f / scale;
  auto section = [&](int q, int rounds, float& a, float& b) {
    for (int rd = 0; rd < rounds; ++rd) {
      const float step = (b - a) * (1.f / 65.f);
      const float xx = a + step * static_cast<float>(l + 1);
      const bool above = m - sturm_below_long(al_s, be_s, m, sc, xx) >= q;
      const int cnt = __builtin_popcountll(__ballot(above));
      const float na = cnt > 0 ? a + step * static_cast<float>(cnt) : a;
      const float nb = cnt < 64 ? a + step * static_cast<float>(cnt + 1) : b;
      a = na;
      b = nb;
    }
  };
  float lo1 = lo * sc, hi1 = hi * sc;
  section(1, 4, lo1, hi1);
  float lo2 = lo * sc, hi2 = hi1;
  section(2, 2, lo2, hi2);
  const float theta = 0.5f * (lo1 + hi1);
  const float mu = hi1 + fmaxf(fabsf(theta) * 1e-6f, 1e-30f);
  for (int i = 0; i < m; ++i) sv[i] = 1.f;
  for (int pass = 0; pass < 2; ++pass) {
    float rden = __builtin_amdgcn_rcpf(fmaxf(mu - al_s[0] * sc, 1e-30f));
    float cprev = -be_s[0] * sc * rden, bprev = sv[0] * rden;
    cp[0] = cprev;
    bp[0] = bprev;
    for (int i = 1; i < m; ++i) {
      const float bi1 = be_s[i - 1] * sc;
      rden = __builtin_amdgcn_rcpf(fmaxf((mu - al_s[i] * sc) + bi1 * cprev, 1e-30f));
      cprev = -be_s[i] * sc * rden;
      bprev = (sv[i] + bi1 * bprev) * rden;
      cp[i] = cprev;
      bp[i] = bprev;
    }
    float nxt = bp[m - 1];
    sv[m - 1] = nxt;
    float n = nxt * nxt;
    for (int i = m - 2; i >= 0; --i) {
      nxt = bp[i] - cp[i] * nxt;
      sv[i] = nxt;
      n += nxt * nxt;
    }
    const float inv = __builtin_amdgcn_rsqf(n);
    for (int i = 0; i < m; ++i) sv[i] *= inv;
  }
  const float res = fabsf(be_s[m - 1] * sc * sv[m - 1]);
  const float gap = theta - hi2;
  const bool conv = res == 0.f || (gap > 0.f && theta > 0.f &&
                                   static_cast<double>(res) * res < kLanczosTol * gap * theta);
  need = gap > 0.f && theta > 0.f ? static_cast<float>(static_cast<double>(res) * res / (kLanczosTol * gap * theta))
                                  : INFINITY;
  if (conv || form) {
#pragma unroll
    for (int tj = 0; tj < NT; ++tj) x[tj] = 0.f;
    for (int i = 0; i < m; ++i) {
      float b[NT];
      load_vec<NT>(basis[i], c, b);
      const float si = sv[i];
#pragma unroll
      for (int tj = 0; tj < NT; ++tj) x[tj] += si * b[tj];
    }
  }
  return conv;
}

// A += K_j^T V_j for this wave's rows.
template <int D>
__device__ __forceinline__ void pair_ktv(const PairLds<uint16_t, D>& s, PairA<D>& A, int w, int l) {
  constexpr int MT = PairA<D>::MT, NT = PairA<D>::NT;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    bf16x8 a[MT];
#pragma unroll
    for (int ti = 0; ti < MT; ++ti)
      a[ti] = *reinterpret_cast<const bf16x8*>(&s.u.tile.kt[16 * (MT * w + ti) + l % 16][32 * ks + 8 * (l / 16)]);
#pragma unroll
    for (int tj = 0; tj < NT; ++tj) {
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(&s.u.tile.vt[16 * tj + l % 16][32 * ks + 8 * (l / 16)]);
#pragma unroll
      for (int ti = 0; ti < MT; ++ti) A.v[ti][tj] = mfma16x16x32(a[ti], b, A.v[ti][tj]);
    }
  }
}
template <int D>
__device__ __forceinline__ void pair_ktv(const PairLds<float, D>& s, PairA<D>& A, int w, int l) {
  const int g = l / 16, c = l % 16;
#pragma unroll
  for (int ti = 0; ti < PairA<D>::MT; ++ti)
#pragma unroll
    for (int tj = 0; tj < PairA<D>::NT; ++tj)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * (PairA<D>::MT * w + ti) + 4 * g + r, col = 16 * tj + c;
        float sum = 0.f;
#pragma unroll 4
        for (int t = 0; t < kBlock; ++t) sum += s.u.tile.kt[row][t] * s.u.tile.vt[col][t];
        A.v[ti][tj][r] += sum;
      }
}

template <typename E, int D>
__global__ __launch_bounds__(kPairThreads) __attribute__((amdgpu_waves_per_eu(2))) void k_block_spectral(const E* __restrict__ K, const E* __restrict__ V,
                                                                 const float* __restrict__ kbar,
                                                                 const float* __restrict__ vsum,
                                                                 const float* __restrict__ hperm,
                                                                 double* __restrict__ M, int L, int T, int nbh) {
  extern __shared__ __align__(16) unsigned char smem[];
  PairLds<E, D>& s = *reinterpret_cast<PairLds<E, D>*>(smem);
  constexpr int MT = PairA<D>::MT, NT = PairA<D>::NT;
  // one workgroup per (head, block), heads fastest and blocks from the end
  // of the sequence back: blocks of nearly i.i.d. keys (text tokens, which
  // DiT layouts append after the image or video tokens) have the smallest
  // spectral gaps and the longest Lanczos runs, and this order starts them
  // first instead of leaving the last head's to run alone at the end
  const int j = T - 1 - static_cast<int>(blockIdx.x / nbh), bh = static_cast<int>(blockIdx.x % nbh);
  const int t = threadIdx.x, w = t / 64, l = t % 64, g = l / 16, c = l % 16;
  const int row0 = j * kBlock, nvalid = min(kBlock, L - row0);

  // A starts as -Hbar (this lane's entries, 16-byte loads of the permuted
  // copy). For bf16 all the K_j and V_j staging items and kbar_j, vsum_j are
  // in flight before the first is waited on (instead of one round trip per
  // staging item), and the Hbar loads (from L2) follow the LDS writes that
  // free the staging registers.
  PairA<D> A;
  const f32x4* hp = reinterpret_cast<const f32x4*>(hperm + static_cast<size_t>(bh) * D * D) + (w * 64 + l) * MT * NT;
  const E* Kh = K + static_cast<size_t>(bh) * L * D;
  const E* Vh = V + static_cast<size_t>(bh) * L * D;
  const size_t o_kv = (static_cast<size_t>(bh) * T + j) * D + t;
  if constexpr (sizeof(E) == 2) {
    constexpr int IPT = 2 * D / kPairThreads;  // staging items per thread
    static_assert(2 * D % kPairThreads == 0, "staging items per thread");
    uint4 rk[IPT][4], rv[IPT][4];
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
      load_item<D>(Kh, row0, nvalid, t + kPairThreads * i, rk[i]);
      load_item<D>(Vh, row0, nvalid, t + kPairThreads * i, rv[i]);
    }
    float kb = 0.f, vs = 0.f;
    if (t < D) {
      kb = kbar[o_kv];
      vs = vsum[o_kv];
    }
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
      store_item(s.u.tile.kt, t + kPairThreads * i, rk[i]);
      store_item(s.u.tile.vt, t + kPairThreads * i, rv[i]);
    }
    if (t < D) {
      s.kbar[t] = kb;
      s.vsum[t] = vs;
    }
#pragma unroll
    for (int ti = 0; ti < MT; ++ti)
#pragma unroll
      for (int tj = 0; tj < NT; ++tj) A.v[ti][tj] = -hp[ti * NT + tj];
  } else {
#pragma unroll
    for (int ti = 0; ti < MT; ++ti)
#pragma unroll
      for (int tj = 0; tj < NT; ++tj) A.v[ti][tj] = -hp[ti * NT + tj];
    stage_transposed<D, kPairThreads>(Kh, row0, nvalid, s.u.tile.kt);
    stage_transposed<D, kPairThreads>(Vh, row0, nvalid, s.u.tile.vt);
    if (t < D) {
      s.kbar[t] = kbar[o_kv];
      s.vsum[t] = vsum[o_kv];
    }
  }
  __syncthreads();
  // A = K_j^T V_j - kbar_j^T vsum_j - Hbar
#pragma unroll
  for (int ti = 0; ti < MT; ++ti)
#pragma unroll
    for (int tj = 0; tj < NT; ++tj)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        A.v[ti][tj][r] -= s.kbar[16 * (MT * w + ti) + 4 * g + r] * s.vsum[16 * tj + c];
  pair_ktv<D>(s, A, w, l);
  lds_barrier();  // the staged tiles are dead from here on (the basis reuses their LDS)

  float(*basis)[D] = s.u.lz.basis[w];
  int par = 0;
  // z <- A^T A-like product: y = A x (if x given) then A^T y, summed over both waves
  auto exchange = [&](float (&z)[NT]) {
    if (g == 0) store_vec<NT>(s.u.lz.zx[par][w], c, z);
    lds_barrier();
    float z0[NT], z1[NT];
    load_vec<NT>(s.u.lz.zx[par][0], c, z0);
    load_vec<NT>(s.u.lz.zx[par][1], c, z1);
#pragma unroll
    for (int tj = 0; tj < NT; ++tj) z[tj] = z0[tj] + z1[tj];
    par ^= 1;
  };

  // start vector x = A^T r for a fixed +-1 pattern r over the rows
  float x[NT];
  {
    float y[MT][4];
#pragma unroll
    for (int ti = 0; ti < MT; ++ti)
#pragma unroll
      for (int r = 0; r < 4; ++r) y[ti][r] = start_sign(16 * (MT * w + ti) + 4 * g + r);
    pair_aty<D>(A, y, x);
    exchange(x);
    // r in the null space of A^T: start from a fixed +-1 pattern over the columns
    if (!(vdot<NT>(x, x) > 0.f)) {
#pragma unroll
      for (int tj = 0; tj < NT; ++tj) x[tj] = start_sign(D + 16 * tj + c);
    }
  }
  bool done = false;
  for (int cyc = 0; cyc < kLanczosCycles && !done; ++cyc) {
    float v[NT], vp[NT];
    {
      const float n2 = vdot<NT>(x, x);
      const float inv = n2 > 0.f ? 1.f / sqrtf(n2) : 0.f;
#pragma unroll
      for (int tj = 0; tj < NT; ++tj) {
        v[tj] = x[tj] * inv;
        vp[tj] = 0.f;
      }
    }
    float beta_prev = 0.f;
    int next = kLanczosCheck, m_prev = 0;  // the step of the next convergence check, and of the last one
    float need_prev = 0.f;
    if (g == 0) store_vec<NT>(basis[0], c, v);
    // three-term recurrence with no reorthogonalisation: once the top Ritz
    // pair converges the basis loses orthogonality (copies of it appear in
    // the tridiagonal, the gap test then fails and the cycle ends with a
    // restart from the Ritz vector), and M_j is re-evaluated from A itself
    for (int k = 0; k < kLanczosK; ++k) {
      float z[NT];
      {
        float y[MT][4];
        pair_ax<D>(A, v, y);
        pair_aty<D>(A, y, z);
      }
      exchange(z);
      const float alpha = vdot<NT>(z, v);
      float wv[NT];
#pragma unroll
      for (int tj = 0; tj < NT; ++tj) wv[tj] = z[tj] - alpha * v[tj] - beta_prev * vp[tj];
      const float beta = sqrtf(vdot<NT>(wv, wv));
      const float binv = beta > 0.f ? __builtin_amdgcn_rcpf(beta) : 0.f;
#pragma unroll
      for (int tj = 0; tj < NT; ++tj) {
        vp[tj] = v[tj];
        v[tj] = wv[tj] * binv;
      }
      beta_prev = beta;
      if (g == 0) store_vec<NT>(basis[k + 1], c, v);
      if (l == 0) {
        s.al[w][k] = alpha;
        s.be[w][k] = beta;
      }
      const int m = k + 1;
      if (m == next) {
        bool conv;
        float need;
        switch (m) {
          case 5: conv = ritz_step<5, D>(s.al[w], s.be[w], basis, l, c, false, x, need); break;
          case 6: conv = ritz_step<6, D>(s.al[w], s.be[w], basis, l, c, false, x, need); break;
          case 7: conv = ritz_step<7, D>(s.al[w], s.be[w], basis, l, c, false, x, need); break;
          case 8: conv = ritz_step<8, D>(s.al[w], s.be[w], basis, l, c, false, x, need); break;
          default:
            conv = ritz_step_long<D>(s.al[w], s.be[w], m, s.rz[w][0], s.rz[w][1], s.rz[w][2], basis, l, c,
                                     m == kLanczosK, x, need);
            break;
        }
        if (conv) {
          done = true;
          break;
        }
        // next check: after every step to 8; then where the decay of the
        // residual bound since the last check (need falls geometrically with
        // the steps) predicts need < 1, at most 8 steps on, 4 without a
        // usable rate. need is the same value in both waves (computed from
        // the same tridiagonal), so both keep the same schedule.
        int ahead = 1;
        if (m >= 8) {
          ahead = 4;
          if (m_prev > 0 && need < INFINITY && need_prev > need) {
            const float rate = (__log2f(need_prev) - __log2f(need)) / static_cast<float>(m - m_prev);
            ahead = min(8, max(1, static_cast<int>(ceilf(__log2f(need) / rate))));
          }
        }
        next = min(m + ahead, kLanczosK);
        need_prev = need;
        m_prev = m;
      }
    }
  }
  // M_j = ||A x|| / ||x|| in fp64 from the fp32 Ritz vector. Each lane's 16
  // row partials are summed over the 16 lanes of its DPP row by a butterfly
  // reduce-scatter (after it lane c holds the whole of its row c), so the
  // 64-bit values cross lanes 15 times instead of 64.
  static_assert(4 * MT <= 16, "at most 16 rows per lane");
  double p[16];  // rows 4 ti + r of this lane (4 MT of them; the rest are zero for D = 64)
#pragma unroll
  for (int i = 4 * MT; i < 16; ++i) p[i] = 0.0;
#pragma unroll
  for (int ti = 0; ti < MT; ++ti)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      double q = 0.0;
#pragma unroll
      for (int tj = 0; tj < NT; ++tj) q += static_cast<double>(A.v[ti][tj][r]) * x[tj];
      p[4 * ti + r] = q;
    }
  const double yrow = butterfly16(p, c);
  const double ysq = row_sum16(yrow * yrow);
  double x2 = 0.0;
#pragma unroll
  for (int tj = 0; tj < NT; ++tj) x2 += static_cast<double>(x[tj]) * x[tj];
  x2 = row_sum16(x2);
  if (c == 0) s.red[w][g] = ysq;
  lds_barrier();
  if (t == 0) {
    const double ys = ((s.red[0][0] + s.red[0][1]) + (s.red[0][2] + s.red[0][3])) +
                      ((s.red[1][0] + s.red[1][1]) + (s.red[1][2] + s.red[1][3]));
    M[static_cast<size_t>(bh) * T + j] = x2 > 0.0 ? sqrt(ys / x2) : 0.0;
  }
}

template <typename E, int D>
int stats_chunks(const paro_problem& p, int* G) {
  const int T = ceil_div(p.L, kBlock);
  const int bh = p.B * p.H;
  // about 1024 workgroups in all, rounded down: two full rounds of the 512
  // that fit at once (256 CUs x 2), rather than two and a sliver whose
  // workgroups each walk a whole chunk alone. For bf16, chunks of at least
  // 8 blocks: every chunk writes a D x D partial sum (64 KB at d = 128) that
  // k_hbar_reduce reads back, which for chunks of 2 blocks (the image shape)
  // is as much traffic as K and V themselves (precompute 0.163 -> 0.152 ms
  // there, 0.227 -> 0.214 ms at 480p; the fp32 path's per-block staging is
  // slower, so it keeps the finer split).
  const int gmin = sizeof(E) == 2 ? 8 : 1;
  int nchunk = max(1, min(T / gmin, 1024 / bh));
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
  const size_t lds3 = sizeof(PairLds<E, D>);
  hipError_t e;
  if (lds1 > 65536 && (e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_block_stats<E, D>),
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               static_cast<int>(lds1))) != hipSuccess)
    return e;
  if (lds3 > 65536 && (e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_block_spectral<E, D>),
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               static_cast<int>(lds3))) != hipSuccess)
    return e;
  float* partials = static_cast<float*>(ws);
  float* hperm = partials + static_cast<size_t>(bh) * nchunk * D * D;
  hipLaunchKernelGGL((k_block_stats<E, D>), dim3(nchunk, bh), dim3(kThreads), lds1, st, K, V, kbar, vsum,
                     partials, p.L, T, G, nchunk);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_hbar_reduce<D>, dim3(ceil_div(D * D, 256), bh), dim3(256), 0, st,
                     static_cast<const float*>(partials), Hbar, hperm, nchunk, T);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((k_block_spectral<E, D>), dim3(static_cast<unsigned>(T * bh)), dim3(kPairThreads), lds3, st, K, V,
                     kbar, vsum, static_cast<const float*>(hperm), M, p.L, T, static_cast<int>(bh));
  return hipGetLastError();
}

}  // namespace

size_t precompute_workspace_bytes(const paro_problem& p) {
  int G = 1;
  const int nchunk = p.dtype == PARO_DTYPE_BF16 ? stats_chunks<uint16_t, 64>(p, &G) : stats_chunks<float, 64>(p, &G);
  // per (b, h): nchunk partial H sums, then Hbar in PairA order
  return static_cast<size_t>(p.B) * p.H * (nchunk + 1) * p.d * p.d * sizeof(float);
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
