// Fused piecewise attention ("PISA: Piecewise Sparse Attention Is Wiser for
// Efficient Diffusion Transformers", section 2, "core algorithm" and
// "hardware implementation": stage 1 exact, stage 2 zeroth-order scan,
// stage 3 global first-order correction, then o = N / D).
//
// bf16 kernel (k_attn_bf16): a workgroup of 8 waves serves 4 consecutive
// query blocks of one (batch, head); each block of 64 rows is split between
// two waves of 32 rows, so every wave fits in 256 registers and each SIMD
// runs two waves whose matrix and vector work interleave.
//  * The exact lists of the 4 blocks are merged into their sorted union; each
//    union tile (64 keys x d) is staged once into LDS for all 8 waves (the
//    global loads of the tile after next sit in registers while the current
//    one is consumed; two LDS buffers; one LDS-only barrier per tile). K is
//    stored row-major and V transposed (V^T[dim][key]); rows are padded so
//    every MFMA operand is one conflict-free ds_read_b128 at a per-lane base
//    plus a compile-time offset.
//  * A wave computes S^T = K Q^T for its 32 queries on
//    v_mfma_f32_32x32x16_bf16 with Q^T held in registers. In the C layout of
//    S^T each lane owns one query and 32 keys of the tile, so the softmax
//    state is per lane.
//  * O^T += V^T P^T with P straight from the S^T accumulators (K rows are read
//    in a permuted order so each lane's 8 consecutive P values are 8
//    consecutive keys of a V^T row).
//  * The softmax reference m is fixed by the first tile a wave sees and never
//    moves, so O needs no rescaling: N and D share the factor exp(-m), which
//    cancels in N / D. A tile whose maximum exceeds m by more than 2^64 (far
//    beyond real attention logits) marks the wave, and after the pass the
//    marked waves recompute their rows with m set to the exact maximum
//    recorded during the first pass.
//  * Stage 2 streams all T centroids in chunks of 32 through the same code
//    (kbar as keys, vsum as values, converted to bf16 while staging), with the
//    blocks of S_i and j >= T masked; the weights add n_j p to D and p to c.
//  * Stage 3 forms r^T = Hbar^T q^T on MFMA (Hbar transposed into LDS in
//    bf16) and adds (scale c) r before the division.
//
// fp32 kernel (k_attn_f32): the same three stages in plain fp32 arithmetic,
// one key at a time; used for fp32 problems.
#include <algorithm>

#include "paro_common.h"

namespace paro {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kQB = 4;                    // query blocks per workgroup
constexpr int kWaves = 2 * kQB;           // two 32-row waves per query block
constexpr int kAttnThreads = 64 * kWaves;
constexpr float kOverflowSlack = 64.f;    // log2 units above the reference max that trigger a rerun

template <int D>
struct Geo {
  static constexpr int CG = D / 8;                         // 16-byte chunks in a K row
  static constexpr int KS = D + 8;                         // K tile row stride (elements)
  static constexpr int VS = 64 + 8;                        // V^T tile row stride
  static constexpr int HS = D + 8;                         // Hbar^T row stride
  static constexpr int KTILE = 64 * KS;
  static constexpr int VTILE = D * VS;
  static constexpr int BUF = KTILE + VTILE;                // one staging buffer (elements)
  static constexpr int NK = D / 16;                        // k-steps of S^T = K Q^T
  static constexpr int NU = D / 32;                        // 32-dim output tiles
  static constexpr int KPT = 64 * CG / kAttnThreads;       // exact-tile K chunks staged per thread
  static constexpr int KCT = (32 * CG + kAttnThreads - 1) / kAttnThreads;  // centroid K chunks per thread
  static constexpr int NR = (KPT > 2 * KCT ? KPT : 2 * KCT) + 2;          // staging registers (16 B)
  static constexpr int VI = NR - 2;                                       // first V register
  static_assert(D * HS <= 2 * BUF, "Hbar^T must fit in the staging buffers");
  static_assert(32 * CG == kAttnThreads || 32 * CG * 2 == kAttnThreads, "V items per thread");
};

// Key (tile row) that MFMA row m of S^T sub-tile t reads, chosen so that
// accumulator register i of a lane in half g holds key 32 t + 16 (i/8) + 8 g + i%8.
__device__ __forceinline__ int perm_key(int t, int m) {
  const int a = m >> 3, g = (m >> 2) & 1, b = m & 3;
  return 32 * t + 16 * (a >> 1) + 8 * g + 4 * (a & 1) + b;
}

__device__ __forceinline__ uint32_t half16(const uint4& v, int e) {
  const uint32_t w = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
  return (e & 1) ? (w >> 16) : (w & 0xFFFFu);
}
__device__ __forceinline__ uint4 to_bf16x8(const float4& a, const float4& b) {
  return make_uint4(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w), pack_bf16x2(b.x, b.y), pack_bf16x2(b.z, b.w));
}
__device__ __forceinline__ float4 as_f4(const uint4& u) { return __builtin_bit_cast(float4, u); }

// ------------------------------------------------------------ staging
// One step's data in flight, NR registers of 16 bytes per thread:
//  exact tile (bf16): r[0..KPT) = K chunks; r[VI..VI+2) = 2 keys x 8 dims of V;
//  centroid chunk (fp32, 32 centroids): r[0..2 KCT) = kbar chunks as float4
//  pairs; r[VI..VI+2) = 1 centroid x 8 dims of vsum.
// V items put consecutive lanes on consecutive keys, so each LDS write
// instruction fills whole V^T rows. Rows past the valid range re-read the last
// valid row (finite values whose keys are masked out): no predicated loads.
template <int D>
struct Stage {
  uint4 r[Geo<D>::NR];
};

template <int D>
__device__ __forceinline__ void load_exact(const uint16_t* __restrict__ Kh, const uint16_t* __restrict__ Vh,
                                           int row0, int nvalid, Stage<D>& st) {
  constexpr int CG = Geo<D>::CG, KPT = Geo<D>::KPT, VI = Geo<D>::VI;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int q = threadIdx.x + kAttnThreads * i;
    const int row = min(q / CG, nvalid - 1), c = q % CG;
    st.r[i] = *reinterpret_cast<const uint4*>(Kh + static_cast<size_t>(row0 + row) * D + 8 * c);
  }
  // item: 32 key pairs (fast) x CG dim groups; with d = 64 the upper half of
  // the threads repeats the lower half's loads and stores nothing
  const int item = threadIdx.x % (32 * CG);
  const int kp = item & 31, dg = item >> 5;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int row = min(2 * kp + e, nvalid - 1);
    st.r[VI + e] = *reinterpret_cast<const uint4*>(Vh + static_cast<size_t>(row0 + row) * D + 8 * dg);
  }
}
template <int D>
__device__ __forceinline__ void store_exact(const Stage<D>& st, uint16_t* buf) {
  constexpr int CG = Geo<D>::CG, KPT = Geo<D>::KPT, KS = Geo<D>::KS, VS = Geo<D>::VS, VI = Geo<D>::VI;
  uint16_t* vt = buf + Geo<D>::KTILE;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int q = threadIdx.x + kAttnThreads * i;
    *reinterpret_cast<uint4*>(buf + (q / CG) * KS + 8 * (q % CG)) = st.r[i];
  }
  if (threadIdx.x < 32 * CG) {
    const int item = threadIdx.x;
    const int kp = item & 31, dg = item >> 5;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      *reinterpret_cast<uint32_t*>(vt + (8 * dg + e) * VS + 2 * kp) =
          half16(st.r[VI], e) | (half16(st.r[VI + 1], e) << 16);
  }
}
// Tail chunk of 32 centroids [j0, j0 + 32): kbar rows -> K tile rows 0..31,
// vsum rows -> keys 0..31 of the V^T tile (fp32 converted to bf16 on store).
template <int D>
__device__ __forceinline__ void load_centroids(const float* __restrict__ kb, const float* __restrict__ vs, int j0,
                                               int T, Stage<D>& st) {
  constexpr int CG = Geo<D>::CG, KCT = Geo<D>::KCT, VI = Geo<D>::VI;
#pragma unroll
  for (int i = 0; i < KCT; ++i) {
    const int q = min(static_cast<int>(threadIdx.x) + kAttnThreads * i, 32 * CG - 1);
    const int row = min(j0 + q / CG, T - 1), c = q % CG;
    const uint4* src = reinterpret_cast<const uint4*>(kb + static_cast<size_t>(row) * D + 8 * c);
    st.r[2 * i] = src[0];
    st.r[2 * i + 1] = src[1];
  }
  const int item = threadIdx.x % (32 * CG);  // 32 centroids (fast) x CG dim groups
  const int kc = item & 31, dg = item >> 5;
  const uint4* src = reinterpret_cast<const uint4*>(vs + static_cast<size_t>(min(j0 + kc, T - 1)) * D + 8 * dg);
  st.r[VI] = src[0];
  st.r[VI + 1] = src[1];
}
template <int D>
__device__ __forceinline__ void store_centroids(const Stage<D>& st, uint16_t* buf) {
  constexpr int CG = Geo<D>::CG, KCT = Geo<D>::KCT, KS = Geo<D>::KS, VS = Geo<D>::VS, VI = Geo<D>::VI;
  uint16_t* vt = buf + Geo<D>::KTILE;
#pragma unroll
  for (int i = 0; i < KCT; ++i) {
    const int q = threadIdx.x + kAttnThreads * i;
    if (q < 32 * CG)
      *reinterpret_cast<uint4*>(buf + (q / CG) * KS + 8 * (q % CG)) =
          to_bf16x8(as_f4(st.r[2 * i]), as_f4(st.r[2 * i + 1]));
  }
  if (threadIdx.x < 32 * CG) {
    const int item = threadIdx.x;
    const int kc = item & 31, dg = item >> 5;
    const float4 x = as_f4(st.r[VI]), y = as_f4(st.r[VI + 1]);
    const float a0[8] = {x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) vt[(8 * dg + e) * VS + kc] = f32_to_bf16(a0[e]);
  }
}

// ------------------------------------------------------------ compute
template <int D>
struct Acc {
  bf16x8 qb[Geo<D>::NK];   // B operand Q^T: query lane % 32 of the wave's rows, dims 16 s + 8 g .. + 8
  f32x16 o[Geo<D>::NU];    // O^T: dims 32 u + 8 (i / 4) + 4 g + i % 4, query lane % 32
  float m;                 // reference max (log2 units), -inf until the first tile
  float mtrue;             // exact running max, for a rerun
  float dsum;              // this lane's part of D
  float csum;              // this lane's part of c
  bool over;               // some logit exceeded m + kOverflowSlack
};

// S^T of 32 keys (kt: the lane's permuted K row and 8-dim half).
template <int D>
__device__ __forceinline__ f32x16 qk_half(const uint16_t* kt, const Acc<D>& a) {
  f32x16 s = f32x16{};
#pragma unroll
  for (int ks = 0; ks < Geo<D>::NK; ++ks)
    s = mfma32x32x16(*reinterpret_cast<const bf16x8*>(kt + 16 * ks), a.qb[ks], s);
  return s;
}

// O^T += V^T P^T for 32 keys (vt: the lane's V^T row base plus the key offset).
template <int D>
__device__ __forceinline__ void pv_half(const uint16_t* vt, const bf16x8 (&pb)[2], Acc<D>& a) {
#pragma unroll
  for (int u = 0; u < Geo<D>::NU; ++u)
#pragma unroll
    for (int s = 0; s < 2; ++s)
      a.o[u] = mfma32x32x16(*reinterpret_cast<const bf16x8*>(vt + 32 * u * Geo<D>::VS + 16 * s), pb[s], a.o[u]);
}

// The lane's 16 keys of 32-key sub-tile t as a 16-bit mask of a 64-bit key mask.
__device__ __forceinline__ uint32_t lane_bits(uint64_t km, int t, int g) {
  return static_cast<uint32_t>((km >> (32 * t + 8 * g)) & 0xFFu) |
         (static_cast<uint32_t>((km >> (32 * t + 16 + 8 * g)) & 0xFFu) << 8);
}

// Softmax weights of one 32-key sub-tile against the fixed reference max.
// kMask: keys with a set bit in lmask get weight 0. kTail: D gains n_j p
// (n_j = 64 except nlast for the key flagged in llast) and c gains p.
template <int D, bool kMask, bool kTail>
__device__ __forceinline__ void softmax_half(f32x16& s, Acc<D>& a, float cl2, uint32_t lmask, uint32_t llast,
                                             float nlast, bf16x8 (&pb)[2]) {
  float v = -INFINITY;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (kMask && ((lmask >> i) & 1u)) s[i] = -INFINITY;
    v = fmaxf(v, s[i]);
  }
  v = fmaxf(v, __shfl_xor(v, 32)) * cl2;
  a.mtrue = fmaxf(a.mtrue, v);
  if (a.m == -INFINITY) a.m = v;
  a.over = a.over || v > a.m + kOverflowSlack;
  const float mref = a.m == -INFINITY ? 0.f : a.m;
  float pv[16];
  float ps = 0.f, pl = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], cl2, -mref));
    pv[i] = p;
    ps += p;
    if (kTail) pl += ((llast >> i) & 1u) ? p : 0.f;
  }
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    uint4 w;
    w.x = pack_bf16x2(pv[8 * c + 0], pv[8 * c + 1]);
    w.y = pack_bf16x2(pv[8 * c + 2], pv[8 * c + 3]);
    w.z = pack_bf16x2(pv[8 * c + 4], pv[8 * c + 5]);
    w.w = pack_bf16x2(pv[8 * c + 6], pv[8 * c + 7]);
    pb[c] = __builtin_bit_cast(bf16x8, w);
  }
  if (kTail) {
    a.dsum += 64.f * ps + (nlast - 64.f) * pl;
    a.csum += ps;
  } else {
    a.dsum += ps;
  }
}

template <int D>
__global__ __launch_bounds__(kAttnThreads) void k_attn_bf16(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const float* __restrict__ kbar, const float* __restrict__ vsum, const float* __restrict__ Hbar,
    const int32_t* __restrict__ idx, uint16_t* __restrict__ O, int L, int T, int keep_k, float scale, int nwg) {
  constexpr int BUF = Geo<D>::BUF, KS = Geo<D>::KS, VS = Geo<D>::VS, HS = Geo<D>::HS;
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* buf = reinterpret_cast<uint16_t*>(smem);  // 2 staging buffers
  const int nw = ceil_div(T, 32);
  uint32_t* masks = reinterpret_cast<uint32_t*>(smem + sizeof(uint16_t) * 2 * BUF);  // [kQB][nw]
  int* sh = reinterpret_cast<int*>(masks + kQB * nw);                               // nu, rerun flags
  uint16_t* ulist = reinterpret_cast<uint16_t*>(sh + 12);                           // [T]

  // XCD-aware order: consecutive workgroup ids go to different XCDs, so hand
  // each XCD a contiguous run of (head, query-block group) items.
  int wg = blockIdx.x;
  const int n8 = (nwg / 8) * 8;
  if (wg < n8) wg = (wg % 8) * (nwg / 8) + wg / 8;
  const int ngrp = ceil_div(T, kQB);
  const int grp = wg % ngrp, bh = wg / ngrp;

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 5, ql = l & 31;
  const int qi = w >> 1;                       // query block of this wave within the group
  const int qblk = grp * kQB + qi;
  const int row = qblk * 64 + 32 * (w & 1) + ql;  // this lane's query row
  const bool qvalid = qblk < T;
  const size_t head = static_cast<size_t>(bh) * L * D;
  const uint16_t* Kh = K + head;
  const uint16_t* Vh = V + head;
  const float cl2 = scale * kLog2e;
  const int nlast = L - 64 * (T - 1);
  // per-lane operand offsets inside a staging buffer
  const int koff = perm_key(0, ql) * KS + 8 * g;              // K rows of sub-tile 0 (+32 KS for 1)
  const int voff = Geo<D>::KTILE + ql * VS + 8 * g;           // V^T rows 32 u + ql (+16 s + 32 t keys)

  Acc<D> a;
  {
    const uint16_t* qp = Q + head + static_cast<size_t>(row) * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < Geo<D>::NK; ++ks) {
      const uint4 v = (qvalid && row < L) ? *reinterpret_cast<const uint4*>(qp + 16 * ks) : make_uint4(0, 0, 0, 0);
      a.qb[ks] = __builtin_bit_cast(bf16x8, v);
    }
    a.m = -INFINITY;
    a.mtrue = -INFINITY;
  }

  // ---- membership masks of the 4 exact lists and their sorted union
  for (int e = tid; e < kQB * nw; e += kAttnThreads) masks[e] = 0u;
  lds_barrier();
  if (qvalid && (w & 1) == 0) {
    const int32_t* irow = idx + (static_cast<size_t>(bh) * T + qblk) * keep_k;
    for (int e = l; e < keep_k; e += 64) {
      const int j = min(max(irow[e], 0), T - 1);
      atomicOr(&masks[qi * nw + (j >> 5)], 1u << (j & 31));
    }
  }
  lds_barrier();
  if (w == 0) {
    int base = 0;
    for (int w0 = 0; w0 < nw; w0 += 64) {
      const int wd = w0 + l;
      uint32_t u = 0;
      if (wd < nw) u = masks[wd] | masks[nw + wd] | masks[2 * nw + wd] | masks[3 * nw + wd];
      const int cnt = __builtin_popcount(u);
      int incl = cnt;
      for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o);
        if (l >= o) incl += v;
      }
      int pos = base + incl - cnt;
      while (u) {
        ulist[pos++] = static_cast<uint16_t>(wd * 32 + __builtin_ctz(u));
        u &= u - 1;
      }
      base += __shfl(incl, 63);
    }
    if (l == 0) sh[0] = base;
  }
  lds_barrier();
  const int nu = sh[0];
  const uint32_t* mymask = masks + qi * nw;
  const float* kb = kbar + static_cast<size_t>(bh) * T * D;
  const float* vs = vsum + static_cast<size_t>(bh) * T * D;
  const int nch = keep_k < T ? ceil_div(T, 32) : 0;

  bool active = qvalid;
#pragma unroll
  for (int u = 0; u < Geo<D>::NU; ++u) a.o[u] = f32x16{};
  a.dsum = 0.f;
  a.csum = 0.f;
  for (int pass = 0; pass < 2; ++pass) {
    if (pass > 0 && active) {  // only rerunning waves start over; the others keep their sums
#pragma unroll
      for (int u = 0; u < Geo<D>::NU; ++u) a.o[u] = f32x16{};
      a.dsum = 0.f;
      a.csum = 0.f;
    }
    a.over = false;

    // ---- stages 1 and 2 as one stream of steps: the nu exact tiles of the
    // union, then the nch chunks of 32 centroids.
    const int nsteps = nu + nch;
    Stage<D> st;
    auto fetch = [&](int step) {
      if (step < nu) {
        const int j = ulist[step];
        load_exact<D>(Kh, Vh, 64 * j, j == T - 1 ? nlast : 64, st);
      } else {
        load_centroids<D>(kb, vs, 32 * (step - nu), T, st);
      }
    };
    auto put = [&](int step, uint16_t* b) {
      if (step < nu)
        store_exact<D>(st, b);
      else
        store_centroids<D>(st, b);
    };
    if (nsteps > 0) {
      fetch(0);
      put(0, buf);
    }
    lds_barrier();
    if (nsteps > 1) fetch(1);
    // Three loops over consecutive step ranges, one compute variant each:
    // full exact tiles, then the partial last block (always last in the
    // ascending union), then the centroid chunks.
    const int nfull = (nu > 0 && ulist[nu - 1] == T - 1 && nlast < 64) ? nu - 1 : nu;
    auto advance = [&](int step) {
      if (step + 1 < nsteps) put(step + 1, buf + ((step + 1) & 1) * BUF);
      if (step + 2 < nsteps) fetch(step + 2);
      lds_barrier();
    };
    for (int step = 0; step < nfull; ++step) {
      const uint16_t* bc = buf + (step & 1) * BUF;
      const int j = ulist[step];
      if (active && ((mymask[j >> 5] >> (j & 31)) & 1u)) {
        f32x16 s0 = qk_half<D>(bc + koff, a);
        f32x16 s1 = qk_half<D>(bc + koff + 32 * KS, a);
        bf16x8 p0[2], p1[2];
        softmax_half<D, false, false>(s0, a, cl2, 0u, 0u, 0.f, p0);
        pv_half<D>(bc + voff, p0, a);
        softmax_half<D, false, false>(s1, a, cl2, 0u, 0u, 0.f, p1);
        pv_half<D>(bc + voff + 32, p1, a);
      }
      advance(step);
    }
    for (int step = nfull; step < nu; ++step) {
      const uint16_t* bc = buf + (step & 1) * BUF;
      const int j = ulist[step];
      if (active && ((mymask[j >> 5] >> (j & 31)) & 1u)) {
        const uint64_t km = ~0ull << nlast;
        f32x16 s0 = qk_half<D>(bc + koff, a);
        f32x16 s1 = qk_half<D>(bc + koff + 32 * KS, a);
        bf16x8 p0[2], p1[2];
        softmax_half<D, true, false>(s0, a, cl2, lane_bits(km, 0, g), 0u, 0.f, p0);
        pv_half<D>(bc + voff, p0, a);
        softmax_half<D, true, false>(s1, a, cl2, lane_bits(km, 1, g), 0u, 0.f, p1);
        pv_half<D>(bc + voff + 32, p1, a);
      }
      advance(step);
    }
    for (int step = nu; step < nsteps; ++step) {
      const uint16_t* bc = buf + (step & 1) * BUF;
      if (active) {
        const int j0 = 32 * (step - nu);
        uint64_t km = 0xFFFFFFFF00000000ull | ((j0 >> 5) < nw ? mymask[j0 >> 5] : 0xFFFFFFFFu);
        if (j0 + 32 > T) km |= ~0ull << (T - j0);
        const int lk = T - 1 - j0;  // chunk-local index of the last (partial) block, if present
        const uint64_t kl = (lk >= 0 && lk < 32) ? (1ull << lk) : 0ull;
        f32x16 s0 = qk_half<D>(bc + koff, a);
        bf16x8 p0[2];
        softmax_half<D, true, true>(s0, a, cl2, lane_bits(km, 0, g), lane_bits(kl, 0, g), static_cast<float>(nlast), p0);
        pv_half<D>(bc + voff, p0, a);
      }
      advance(step);
    }

    // ---- rerun the rows whose logits outgrew their reference max
    const bool mine = active && __any(a.over);
    if (l == 0) sh[1 + w] = mine ? 1 : 0;
    lds_barrier();
    bool any = false;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) any = any || sh[1 + v];
    lds_barrier();
    if (!any) break;
    active = mine;
    if (mine) a.m = a.mtrue;
  }

  // ---- stage 3: global first-order correction, then N / D
  const float csum = a.csum + __shfl_xor(a.csum, 32);
  const float dsum = a.dsum + __shfl_xor(a.dsum, 32);
  if (nch > 0) {
    // Hbar^T in bf16: ht[v][k] = Hbar[k][v], rows padded to HS
    const float* Hh = Hbar + static_cast<size_t>(bh) * D * D;
    for (int item = tid; item < (D / 4) * Geo<D>::CG; item += kAttnThreads) {
      const int kg = item % (D / 4), vg = item / (D / 4);
      float f[4][8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float4* src = reinterpret_cast<const float4*>(Hh + (4 * kg + e) * D + 8 * vg);
        const float4 x = src[0], y = src[1];
        f[e][0] = x.x; f[e][1] = x.y; f[e][2] = x.z; f[e][3] = x.w;
        f[e][4] = y.x; f[e][5] = y.y; f[e][6] = y.z; f[e][7] = y.w;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e)
        *reinterpret_cast<uint2*>(buf + (8 * vg + e) * HS + 4 * kg) =
            make_uint2(pack_bf16x2(f[0][e], f[1][e]), pack_bf16x2(f[2][e], f[3][e]));
    }
    lds_barrier();
  }
  // MFMAs need the whole wave: only the stores are guarded per lane.
  if (qvalid) {
    const uint16_t* hrow = buf + ql * HS + 8 * g;
    const float inv = 1.f / dsum;
    uint16_t* op = O + head + static_cast<size_t>(row) * D;
#pragma unroll
    for (int u = 0; u < Geo<D>::NU; ++u) {
      f32x16 o = a.o[u];
      if (nch > 0) {
        f32x16 r = f32x16{};
#pragma unroll
        for (int ks = 0; ks < Geo<D>::NK; ++ks)
          r = mfma32x32x16(*reinterpret_cast<const bf16x8*>(hrow + 32 * u * HS + 16 * ks), a.qb[ks], r);
        o += (scale * csum) * r;
      }
      if (row < L) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int dim = 32 * u + 8 * q + 4 * g;
          *reinterpret_cast<uint2*>(op + dim) = make_uint2(pack_bf16x2(o[4 * q] * inv, o[4 * q + 1] * inv),
                                                           pack_bf16x2(o[4 * q + 2] * inv, o[4 * q + 3] * inv));
        }
      }
    }
  }
}

// ------------------------------------------------------------------ fp32
constexpr int kF32Threads = 256;

template <int D>
__global__ __launch_bounds__(kF32Threads) void k_attn_f32(const float* __restrict__ Q, const float* __restrict__ K,
                                                          const float* __restrict__ V, const float* __restrict__ kbar,
                                                          const float* __restrict__ vsum,
                                                          const float* __restrict__ Hbar,
                                                          const int32_t* __restrict__ idx, float* __restrict__ O,
                                                          int L, int T, int keep_k, float scale) {
  constexpr int DP = D / 4;  // dims per thread
  extern __shared__ __align__(16) unsigned char smem[];
  float(*kt)[D] = reinterpret_cast<float(*)[D]>(smem);
  float(*vt)[D] = reinterpret_cast<float(*)[D]>(smem + sizeof(float) * 64 * D);
  uint32_t* selmask = reinterpret_cast<uint32_t*>(smem + 2 * sizeof(float) * 64 * D);
  const int nw = ceil_div(T, 32);
  const int qblk = blockIdx.x, bh = blockIdx.y;
  const int tid = threadIdx.x, r = tid / 4, part = tid % 4;
  const size_t head = static_cast<size_t>(bh) * L * D;
  const int32_t* irow = idx + (static_cast<size_t>(bh) * T + qblk) * keep_k;
  const int row = qblk * 64 + r;
  const bool valid = row < L;
  float q[DP], o[DP];
  for (int e = 0; e < DP; ++e) {
    q[e] = valid ? Q[head + static_cast<size_t>(row) * D + part * DP + e] * scale : 0.f;
    o[e] = 0.f;
  }
  float m = -INFINITY, dsum = 0.f, csum = 0.f;
  const int nlast = L - 64 * (T - 1);

  auto key_step = [&](const float* kk, const float* vv, float weight, bool tail) {
    float x = 0.f;
    for (int e = 0; e < DP; ++e) x += q[e] * kk[part * DP + e];
    x += __shfl_xor(x, 1);
    x += __shfl_xor(x, 2);
    const float mnew = fmaxf(m, x);
    const float alpha = expf(m - mnew);
    const float p = expf(x - mnew);
    m = mnew;
    dsum = dsum * alpha + p * weight;
    if (tail) csum = csum * alpha + p;
    for (int e = 0; e < DP; ++e) o[e] = o[e] * alpha + p * vv[part * DP + e];
  };

  for (int it = 0; it < keep_k; ++it) {
    const int j = min(max(irow[it], 0), T - 1);
    const int nv = j == T - 1 ? nlast : 64;
    __syncthreads();
    for (int e = tid; e < 64 * D; e += kF32Threads) {
      const int tk = e / D, dm = e % D;
      kt[tk][dm] = tk < nv ? K[head + static_cast<size_t>(64 * j + tk) * D + dm] : 0.f;
      vt[tk][dm] = tk < nv ? V[head + static_cast<size_t>(64 * j + tk) * D + dm] : 0.f;
    }
    __syncthreads();
    for (int tk = 0; tk < nv; ++tk) key_step(kt[tk], vt[tk], 1.f, false);
  }
  if (keep_k < T) {
    __syncthreads();
    for (int wd = tid; wd < nw; wd += kF32Threads) selmask[wd] = 0u;
    __syncthreads();
    for (int e = tid; e < keep_k; e += kF32Threads) {
      const int jj = min(max(irow[e], 0), T - 1);
      atomicOr(&selmask[jj >> 5], 1u << (jj & 31));
    }
    __syncthreads();
    const float* kb = kbar + static_cast<size_t>(bh) * T * D;
    const float* vs = vsum + static_cast<size_t>(bh) * T * D;
    for (int j = 0; j < T; ++j) {
      if ((selmask[j >> 5] >> (j & 31)) & 1u) continue;
      key_step(kb + static_cast<size_t>(j) * D, vs + static_cast<size_t>(j) * D,
               j == T - 1 ? static_cast<float>(nlast) : 64.f, true);
    }
  }
  // correction r = q' Hbar for this thread's dims (q' needs the whole row)
  const float* Hh = Hbar + static_cast<size_t>(bh) * D * D;
  float rr[DP];
  for (int e = 0; e < DP; ++e) rr[e] = 0.f;
  if (valid) {
    const float* qrow = Q + head + static_cast<size_t>(row) * D;
    for (int k = 0; k < D; ++k) {
      const float qk = qrow[k] * scale;
      for (int e = 0; e < DP; ++e) rr[e] += qk * Hh[k * D + part * DP + e];
    }
    float* op = O + head + static_cast<size_t>(row) * D + part * DP;
    for (int e = 0; e < DP; ++e) op[e] = (o[e] + csum * rr[e]) / dsum;
  }
}

template <int D>
hipError_t launch_bf16(const paro_problem& p, const void* Q, const void* K, const void* V, const float* kbar,
                       const float* vsum, const float* Hbar, const int32_t* idx, int keep_k, void* O,
                       hipStream_t s) {
  const int T = ceil_div(p.L, 64);
  const int nw = ceil_div(T, 32);
  const size_t lds = sizeof(uint16_t) * 2 * Geo<D>::BUF + sizeof(uint32_t) * kQB * nw + 12 * sizeof(int) +
                     sizeof(uint16_t) * T;
  const size_t lds_al = (lds + 15) / 16 * 16;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_attn_bf16<D>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds_al));
  if (e != hipSuccess) return e;
  const int nwg = ceil_div(T, kQB) * p.B * p.H;
  hipLaunchKernelGGL(k_attn_bf16<D>, dim3(nwg), dim3(kAttnThreads), lds_al, s,
                     static_cast<const uint16_t*>(Q), static_cast<const uint16_t*>(K),
                     static_cast<const uint16_t*>(V), kbar, vsum, Hbar, idx, static_cast<uint16_t*>(O), p.L, T,
                     keep_k, static_cast<float>(p.scale), nwg);
  return hipGetLastError();
}

template <int D>
hipError_t launch_f32(const paro_problem& p, const void* Q, const void* K, const void* V, const float* kbar,
                      const float* vsum, const float* Hbar, const int32_t* idx, int keep_k, void* O,
                      hipStream_t s) {
  const int T = ceil_div(p.L, 64);
  const size_t lds = 2 * sizeof(float) * 64 * D + sizeof(uint32_t) * ceil_div(T, 32);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_attn_f32<D>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_attn_f32<D>, dim3(T, p.B * p.H), dim3(kF32Threads), lds, s, static_cast<const float*>(Q),
                     static_cast<const float*>(K), static_cast<const float*>(V), kbar, vsum, Hbar, idx,
                     static_cast<float*>(O), p.L, T, keep_k, static_cast<float>(p.scale));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const paro_problem& p, const void* Q, const void* K, const void* V, const float* kbar,
                            const float* vsum, const float* Hbar, const int32_t* idx, int keep_k, void* O,
                            hipStream_t s) {
  if (p.dtype == PARO_DTYPE_BF16)
    return p.d == 128 ? launch_bf16<128>(p, Q, K, V, kbar, vsum, Hbar, idx, keep_k, O, s)
                      : launch_bf16<64>(p, Q, K, V, kbar, vsum, Hbar, idx, keep_k, O, s);
  return p.d == 128 ? launch_f32<128>(p, Q, K, V, kbar, vsum, Hbar, idx, keep_k, O, s)
                    : launch_f32<64>(p, Q, K, V, kbar, vsum, Hbar, idx, keep_k, O, s);
}

}  // namespace paro
