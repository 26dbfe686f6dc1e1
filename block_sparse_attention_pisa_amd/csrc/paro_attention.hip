// Fused piecewise attention ("PISA: Piecewise Sparse Attention Is Wiser for
// Efficient Diffusion Transformers", section 2, "core algorithm" and
// "hardware implementation": stage 1 exact, stage 2 zeroth-order scan,
// stage 3 global first-order correction, then o = N / D).
//
// bf16 kernel (k_attn_bf16): one workgroup of 2 waves per query block of 64
// rows; each wave owns 32 query rows. Per kv tile of 64 keys:
//   S^T = K Q^T  (v_mfma_f32_32x32x16_bf16, A = K rows from LDS, B = Q^T held
//                 in registers for the whole kernel). In the C layout of S^T
//                 every lane holds one query and 32 of the tile's keys, so
//                 the online-softmax state (running max m, denominator D,
//                 tail weight c) is per lane and the row max needs one
//                 cross-half exchange.
//   O^T += V^T P^T (A = V^T from an LDS tile stored transposed, B = P in
//                 registers straight from the S^T accumulators: the K rows
//                 are read in a permuted order so that each lane's 8
//                 consecutive P values match 8 consecutive keys of V^T).
// Stage 1 walks the exact blocks of idx in ascending order with the next
// tile's global loads in flight during the current tile's MFMAs. Stage 2
// scans all T centroids in chunks of 64 through the same code path (kbar as
// keys, vsum as values, both rounded to bf16), with blocks of S_i and j >= T
// masked, adding n_j * p to D and p to c. Stage 3 forms r^T = Hbar^T q^T on
// MFMA (Hbar rounded to bf16, transposed into LDS) and adds
// (scale * c) * r before the final division.
//
// fp32 kernel (k_attn_f32): the same three stages in plain fp32 arithmetic,
// one key at a time; used for fp32 problems.
#include <algorithm>

#include "paro_common.h"

namespace paro {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

// ------------------------------------------------------------------ bf16
constexpr int kAttnThreads = 128;

template <int D>
struct AttnLds {
  static constexpr int KS = D + 8;   // row stride of the key tile
  static constexpr int VS = 64 + 8;  // row stride of the transposed value tile
  uint16_t ks[64][KS];
  uint16_t vt[D][VS];
};
// Hbar^T staged in bf16 reuses the tile region after both loops.
template <int D>
struct HtLds {
  uint16_t ht[D][D + 8];
};

// Key (row of the K tile) that MFMA row m of S^T sub-tile t reads, chosen so
// that accumulator register i of a lane in half g holds key
// 32 t + 16 (i / 8) + 8 g + (i % 8).
__device__ __forceinline__ int perm_key(int t, int m) {
  const int a = m >> 3, g = (m >> 2) & 1, b = m & 3;
  return 32 * t + 16 * (a >> 1) + 8 * g + 4 * (a & 1) + b;
}

template <int D>
struct TileRegs {
  uint4 k[D / 16];     // 64 rows x D/8 chunks of 16 B = 8D chunks / 128 threads
  uint4 v[D / 64][4];  // 16 token groups x D/8 dim groups = 2D items / 128 threads
};

// Global -> registers for one exact kv tile (rows >= nvalid zero-filled).
template <int D>
__device__ __forceinline__ void load_tile(const uint16_t* __restrict__ Kh, const uint16_t* __restrict__ Vh,
                                          int row0, int nvalid, TileRegs<D>& r) {
  constexpr int CG = D / 8;
#pragma unroll
  for (int i = 0; i < D / 16; ++i) {
    const int c = threadIdx.x + kAttnThreads * i;
    const int row = c / CG, cg = c % CG;
    r.k[i] = row < nvalid ? *reinterpret_cast<const uint4*>(Kh + static_cast<size_t>(row0 + row) * D + 8 * cg)
                          : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < D / 64; ++i) {
    const int item = threadIdx.x + kAttnThreads * i;
    const int tg = item / CG, dg = item % CG;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int tok = 4 * tg + q;
      r.v[i][q] = tok < nvalid
                      ? *reinterpret_cast<const uint4*>(Vh + static_cast<size_t>(row0 + tok) * D + 8 * dg)
                      : make_uint4(0, 0, 0, 0);
    }
  }
}

__device__ __forceinline__ uint32_t half16(const uint4& v, int e) {
  const uint32_t w = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
  return (e & 1) ? (w >> 16) : (w & 0xFFFFu);
}

template <int D>
__device__ __forceinline__ void store_tile(const TileRegs<D>& r, AttnLds<D>& s) {
  constexpr int CG = D / 8;
#pragma unroll
  for (int i = 0; i < D / 16; ++i) {
    const int c = threadIdx.x + kAttnThreads * i;
    *reinterpret_cast<uint4*>(&s.ks[c / CG][8 * (c % CG)]) = r.k[i];
  }
#pragma unroll
  for (int i = 0; i < D / 64; ++i) {
    const int item = threadIdx.x + kAttnThreads * i;
    const int tg = item / CG, dg = item % CG;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t w0 = half16(r.v[i][0], e) | (half16(r.v[i][1], e) << 16);
      const uint32_t w1 = half16(r.v[i][2], e) | (half16(r.v[i][3], e) << 16);
      *reinterpret_cast<uint2*>(&s.vt[8 * dg + e][4 * tg]) = make_uint2(w0, w1);
    }
  }
}

// Tail chunk: centroids [64 c, 64 c + 64) of kbar / vsum (fp32 -> bf16) into LDS.
template <int D>
__device__ __forceinline__ void stage_centroids(const float* __restrict__ kb, const float* __restrict__ vs,
                                                int j0, int T, AttnLds<D>& s) {
  constexpr int CG = D / 8;
#pragma unroll
  for (int i = 0; i < D / 16; ++i) {
    const int c = threadIdx.x + kAttnThreads * i;
    const int row = c / CG, cg = c % CG;
    uint4 o = make_uint4(0, 0, 0, 0);
    if (j0 + row < T) {
      const float4* src = reinterpret_cast<const float4*>(kb + static_cast<size_t>(j0 + row) * D + 8 * cg);
      const float4 x = src[0], y = src[1];
      o = make_uint4(pack_bf16x2(x.x, x.y), pack_bf16x2(x.z, x.w), pack_bf16x2(y.x, y.y), pack_bf16x2(y.z, y.w));
    }
    *reinterpret_cast<uint4*>(&s.ks[row][8 * cg]) = o;
  }
#pragma unroll
  for (int i = 0; i < D / 64; ++i) {
    const int item = threadIdx.x + kAttnThreads * i;
    const int tg = item / CG, dg = item % CG;
    float f[4][8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int jj = j0 + 4 * tg + q;
      if (jj < T) {
        const float4* src = reinterpret_cast<const float4*>(vs + static_cast<size_t>(jj) * D + 8 * dg);
        const float4 x = src[0], y = src[1];
        f[q][0] = x.x; f[q][1] = x.y; f[q][2] = x.z; f[q][3] = x.w;
        f[q][4] = y.x; f[q][5] = y.y; f[q][6] = y.z; f[q][7] = y.w;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) f[q][e] = 0.f;
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e)
      *reinterpret_cast<uint2*>(&s.vt[8 * dg + e][4 * tg]) =
          make_uint2(pack_bf16x2(f[0][e], f[1][e]), pack_bf16x2(f[2][e], f[3][e]));
  }
}

template <int D>
struct AttnState {
  bf16x8 qb[D / 16];    // B operand Q^T: query (lane % 32), dims 16 s + 8 g .. + 8
  f32x16 o[D / 32];     // O^T accumulators, dims 32 u + 8 (i / 4) + 4 g + i % 4
  float m;              // running max (log2 domain), equal in both halves
  float dsum;           // this lane's part of D
  float csum;           // this lane's part of c = sum of tail weights
};

// One 64-key tile from LDS. Keys whose mask bit is set get weight 0.
// kTail adds n_j * p to D (instead of p) and p to c.
template <int D, bool kTail>
__device__ __forceinline__ void tile_step(const AttnLds<D>& s, AttnState<D>& st, float cl2, uint64_t keymask,
                                          int nlast_key, float nlast) {
  const int l = threadIdx.x % 64, g = l / 32, ql = l % 32;
  f32x16 sacc[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    sacc[t] = f32x16{};
    const uint16_t* krow = &s.ks[perm_key(t, ql)][8 * g];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
      sacc[t] = mfma32x32x16(*reinterpret_cast<const bf16x8*>(krow + 16 * ks), st.qb[ks], sacc[t]);
  }
  // logits in log2 units, masked keys -> -inf
  float mx = -INFINITY;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = 32 * t + 16 * (i / 8) + 8 * g + (i % 8);
      const float x = ((keymask >> key) & 1ull) ? -INFINITY : sacc[t][i] * cl2;
      sacc[t][i] = x;
      mx = fmaxf(mx, x);
    }
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  // While every key seen so far is masked the max stays -inf; subtracting 0
  // instead keeps every weight (and alpha) exactly 0 without a branch.
  const float mnew = fmaxf(st.m, mx);
  const float mref = mnew == -INFINITY ? 0.f : mnew;
  const float alpha = __builtin_amdgcn_exp2f(st.m - mref);
  st.m = mnew;
  float psum = 0.f, pw = 0.f;
  bf16x8 pb[4];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = __builtin_amdgcn_exp2f(sacc[t][i] - mref);
      psum += p;
      if (kTail) {
        const int key = 32 * t + 16 * (i / 8) + 8 * g + (i % 8);
        pw += key == nlast_key ? p * nlast : p * 64.f;
      }
      pb[2 * t + i / 8][i % 8] = static_cast<__bf16>(p);
    }
  if (kTail) {
    st.dsum = st.dsum * alpha + pw;
    st.csum = st.csum * alpha + psum;
  } else {
    st.dsum = st.dsum * alpha + psum;
  }
#pragma unroll
  for (int u = 0; u < D / 32; ++u) {
    st.o[u] *= alpha;
    const uint16_t* vrow = &s.vt[32 * u + ql][8 * g];
#pragma unroll
    for (int sp = 0; sp < 4; ++sp)
      st.o[u] = mfma32x32x16(*reinterpret_cast<const bf16x8*>(vrow + 16 * sp), pb[sp], st.o[u]);
  }
}

template <int D>
__global__ __launch_bounds__(kAttnThreads) void k_attn_bf16(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const float* __restrict__ kbar, const float* __restrict__ vsum, const float* __restrict__ Hbar,
    const int32_t* __restrict__ idx, uint16_t* __restrict__ O, int L, int T, int keep_k, float scale,
    int nwg) {
  extern __shared__ __align__(16) unsigned char smem[];
  AttnLds<D>& s = *reinterpret_cast<AttnLds<D>*>(smem);
  uint32_t* selmask = reinterpret_cast<uint32_t*>(smem + sizeof(AttnLds<D>));
  const int nw = ceil_div(T, 32);

  // XCD-aware order: consecutive workgroup ids land on different XCDs, so
  // give each XCD a contiguous run of (head, query block) work items.
  int wg = blockIdx.x;
  const int n8 = (nwg / 8) * 8;
  if (wg < n8) wg = (wg % 8) * (nwg / 8) + wg / 8;
  const int qblk = wg % T, bh = wg / T;

  const int tid = threadIdx.x, w = tid / 64, l = tid % 64, g = l / 32, ql = l % 32;
  const size_t head = static_cast<size_t>(bh) * L * D;
  const uint16_t* Kh = K + head;
  const uint16_t* Vh = V + head;
  const int32_t* irow = idx + (static_cast<size_t>(bh) * T + qblk) * keep_k;
  const float cl2 = scale * kLog2e;

  AttnState<D> st;
  const int qrow = qblk * 64 + 32 * w + ql;
  {
    const uint16_t* qp = Q + head + static_cast<size_t>(qrow) * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      uint4 v = qrow < L ? *reinterpret_cast<const uint4*>(qp + 16 * ks) : make_uint4(0, 0, 0, 0);
      st.qb[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }
#pragma unroll
  for (int u = 0; u < D / 32; ++u) st.o[u] = f32x16{};
  st.m = -INFINITY;
  st.dsum = 0.f;
  st.csum = 0.f;

  const int nlast = L - 64 * (T - 1);  // valid keys in the last block

  // ---- stage 1: exact blocks
  if (keep_k > 0) {
    TileRegs<D> regs;
    int j = min(max(irow[0], 0), T - 1);
    load_tile<D>(Kh, Vh, 64 * j, j == T - 1 ? nlast : 64, regs);
    for (int it = 0; it < keep_k; ++it) {
      const int nvalid = j == T - 1 ? nlast : 64;
      __syncthreads();
      store_tile<D>(regs, s);
      __syncthreads();
      if (it + 1 < keep_k) {
        j = min(max(irow[it + 1], 0), T - 1);
        load_tile<D>(Kh, Vh, 64 * j, j == T - 1 ? nlast : 64, regs);
      }
      const uint64_t km = nvalid == 64 ? 0ull : (~0ull << nvalid);
      tile_step<D, false>(s, st, cl2, km, -1, 0.f);
    }
  }

  // ---- stage 2: zeroth-order scan over the centroids of U_i
  if (keep_k < T) {
    for (int wd = tid; wd < nw; wd += kAttnThreads) selmask[wd] = 0u;
    __syncthreads();
    for (int e = tid; e < keep_k; e += kAttnThreads) {
      const int jj = min(max(irow[e], 0), T - 1);
      atomicOr(&selmask[jj >> 5], 1u << (jj & 31));
    }
    for (int j0 = 0; j0 < T; j0 += 64) {
      __syncthreads();
      stage_centroids<D>(kbar + static_cast<size_t>(bh) * T * D, vsum + static_cast<size_t>(bh) * T * D, j0, T, s);
      __syncthreads();
      uint64_t km = 0;
      for (int b = 0; b < 2; ++b) {
        const int wd = j0 / 32 + b;
        const uint32_t word = wd < nw ? selmask[wd] : 0xFFFFFFFFu;
        km |= static_cast<uint64_t>(word) << (32 * b);
      }
      if (j0 + 64 > T) km |= ~0ull << (T - j0);
      tile_step<D, true>(s, st, cl2, km, T - 1 - j0, static_cast<float>(nlast));
    }
  }

  // ---- stage 3: global first-order correction, then N / D
  const float csum = st.csum + __shfl_xor(st.csum, 32);
  const float dsum = st.dsum + __shfl_xor(st.dsum, 32);
  __syncthreads();
  HtLds<D>& h = *reinterpret_cast<HtLds<D>*>(smem);
  {
    const float* Hh = Hbar + static_cast<size_t>(bh) * D * D;
    for (int e = tid; e < D * D; e += kAttnThreads) {
      const int kr = e / D, vc = e % D;  // Hbar[kr][vc] -> ht[vc][kr]
      h.ht[vc][kr] = f32_to_bf16(Hh[e]);
    }
  }
  __syncthreads();
  const float cs = scale * csum;
  const float inv = 1.f / dsum;
#pragma unroll
  for (int u = 0; u < D / 32; ++u) {
    f32x16 r = f32x16{};
    const uint16_t* hrow = &h.ht[32 * u + ql][8 * g];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
      r = mfma32x32x16(*reinterpret_cast<const bf16x8*>(hrow + 16 * ks), st.qb[ks], r);
    st.o[u] += cs * r;
  }
  if (qrow < L) {
    uint16_t* op = O + head + static_cast<size_t>(qrow) * D;
#pragma unroll
    for (int u = 0; u < D / 32; ++u)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int dim = 32 * u + 8 * a + 4 * g;
        const uint2 v = make_uint2(pack_bf16x2(st.o[u][4 * a] * inv, st.o[u][4 * a + 1] * inv),
                                   pack_bf16x2(st.o[u][4 * a + 2] * inv, st.o[u][4 * a + 3] * inv));
        *reinterpret_cast<uint2*>(op + dim) = v;
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
  const size_t lds = std::max(sizeof(AttnLds<D>), sizeof(HtLds<D>)) + sizeof(uint32_t) * ceil_div(T, 32);
  const size_t lds_al = (lds + 15) / 16 * 16;
  hipError_t e;
  if (lds_al > 65536 &&
      (e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_attn_bf16<D>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds_al))) != hipSuccess)
    return e;
  const int nwg = T * p.B * p.H;
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
