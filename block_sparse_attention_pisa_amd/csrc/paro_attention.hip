// Fused piecewise attention ("PISA: Piecewise Sparse Attention Is Wiser for
// Efficient Diffusion Transformers", section 2, "core algorithm" and
// "hardware implementation": stage 1 exact, stage 2 zeroth-order scan,
// stage 3 global first-order correction, then o = N / D).
//
// bf16 kernel (k_attn_bf16): a workgroup of 8 waves serves 4 consecutive
// query blocks of one (batch, head); each block of 64 rows is split between
// two waves of 32 rows, so every wave fits in 256 registers and each SIMD
// runs two waves whose matrix and vector work interleave. The grid is
// persistent (one workgroup per CU) and takes these items from per-XCD
// queues in the workspace.
//  * The exact lists of the 4 blocks are merged into their sorted union; each
//    union tile (64 keys x d) is staged once into LDS for all 8 waves by
//    direct global-to-LDS loads, two tiles ahead into three buffers, one
//    LDS-only barrier per tile. K and V rows are stored whole, in 1 KB
//    regions whose spacing keeps every operand read free of bank conflicts:
//    a K operand is one ds_read_b128, a V^T operand two transposing reads
//    (ds_read_b64_tr_b16, new in CDNA4), each at a per-lane base plus a
//    compile-time offset, so V needs no transpose on its way in.
//  * A wave computes S^T = K Q^T for its 32 queries on
//    v_mfma_f32_32x32x16_bf16 with Q^T held in registers, the accumulators
//    starting at -m (the softmax reference). In the C layout of S^T each
//    lane owns one query and 32 keys of the tile, so the softmax state is
//    per lane.
//  * O^T += V^T P^T with P straight from the S^T accumulators (K rows are read
//    in a permuted order so each lane's 8 consecutive P values are 8
//    consecutive keys, the 8 keys its V^T operand holds).
//  * The softmax reference m is fixed by the first tile a wave sees (the
//    largest logit of centroid chunk 0 among the blocks that carry weight)
//    and never moves, so O needs no rescaling: N and D share the factor
//    exp(-m), which cancels in N / D. A tile whose weight sum reaches 2^64
//    (some logit at least 64 log2 units above m, far beyond real attention
//    logits) marks the wave, and so does a row whose D ends below 2^-64
//    (every weighted logit far below m); after the pass the marked waves
//    recompute their rows with m set to the exact maximum, found by a
//    max-only pass.
//  * Stage 2 streams all T centroids in chunks of 64 through the same staging
//    and the same pipelined tile code as the exact tiles (kbar as keys, vsum
//    as values, rounded to bf16 by a small kernel into a caller workspace),
//    with the blocks of S_i and j >= T masked; the weights add n_j p to D and
//    p to c.
//  * Stage 3 forms r^T = Hbar^T q^T on MFMA (Hbar transposed into LDS in
//    bf16) and adds (scale c) r before the division.
//  * With F8 (paro_attention_fp8) S^T of every tile runs on the fp8 matrix
//    cores instead: K, kbar and q' rounded to e4m3 with per-row power-of-two
//    scales that the MFMA applies; softmax, P V and stage 3 are unchanged.
//
// fp32 kernel (k_attn_f32): the same three stages in plain fp32 arithmetic,
// one key at a time; used for fp32 problems.
#include <algorithm>
#include <atomic>
#include <mutex>

#include "paro_common.h"

// Device scratch of paro_attention_noalloc, for callers that cannot allocate:
// it holds the bf16 copies of kbar and vsum and the work-queue counters that
// paro_attention otherwise keeps in the caller's workspace. Every GPU the
// library runs on holds its own copy until the process ends; calls on one
// GPU share it.
static __device__ __align__(256) unsigned char scratch[PARO_NOALLOC_SCRATCH_BYTES];

namespace paro {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kQB = 4;                    // query blocks per workgroup
constexpr int kWaves = 2 * kQB;           // two 32-row waves per query block
constexpr int kAttnThreads = 64 * kWaves;
constexpr int kQueueStride = 16;          // ints between the item queues' counters (64 bytes)
constexpr int kQueueInts = 8 * kQueueStride;
// tail modes (the PARO_TAIL_* codes of the ABI; 2 = zeroth order only: tail on, correction off)
constexpr int kModePisa = 0, kModeDrop = 1;

// Tile geometry. A staged tile (64 K rows, then 64 V rows) lives in LDS as
// 1 KB regions, each filled by one wave-wide direct global-to-LDS load (lane
// i writes bytes 16 i .. 16 i + 16 of the region): region r of the K (V)
// part holds tile rows r, r + NREG, r + 2 NREG, ... as whole rows, so every
// such load reads complete rows of the tensor. Regions are KREG (VREG) bytes
// apart; the 16 (64) bytes beyond the 1 KB shift each region's LDS banks, so
// that the K operand reads of 16 consecutive rows (one 16-lane group of
// ds_read_b128, same dims) fall in 16 different bank quads, and the
// transposing V reads of 4 consecutive rows (64 bytes each) fall in 4
// regions 64 bytes apart: no bank conflicts, and every operand address is a
// per-lane base plus constants.
// bf16: K rows of 2 D bytes, NREG = 64 / RR regions of RR = 512 / D rows.
// F8: K (and the centroid keys) as e4m3 rows of D bytes, NREG8 = D / 16
// regions of 1024 / D rows, then the 64 row-scale (E8M0) bytes at KSC; V
// as in bf16.
template <int D, bool F8 = false>
struct Geo {
  static constexpr int CG = D / 8;                         // 16-byte chunks in a bf16 row
  static constexpr int HS = D + 8;                         // fp8 stage 3: Hbar^T row stride
  static constexpr int RR = 512 / D;                       // bf16 K and V: tile rows per 1 KB region
  static constexpr int NREG = 64 / RR;                     // bf16 K and V: regions per 64 rows
  static constexpr int NREG8 = D / 16;                     // e4m3 K: regions per 64 rows
  static constexpr int KREG = 1024 + 16, VREG = 1024 + 64; // bytes from one region to the next
  static constexpr int KSC = NREG8 * KREG;                 // fp8: byte offset of the row-scale bytes
  // K part (elements of 2 bytes); fp8: the e4m3 regions, then the scales
  static constexpr int KTILE = F8 ? (KSC + 64) / 2 : NREG * KREG / 2;
  static constexpr int VTILE = NREG * VREG / 2;
  static constexpr int BUF = KTILE + VTILE;                // one staging buffer (elements)
  static constexpr int NBUF = 3;                           // staging buffers in LDS
  // element offsets, from a lane's operand address, of the same dims 32 key
  // rows on (bf16 K), and 4, 16 and 32 key rows on (V); fp8 K: 32 rows on
  // are K32B bytes on
  static constexpr int K32 = 32 / NREG * D;
  static constexpr int K32B = 32 / NREG8 * D;
  static constexpr int V4 = 4 * VREG / 2;
  static constexpr int V16 = 16 / NREG * D;
  static constexpr int V32 = 32 / NREG * D;
  // direct loads per wave and tile: bf16 NREG / 8 K and V regions each;
  // fp8 d = 128 one e4m3 region, two V regions and one load of scale bytes,
  // d = 64 one V region and either the e4m3 region (waves 0-3) or scales
  static constexpr int DMA_OPS = F8 ? (D == 128 ? 4 : 2) : 2 * NREG / kWaves;
  static constexpr int NK = D / 16;                        // bf16 k-steps of S^T = K Q^T over the D dims
  static constexpr int NK8 = D / 64;                       // fp8 k-steps
  static constexpr int NU = D / 32;                        // 32-dim output tiles
  static_assert(D * HS <= NBUF * BUF, "Hbar^T must fit in the staging buffers");
  // each wave loads whole regions; a lane's V rows 8 g + k (k < 4) and those
  // 4 rows on stay in one row of regions; +16 and +32 key rows are whole rows
  // of regions on
  static_assert(NREG % kWaves == 0 && 11 % NREG + 4 < NREG && 16 % NREG == 0, "region geometry");
  static_assert((D == 128 && NREG8 == kWaves) || (D == 64 && 2 * NREG8 == kWaves), "fp8 regions per wave");
  static_assert(KTILE % 8 == 0, "V tile alignment");
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
// Global loads are raw buffer loads: the buffer descriptor (base and size,
// in scalar registers) is built per tile, so each thread's offsets inside a
// tile are constants and rows past the end of the tensor read as zeros
// (their keys are masked out; their values carry zero weight).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ uint4 bload(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// bf16 path: per-lane source offsets (bytes, constant) of this wave's direct
// loads. Wave w loads regions PW w .. PW w + PW - 1 of the K and the V part;
// lane i of the load of region r supplies tile row r + NREG (i / (D / 8)),
// bytes 16 (i % (D / 8)) .. + 16, which lands at byte 16 i of the region.
typedef __attribute__((address_space(3))) void lds_void;
template <int D>
struct DmaOffs {
  static constexpr int PW = Geo<D>::NREG / kWaves;
  uint32_t off[PW];
  int reg0;  // this wave's first region (uniform)
  __device__ __forceinline__ void init() {
    constexpr int NREG = Geo<D>::NREG;
    reg0 = PW * __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    const int i = threadIdx.x & 63;
#pragma unroll
    for (int p = 0; p < PW; ++p)
      off[p] = static_cast<uint32_t>((reg0 + p + NREG * (i / (D / 8))) * 2 * D + 16 * (i % (D / 8)));
  }
};
// bf16 path: one tile (keys kr, values vr, both bf16 [rows][D], `rows` valid
// rows from the base on; the rest read as zeros) into staging buffer b by
// direct global-to-LDS loads, DMA_OPS per wave. Their LDS writes land
// asynchronously: they are counted by vmcnt, which the caller waits on
// before the barrier that publishes the tile.
template <int D>
__device__ __forceinline__ void dma_rows(const uint16_t* kr, const uint16_t* vr, int rows, uint16_t* b,
                                         const DmaOffs<D>& of) {
  const auto rk = make_rsrc(kr, static_cast<uint32_t>(rows * D * 2));
  const auto rv = make_rsrc(vr, static_cast<uint32_t>(rows * D * 2));
  unsigned char* kb = reinterpret_cast<unsigned char*>(b);
  unsigned char* vb = kb + 2 * Geo<D>::KTILE;
#pragma unroll
  for (int p = 0; p < DmaOffs<D>::PW; ++p) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(kb + (of.reg0 + p) * Geo<D>::KREG), 16, of.off[p], 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(vb + (of.reg0 + p) * Geo<D>::VREG), 16, of.off[p], 0, 0, 0);
  }
}
// fp8 path: this wave's direct loads of a tile (DMA_OPS of them): V regions
// as DmaOffs; d = 128: e4m3 region w and scale bytes 8 w .. + 8 (lanes 0-1);
// d = 64: e4m3 region w (waves 0-3) or scale bytes 16 (w - 4) .. + 16 (waves
// 4-7, lanes 0-3). Lane i of an e4m3 load supplies tile row r + NREG8 (i / (D
// / 16)), bytes 16 (i % (D / 16)) .. + 16; a scale load writes 4 bytes per lane.
template <int D>
struct DmaOffs8 {
  DmaOffs<D> v;
  uint32_t koff, soff;
  int w;                    // this wave (uniform)
  bool has_k;               // loads an e4m3 region (else scale bytes, d = 64)
  int sbase, slanes;        // scale bytes of this wave: first byte, lanes
  __device__ __forceinline__ void init() {
    constexpr int NREG8 = Geo<D, true>::NREG8;
    v.init();
    w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    const int i = threadIdx.x & 63;
    has_k = D == 128 || w < 4;
    koff = static_cast<uint32_t>((w + NREG8 * (i / (D / 16))) * D + 16 * (i % (D / 16)));
    sbase = D == 128 ? 8 * w : 16 * (w - 4);
    slanes = D == 128 ? 2 : 4;
    soff = static_cast<uint32_t>(sbase + 4 * i);
  }
};
template <int D>
__device__ __forceinline__ void dma_rows8(const uint8_t* kr, const uint16_t* vr, const uint8_t* ke, int rows,
                                          uint16_t* b, const DmaOffs8<D>& of) {
  constexpr int KREG = Geo<D, true>::KREG, VREG = Geo<D, true>::VREG;
  unsigned char* kb = reinterpret_cast<unsigned char*>(b);
  unsigned char* vb = kb + 2 * Geo<D, true>::KTILE;
  const auto rv = make_rsrc(vr, static_cast<uint32_t>(rows * D * 2));
#pragma unroll
  for (int p = 0; p < DmaOffs<D>::PW; ++p)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(vb + (of.v.reg0 + p) * VREG), 16, of.v.off[p], 0, 0, 0);
  if (of.has_k) {
    const auto rk = make_rsrc(kr, static_cast<uint32_t>(rows * D));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(kb + of.w * KREG), 16, of.koff, 0, 0, 0);
  }
  if (D == 128 || !of.has_k) {
    // the range check of a raw buffer load is per dword, so the scale bytes'
    // range is rounded up to whole dwords (the bytes past the last row belong
    // to masked keys; they lie inside the caller's workspace)
    const auto rs = make_rsrc(ke, static_cast<uint32_t>((rows + 3) & ~3));
    if ((threadIdx.x & 63) < of.slanes)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(kb + Geo<D, true>::KSC + of.sbase), 4, of.soff, 0, 0, 0);
  }
}
// Wait until at most N of this wave's global loads (direct loads included)
// are outstanding (N < 16; expcnt and lgkmcnt left alone).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}
// ------------------------------------------------------------ fp8
typedef int i32x8 __attribute__((ext_vector_type(8)));

// E8M0 code (exponent + 127) of the smallest power-of-two scale 2^e that
// brings values of magnitude <= amax into the e4m3 range: amax 2^-e <= 448.
__device__ __forceinline__ int e8m0_of(float amax) {
  if (!(amax > 0.f)) return 127;
  int p;
  const float fr = frexpf(amax, &p);  // amax = fr 2^p, fr in [0.5, 1)
  const int e = p - 9 + (fr * 512.f > 448.f ? 1 : 0);
  return min(254, max(0, e + 127));
}
// Four floats (already scaled) -> four e4m3 bytes in one dword, first value
// in the low byte (round to nearest even).
__device__ __forceinline__ int pack_fp8x4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// kbar and vsum (fp32 [BH][T][D]) rounded to bf16 for the matrix cores; also
// clears the item queues of the attention launch that follows (when given).
__global__ __launch_bounds__(256) void k_centroids_bf16(const float* __restrict__ kbar, const float* __restrict__ vsum,
                                                        uint16_t* __restrict__ kb16, uint16_t* __restrict__ vs16,
                                                        size_t n8, int* __restrict__ queues) {
  const size_t e = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (queues && e < kQueueInts) queues[e] = 0;
  if (e >= n8) return;
  const float4* v4 = reinterpret_cast<const float4*>(vsum) + 2 * e;
  reinterpret_cast<uint4*>(vs16)[e] = to_bf16x8(v4[0], v4[1]);
  if (kb16) {  // (the fp8 path keeps the centroid keys in e4m3 instead)
    const float4* k4 = reinterpret_cast<const float4*>(kbar) + 2 * e;
    reinterpret_cast<uint4*>(kb16)[e] = to_bf16x8(k4[0], k4[1]);
  }
}

// Rows of D values (bf16 bits or fp32) -> e4m3 rows of D bytes, each row
// scaled by the smallest power of two 2^e that brings it into the e4m3 range
// (ex[row] = e + 127, the E8M0 code the fp8 MFMA applies). Consecutive lanes
// share a row (16-byte loads), so the row maximum is a shuffle reduction.
template <typename E, int D>
__global__ __launch_bounds__(256) void k_quant_rows(const E* __restrict__ src, size_t nrows, uint8_t* __restrict__ dst,
                                                    uint8_t* __restrict__ ex) {
  constexpr int EPT = 16 / static_cast<int>(sizeof(E));  // elements per thread
  constexpr int TPR = D / EPT;                            // threads per row (divides 64)
  const size_t t = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  const size_t r = t / TPR;
  const int c = static_cast<int>(t % TPR);
  const bool ok = r < nrows;
  float x[EPT];
  const uint4 v = ok ? *reinterpret_cast<const uint4*>(src + r * D + static_cast<size_t>(c) * EPT) : make_uint4(0, 0, 0, 0);
  if constexpr (EPT == 8) {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = bf16_to_f32(static_cast<uint16_t>(half16(v, e)));
  } else {
    const float4 f = as_f4(v);
    x[0] = f.x; x[1] = f.y; x[2] = f.z; x[3] = f.w;
  }
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < EPT; ++e) amax = fmaxf(amax, fabsf(x[e]));
#pragma unroll
  for (int o = 1; o < TPR; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  const int code = e8m0_of(amax);
  const int sh = 127 - code;
  if (!ok) return;
  uint8_t* out = dst + r * D + static_cast<size_t>(c) * EPT;
  if constexpr (EPT == 8) {
    *reinterpret_cast<uint2*>(out) =
        make_uint2(static_cast<uint32_t>(pack_fp8x4(ldexpf(x[0], sh), ldexpf(x[1], sh), ldexpf(x[2], sh), ldexpf(x[3], sh))),
                   static_cast<uint32_t>(pack_fp8x4(ldexpf(x[4], sh), ldexpf(x[5], sh), ldexpf(x[6], sh), ldexpf(x[7], sh))));
  } else {
    *reinterpret_cast<uint32_t*>(out) =
        static_cast<uint32_t>(pack_fp8x4(ldexpf(x[0], sh), ldexpf(x[1], sh), ldexpf(x[2], sh), ldexpf(x[3], sh)));
  }
  if (c == 0) ex[r] = static_cast<uint8_t>(code);
}

// ------------------------------------------------------------ compute
template <int D>
struct Acc {
  bf16x8 qb[Geo<D>::NK];   // B operand (scale log2(e) Q)^T in bf16: query lane % 32, dims 16 s + 8 g .. + 8
  i32x8 q8[Geo<D>::NK8];   // fp8 path: B operand (scale log2(e) Q)^T 2^-qe in e4m3: dims 64 s + 32 g .. + 32
  int qe;                  // fp8 path: E8M0 code of the lane's query scale
  f32x16 nm;               // -m in every element: the C operand that starts each S^T chain
  f32x16 o[Geo<D>::NU];    // O^T: dims 32 u + 8 (i / 4) + 4 g + i % 4, query lane % 32
  float m;                 // softmax reference (log2 units); the logits S^T come out as logit - m
  float dsum;              // this lane's part of D
  float csum;              // this lane's part of c
  bool over;               // some logit exceeded m + 64 (log2 units)
};

// S^T of 32 keys (kt: the lane's permuted K row and 8-dim half), in log2
// units relative to the reference: scale log2(e) q.k - m.
template <int D>
__device__ __forceinline__ f32x16 qk_half(const uint16_t* kt, const Acc<D>& a) {
  f32x16 s = a.nm;
#pragma unroll
  for (int ks = 0; ks < Geo<D>::NK; ++ks)
    s = mfma32x32x16(*reinterpret_cast<const bf16x8*>(kt + 16 * ks), a.qb[ks], s);
  return s;
}

// 32 bytes of a staged e4m3 K row as an fp8 MFMA operand. (p is
// restrict-qualified so that the reads carry alias-scope information:
// without it the compiler makes them wait for every direct global-to-LDS
// load in flight; the kernel's own waits before each barrier order those
// loads with the reads.)
__device__ __forceinline__ i32x8 k8_op(const uint8_t* __restrict__ p) {
  const uint4 lo = *reinterpret_cast<const uint4*>(p);
  const uint4 hi = *reinterpret_cast<const uint4*>(p + 16);
  return i32x8{static_cast<int>(lo.x), static_cast<int>(lo.y), static_cast<int>(lo.z), static_cast<int>(lo.w),
               static_cast<int>(hi.x), static_cast<int>(hi.y), static_cast<int>(hi.z), static_cast<int>(hi.w)};
}

// fp8 path: S^T of 32 keys (kt: the lane's permuted fp8 K row plus 32 g
// bytes; sa: the E8M0 code of that row's scale). The two operands carry
// their power-of-two scales into the MFMA, which applies them.
template <int D>
__device__ __forceinline__ f32x16 qk_half8(const uint8_t* kt, int sa, const Acc<D>& a) {
  f32x16 s = a.nm;
#pragma unroll
  for (int st = 0; st < Geo<D>::NK8; ++st)
    s = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(k8_op(kt + 64 * st), a.q8[st], s, 0, 0, 0, sa, 0, a.qe);
  return s;
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
// V^T operand (8 keys x 1 dim per lane) from the V tile (rows of V as
// loaded): two transposing reads, keys key0 .. key0 + 3 and key0 + 4 ..
// key0 + 7, where p is the lane's supplier address (see voff in the kernel).
// (p is restrict-qualified so that the reads carry alias-scope information:
// without it the compiler makes every LDS read that lacks such information
// wait for all direct global-to-LDS loads in flight, including those of the
// tiles still being prefetched; the kernel's own waits before each barrier
// order the direct loads with the reads.)
template <int D, bool F8>
__device__ __forceinline__ bf16x8 v_op(const uint16_t* __restrict__ p) {
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(const_cast<uint16_t*>(p)));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(const_cast<uint16_t*>(p + Geo<D, F8>::V4)));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// O^T += V^T P^T for 32 keys (vt: the lane's supplier base plus the key offset).
template <int D, bool F8>
__device__ __forceinline__ void pv_half(const uint16_t* vt, const bf16x8 (&pb)[2], Acc<D>& a) {
#pragma unroll
  for (int u = 0; u < Geo<D>::NU; ++u)
#pragma unroll
    for (int s = 0; s < 2; ++s) a.o[u] = mfma32x32x16(v_op<D, F8>(vt + s * Geo<D, F8>::V16 + 32 * u), pb[s], a.o[u]);
}

// Lane predicate for accumulator register i of a 32-key S^T half: whether the
// key the lane holds (16 (i / 8) + 8 g + i % 8, g = lane / 32) has its bit set
// in the wave-uniform key mask km. Built as a scalar lane mask, so applying it
// costs one v_cndmask per register.
__device__ __forceinline__ bool key_bit(uint32_t km, int i) {
  const int b0 = 16 * (i >> 3) + (i & 7);
  const uint64_t lo = ((km >> b0) & 1u) ? 0x00000000FFFFFFFFull : 0ull;
  const uint64_t hi = ((km >> (b0 + 8)) & 1u) ? 0xFFFFFFFF00000000ull : 0ull;
  return __builtin_amdgcn_inverse_ballot_w64(lo | hi);
}

// Maximum of S^T for this lane's query over the 32 keys, leaving out the
// keys of the wave-uniform mask km.
__device__ __forceinline__ float half_max_masked(const f32x16& s, uint32_t km) {
  float v = -INFINITY;
#pragma unroll
  for (int i = 0; i < 16; ++i) v = fmaxf(v, key_bit(km, i) ? -INFINITY : s[i]);
  return fmaxf(v, __shfl_xor(v, 32));
}
// Sets the softmax reference m (log2 units) of this lane's query.
template <int D>
__device__ __forceinline__ void set_reference(Acc<D>& a, float m) {
  a.m = m;
#pragma unroll
  for (int i = 0; i < 16; ++i) a.nm[i] = -m;
}

// Softmax weights exp2(S^T) of one 32-key sub-tile (the reference is already
// in the accumulators, which start at -m; kShift adds shift first), with no data-dependent
// branches; returns this lane's sum of the bf16-rounded weights, which is
// also what the numerator sees.
// kMask: keys whose bit is set in the wave-uniform mask km get weight 0.
// kLast: pl receives the (bf16-rounded) weight of the key flagged in kl.
// A weight of 2^64 or more (logits far above the reference) sets a.over.
template <int D, bool kMask, bool kLast, bool kShift = false>
__device__ __forceinline__ float softmax_half(f32x16& s, Acc<D>& a, float shift, uint32_t km, uint32_t kl,
                                              bf16x8 (&pb)[2], float& pl) {
  if (kMask) {
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = key_bit(km, i) ? -INFINITY : s[i];
  }
  float pv[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) pv[i] = __builtin_amdgcn_exp2f(kShift ? s[i] + shift : s[i]);
  uint32_t w[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) w[c] = pack_bf16x2(pv[2 * c], pv[2 * c + 1]);
  pb[0] = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
  pb[1] = __builtin_bit_cast(bf16x8, make_uint4(w[4], w[5], w[6], w[7]));
  const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3F803F80u);
  float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    ps0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[c]), ones, ps0, false);
    ps1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[4 + c]), ones, ps1, false);
  }
  const float ps = ps0 + ps1;
  if (kLast) {
    float x = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) x += key_bit(kl, i) ? bf16_to_f32(f32_to_bf16(pv[i])) : 0.f;
    pl = x;
  }
  a.over = a.over || !(ps < 0x1p64f);
  return ps;
}

// Scheduling-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSgValu = 0x002, kSgMfma = 0x008, kSgDsRead = 0x100;

// One exact tile (64 keys) for this wave's 32 queries: S^T = K Q^T for both
// 32-key halves, the weights of each half, O^T += V^T P^T. Written as a
// software pipeline so the matrix cores and the vector ALU overlap inside
// the wave: the K operands of half 1 load during the MFMAs of half 0, the
// softmax of half 0 runs between the MFMAs of half 1, the softmax of half 1
// between the P V MFMAs of half 0, and every V operand is read one phase
// ahead. kMask: the uniform 64-bit key mask km zeroes keys (partial block,
// centroids outside the tail). kLast: pl receives the weight of the key
// flagged in kl. Returns this lane's sum of the weights.
template <int D, bool kMask, bool kLast = false>
__device__ __forceinline__ float exact_tile(const uint16_t* bc, int koff, int voff, Acc<D>& a, uint64_t km,
                                            uint64_t kl, float& pl) {
  constexpr int NK = Geo<D>::NK, NU = Geo<D>::NU, K32 = Geo<D>::K32, V16 = Geo<D>::V16, V32 = Geo<D>::V32;
  constexpr int NV = 2 * NU;
  constexpr int kValu = kMask ? 52 : 36;  // VALU instructions of one softmax half (approximate)
  const uint16_t* kp = bc + koff;
  const uint16_t* vp = bc + voff;
  constexpr int NKX = NK;
  bf16x8 k0[NK], k1[NK], v0[NV], v1[NV];
  // region 1: K operands of half 0
#pragma unroll
  for (int ks = 0; ks < NK; ++ks) k0[ks] = *reinterpret_cast<const bf16x8*>(kp + 16 * ks);
  __builtin_amdgcn_sched_barrier(0);
  // region 2: S^T half 0 | K operands of half 1
#pragma unroll
  for (int ks = 0; ks < NK; ++ks) k1[ks] = *reinterpret_cast<const bf16x8*>(kp + K32 + 16 * ks);
  f32x16 s0 = a.nm, s1 = a.nm;
#pragma unroll
  for (int ks = 0; ks < NK; ++ks) s0 = mfma32x32x16(k0[ks], a.qb[ks], s0);
#pragma unroll
  for (int i = 0; i < NKX; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  // region 3: S^T half 1 | softmax of half 0 | V operands of half 0
#pragma unroll
  for (int u = 0; u < NU; ++u)
#pragma unroll
    for (int h = 0; h < 2; ++h) v0[2 * u + h] = v_op<D, false>(vp + h * V16 + 32 * u);
#pragma unroll
  for (int ks = 0; ks < NK; ++ks) s1 = mfma32x32x16(k1[ks], a.qb[ks], s1);
  float pl0 = 0.f, pl1 = 0.f;
  bf16x8 p0[2], p1[2];
  float ps = softmax_half<D, kMask, kLast>(s0, a, 0.f, static_cast<uint32_t>(km), static_cast<uint32_t>(kl), p0, pl0);
#pragma unroll
  for (int i = 0; i < NKX; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kSgValu, (kValu + NKX - 1) / NKX, 0);
    __builtin_amdgcn_sched_group_barrier(kSgDsRead, (NV + NKX - 1) / NKX, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  // region 4: P V half 0 | softmax of half 1 | V operands of half 1
#pragma unroll
  for (int u = 0; u < NU; ++u)
#pragma unroll
    for (int h = 0; h < 2; ++h) v1[2 * u + h] = v_op<D, false>(vp + V32 + h * V16 + 32 * u);
#pragma unroll
  for (int u = 0; u < NU; ++u)
#pragma unroll
    for (int h = 0; h < 2; ++h) a.o[u] = mfma32x32x16(v0[2 * u + h], p0[h], a.o[u]);
  ps += softmax_half<D, kMask, kLast>(s1, a, 0.f, static_cast<uint32_t>(km >> 32), static_cast<uint32_t>(kl >> 32), p1,
                                      pl1);
  if (kLast) pl = pl0 + pl1;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kSgValu, (kValu + NV - 1) / NV, 0);
    __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  // region 5: P V half 1
#pragma unroll
  for (int u = 0; u < NU; ++u)
#pragma unroll
    for (int h = 0; h < 2; ++h) a.o[u] = mfma32x32x16(v1[2 * u + h], p1[h], a.o[u]);
  return ps;
}

// exact_tile with S^T = K Q^T on the fp8 matrix cores (two 32x32x64 e4m3
// MFMAs per 32 keys instead of eight bf16 ones); kb: the lane's fp8 K row
// base (tile base + perm_key(0, ql) row + 32 g bytes), sc: the tile's
// row-scale bytes. Softmax and P V are those of exact_tile.
template <int D, bool kMask, bool kLast = false>
__device__ __forceinline__ float exact_tile8(const uint8_t* kb, const uint8_t* sc, int ql, const uint16_t* bc,
                                             int voff, Acc<D>& a, uint64_t km, uint64_t kl, float& pl) {
  constexpr int NK8 = Geo<D>::NK8, NU = Geo<D>::NU, K32B = Geo<D, true>::K32B, V16 = Geo<D, true>::V16,
                V32 = Geo<D, true>::V32;
  constexpr int NV = 2 * NU;
  constexpr int kValu = kMask ? 52 : 36;
  constexpr int NKX = NK8;
  const uint16_t* vp = bc + voff;
  i32x8 k0[NK8], k1[NK8];
  bf16x8 v0[NV], v1[NV];
  // region 1: K operands of half 0, the row scales of both halves
#pragma unroll
  for (int st = 0; st < NK8; ++st) k0[st] = k8_op(kb + 64 * st);
  const int sa0 = sc[perm_key(0, ql)], sa1 = sc[perm_key(1, ql)];
  __builtin_amdgcn_sched_barrier(0);
  // region 2: S^T half 0 | K operands of half 1
#pragma unroll
  for (int st = 0; st < NK8; ++st) k1[st] = k8_op(kb + K32B + 64 * st);
  f32x16 s0 = a.nm, s1 = a.nm;
#pragma unroll
  for (int st = 0; st < NK8; ++st)
    s0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(k0[st], a.q8[st], s0, 0, 0, 0, sa0, 0, a.qe);
#pragma unroll
  for (int i = 0; i < NKX; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kSgDsRead, 2, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  // region 3: S^T half 1 | softmax of half 0 | V operands of half 0
#pragma unroll
  for (int u = 0; u < NU; ++u)
#pragma unroll
    for (int h = 0; h < 2; ++h) v0[2 * u + h] = v_op<D, true>(vp + h * V16 + 32 * u);
#pragma unroll
  for (int st = 0; st < NK8; ++st)
    s1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(k1[st], a.q8[st], s1, 0, 0, 0, sa1, 0, a.qe);
  float pl0 = 0.f, pl1 = 0.f;
  bf16x8 p0[2], p1[2];
  float ps = softmax_half<D, kMask, kLast>(s0, a, 0.f, static_cast<uint32_t>(km), static_cast<uint32_t>(kl), p0, pl0);
#pragma unroll
  for (int i = 0; i < NKX; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kSgValu, (kValu + NKX - 1) / NKX, 0);
    __builtin_amdgcn_sched_group_barrier(kSgDsRead, (NV + NKX - 1) / NKX, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  // region 4: P V half 0 | softmax of half 1 | V operands of half 1
#pragma unroll
  for (int u = 0; u < NU; ++u)
#pragma unroll
    for (int h = 0; h < 2; ++h) v1[2 * u + h] = v_op<D, true>(vp + V32 + h * V16 + 32 * u);
#pragma unroll
  for (int u = 0; u < NU; ++u)
#pragma unroll
    for (int h = 0; h < 2; ++h) a.o[u] = mfma32x32x16(v0[2 * u + h], p0[h], a.o[u]);
  ps += softmax_half<D, kMask, kLast>(s1, a, 0.f, static_cast<uint32_t>(km >> 32), static_cast<uint32_t>(kl >> 32), p1,
                                      pl1);
  if (kLast) pl = pl0 + pl1;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kSgValu, (kValu + NV - 1) / NV, 0);
    __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  // region 5: P V half 1
#pragma unroll
  for (int u = 0; u < NU; ++u)
#pragma unroll
    for (int h = 0; h < 2; ++h) a.o[u] = mfma32x32x16(v1[2 * u + h], p1[h], a.o[u]);
  return ps;
}

// The exact list of query block qblk: fixed-length rows (offs == nullptr,
// row stride keep) or CSR rows (offs [B H][T + 1], head stride keep),
// clamped so that a malformed list can never read outside idx.
__device__ __forceinline__ const int32_t* exact_list(const int32_t* idx, const int32_t* offs, int bh, int T, int qblk,
                                                     int keep, int& cnt) {
  if (!offs) {
    cnt = keep;
    return idx + (static_cast<size_t>(bh) * T + qblk) * keep;
  }
  const int32_t* o = offs + static_cast<size_t>(bh) * (T + 1) + qblk;
  const int s0 = min(max(o[0], 0), keep);
  cnt = min(max(o[1] - o[0], 0), min(T, keep - s0));
  return idx + static_cast<size_t>(bh) * keep + s0;
}

// One tile through the bf16 or the fp8 (F8) S^T path.
template <int D, bool F8, bool kMask, bool kLast = false>
__device__ __forceinline__ float run_tile(const uint16_t* bc, int koff, int koff8, int ql, int voff, Acc<D>& a,
                                          uint64_t km, uint64_t kl, float& pl) {
  if constexpr (F8) {
    const uint8_t* b8 = reinterpret_cast<const uint8_t*>(bc);
    return exact_tile8<D, kMask, kLast>(b8 + koff8, b8 + Geo<D, true>::KSC, ql, bc, voff, a, km, kl, pl);
  } else {
    return exact_tile<D, kMask, kLast>(bc, koff, voff, a, km, kl, pl);
  }
}

// F8: the exact keys come from k8 (e4m3 rows) and ke (their E8M0 scales), the
// centroid keys from kb8 and kbe; otherwise from K and kb16 (bf16).
template <int D, bool F8>
__global__ __launch_bounds__(kAttnThreads) void k_attn_bf16(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ kb16, const uint16_t* __restrict__ vs16, const float* __restrict__ Hbar,
    const int32_t* __restrict__ idx, uint16_t* __restrict__ O, int L, int T, int keep_k, float scale, int nwg,
    int mode, const uint8_t* __restrict__ k8, const uint8_t* __restrict__ ke, const uint8_t* __restrict__ kb8,
    const uint8_t* __restrict__ kbe, const int32_t* __restrict__ offs, int* __restrict__ queues) {
  const bool tail = mode != kModeDrop, corr = mode == kModePisa;
  constexpr int BUF = Geo<D, F8>::BUF, NBUF = Geo<D, F8>::NBUF, NREG8 = Geo<D>::NREG8;
  constexpr int HS = Geo<D>::HS, NREG = Geo<D>::NREG;
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* buf = reinterpret_cast<uint16_t*>(smem);  // NBUF staging buffers
  const int nw = ceil_div(T, 32);
  uint32_t* masks = reinterpret_cast<uint32_t*>(smem + sizeof(uint16_t) * NBUF * BUF);  // [kQB][nw]
  uint32_t* ubits = masks + kQB * nw;  // [kQB][nw]: bit e = union tile e belongs to S_i of q-block qi
  int* sh = reinterpret_cast<int*>(ubits + kQB * nw);  // nu, rerun flags, next item (10)
  uint16_t* ulist = reinterpret_cast<uint16_t*>(sh + 12);                           // [T]

  // The grid is persistent (at most one workgroup per CU) and takes the
  // nwg (head, query-block group) items from 8 queues, so a CU moves from
  // one item straight to the next (no workgroup launch between them) and an
  // item's set-up overlaps the previous item's last stores. Workgroups go to
  // the XCDs round robin (b % 8), and queue x holds a contiguous run of
  // items (whole heads), served in order to the workgroups b % 8 = x: the
  // items in flight on one XCD stay neighbours, whose exact lists share most
  // key blocks in that XCD's L2, however unevenly the items run. The first
  // gridDim.x / 8 items of each queue are handed out by position (workgroup
  // 8 i + x takes item i of queue x), the rest by an atomic counter per
  // queue; a workgroup whose queue is empty serves the others. The next
  // item is claimed during the current one (stage 3) and passed on in LDS.
  const int per_q = nwg / 8, g8 = static_cast<int>(gridDim.x) / 8;
  auto queue_len = [&](int x) { return per_q + (x < nwg - 8 * per_q ? 1 : 0); };
  auto queue_item = [&](int x, int i) { return i < per_q ? x * per_q + i : 8 * per_q + x; };
  int* const own_queue = queues + kQueueStride * (blockIdx.x & 7);
  // the claimed item, given this workgroup's take from its own queue. Once
  // that queue is empty the other seven counters are read together (one
  // round trip, however many are empty) and the first queue seen with items
  // left is taken from; a take that lost the race for its last item reads
  // again. Counters only grow, so each pass that fails has seen a queue run
  // empty, and after at most 8 passes every queue reads empty.
  auto claim = [&](int own) -> int {
    const int x0 = blockIdx.x & 7;
    if (g8 + own < queue_len(x0)) return queue_item(x0, g8 + own);
    for (;;) {
      int seen[7];
#pragma unroll
      for (int t = 0; t < 7; ++t)
        seen[t] = __hip_atomic_load(queues + kQueueStride * ((x0 + 1 + t) & 7), __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
      int x = -1;
#pragma unroll
      for (int t = 6; t >= 0; --t)
        if (g8 + seen[t] < queue_len((x0 + 1 + t) & 7)) x = (x0 + 1 + t) & 7;
      if (x < 0) return -1;
      const int i = g8 + atomicAdd(queues + kQueueStride * x, 1);
      if (i < queue_len(x)) return queue_item(x, i);
    }
  };
  int wg = blockIdx.x;
  {
    const int x0 = wg & 7, i0 = wg >> 3;
    if (wg < 8 * g8 && i0 < queue_len(x0)) {
      wg = queue_item(x0, i0);
    } else {
      if (threadIdx.x == 0) sh[10] = claim(atomicAdd(own_queue, 1));
      lds_barrier();
      wg = sh[10];
    }
  }
  for (; wg >= 0;) {
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
  // bf16: the lane's K row of sub-tile 0, dims 8 g .. + 8 (+K32 for sub-tile 1)
  const int krow = perm_key(0, ql);
  const int koff = (krow % NREG) * (Geo<D>::KREG / 2) + (krow / NREG) * D + 8 * g;
  // fp8: bytes, the lane's e4m3 row of sub-tile 0, dims 32 g .. (+K32B for sub-tile 1)
  const int koff8 = (krow % NREG8) * Geo<D>::KREG + (krow / NREG8) * D + 32 * g;
  // supplier address of the transposing V reads: in 16-lane group G = l / 16,
  // lane 4 k + j reads row (key) 8 g + k, dims 16 (G % 2) + 4 j .. + 4, so
  // that the group's output lane i gets dim 16 (G % 2) + i of keys .. + 3
  const int vrow = 8 * g + (l & 15) / 4, vdim = 16 * ((l >> 4) & 1) + 4 * (l & 3);
  const int voff = Geo<D, F8>::KTILE + vdim +
                   (vrow % NREG) * (Geo<D>::VREG / 2) + (vrow / NREG) * D;

  Acc<D> a;
  {
    const uint16_t* qp = Q + head + static_cast<size_t>(row) * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < Geo<D>::NK; ++ks) {
      const uint4 v = (qvalid && row < L) ? *reinterpret_cast<const uint4*>(qp + 16 * ks) : make_uint4(0, 0, 0, 0);
      const uint32_t x[4] = {v.x, v.y, v.z, v.w};
      uint32_t y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        y[e] = pack_bf16x2(bf16_to_f32(static_cast<uint16_t>(x[e])) * cl2, bf16_to_f32(static_cast<uint16_t>(x[e] >> 16)) * cl2);
      a.qb[ks] = __builtin_bit_cast(bf16x8, make_uint4(y[0], y[1], y[2], y[3]));
    }
    set_reference(a, 0.f);
  }
  if constexpr (F8) {
    // e4m3 copy of the lane's query dims 64 s + 32 g .. + 32, with one
    // power-of-two scale per query (both lanes of the query agree on it)
    constexpr int NK8 = Geo<D>::NK8;
    float x[NK8][32];
    float amax = 0.f;
    const uint16_t* qp = Q + head + static_cast<size_t>(row) * D + 32 * g;
#pragma unroll
    for (int st = 0; st < NK8; ++st)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint4 v = (qvalid && row < L) ? *reinterpret_cast<const uint4*>(qp + 64 * st + 8 * c) : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          x[st][8 * c + e] = bf16_to_f32(static_cast<uint16_t>(half16(v, e))) * cl2;
          amax = fmaxf(amax, fabsf(x[st][8 * c + e]));
        }
      }
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    a.qe = e8m0_of(amax);
    const int ex = 127 - a.qe;
#pragma unroll
    for (int st = 0; st < NK8; ++st)
#pragma unroll
      for (int wd = 0; wd < 8; ++wd)
        a.q8[st][wd] = pack_fp8x4(ldexpf(x[st][4 * wd], ex), ldexpf(x[st][4 * wd + 1], ex),
                                  ldexpf(x[st][4 * wd + 2], ex), ldexpf(x[st][4 * wd + 3], ex));
    // the bf16 operand of the correction holds the same rounded q' (an e4m3
    // value times a power of two is exact in bf16), so every use of q' on
    // this path sees one rounding
    const uint16_t* qb16 = Q + head + static_cast<size_t>(row) * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < Geo<D>::NK; ++ks) {
      const uint4 v = (qvalid && row < L) ? *reinterpret_cast<const uint4*>(qb16 + 16 * ks) : make_uint4(0, 0, 0, 0);
      float r[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float y = bf16_to_f32(static_cast<uint16_t>(half16(v, e))) * cl2;
        const int c8 = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(y, ex), 0.f, 0, false);
        r[e] = ldexpf(__builtin_amdgcn_cvt_f32_fp8(c8, 0), -ex);
      }
      a.qb[ks] = __builtin_bit_cast(bf16x8, make_uint4(pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3]),
                                                      pack_bf16x2(r[4], r[5]), pack_bf16x2(r[6], r[7])));
    }
  }
  DmaOffs8<D> of8;
  DmaOffs<D> ofd;
  const uint16_t* kb = kb16 + static_cast<size_t>(bh) * T * D;
  const uint16_t* vs = vs16 + static_cast<size_t>(bh) * T * D;
  // step 0 (centroid chunk 0) does not depend on the exact lists: its direct
  // loads go out now and overlap the set-up below
  if constexpr (F8) {
    of8.init();
    dma_rows8<D>(kb8 + static_cast<size_t>(bh) * T * D, vs, kbe + static_cast<size_t>(bh) * T, min(64, T), buf, of8);
  } else {
    ofd.init();
    dma_rows<D>(kb, vs, min(64, T), buf, ofd);
  }

  // ---- membership masks of the 4 exact lists and their sorted union
  // (the first entries of each list are loaded before the masks are
  // cleared, so that round trip overlaps the clearing barrier)
  constexpr int kPre = 3;
  int cnt = 0, jpre[kPre];
  const int32_t* irow = nullptr;
  if (qvalid && (w & 1) == 0) {
    irow = exact_list(idx, offs, bh, T, qblk, keep_k, cnt);
#pragma unroll
    for (int r = 0; r < kPre; ++r) jpre[r] = l + 64 * r < cnt ? irow[l + 64 * r] : 0;
  }
  for (int e = tid; e < kQB * nw; e += kAttnThreads) masks[e] = 0u;
  lds_barrier();
  if (qvalid && (w & 1) == 0) {
#pragma unroll
    for (int r = 0; r < kPre; ++r)
      if (l + 64 * r < cnt) {
        const int j = min(max(jpre[r], 0), T - 1);
        atomicOr(&masks[qi * nw + (j >> 5)], 1u << (j & 31));
      }
    for (int e = l + 64 * kPre; e < cnt; e += 64) {
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
  // which union tiles each q-block computes, as bitmaps over the union
  for (int e0 = 64 * w; e0 < nu; e0 += 64 * kWaves) {
    const int e = e0 + l;
    const int j = e < nu ? ulist[e] : 0;
#pragma unroll
    for (int q = 0; q < kQB; ++q) {
      const uint64_t b = __ballot(e < nu && ((masks[q * nw + (j >> 5)] >> (j & 31)) & 1u));
      if (l == 0) {
        ubits[q * nw + (e0 >> 5)] = static_cast<uint32_t>(b);
        if ((e0 >> 5) + 1 < nw) ubits[q * nw + (e0 >> 5) + 1] = static_cast<uint32_t>(b >> 32);
      }
    }
  }
  lds_barrier();
  const uint32_t* mymask = masks + qi * nw;
  const uint32_t* mybits = ubits + qi * nw;
  // stage 2 chunks (none when U_i is empty or the tail is dropped; step 0
  // still stages centroid chunk 0 for the softmax reference)
  bool any_tail = keep_k < T;  // some query block of the group has a non-empty U_i
  if (offs) {
    any_tail = false;
    for (int q = 0; q < kQB; ++q) {
      int cq;
      if (grp * kQB + q < T) {
        exact_list(idx, offs, bh, T, grp * kQB + q, keep_k, cq);
        any_tail = any_tail || cq < T;
      }
    }
  }
  const int nch = (tail && any_tail) ? ceil_div(T, 64) : 0;

  bool active = qvalid;
#pragma unroll
  for (int u = 0; u < Geo<D>::NU; ++u) a.o[u] = f32x16{};
  a.dsum = 0.f;
  a.csum = 0.f;

  // One stream of staged steps: step 0 = centroid chunk 0 (it also sets the
  // softmax reference), steps 1..nu = the exact tiles of the union, then
  // centroid chunks 1..nch-1. Chunk c covers blocks [64 c, 64 c + 64).
  const int nsteps = 1 + nu + (nch > 1 ? nch - 1 : 0);
  // staging buffer of the current step (step % NBUF, kept by rotation)
  int slot = 0;
  auto slot_after = [&](int k) { return slot + k < NBUF ? slot + k : slot + k - NBUF; };
  auto cur = [&]() -> uint16_t* { return buf + slot * BUF; };
  // start the direct loads of a step into LDS buffer dst
  auto fetch = [&](int step, uint16_t* dst) {
    if (step >= 1 && step <= nu) {
      const int j = __builtin_amdgcn_readfirstlane(ulist[step - 1]);
      const size_t base = static_cast<size_t>(64 * j) * D;
      if constexpr (F8)
        dma_rows8<D>(k8 + head + base, Vh + base, ke + static_cast<size_t>(bh) * L + 64 * j, min(64, L - 64 * j), dst,
                     of8);
      else
        dma_rows<D>(Kh + base, Vh + base, min(64, L - 64 * j), dst, ofd);
    } else {
      const int c = step == 0 ? 0 : step - nu;
      const size_t base = static_cast<size_t>(64 * c) * D;
      if constexpr (F8)
        dma_rows8<D>(kb8 + static_cast<size_t>(bh) * T * D + base, vs + base,
                     kbe + static_cast<size_t>(bh) * T + 64 * c, min(64, T - 64 * c), dst, of8);
      else
        dma_rows<D>(kb + base, vs + base, min(64, T - 64 * c), dst, ofd);
    }
  };
  // S^T of sub-tile t (keys 32 t ..) of a staged tile, either path
  auto s_half = [&](const uint16_t* bc, int t) -> f32x16 {
    if constexpr (F8) {
      const uint8_t* b8 = reinterpret_cast<const uint8_t*>(bc);
      return qk_half8<D>(b8 + koff8 + t * Geo<D>::K32B, b8[Geo<D, true>::KSC + perm_key(t, ql)], a);
    } else {
      return qk_half<D>(bc + koff + t * Geo<D>::K32, a);
    }
  };
  // after step: publish step + 1 in LDS (three buffers, loads two steps
  // ahead): wait for this wave's loads of step + 1 (those of step + 2 may
  // stay in flight), then, past the barrier, every wave is done with step's
  // buffer, which takes step + 3.
  constexpr int OPS = Geo<D, F8>::DMA_OPS;
  auto advance = [&](int step) {
    if (step + 2 < nsteps)
      wait_vm<OPS>();
    else
      wait_vm<0>();
    lds_barrier();
    if (step + 3 < nsteps) fetch(step + 3, cur());
    slot = slot_after(1);
  };
  // (pre0: the loads of step 0 were issued already)
  auto start = [&](bool pre0) {
    slot = 0;
    if (!pre0) fetch(0, buf);
    if (nsteps > 1) fetch(1, buf + BUF);
    if (nsteps > 2) fetch(2, buf + 2 * BUF);
    if (nsteps > 2)
      wait_vm<2 * OPS>();
    else if (nsteps > 1)
      wait_vm<OPS>();
    else
      wait_vm<0>();
    lds_barrier();
  };
  // whether this wave computes union tile `step`: one 64-bit word of its
  // bitmap per 64 tiles, held in scalar registers
  int mblk = -1;
  uint64_t mword = 0;
  auto mine_tile = [&](int step) {
    const int e = step - 1;
    if ((e >> 6) != mblk) {
      mblk = e >> 6;
      const int i0 = 2 * mblk;
      const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(mybits[i0]));
      const uint32_t hi = i0 + 1 < nw ? static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(mybits[i0 + 1])) : 0u;
      mword = (static_cast<uint64_t>(hi) << 32) | lo;
    }
    return active && ((mword >> (e & 63)) & 1ull);
  };
  // keys of centroid chunk c left out of the tail: the blocks of S_i (this
  // wave's membership words 2 c, 2 c + 1) and blocks >= T
  auto past_T = [&](int c) {
    const int left = T - 64 * c;
    return left < 64 ? ~0ull << left : 0ull;
  };
  auto chunk_mask = [&](int c) {
    // (readfirstlane yields a signed int: widen through uint32_t, not sign-extended)
    uint64_t km = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(mymask[2 * c]));
    if (2 * c + 1 < nw)
      km |= static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(mymask[2 * c + 1]))) << 32;
    return km | past_T(c);
  };
  const uint64_t past_nlast = ~0ull << nlast;        // keys past the end of the last block
  // exact tiles 1..nfull are full blocks; a partial last block is always last
  const int nfull = (nu > 0 && ulist[nu - 1] == T - 1 && nlast < 64) ? nu - 1 : nu;

  for (int pass = 0; pass < 2; ++pass) {
    if (pass > 0) {
      // A wave whose logits outgrew the reference by 2^64 or more: find the
      // exact maximum of everything it weighs (exact keys, and centroids,
      // which never exceed the keys of their own block), then start over.
      float mx = -INFINITY;
      start(false);
      for (int step = 0; step < nsteps; ++step) {
        const uint16_t* bc = cur();
        if (step >= 1 && step <= nu) {
          if (mine_tile(step)) {
            const uint64_t km = step > nfull ? past_nlast : 0ull;
            const f32x16 s0 = s_half(bc, 0);
            const f32x16 s1 = s_half(bc, 1);
            mx = fmaxf(mx, fmaxf(half_max_masked(s0, static_cast<uint32_t>(km)),
                                 half_max_masked(s1, static_cast<uint32_t>(km >> 32))));
          }
        } else if (active && nch > 0) {
          // (centroids count only where some carry weight: with no tail
          // chunk 0 is staged for the reference alone)
          const uint64_t km = past_T(step == 0 ? 0 : step - nu);
          const f32x16 s0 = s_half(bc, 0);
          const f32x16 s1 = s_half(bc, 1);
          mx = fmaxf(mx, fmaxf(half_max_masked(s0, static_cast<uint32_t>(km)),
                               half_max_masked(s1, static_cast<uint32_t>(km >> 32))));
        }
        advance(step);
      }
      if (active) {
        // mx is relative to the current reference; a row with nothing to
        // weigh (keep-or-drop with an empty S_i: 0 / 0 by definition) keeps it
        if (mx > -INFINITY) set_reference(a, a.m + mx);
#pragma unroll
        for (int u = 0; u < Geo<D>::NU; ++u) a.o[u] = f32x16{};
        a.dsum = 0.f;
        a.csum = 0.f;
      }
    }
    a.over = false;
    start(pass == 0);
    float pl = 0.f;
    // ---- step 0: centroid chunk 0
    {
      if (active) {
        f32x16 s0 = s_half(buf, 0);
        f32x16 s1 = s_half(buf, 1);
        float shift = 0.f;
        if (pass == 0) {
          // reference: the largest centroid logit of the chunk (computed with
          // the reference 0) over the blocks that carry weight: every block
          // below T when the tail is on, only the blocks of S_i when it is
          // not. A centroid logit is the mean of its block's key logits, so
          // the reference never exceeds the largest logit that carries
          // weight. With no such block in the chunk the reference stays 0;
          // a row whose weights then all underflow is caught after the pass.
          const uint64_t km = nch > 0 ? past_T(0) : ~(chunk_mask(0) & ~past_T(0));
          float v = fmaxf(half_max_masked(s0, static_cast<uint32_t>(km)),
                          half_max_masked(s1, static_cast<uint32_t>(km >> 32)));
          if (!(v > -INFINITY)) v = 0.f;
          set_reference(a, v);
          shift = -v;
        }
        if (nch > 0) {
          const uint64_t km = chunk_mask(0);
          const uint64_t kl = nch == 1 ? 1ull << (T - 1) : 0ull;
          bf16x8 p0[2], p1[2];
          float pl0 = 0.f, pl1 = 0.f;
          float ps = softmax_half<D, true, true, true>(s0, a, shift, static_cast<uint32_t>(km),
                                                       static_cast<uint32_t>(kl), p0, pl0);
          ps += softmax_half<D, true, true, true>(s1, a, shift, static_cast<uint32_t>(km >> 32),
                                                  static_cast<uint32_t>(kl >> 32), p1, pl1);
          pv_half<D, F8>(buf + voff, p0, a);
          pv_half<D, F8>(buf + voff + Geo<D, F8>::V32, p1, a);
          a.dsum += 64.f * ps + (static_cast<float>(nlast) - 64.f) * (pl0 + pl1);
          a.csum += ps;
        }
      }
      advance(0);
    }
    // ---- exact tiles: full blocks, then the partial last block
    for (int step = 1; step <= nfull; ++step) {
      const uint16_t* bc = cur();
      if (mine_tile(step)) a.dsum += run_tile<D, F8, false>(bc, koff, koff8, ql, voff, a, 0ull, 0ull, pl);
      advance(step);
    }
    for (int step = nfull + 1; step <= nu; ++step) {
      const uint16_t* bc = cur();
      if (mine_tile(step)) a.dsum += run_tile<D, F8, true>(bc, koff, koff8, ql, voff, a, past_nlast, 0ull, pl);
      advance(step);
    }
    // ---- centroid chunks 1..nch-2, then the last chunk (block T - 1 with its
    // weight n_{T-1})
    for (int step = nu + 1; step < nsteps - 1; ++step) {
      const uint16_t* bc = cur();
      if (active) {
        const float ps = run_tile<D, F8, true>(bc, koff, koff8, ql, voff, a, chunk_mask(step - nu), 0ull, pl);
        a.dsum += 64.f * ps;
        a.csum += ps;
      }
      advance(step);
    }
    if (nch > 1) {
      const int c = nch - 1;  // step nsteps - 1
      const uint16_t* bc = cur();
      if (active) {
        const float ps =
            run_tile<D, F8, true, true>(bc, koff, koff8, ql, voff, a, chunk_mask(c), 1ull << (T - 1 - 64 * c), pl);
        a.dsum += 64.f * ps + (static_cast<float>(nlast) - 64.f) * pl;
        a.csum += ps;
      }
      lds_barrier();
    }

    // ---- rerun the rows whose logits outgrew their reference max, and the
    // rows whose weights all fell below 2^-64 of it (D would lose its
    // precision or underflow to 0)
    if (pass == 0 && active) {
      const float drow = a.dsum + __shfl_xor(a.dsum, 32);
      a.over = a.over || !(drow >= 0x1p-64f);
    }
    const bool mine = active && __any(a.over);
    if (l == 0) sh[1 + w] = mine ? 1 : 0;
    lds_barrier();
    bool any = false;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) any = any || sh[1 + v];
    lds_barrier();
    if (!any) break;
    active = mine;
  }

  // ---- stage 3: global first-order correction, then N / D
  const float csum = a.csum + __shfl_xor(a.csum, 32);
  const float dsum = a.dsum + __shfl_xor(a.dsum, 32);
  // the per-lane indices again, from an opaque copy of the thread id: the
  // compiler recomputes them here instead of keeping them live (and spilled
  // to memory) across the tile loops
  int t3 = threadIdx.x;
  asm volatile("" : "+v"(t3));
  const int g3 = (t3 >> 5) & 1, ql3 = t3 & 31;
  const int row3 = (grp * kQB + (t3 >> 7)) * 64 + 32 * ((t3 >> 6) & 1) + ql3;
  // the next item: the take from the own queue is issued here and returns
  // ahead of the Hbar loads below (memory returns in order), so waiting for
  // those loads covers it; every wave read the slot sh[10] before this
  // item's first barrier. (The address goes through an opaque zero so the
  // compiler's wave aggregation of atomics, which reads the result back at
  // once, leaves this one alone.)
  int own = 0;
  {
    int z = 0;
    asm volatile("" : "+v"(z));
    if (t3 == 0) own = atomicAdd(own_queue + z, 1);
  }
  if (nch > 0 && corr) {
    // Hbar^T in bf16: ht[v][k] = Hbar[k][v], rows padded to HS
    const float* Hh = Hbar + static_cast<size_t>(bh) * D * D;
    for (int item = t3; item < (D / 4) * Geo<D>::CG; item += kAttnThreads) {
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
  if (t3 == 0) sh[10] = claim(own);
  // MFMAs need the whole wave: only the stores are guarded per lane.
  if (qvalid) {
    const uint16_t* hrow = buf + ql3 * HS + 8 * g3;
    const float inv = 1.f / dsum;
    uint16_t* op = O + static_cast<size_t>(bh) * L * D + static_cast<size_t>(row3) * D;
#pragma unroll
    for (int u = 0; u < Geo<D>::NU; ++u) {
      f32x16 o = a.o[u];
      if (nch > 0 && corr) {
        f32x16 r = f32x16{};
#pragma unroll
        for (int ks = 0; ks < Geo<D>::NK; ++ks)
          r = mfma32x32x16(*reinterpret_cast<const bf16x8*>(hrow + 32 * u * HS + 16 * ks), a.qb[ks], r);
        o += (kLn2 * csum) * r;  // r = Hbar^T (scale log2(e) q): scale c Hbar^T q = ln2 c r
      }
      if (row3 < L) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int dim = 32 * u + 8 * q + 4 * g3;
          *reinterpret_cast<uint2*>(op + dim) = make_uint2(pack_bf16x2(o[4 * q] * inv, o[4 * q + 1] * inv),
                                                           pack_bf16x2(o[4 * q + 2] * inv, o[4 * q + 3] * inv));
        }
      }
    }
  }
  lds_barrier();  // every wave is done with this item's LDS before the next item writes it
  wg = sh[10];
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
                                                          int L, int T, int keep_k, float scale, int mode,
                                                          const int32_t* __restrict__ offs) {
  const bool tail = mode != kModeDrop, corr = mode == kModePisa;
  constexpr int DP = D / 4;  // dims per thread
  extern __shared__ __align__(16) unsigned char smem[];
  float(*kt)[D] = reinterpret_cast<float(*)[D]>(smem);
  float(*vt)[D] = reinterpret_cast<float(*)[D]>(smem + sizeof(float) * 64 * D);
  uint32_t* selmask = reinterpret_cast<uint32_t*>(smem + 2 * sizeof(float) * 64 * D);
  const int nw = ceil_div(T, 32);
  const int qblk = blockIdx.x, bh = blockIdx.y;
  const int tid = threadIdx.x, r = tid / 4, part = tid % 4;
  const size_t head = static_cast<size_t>(bh) * L * D;
  int cnt;
  const int32_t* irow = exact_list(idx, offs, bh, T, qblk, keep_k, cnt);
  const int row = qblk * 64 + r;
  const bool valid = row < L;
  float q[DP], o[DP];
  for (int e = 0; e < DP; ++e) {
    q[e] = valid ? Q[head + static_cast<size_t>(row) * D + part * DP + e] * scale : 0.f;
    o[e] = 0.f;
  }
  float m = -INFINITY, dsum = 0.f, csum = 0.f;
  const int nlast = L - 64 * (T - 1);

  auto key_step = [&](const float* kk, const float* vv, float weight, bool in_tail) {
    float x = 0.f;
    for (int e = 0; e < DP; ++e) x += q[e] * kk[part * DP + e];
    x += __shfl_xor(x, 1);
    x += __shfl_xor(x, 2);
    const float mnew = fmaxf(m, x);
    const float alpha = expf(m - mnew);
    const float p = expf(x - mnew);
    m = mnew;
    dsum = dsum * alpha + p * weight;
    if (in_tail) csum = csum * alpha + p;
    for (int e = 0; e < DP; ++e) o[e] = o[e] * alpha + p * vv[part * DP + e];
  };

  for (int it = 0; it < cnt; ++it) {
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
  if (tail && cnt < T) {
    __syncthreads();
    for (int wd = tid; wd < nw; wd += kF32Threads) selmask[wd] = 0u;
    __syncthreads();
    for (int e = tid; e < cnt; e += kF32Threads) {
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
    for (int e = 0; e < DP; ++e) op[e] = (o[e] + (corr ? csum * rr[e] : 0.f)) / dsum;
  }
}

// Workspace of the bf16 problems (byte offsets, each region 256-byte aligned).
// bf16 path: [kb16 | vs16 | queues], kbar and vsum in bf16, each [B H][T][D],
// and the 8 item-queue counters of the persistent grid (kQueueInts ints).
// fp8 path: [k8 | ke | kb8 | kbe | vs16 | queues]: K in e4m3 [B H][L][D] and
// its row scale codes [B H][L], kbar likewise ([B H][T][D], [B H][T]), vsum
// in bf16, and the 8 item-queue counters.
struct WsLayout {
  size_t k8, ke, kb8, kbe, vs16, kb16, queues, total;
};
__host__ inline size_t up256(size_t x) { return (x + 255) / 256 * 256; }
__host__ inline WsLayout ws_layout(const paro_problem& p, bool fp8) {
  const size_t bh = static_cast<size_t>(p.B) * p.H, T = ceil_div(p.L, 64), d = p.d;
  WsLayout w{};
  if (fp8) {
    w.k8 = 0;
    w.ke = up256(bh * p.L * d);
    w.kb8 = w.ke + up256(bh * p.L);
    w.kbe = w.kb8 + up256(bh * T * d);
    w.vs16 = w.kbe + up256(bh * T);
    w.queues = w.vs16 + up256(bh * T * d * 2);
    w.total = w.queues + up256(sizeof(int) * kQueueInts);
  } else {
    w.kb16 = 0;
    w.vs16 = up256(bh * T * d * 2);
    w.queues = w.vs16 + up256(bh * T * d * 2);
    w.total = w.queues + up256(sizeof(int) * kQueueInts);
  }
  return w;
}

// Workgroups of the persistent attention grid: one per CU of the current
// device (its LDS holds one), rounded down to a multiple of 8 so that every
// workgroup stays on one XCD's run of items; looked up once per device.
int persistent_workgroups() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 8) cus = 256;
    n = cus / 8 * 8;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <int D, bool F8>
hipError_t launch_bf16(const paro_problem& p, const void* Q, const void* K, const void* V, const float* kbar,
                       const float* vsum, const float* Hbar, const int32_t* idx, int keep_k, void* O, int mode,
                       void* ws, hipStream_t s, const int32_t* offs) {
  const int T = ceil_div(p.L, 64);
  const size_t bh = static_cast<size_t>(p.B) * p.H;
  const size_t n = bh * T * D;
  const WsLayout lay = ws_layout(p, F8);
  unsigned char* wb = static_cast<unsigned char*>(ws);
  uint16_t* kb16 = F8 ? nullptr : reinterpret_cast<uint16_t*>(wb + lay.kb16);
  uint16_t* vs16 = reinterpret_cast<uint16_t*>(wb + lay.vs16);
  int* queues = reinterpret_cast<int*>(wb + lay.queues);
  uint8_t *k8 = nullptr, *ke = nullptr, *kb8 = nullptr, *kbe = nullptr;
  hipLaunchKernelGGL(k_centroids_bf16, dim3(static_cast<unsigned>((n / 8 + 255) / 256)), dim3(256), 0, s, kbar, vsum,
                     kb16, vs16, n / 8, queues);
  if (F8) {
    k8 = wb + lay.k8;
    ke = wb + lay.ke;
    kb8 = wb + lay.kb8;
    kbe = wb + lay.kbe;
    const size_t krows = bh * p.L, crows = bh * T;
    hipLaunchKernelGGL((k_quant_rows<uint16_t, D>), dim3(static_cast<unsigned>((krows * (D / 8) + 255) / 256)), dim3(256),
                       0, s, static_cast<const uint16_t*>(K), krows, k8, ke);
    hipLaunchKernelGGL((k_quant_rows<float, D>), dim3(static_cast<unsigned>((crows * (D / 4) + 255) / 256)), dim3(256), 0,
                       s, kbar, crows, kb8, kbe);
  }
  const int nw = ceil_div(T, 32);
  const size_t lds = sizeof(uint16_t) * Geo<D, F8>::NBUF * Geo<D, F8>::BUF + 2 * sizeof(uint32_t) * kQB * nw + 12 * sizeof(int) +
                     sizeof(uint16_t) * T;
  const size_t lds_al = (lds + 15) / 16 * 16;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_attn_bf16<D, F8>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds_al));
  if (e != hipSuccess) return e;
  const int nwg = ceil_div(T, kQB) * p.B * p.H;
  const int grid = std::min(nwg, persistent_workgroups());
  hipLaunchKernelGGL((k_attn_bf16<D, F8>), dim3(grid), dim3(kAttnThreads), lds_al, s,
                     static_cast<const uint16_t*>(Q), static_cast<const uint16_t*>(K),
                     static_cast<const uint16_t*>(V), kb16, vs16, Hbar, idx, static_cast<uint16_t*>(O), p.L, T,
                     keep_k, static_cast<float>(p.scale), nwg, mode, k8, ke, kb8, kbe, offs, queues);
  return hipGetLastError();
}

template <int D>
hipError_t launch_f32(const paro_problem& p, const void* Q, const void* K, const void* V, const float* kbar,
                      const float* vsum, const float* Hbar, const int32_t* idx, int keep_k, void* O, int mode,
                      hipStream_t s, const int32_t* offs) {
  const int T = ceil_div(p.L, 64);
  const size_t lds = 2 * sizeof(float) * 64 * D + sizeof(uint32_t) * ceil_div(T, 32);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_attn_f32<D>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_attn_f32<D>, dim3(T, p.B * p.H), dim3(kF32Threads), lds, s, static_cast<const float*>(Q),
                     static_cast<const float*>(K), static_cast<const float*>(V), kbar, vsum, Hbar, idx,
                     static_cast<float*>(O), p.L, T, keep_k, static_cast<float>(p.scale), mode, offs);
  return hipGetLastError();
}

}  // namespace

size_t attention_workspace_bytes(const paro_problem& p) {
  if (p.dtype != PARO_DTYPE_BF16) return 0;
  return ws_layout(p, false).total;
}

hipError_t launch_fp8_rows(const void* src, int dtype, size_t nrows, int d, uint8_t* dst, uint8_t* ex, hipStream_t s) {
  const size_t threads = nrows * static_cast<size_t>(d) / (dtype == PARO_DTYPE_BF16 ? 8 : 4);
  const dim3 grid(static_cast<unsigned>((threads + 255) / 256));
  if (dtype == PARO_DTYPE_BF16) {
    if (d == 128)
      hipLaunchKernelGGL((k_quant_rows<uint16_t, 128>), grid, dim3(256), 0, s, static_cast<const uint16_t*>(src), nrows, dst, ex);
    else
      hipLaunchKernelGGL((k_quant_rows<uint16_t, 64>), grid, dim3(256), 0, s, static_cast<const uint16_t*>(src), nrows, dst, ex);
  } else {
    if (d == 128)
      hipLaunchKernelGGL((k_quant_rows<float, 128>), grid, dim3(256), 0, s, static_cast<const float*>(src), nrows, dst, ex);
    else
      hipLaunchKernelGGL((k_quant_rows<float, 64>), grid, dim3(256), 0, s, static_cast<const float*>(src), nrows, dst, ex);
  }
  return hipGetLastError();
}

size_t attention_fp8_workspace_bytes(const paro_problem& p) {
  if (p.dtype != PARO_DTYPE_BF16) return 0;
  return ws_layout(p, true).total;
}

hipError_t launch_attention_fp8(const paro_problem& p, const void* Q, const void* K, const void* V, const float* kbar,
                                const float* vsum, const float* Hbar, const int32_t* idx, int keep_k, void* O,
                                int mode, void* ws, hipStream_t s) {
  return p.d == 128 ? launch_bf16<128, true>(p, Q, K, V, kbar, vsum, Hbar, idx, keep_k, O, mode, ws, s, nullptr)
                    : launch_bf16<64, true>(p, Q, K, V, kbar, vsum, Hbar, idx, keep_k, O, mode, ws, s, nullptr);
}

// Per-device address of the static attention scratch (see `scratch` below):
// the host-side name of a __device__ array is only a stand-in, so kernels are
// given the address the runtime reports for the current device, looked up
// once per device.
namespace {
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices];
}  // namespace

hipError_t attention_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_attention(const paro_problem& p, const void* Q, const void* K, const void* V, const float* kbar,
                            const float* vsum, const float* Hbar, const int32_t* idx, int keep_k, void* O, int mode,
                            void* ws, hipStream_t s, const int32_t* offs) {
  if (p.dtype == PARO_DTYPE_BF16)
    return p.d == 128 ? launch_bf16<128, false>(p, Q, K, V, kbar, vsum, Hbar, idx, keep_k, O, mode, ws, s, offs)
                      : launch_bf16<64, false>(p, Q, K, V, kbar, vsum, Hbar, idx, keep_k, O, mode, ws, s, offs);
  return p.d == 128 ? launch_f32<128>(p, Q, K, V, kbar, vsum, Hbar, idx, keep_k, O, mode, s, offs)
                    : launch_f32<64>(p, Q, K, V, kbar, vsum, Hbar, idx, keep_k, O, mode, s, offs);
}

}  // namespace paro
