// Geometric token reordering before blocking ("PAROAttention: Pattern-Aware
// ReOrdering for Efficient Sparse and Quantized Attention in Visual
// Generation Models", abstract): the rows of a [B, H, L, d] tensor are moved
// into the tiled raster order of a (t, y, x) latent grid, or back.
//
// The order is never stored. A position i maps to its raster source by
// inverting the box enumeration arithmetically: every t-slab before the
// current one is full (tile_t * y * x tokens), every band of rows before the
// current one in a slab is full, and every box before the current one in a
// band is full, because only the last slab, band and box along each axis
// are cut short.
//
// The copy is a pure HBM stream (one read and one write of every row). A
// workgroup handles one block of 64 positions for 8 (batch, head) pairs: the
// 64 sources go to LDS once, then each thread moves 16-byte chunks, several
// rows and two heads at a time so that many loads are in flight.
#include "paro_common.h"

namespace paro {

__host__ __device__ constexpr int imin(int a, int b) { return a < b ? a : b; }

// Raster index of the token at tiled position i (N = t * y * x grid tokens).
// The tile extents must not exceed the grid extents (the ABI layer clamps
// them), so every product below stays within N.
__host__ __device__ int reorder_source(const paro_grid& g, int N, int i) {
  if (i >= N) return i;  // tokens after the grid keep their places
  const int slab = g.tile_t * g.y * g.x;
  const int a = i / slab;
  int r = i - a * slab;
  const int st = imin(g.tile_t, g.t - a * g.tile_t);  // frames in this slab
  const int band = st * g.tile_y * g.x;
  const int b = r / band;
  r -= b * band;
  const int sy = imin(g.tile_y, g.y - b * g.tile_y);  // rows in this band
  const int box = st * sy * g.tile_x;
  const int c = r / box;
  r -= c * box;
  const int sx = imin(g.tile_x, g.x - c * g.tile_x);  // columns in this box
  const int dt = r / (sy * sx);
  r -= dt * sy * sx;
  const int dy = r / sx, dx = r - dy * sx;
  return ((a * g.tile_t + dt) * g.y + b * g.tile_y + dy) * g.x + c * g.tile_x + dx;
}

namespace {

constexpr int kReorderThreads = 256;
constexpr int kHeadsPerWg = 8;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// CPR: 16-byte chunks per token row (d * element size / 16).
template <int CPR>
__global__ __launch_bounds__(kReorderThreads) void k_reorder(const u32x4* __restrict__ X, u32x4* __restrict__ Y,
                                                             paro_grid g, int N, int L, int BH, int gather) {
  constexpr int RPI = kReorderThreads / CPR;  // rows per pass of the workgroup
  constexpr int NR = kBlock / RPI;            // rows per thread
  __shared__ int src[kBlock];
  const int i0 = blockIdx.x * kBlock;
  const int tid = threadIdx.x;
  if (tid < kBlock) src[tid] = i0 + tid < L ? reorder_source(g, N, i0 + tid) : 0;
  __syncthreads();
  const int c = tid % CPR, r0 = tid / CPR;
  size_t in_off[NR], out_off[NR];
  bool ok[NR];
#pragma unroll
  for (int k = 0; k < NR; ++k) {
    const int r = r0 + k * RPI, i = i0 + r;
    ok[k] = i < L;
    const int s = src[r];
    in_off[k] = static_cast<size_t>(gather ? s : i) * CPR + c;
    out_off[k] = static_cast<size_t>(gather ? i : s) * CPR + c;
  }
  const int h0 = blockIdx.y * kHeadsPerWg, h1 = min(BH, h0 + kHeadsPerWg);
  const size_t hstride = static_cast<size_t>(L) * CPR;
  int h = h0;
  for (; h + 1 < h1; h += 2) {
    const u32x4* x0 = X + h * hstride;
    const u32x4* x1 = x0 + hstride;
    u32x4 v0[NR], v1[NR];
#pragma unroll
    for (int k = 0; k < NR; ++k)
      if (ok[k]) {
        v0[k] = __builtin_nontemporal_load(x0 + in_off[k]);
        v1[k] = __builtin_nontemporal_load(x1 + in_off[k]);
      }
    u32x4* y0 = Y + h * hstride;
    u32x4* y1 = y0 + hstride;
#pragma unroll
    for (int k = 0; k < NR; ++k)
      if (ok[k]) {
        __builtin_nontemporal_store(v0[k], y0 + out_off[k]);
        __builtin_nontemporal_store(v1[k], y1 + out_off[k]);
      }
  }
  if (h < h1) {
    const u32x4* x0 = X + h * hstride;
    u32x4* y0 = Y + h * hstride;
#pragma unroll
    for (int k = 0; k < NR; ++k)
      if (ok[k]) __builtin_nontemporal_store(__builtin_nontemporal_load(x0 + in_off[k]), y0 + out_off[k]);
  }
}

template <int CPR>
hipError_t launch(const paro_problem& p, const paro_grid& g, int N, int direction, const void* X, void* Y,
                  hipStream_t s) {
  const int BH = p.B * p.H;
  const dim3 grid(ceil_div(p.L, kBlock), ceil_div(BH, kHeadsPerWg));
  hipLaunchKernelGGL(k_reorder<CPR>, grid, dim3(kReorderThreads), 0, s, static_cast<const u32x4*>(X),
                     static_cast<u32x4*>(Y), g, N, p.L, BH, direction == PARO_REORDER_GATHER ? 1 : 0);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_reorder(const paro_problem& p, const paro_grid& g, int direction, const void* X, void* Y,
                          hipStream_t s) {
  const int N = g.t * g.y * g.x;
  const int row_bytes = p.d * (p.dtype == PARO_DTYPE_BF16 ? 2 : 4);
  switch (row_bytes / 16) {
    case 8: return launch<8>(p, g, N, direction, X, Y, s);
    case 16: return launch<16>(p, g, N, direction, X, Y, s);
    default: return launch<32>(p, g, N, direction, X, Y, s);
  }
}

}  // namespace paro
