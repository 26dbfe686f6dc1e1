// Internal helpers shared by the gfx950 kernels of libparo (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "paro.h"

namespace paro {

constexpr int kBlock = 64;  // tokens per block (the only supported block size)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------- bf16 bits
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// Round-to-nearest-even float -> bf16 bits (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// Two floats -> packed bf16 pair (lo in bits 0..15), round-to-nearest-even,
// one v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// ------------------------------------------------------- element loads
// Element type of Q/K/V in memory: uint16_t (bf16 bits) or float.
template <typename E>
__device__ __forceinline__ float load_elem(const E* p);
template <>
__device__ __forceinline__ float load_elem<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }
template <>
__device__ __forceinline__ float load_elem<float>(const float* p) { return *p; }

// ------------------------------------------------------------------ DPP
// row_ror:n rotates values by n lanes inside each row of 16 lanes.
template <int N>
__device__ __forceinline__ float ror16(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x120 + N, 0xF, 0xF, false));
}
template <int N>
__device__ __forceinline__ double ror16(double v) {
  int2 x = __builtin_bit_cast(int2, v);
  x.x = __builtin_amdgcn_update_dpp(0, x.x, 0x120 + N, 0xF, 0xF, false);
  x.y = __builtin_amdgcn_update_dpp(0, x.y, 0x120 + N, 0xF, 0xF, false);
  return __builtin_bit_cast(double, x);
}
// Sum over the 16 lanes of a DPP row; every lane of the row receives the total.
template <typename F>
__device__ __forceinline__ F row_sum16(F v) {
  v += ror16<8>(v);
  v += ror16<4>(v);
  v += ror16<2>(v);
  v += ror16<1>(v);
  return v;
}
__device__ __forceinline__ double readlane_f64(double v, int lane) {
  int2 x = __builtin_bit_cast(int2, v);
  x.x = __builtin_amdgcn_readlane(x.x, lane);
  x.y = __builtin_amdgcn_readlane(x.y, lane);
  return __builtin_bit_cast(double, x);
}
// Full 64-lane sum in a fixed order; the result is wave-uniform.
__device__ __forceinline__ double wave_sum_f64(double v) {
  v = row_sum16(v);
  return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}

// ----------------------------------------------------------------- MFMA
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__host__ __device__ constexpr int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Workgroup barrier for data exchanged through LDS only: waits for this
// wave's LDS operations (lgkmcnt(0)) but leaves global loads in flight, unlike
// __syncthreads(), whose release fence also drains every outstanding global
// load. The empty asm statements keep the compiler from moving memory
// accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt and expcnt at their maxima, lgkmcnt = 0
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace paro

// ----------------------------------------------------- launcher prototypes
// Host-side launchers (defined with the kernels). Arguments are validated by
// the ABI layer before these are called; each returns a hipError_t.
namespace paro {
size_t precompute_workspace_bytes(const paro_problem& p);
hipError_t launch_precompute(const paro_problem& p, const void* K, const void* V, float* kbar,
                             float* vsum, float* Hbar, double* M, void* ws, hipStream_t s);
hipError_t launch_route(const paro_problem& p, const void* Q, const float* kbar, const double* M,
                        int keep_k, double lambda, int32_t* idx, hipStream_t s);
// offs: CSR row offsets [B H][T + 1] (keep_k is then the per-head stride of
// idx), or nullptr for rows of keep_k.
hipError_t launch_attention(const paro_problem& p, const void* Q, const void* K, const void* V,
                            const float* kbar, const float* vsum, const float* Hbar, const int32_t* idx,
                            int keep_k, void* O, int mode, void* ws, hipStream_t s,
                            const int32_t* offs = nullptr);
size_t attention_workspace_bytes(const paro_problem& p);
// Address of this device's static attention scratch (PARO_NOALLOC_SCRATCH_BYTES
// bytes), looked up with hipGetSymbolAddress on the first call per device.
hipError_t attention_scratch(void** out);
hipError_t launch_attention_fp8(const paro_problem& p, const void* Q, const void* K, const void* V,
                                const float* kbar, const float* vsum, const float* Hbar, const int32_t* idx,
                                int keep_k, void* O, int mode, void* ws, hipStream_t s);
size_t attention_fp8_workspace_bytes(const paro_problem& p);
hipError_t launch_fp8_rows(const void* src, int dtype, size_t nrows, int d, uint8_t* dst, uint8_t* ex, hipStream_t s);
// g must have its tile extents clamped to the grid extents.
hipError_t launch_reorder(const paro_problem& p, const paro_grid& g, int direction, const void* X, void* Y,
                          hipStream_t s);
__host__ __device__ int reorder_source(const paro_grid& g, int N, int i);
int route_rows_per_group(int T, int d);
size_t route_budget_workspace_bytes(const paro_problem& p);
hipError_t launch_route_budget(const paro_problem& p, const void* Q, const float* kbar, const double* M, int k_total,
                               int k_min, double lambda, int64_t* wq, int32_t* offsets, int32_t* idx, void* ws,
                               hipStream_t s);
}  // namespace paro
