// Measurement helpers of libparo_peaks (include/paro_peaks.h): the practical
// bf16 matrix-core rate and HBM read rate of the GPU, against which the PISA
// kernels' rates are also reported. Not part of the PISA path.
#include <hip/hip_runtime.h>

#include "paro_peaks.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kChains = 8;

__global__ __launch_bounds__(256) void k_peak_mfma(int iters, float* __restrict__ sink) {
  const int l = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = static_cast<__bf16>(1.0f / static_cast<float>(1 + ((l + e) & 7)));
    b[e] = static_cast<__bf16>(static_cast<float>((l * 3 + e) & 3) * 0.25f);
  }
  f32x16 c[kChains];
#pragma unroll
  for (int i = 0; i < kChains; ++i) c[i] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < kChains; ++i) c[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[i], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kChains; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += c[i][e];
  __shared__ float red[256];
  red[threadIdx.x] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.f;
    for (int i = 0; i < 256; ++i) t += red[i];
    sink[blockIdx.x] = t;
  }
}

__global__ __launch_bounds__(256) void k_peak_read(const u32x4* __restrict__ src, size_t n16,
                                                   float* __restrict__ sink) {
  uint32_t acc = 0;
  const size_t stride = static_cast<size_t>(gridDim.x) * 256;
  size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 x0 = __builtin_nontemporal_load(src + i);
    const u32x4 x1 = __builtin_nontemporal_load(src + i + stride);
    const u32x4 x2 = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4 x3 = __builtin_nontemporal_load(src + i + 3 * stride);
    acc ^= (x0.x ^ x0.y ^ x0.z ^ x0.w) ^ (x1.x ^ x1.y ^ x1.z ^ x1.w) ^ (x2.x ^ x2.y ^ x2.z ^ x2.w) ^
           (x3.x ^ x3.y ^ x3.z ^ x3.w);
  }
  for (; i < n16; i += stride) {
    const u32x4 x = __builtin_nontemporal_load(src + i);
    acc ^= x.x ^ x.y ^ x.z ^ x.w;
  }
  __shared__ uint32_t red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
    for (int k = 0; k < 256; ++k) t ^= red[k];
    sink[blockIdx.x] = static_cast<float>(t & 0xFFFF);
  }
}

}  // namespace

extern "C" {

int paro_peak_mfma_bf16(int32_t workgroups, int32_t iters, float* sink, void* stream) {
  if (workgroups < 1 || workgroups > (1 << 20) || iters < 1 || iters > (1 << 20)) return -2;
  if (!sink) return -1;
  hipLaunchKernelGGL(k_peak_mfma, dim3(workgroups), dim3(256), 0, static_cast<hipStream_t>(stream), iters, sink);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

int paro_peak_read(const void* src, size_t bytes, int32_t workgroups, float* sink, void* stream) {
  if (bytes < 16 || bytes % 16 || workgroups < 1 || workgroups > (1 << 20)) return -2;
  if (!src || !sink) return -1;
  hipLaunchKernelGGL(k_peak_read, dim3(workgroups), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(src), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // extern "C"
