// C ABI of libparo: host-side argument validation, then the kernel launchers.
// Validation touches no HIP API, so every error path runs without a device
// and nothing is launched when an argument is rejected.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <initializer_list>

#include "paro_common.h"

namespace {

int check_problem(const paro_problem* p) {
  if (!p) return PARO_ERR_NULL;
  if (p->dtype != PARO_DTYPE_BF16 && p->dtype != PARO_DTYPE_FP32) return PARO_ERR_DTYPE;
  if (p->B < 1 || p->H < 1 || p->L < 1) return PARO_ERR_SHAPE;
  if (p->block != paro::kBlock) return PARO_ERR_SHAPE;
  if (p->d != 64 && p->d != 128) return PARO_ERR_SHAPE;
  if (static_cast<int64_t>(p->B) * p->H > 65535) return PARO_ERR_SHAPE;
  const int64_t T = (static_cast<int64_t>(p->L) + p->block - 1) / p->block;
  if (T > PARO_MAX_BLOCKS) return PARO_ERR_SHAPE;
  if (T * p->B * p->H > INT32_MAX) return PARO_ERR_SHAPE;
  if (static_cast<int64_t>(p->B) * p->H * p->L * p->d > INT32_MAX) return PARO_ERR_SHAPE;
  if (!std::isfinite(p->scale) || !(p->scale > 0.0)) return PARO_ERR_ARG;
  return PARO_OK;
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

int check_ptrs(std::initializer_list<const void*> ptrs) {
  for (const void* q : ptrs)
    if (!q) return PARO_ERR_NULL;
  for (const void* q : ptrs)
    if (!aligned16(q)) return PARO_ERR_ALIGN;
  return PARO_OK;
}

int num_blocks(const paro_problem* p) { return (p->L + p->block - 1) / p->block; }

int from_hip(hipError_t e) { return e == hipSuccess ? PARO_OK : PARO_ERR_HIP; }

// Checks a token grid against L and returns it with the tile extents clamped
// to the grid extents (the same order, and products that stay within L).
int check_grid(const paro_grid* g, int32_t L, paro_grid* out) {
  if (!g) return PARO_ERR_NULL;
  if (g->t < 1 || g->y < 1 || g->x < 1 || g->tile_t < 1 || g->tile_y < 1 || g->tile_x < 1) return PARO_ERR_SHAPE;
  if (static_cast<int64_t>(g->t) * g->y * g->x > L) return PARO_ERR_SHAPE;
  *out = *g;
  out->tile_t = std::min(g->tile_t, g->t);
  out->tile_y = std::min(g->tile_y, g->y);
  out->tile_x = std::min(g->tile_x, g->x);
  return PARO_OK;
}

}  // namespace

extern "C" {

size_t paro_route_budget_workspace_bytes(const paro_problem* p) {
  if (check_problem(p) != PARO_OK || paro::route_rows_per_group(num_blocks(p), p->d) < 1) return 0;
  return paro::route_budget_workspace_bytes(*p);
}

int paro_route_budget(const paro_problem* p, const void* Q, const float* kbar, const double* M, int32_t k_total,
                      int32_t k_min, double lambda, int64_t* weights, int32_t* offsets, int32_t* idx, void* workspace,
                      size_t workspace_bytes, void* stream) {
  int rc = check_problem(p);
  if (rc != PARO_OK) return rc;
  const int64_t T = num_blocks(p);
  if (paro::route_rows_per_group(static_cast<int>(T), p->d) < 1) return PARO_ERR_SHAPE;
  if (k_min < 0 || k_total < T * k_min || k_total > T * T || k_total < 1) return PARO_ERR_SHAPE;
  if (!std::isfinite(lambda)) return PARO_ERR_ARG;
  if ((rc = check_ptrs({Q, kbar, M, weights, offsets, idx, workspace})) != PARO_OK) return rc;
  if (workspace_bytes < paro::route_budget_workspace_bytes(*p)) return PARO_ERR_WORKSPACE;
  return from_hip(paro::launch_route_budget(*p, Q, kbar, M, k_total, k_min, lambda, weights, offsets, idx, workspace,
                                            static_cast<hipStream_t>(stream)));
}

int paro_attention_csr(const paro_problem* p, const void* Q, const void* K, const void* V, const float* kbar,
                       const float* vsum, const float* Hbar, const int32_t* offsets, const int32_t* idx,
                       int32_t k_stride, int32_t mode, void* O, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_problem(p);
  if (rc != PARO_OK) return rc;
  if (k_stride < 0) return PARO_ERR_SHAPE;
  if (mode != PARO_TAIL_PISA && mode != PARO_TAIL_DROP && mode != PARO_TAIL_ZEROTH) return PARO_ERR_ARG;
  if ((rc = check_ptrs({Q, K, V, kbar, vsum, Hbar, O, offsets})) != PARO_OK) return rc;
  if (k_stride > 0 && (rc = check_ptrs({idx})) != PARO_OK) return rc;
  const size_t need = paro::attention_workspace_bytes(*p);
  if (workspace_bytes < need) return PARO_ERR_WORKSPACE;
  if (need > 0 && (rc = check_ptrs({workspace})) != PARO_OK) return rc;
  return from_hip(paro::launch_attention(*p, Q, K, V, kbar, vsum, Hbar, idx, k_stride, O, mode, workspace,
                                         static_cast<hipStream_t>(stream), offsets));
}

size_t paro_attention_fp8_workspace_bytes(const paro_problem* p) {
  if (check_problem(p) != PARO_OK) return 0;
  return paro::attention_fp8_workspace_bytes(*p);
}

int paro_attention_fp8(const paro_problem* p, const void* Q, const void* K, const void* V, const float* kbar,
                       const float* vsum, const float* Hbar, const int32_t* idx, int32_t keep_k, int32_t mode, void* O,
                       void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_problem(p);
  if (rc != PARO_OK) return rc;
  if (p->dtype != PARO_DTYPE_BF16) return PARO_ERR_DTYPE;
  const int T = num_blocks(p);
  if (keep_k < 0 || keep_k > T) return PARO_ERR_SHAPE;
  if (mode != PARO_TAIL_PISA && mode != PARO_TAIL_DROP && mode != PARO_TAIL_ZEROTH) return PARO_ERR_ARG;
  if ((rc = check_ptrs({Q, K, V, kbar, vsum, Hbar, O, workspace})) != PARO_OK) return rc;
  if (keep_k > 0 && (rc = check_ptrs({idx})) != PARO_OK) return rc;
  if (workspace_bytes < paro::attention_fp8_workspace_bytes(*p)) return PARO_ERR_WORKSPACE;
  return from_hip(paro::launch_attention_fp8(*p, Q, K, V, kbar, vsum, Hbar, idx, keep_k, O, mode, workspace,
                                             static_cast<hipStream_t>(stream)));
}

int paro_fp8_rows(const void* src, int32_t dtype, int64_t nrows, int32_t d, uint8_t* dst, uint8_t* scales,
                  void* stream) {
  if (dtype != PARO_DTYPE_BF16 && dtype != PARO_DTYPE_FP32) return PARO_ERR_DTYPE;
  if (nrows < 1 || (d != 64 && d != 128) || nrows * d > INT64_C(1) << 40) return PARO_ERR_SHAPE;
  int rc;
  if ((rc = check_ptrs({src, dst})) != PARO_OK) return rc;
  if (!scales) return PARO_ERR_NULL;
  return from_hip(paro::launch_fp8_rows(src, dtype, static_cast<size_t>(nrows), d, dst, scales,
                                        static_cast<hipStream_t>(stream)));
}

int paro_reorder(const paro_problem* p, const paro_grid* g, int32_t direction, const void* X, void* Y,
                 void* stream) {
  int rc = check_problem(p);
  if (rc != PARO_OK) return rc;
  paro_grid gc;
  if ((rc = check_grid(g, p->L, &gc)) != PARO_OK) return rc;
  if (direction != PARO_REORDER_GATHER && direction != PARO_REORDER_SCATTER) return PARO_ERR_ARG;
  if ((rc = check_ptrs({X, Y})) != PARO_OK) return rc;
  if (X == Y) return PARO_ERR_ARG;
  return from_hip(paro::launch_reorder(*p, gc, direction, X, Y, static_cast<hipStream_t>(stream)));
}

int32_t paro_reorder_source(const paro_grid* g, int32_t L, int32_t i) {
  paro_grid gc;
  if (L < 1 || check_grid(g, L, &gc) != PARO_OK || i < 0 || i >= L) return -1;
  return paro::reorder_source(gc, gc.t * gc.y * gc.x, i);
}

int32_t paro_num_blocks(int32_t L, int32_t block) {
  if (L < 1 || block < 1) return -1;
  return static_cast<int32_t>((static_cast<int64_t>(L) + block - 1) / block);
}

int paro_version(void) { return PARO_VERSION; }

const char* paro_status_string(int status) {
  switch (status) {
    case PARO_OK: return "ok";
    case PARO_ERR_NULL: return "a required pointer is NULL";
    case PARO_ERR_SHAPE: return "unsupported shape (B, H, L, d, block, keep_k or number of blocks)";
    case PARO_ERR_DTYPE: return "unknown dtype code";
    case PARO_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case PARO_ERR_WORKSPACE: return "workspace smaller than the call's *_workspace_bytes()";
    case PARO_ERR_HIP: return "a kernel launch reported a HIP error";
    case PARO_ERR_ARG: return "scale must be finite and > 0, lambda finite, mode or direction known, X != Y";
    default: return "unknown status";
  }
}

size_t paro_precompute_workspace_bytes(const paro_problem* p) {
  if (check_problem(p) != PARO_OK) return 0;
  return paro::precompute_workspace_bytes(*p);
}

int paro_precompute(const paro_problem* p, const void* K, const void* V, float* kbar, float* vsum, float* Hbar,
                    double* M, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_problem(p);
  if (rc != PARO_OK) return rc;
  if ((rc = check_ptrs({K, V, kbar, vsum, Hbar, M, workspace})) != PARO_OK) return rc;
  if (workspace_bytes < paro::precompute_workspace_bytes(*p)) return PARO_ERR_WORKSPACE;
  return from_hip(paro::launch_precompute(*p, K, V, kbar, vsum, Hbar, M, workspace,
                                          static_cast<hipStream_t>(stream)));
}

int paro_route(const paro_problem* p, const void* Q, const float* kbar, const double* M, int32_t keep_k,
               double lambda, int32_t* idx, void* stream) {
  int rc = check_problem(p);
  if (rc != PARO_OK) return rc;
  const int T = num_blocks(p);
  if (keep_k < 0 || keep_k > T) return PARO_ERR_SHAPE;
  if (paro::route_rows_per_group(T, p->d) < 1) return PARO_ERR_SHAPE;
  if (!std::isfinite(lambda)) return PARO_ERR_ARG;
  if ((rc = check_ptrs({Q, kbar, M})) != PARO_OK) return rc;
  if (keep_k > 0 && (rc = check_ptrs({idx})) != PARO_OK) return rc;
  return from_hip(paro::launch_route(*p, Q, kbar, M, keep_k, lambda, idx, static_cast<hipStream_t>(stream)));
}

size_t paro_attention_workspace_bytes(const paro_problem* p) {
  if (check_problem(p) != PARO_OK) return 0;
  return paro::attention_workspace_bytes(*p);
}

int paro_attention_mode(const paro_problem* p, const void* Q, const void* K, const void* V, const float* kbar,
                        const float* vsum, const float* Hbar, const int32_t* idx, int32_t keep_k, int32_t mode,
                        void* O, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_problem(p);
  if (rc != PARO_OK) return rc;
  const int T = num_blocks(p);
  if (keep_k < 0 || keep_k > T) return PARO_ERR_SHAPE;
  if (mode != PARO_TAIL_PISA && mode != PARO_TAIL_DROP && mode != PARO_TAIL_ZEROTH) return PARO_ERR_ARG;
  if ((rc = check_ptrs({Q, K, V, kbar, vsum, Hbar, O})) != PARO_OK) return rc;
  if (keep_k > 0 && (rc = check_ptrs({idx})) != PARO_OK) return rc;
  const size_t need = paro::attention_workspace_bytes(*p);
  if (workspace_bytes < need) return PARO_ERR_WORKSPACE;
  if (need > 0 && (rc = check_ptrs({workspace})) != PARO_OK) return rc;
  return from_hip(paro::launch_attention(*p, Q, K, V, kbar, vsum, Hbar, idx, keep_k, O, mode, workspace,
                                         static_cast<hipStream_t>(stream)));
}

int paro_attention_noalloc(const paro_problem* p, const void* Q, const void* K, const void* V, const float* kbar,
                           const float* vsum, const float* Hbar, const int32_t* idx, int32_t keep_k, int32_t mode,
                           void* O, void* stream) {
  int rc = check_problem(p);
  if (rc != PARO_OK) return rc;
  const int T = num_blocks(p);
  if (keep_k < 0 || keep_k > T) return PARO_ERR_SHAPE;
  if (mode != PARO_TAIL_PISA && mode != PARO_TAIL_DROP && mode != PARO_TAIL_ZEROTH) return PARO_ERR_ARG;
  if ((rc = check_ptrs({Q, K, V, kbar, vsum, Hbar, O})) != PARO_OK) return rc;
  if (keep_k > 0 && (rc = check_ptrs({idx})) != PARO_OK) return rc;
  const size_t need = paro::attention_workspace_bytes(*p);
  if (need > PARO_NOALLOC_SCRATCH_BYTES) return PARO_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0 && (rc = from_hip(paro::attention_scratch(&ws))) != PARO_OK) return rc;
  return from_hip(paro::launch_attention(*p, Q, K, V, kbar, vsum, Hbar, idx, keep_k, O, mode, ws,
                                         static_cast<hipStream_t>(stream)));
}

int paro_attention(const paro_problem* p, const void* Q, const void* K, const void* V, const float* kbar,
                   const float* vsum, const float* Hbar, const int32_t* idx, int32_t keep_k, void* O,
                   void* workspace, size_t workspace_bytes, void* stream) {
  return paro_attention_mode(p, Q, K, V, kbar, vsum, Hbar, idx, keep_k, PARO_TAIL_PISA, O, workspace,
                             workspace_bytes, stream);
}

}  // extern "C"
