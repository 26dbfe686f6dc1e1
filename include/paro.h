/*
 * paro.h - C ABI of the PISA block-sparse attention hot path on AMD CDNA4
 * (gfx950 / MI355X).
 *
 * Method: "PISA: Piecewise Sparse Attention Is Wiser for Efficient Diffusion
 * Transformers" (technical summary), section 2. For every query block i the
 * key/value blocks are split into an exact set S_i (the top-k blocks of a
 * covariance-aware score) and a tail U_i (all other blocks). The output is
 * o_t = N_t / D_t where
 *   N_t = sum_{j in S_i} sum_n exp(q'_t k_{j,n}) v_{j,n}
 *       + sum_{j in U_i} alpha_{t,j} vsum_j
 *       + (q'_t Hbar) sum_{j in U_i} alpha_{t,j},
 *   D_t = sum_{j in S_i} sum_n exp(q'_t k_{j,n}) + sum_{j in U_i} alpha_{t,j} n_j,
 *   alpha_{t,j} = exp(q'_t kbar_j), q'_t = scale * q_t,
 *   kbar_j = mean of the keys of block j, vsum_j = sum of its values,
 *   H_j = sum_n (k_{j,n} - kbar_j)^T v_{j,n}, Hbar = mean of H_j over all blocks,
 *   M_j = ||H_j - Hbar||_2 (largest singular value).
 * The denominator and the exact definition of H_j are not printed on the page;
 * the forms above are the ones under which the correction is the first-order
 * Taylor term of the exact block sums (its first-order part of the
 * denominator is zero).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Q, K, V, O: contiguous [B, H, L, d] tensors, d fastest, in device
 *   memory, element type given by paro_problem.dtype (bf16 bits or fp32).
 * - Blocks: T = ceil(L / block) blocks of `block` consecutive tokens; the last
 *   block may be partial (n_{T-1} = L - block*(T-1) valid tokens). Padded
 *   positions never contribute to any statistic, score or output.
 * - Every pointer is a device pointer aligned to 16 bytes. The caller owns
 *   every buffer; the library never allocates, frees, keeps or frees a pointer
 *   after return. Outputs are fully overwritten; inputs are never written;
 *   outputs must not alias inputs.
 * - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *   All work is enqueued on it asynchronously; the library never
 *   synchronizes, allocates or sets memory, so every call can be recorded
 *   into a HIP graph by stream capture (the launches are its only work).
 *   Device faults surface at the caller's next synchronization.
 * - Return value: PARO_OK (0) or a negative PARO_ERR_* code. Arguments are
 *   validated on the host before anything is launched; on an error nothing
 *   is launched and no output is touched. The library never prints or aborts.
 *   NaN/Inf inputs are not detected.
 * - Supported: block == 64; d in {64, 128}; 1 <= B, H; B*H <= 65535; 1 <= L;
 *   B*H*L*d < 2^31 elements per tensor; T <= PARO_MAX_BLOCKS. Anything
 *   else returns PARO_ERR_SHAPE.
 */
#ifndef PARO_H_
#define PARO_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PARO_VERSION 100

#define PARO_OK 0
#define PARO_ERR_NULL (-1)      /* a required pointer is NULL */
#define PARO_ERR_SHAPE (-2)     /* unsupported B, H, L, d, block, keep_k or T */
#define PARO_ERR_DTYPE (-3)     /* unknown dtype code */
#define PARO_ERR_ALIGN (-4)     /* a pointer is not 16-byte aligned */
#define PARO_ERR_WORKSPACE (-5) /* workspace smaller than the call's *_workspace_bytes() */
#define PARO_ERR_HIP (-6)       /* a kernel launch reported a HIP error */
#define PARO_ERR_ARG (-7)       /* scale not finite and > 0, lambda not finite, unknown mode or direction, X == Y */

#define PARO_TAIL_PISA 0  /* paro_attention_mode: zeroth-order tail and first-order correction */
#define PARO_TAIL_DROP 1  /* paro_attention_mode: tail dropped (keep-or-drop sparse attention) */
#define PARO_TAIL_ZEROTH 2 /* paro_attention_mode: zeroth-order tail only, no first-order correction */

#define PARO_DTYPE_BF16 0
#define PARO_DTYPE_FP32 1

#define PARO_MAX_BLOCKS 16384

typedef struct paro_problem {
  int32_t B;      /* batch */
  int32_t H;      /* heads */
  int32_t L;      /* tokens per sequence */
  int32_t d;      /* head dimension (64 or 128) */
  int32_t block;  /* tokens per block (64) */
  int32_t dtype;  /* PARO_DTYPE_BF16 or PARO_DTYPE_FP32: Q, K, V and O */
  double scale;   /* softmax scale (q' = scale * q), finite and > 0; usually 1/sqrt(d) */
} paro_problem;

/*
 * paro_precompute - block statistics (section 2, "hardware implementation",
 * pre-computation step, and "covariance-aware routing" for M_j).
 *
 * in : K, V [B, H, L, d] (dtype)
 * out: kbar [B, H, T, d] fp32   mean of the valid keys of block j
 *      vsum [B, H, T, d] fp32   sum of the valid values of block j
 *      Hbar [B, H, d, d] fp32   mean over all T blocks of H_j; row = key dim,
 *                               column = value dim
 *      M    [B, H, T]    fp64   largest singular value of H_j - Hbar
 *                               (restarted Lanczos on A^T A in fp32;
 *                               final ||A x|| / ||x|| in fp64)
 * workspace: device scratch of at least paro_precompute_workspace_bytes(p)
 *            bytes (per-chunk partial sums of H_j); contents on entry are
 *            ignored and undefined on return.
 * H_j itself is never written to memory.
 */
int paro_precompute(const paro_problem* p, const void* K, const void* V, float* kbar,
                    float* vsum, float* Hbar, double* M, void* workspace,
                    size_t workspace_bytes, void* stream);

/* Bytes of device workspace paro_precompute needs for this problem (0 on bad shape). */
size_t paro_precompute_workspace_bytes(const paro_problem* p);

/*
 * paro_route - covariance-aware top-k routing (section 2, "covariance-aware
 * routing"): score_ij = scale * qbar_i . kbar_j + lambda * M_j with qbar_i the
 * mean of the valid queries of block i. S_i = the keep_k highest scores of
 * row i, exact ties resolved toward the lower j, written in ascending j.
 *
 * in : Q [B, H, L, d] (dtype); kbar, M from paro_precompute; 0 <= keep_k <= T;
 *      lambda finite.
 * out: idx [B, H, T, keep_k] int32 (nothing is written when keep_k == 0).
 * qbar is summed in fp64 and rounded to fp32; the dot products qbar . kbar
 * are fp32 (error ~1e-7); scale * dot + lambda * M and the selection are
 * fp64.
 */
int paro_route(const paro_problem* p, const void* Q, const float* kbar, const double* M,
               int32_t keep_k, double lambda, int32_t* idx, void* stream);

/*
 * paro_attention - the fused piecewise attention (section 2, "core
 * algorithm" and the stage 1 / stage 2 / stage 3 pipeline): stage 1 exact
 * online softmax over the blocks listed in idx; stage 2 zeroth-order terms of
 * every other block from kbar and vsum, sharing the same running maximum;
 * stage 3 the global first-order correction (q' Hbar) * sum alpha; then N / D.
 *
 * in : Q, K, V [B, H, L, d] (dtype); kbar, vsum, Hbar from paro_precompute;
 *      idx [B, H, T, keep_k] int32: for every row, keep_k distinct block
 *      indices in [0, T) in ascending order (as paro_route writes them);
 *      0 <= keep_k <= T.
 * out: O [B, H, L, d] (dtype; rows >= L of the last block are not written).
 * workspace: device scratch of at least paro_attention_workspace_bytes(p)
 *            bytes (bf16 copies of kbar and vsum for the matrix cores and
 *            512 bytes of work-queue counters; 0 bytes, so NULL is allowed,
 *            for fp32 problems); contents on entry are ignored and undefined
 *            on return. Two calls that run at once must not share one
 *            workspace.
 * bf16 problems use bf16 MFMA products with fp32 accumulation (tail
 * centroids, value sums and Hbar rounded to bf16 for the matrix cores);
 * fp32 problems use fp32 arithmetic throughout. An idx row that breaks the
 * stated contract gives undefined output values (never an out-of-bounds access).
 */
int paro_attention(const paro_problem* p, const void* Q, const void* K, const void* V,
                   const float* kbar, const float* vsum, const float* Hbar,
                   const int32_t* idx, int32_t keep_k, void* O, void* workspace,
                   size_t workspace_bytes, void* stream);

/* Bytes of device workspace paro_attention and paro_attention_mode need for
 * this problem (0 on bad shape, and 0 for fp32 problems). */
size_t paro_attention_workspace_bytes(const paro_problem* p);

/*
 * paro_attention_mode - paro_attention with the treatment of the tail U_i
 * chosen by `mode`:
 *   PARO_TAIL_PISA: the method (same as paro_attention);
 *   PARO_TAIL_DROP: U_i is dropped (no stage 2, no stage 3): softmax
 *     attention renormalised over the blocks of S_i (with keep_k = 0 nothing
 *     is left and every output is 0/0, NaN), i.e. the keep-or-drop
 *     sparse attention that section 1 (problem definition) describes as the
 *     approach the method improves on, and the exact phase of the method on
 *     its own.
 *   PARO_TAIL_ZEROTH: stages 1 and 2 only (the zeroth-order tail terms
 *     without the first-order correction of stage 3), the ablation that
 *     isolates what the correction adds (section 2, the third term of the
 *     numerator).
 * Same arguments and contract as paro_attention; an unknown mode returns
 * PARO_ERR_ARG.
 */
int paro_attention_mode(const paro_problem* p, const void* Q, const void* K, const void* V,
                        const float* kbar, const float* vsum, const float* Hbar,
                        const int32_t* idx, int32_t keep_k, int32_t mode, void* O,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * paro_attention_noalloc - paro_attention_mode for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the workspace of paro_attention_mode
 * (the bf16 copies of kbar and vsum, the work-queue counters) lives in a
 * static device array of PARO_NOALLOC_SCRATCH_BYTES bytes inside the
 * library instead of a caller buffer. Nothing is allocated or freed by the
 * call.
 *   - Same arguments, results and errors as paro_attention_mode, minus the
 *     workspace. A problem whose paro_attention_workspace_bytes() exceeds
 *     PARO_NOALLOC_SCRATCH_BYTES returns PARO_ERR_WORKSPACE (the 720p video
 *     shape, B*H = 40, T = 1182, d = 128, needs 24.2 MB; fp32 problems need
 *     none).
 *   - The array of the current device is used (hipGetDevice); `stream` must
 *     belong to that device. Its address is looked up once per device on the
 *     first call (a failure there returns PARO_ERR_HIP).
 *   - Every GPU holds its own array until the process ends, and every call
 *     on one GPU shares it: calls that overlap on one GPU (on different
 *     streams, or from several threads without ordering) race and give
 *     undefined results. Calls ordered on one stream are safe; each call
 *     overwrites what it reads before reading it.
 */
#define PARO_NOALLOC_SCRATCH_BYTES (32u << 20)
int paro_attention_noalloc(const paro_problem* p, const void* Q, const void* K, const void* V,
                           const float* kbar, const float* vsum, const float* Hbar,
                           const int32_t* idx, int32_t keep_k, int32_t mode, void* O, void* stream);

/*
 * Geometric token reordering before blocking ("PAROAttention: Pattern-Aware
 * ReOrdering for Efficient Sparse and Quantized Attention in Visual
 * Generation Models", abstract: visual tokens are reordered so that their
 * locally aggregating attention becomes block-wise before sparsification;
 * "Adaptive Vector Quantized Attention" review, supplementary analysis: the
 * token order measurably changes the quality of a blockwise approximation).
 * The pages fix no concrete permutation; the order used here is the tiled
 * raster order:
 *   - the first t*y*x of the L tokens form a (t, y, x) latent grid in raster
 *     order (x fastest); tokens after it (text tokens) keep their places;
 *   - the grid is cut into boxes of tile_t x tile_y x tile_x tokens (boxes at
 *     the far edges are cut short), the boxes are listed in raster order and
 *     the tokens of each box in raster order.
 * With tile = 2 x 4 x 8 or 4 x 4 x 4 every full box is exactly one block of
 * 64 tokens, a compact piece of the latent instead of a slice of one row.
 */
typedef struct paro_grid {
  int32_t t, y, x;                /* latent grid extents, each >= 1, t*y*x <= L */
  int32_t tile_t, tile_y, tile_x; /* box extents, each >= 1 (larger than the grid = whole extent) */
} paro_grid;

#define PARO_REORDER_GATHER 0  /* Y[b,h,i,:] = X[b,h,src(i),:]: raster order -> tiled order */
#define PARO_REORDER_SCATTER 1 /* Y[b,h,src(i),:] = X[b,h,i,:]: tiled order -> raster order */

/*
 * paro_reorder - moves the token rows of X [B, H, L, d] (dtype of p) into
 * Y [B, H, L, d] in the tiled order of g (direction PARO_REORDER_GATHER) or
 * back (PARO_REORDER_SCATTER), where src(i) is the raster index of the
 * token at tiled position i. Rows are copied bit for bit. X and Y must not
 * overlap (X == Y returns PARO_ERR_ARG; a partial overlap is not detected).
 * A grid that does not fit L, or a non-positive extent, returns
 * PARO_ERR_SHAPE; an unknown direction PARO_ERR_ARG. p->scale is ignored.
 */
int paro_reorder(const paro_problem* p, const paro_grid* g, int32_t direction, const void* X, void* Y,
                 void* stream);

/* src(i) of paro_reorder, computed on the host: the raster index of the token
 * at tiled position i for L tokens, or -1 when g does not fit L or i is not
 * in [0, L). */
int32_t paro_reorder_source(const paro_grid* g, int32_t L, int32_t i);

/*
 * paro_route_budget - routing with per-query-block budgets ("Sparsity Should
 * Be ALLOTted by Output: Training-Free Allocation of Block-Sparse Attention
 * for Video Diffusion Transformers", review sections 1-3: a fixed total
 * budget of block-sparse attention shared out by what each output needs).
 * The page gives no estimator; the one used here, per (batch, head):
 *   - need of query block i: w_i = exp(H_i), H_i the entropy of the
 *     zeroth-order block masses p_ij proportional to n_j exp(scale qbar_i .
 *     kbar_j) (the effective number of blocks its attention spreads over),
 *     written to weights as wq_i = w_i 2^16 rounded to nearest (fp64);
 *   - R = k_total - T k_min is shared in proportion to wq with integer
 *     arithmetic: k_i = k_min + floor(R wq_i / S) (S = sum wq), and the
 *     R - sum of the floors leftover blocks go to the rows of largest
 *     remainder R wq_i mod S, ties to the lower i. A row holds at most T
 *     blocks: every row whose floor share reaches T - k_min is set to T,
 *     and the rest of R is shared again among the other rows by the same
 *     rule until no share reaches that cap, so offsets[h][T] = k_total;
 *   - S_i = the k_i best blocks of row i by the covariance-aware score, as in
 *     paro_route (ties to the lower j, ascending).
 * out: weights [B, H, T] int64; offsets [B, H, T + 1] int32, row i of head h
 *      in idx[h k_total + offsets[h][i] .. h k_total + offsets[h][i + 1]);
 *      idx [B, H, k_total] int32 (entries past offsets[h][T] are not written).
 * in : T k_min <= k_total <= T^2, k_total >= 1, k_min >= 0, lambda finite.
 * workspace: at least paro_route_budget_workspace_bytes(p) bytes (qbar).
 */
int paro_route_budget(const paro_problem* p, const void* Q, const float* kbar, const double* M,
                      int32_t k_total, int32_t k_min, double lambda, int64_t* weights,
                      int32_t* offsets, int32_t* idx, void* workspace, size_t workspace_bytes,
                      void* stream);

/* Bytes of device workspace paro_route_budget needs (0 on bad shape). */
size_t paro_route_budget_workspace_bytes(const paro_problem* p);

/*
 * paro_attention_csr - paro_attention_mode on exact lists of any lengths:
 * row i of head h is idx[h k_stride + offsets[h][i] ..
 * h k_stride + offsets[h][i + 1]) (as paro_route_budget writes them), each
 * list ascending with distinct indices in [0, T). Lists are clamped to
 * [0, k_stride) and to T entries, so a malformed list gives undefined output
 * values but never an out-of-bounds access. Same workspace as paro_attention.
 */
int paro_attention_csr(const paro_problem* p, const void* Q, const void* K, const void* V,
                       const float* kbar, const float* vsum, const float* Hbar,
                       const int32_t* offsets, const int32_t* idx, int32_t k_stride, int32_t mode,
                       void* O, void* workspace, size_t workspace_bytes, void* stream);

/*
 * paro_attention_fp8 - paro_attention_mode with the key-query products on
 * the fp8 matrix cores, for bf16 problems. "PAROAttention: Pattern-Aware
 * ReOrdering for Efficient Sparse and Quantized Attention in Visual
 * Generation Models" (abstract) runs block-sparse attention at reduced
 * bitwidth (INT8/INT4); here the same idea uses the e4m3 format that the
 * CDNA4 matrix cores multiply at twice the bf16 rate:
 *   - q' = scale * q is rounded to e4m3 with one power-of-two scale per query
 *     row, K and kbar with one power-of-two scale per row (paro_fp8_rows);
 *   - every logit q'.k (exact keys) and q'.kbar (tail centroids) is an e4m3
 *     product summed in fp32, the scales applied inside the MFMA;
 *   - the first-order correction (q' Hbar) uses the same rounded q';
 *   - the softmax weights, P V and the tail sums are as in paro_attention
 *     (bf16 operands, fp32 sums).
 * That is, the method evaluated on q', K and kbar rounded to e4m3 as stated.
 * Same arguments and contract as paro_attention_mode; fp32 problems return
 * PARO_ERR_DTYPE. workspace: at least paro_attention_fp8_workspace_bytes(p)
 * bytes (the e4m3 copies of K and kbar with their scales, bf16 vsum and 512
 * bytes of work-queue counters); two calls that run at once must not share
 * one workspace.
 */
int paro_attention_fp8(const paro_problem* p, const void* Q, const void* K, const void* V,
                       const float* kbar, const float* vsum, const float* Hbar,
                       const int32_t* idx, int32_t keep_k, int32_t mode, void* O,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace paro_attention_fp8 needs (0 on bad shape and for fp32 problems). */
size_t paro_attention_fp8_workspace_bytes(const paro_problem* p);

/*
 * paro_fp8_rows - the row quantiser of paro_attention_fp8: each of the nrows
 * rows of d values (dtype PARO_DTYPE_BF16 bits or PARO_DTYPE_FP32) is scaled
 * by 2^-e, with e the smallest integer, but no less than -127, such that
 * the row's largest |x| times 2^-e is at most 448 (e = 0 for an all-zero
 * row), and rounded to nearest even e4m3 (OCP FP8 E4M3: 4 exponent bits,
 * bias 7, 3 mantissa bits).
 * out: dst [nrows][d] e4m3 bytes; scales [nrows] the E8M0 codes e + 127.
 * d in {64, 128}; src and dst 16-byte aligned device pointers.
 */
int paro_fp8_rows(const void* src, int32_t dtype, int64_t nrows, int32_t d, uint8_t* dst,
                  uint8_t* scales, void* stream);

/* T = ceil(L / block), or -1 when L < 1 or block < 1. */
int32_t paro_num_blocks(int32_t L, int32_t block);

/* Static description of a status code (never NULL). */
const char* paro_status_string(int status);

/* PARO_VERSION of the loaded library. */
int paro_version(void);

#ifdef __cplusplus
}
#endif
#endif /* PARO_H_ */
