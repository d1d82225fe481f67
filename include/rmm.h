/*
 * rmm.h -- C ABI of the fused RMSNorm+MatMul library for MI355X (gfx950).
 *
 * The operation is the worked example of the Mirage paper review ("Mirage: A
 * Multi-Level Superoptimizer for Tensor Programs", section "核心概念 /
 * μGraph示例"): RMSNorm followed by MatMul, computed by one kernel that never
 * writes the normalised activations to memory.  The same page's abstract
 * expression (section "核心公式 / 抽象表达式"),
 *     E(O) = sum(k, div(mul(I1, I2), I3)),
 * is a k-sum of a product divided by a per-row value that does not depend on
 * k, so the division can be applied once, after the k-sum:
 *
 *     Y[m,n] = ( sum_k X[m,k] * g[k] * W[k,n] ) / sqrt( sum_k X[m,k]^2 / K + eps )
 *
 * The pages name RMSNorm without defining it; the reading used is the usual
 * one (RMS over the contraction dimension K, eps inside the square root, a
 * per-k gain g).  The gated variant follows the GatedMLP benchmark row of
 * the same page (section "五、实验结果"), read as SwiGLU:
 *
 *     Y = silu(norm(X) W1) * (norm(X) W3),   silu(z) = z / (1 + exp(-z))
 *
 * Layouts (all row-major, packed, no strides):
 *   X  : M x K   (X[m*K + k])
 *   g  : K
 *   W, W1, W3 : K x N   (W[k*N + n]; rows indexed by k)
 *   Y  : M x N   (Y[m*N + n])
 * dtype selects the storage type of X, g, W*, Y together; products are summed
 * in fp32 whatever the dtype.  With RMM_DTYPE_BF16 the operand X[m,k]*g[k] is
 * formed exactly in fp32 (a product of two bf16 values); the plain product
 * rounds it once (round to nearest even) to bf16 before the matrix-core
 * product, while the gated product and the low-rank adapter carry it exactly
 * as two bf16 parts hi + lo (two matrix-core products), because the gate
 * multiplies one product's error by the other and the adapter's two terms can
 * cancel.  Y is rounded once from fp32 to bf16 (nearest even).
 *
 * Ownership and ordering.  Every data pointer is a DEVICE pointer owned by the
 * caller; the library keeps none after it returns, allocates nothing and
 * never synchronises.  Calls are stream ordered: they validate on the host,
 * enqueue on `stream` (NULL = the default stream) and return; Y is valid once
 * the stream has reached that point.
 *
 * Workspace.  The split-K forms (the decode variant, the stream variant's
 * split form, the prefill split for few output tiles) combine partial k-sums
 * across workgroups through a caller-owned workspace.  `ws` may be NULL: the library
 * then picks a variant that needs none (correct, slower).  A non-NULL `ws` must
 * be zero-filled before its first use.  Every layout keeps its arrival
 * counters in the workspace's first 64 KiB and its partial sums after that;
 * a call resets its counters to zero and overwrites its partial-sum slots
 * before reading them, so one workspace serves any sequence of calls -- any
 * entry point, shape, dtype, variant or split count -- without clearing, as
 * long as each call runs to completion (a call forced to a split count
 * needing more than 16320 counters returns RMM_ERR_VARIANT).  One workspace
 * must not be used by two calls that may run at the same time.  A non-NULL
 * `ws` must be 16-byte aligned (hipMalloc's are), else RMM_ERR_WORKSPACE.
 * ws_bytes below rmm_workspace_bytes*() returns RMM_ERR_WORKSPACE, except
 * where AUTO picks the prefill split: it then takes the best count that fits
 * (down to no split).
 *
 * Errors.  Validation happens on the host before any HIP call, in this order:
 *   RMM_ERR_NULL      a NULL data pointer (when M*N > 0)
 *   RMM_ERR_SHAPE     M < 0, N < 0, K <= 0 (the mean over an empty row is
 *                     undefined), an adapter rank outside 1..64, or an
 *                     element count that overflows int64
 *   RMM_ERR_EPS       eps negative or not finite (eps = 0 is allowed)
 *   RMM_ERR_DTYPE     unknown dtype
 *   RMM_ERR_ALIAS     Y's byte range overlaps an input or the workspace
 *   RMM_ERR_VARIANT   a forced variant/split count cannot run this call
 *   RMM_ERR_WORKSPACE ws non-NULL and ws_bytes too small or ws not 16-byte aligned
 * M == 0 or N == 0 is a no-op returning RMM_OK.  A failed launch returns
 * RMM_ERR_HIP; rmm_last_hip_error() gives the hipError_t (thread local).
 * Input values are not checked: NaN/Inf propagate (with eps = 0 an all-zero
 * row gives 0 * inf = NaN).  No C++ exception crosses this interface.
 */
#ifndef RMM_H
#define RMM_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RMM_ABI_VERSION 1

typedef enum { RMM_DTYPE_F32 = 0, RMM_DTYPE_BF16 = 1 } rmm_dtype;

typedef enum {
  RMM_OK = 0,
  RMM_ERR_NULL = 1,
  RMM_ERR_SHAPE = 2,
  RMM_ERR_EPS = 3,
  RMM_ERR_DTYPE = 4,
  RMM_ERR_ALIAS = 5,
  RMM_ERR_WORKSPACE = 6,
  RMM_ERR_HIP = 7,
  RMM_ERR_VARIANT = 8,
  RMM_ERR_SCRATCH = 9
} rmm_status;

/* Kernel variants.  AUTO picks by shape (gated: DECODE for M <= 16 when a
 * workspace is passed, STREAM up to 64 rows with a workspace and up to 128
 * without, PREFILL above); the others force one (tests, bench).
 * The fast variants need bf16, K % 8 == 0, N % 8 == 0, 16-byte aligned
 * pointers, and X and each weight below 2 GiB (except fp32 DECODE, below).
 *   GENERIC : any shape, alignment and dtype; VALU fp32 products.
 *   DECODE  : bf16: M <= 32 (gated: M <= 16; with the adapter M <= 128 as
 *             one launch per 32-row block); streams W once with split-K
 *             across workgroups, bf16 matrix-core (MFMA) products, fp32
 *             partials combined by the last-arriving workgroup.
 *             fp32: M <= 32 (16 rows per launch), not gated, no adapter,
 *             16-byte aligned pointers; the same split-K scheme with fp32 fused
 *             multiply-adds (no bf16 rounding).  Bandwidth-bound.
 *   PREFILL : LDS-tiled MFMA GEMM with the row sum of squares fused into
 *             its k-loop (gated: both products in one tile).  Matrix-core-
 *             bound shapes.  Calls with few output tiles (at most 128 tiles:
 *             256 x 256 plain, 128 rows x 128 columns of each weight gated)
 *             and a workspace split K into ranges of whole 64-deep steps:
 *             each workgroup writes its range's fp32 sums (both products'
 *             when gated) and row sums of squares to the workspace, and a
 *             second kernel adds the ranges in order, applies 1/RMS (and the
 *             gate).  AUTO takes this form above 64 rows when a workspace
 *             is passed, with a count whose partial sums fit in that
 *             workspace.
 *   STREAM  : gated: any M; plain: M <= 128, or M <= 256 with N <= 4096
 *             (above 64 rows: one launch per 64-row block); each
 *             workgroup streams 64-column strips of W (W1 and W3 when
 *             gated) over all of K through LDS.  With a workspace
 *             and at most 128 strips, the split form: every workgroup takes
 *             an equal share of the strips' k-steps, partial sums combined
 *             in the workspace.  Bandwidth-bound shapes.                  */
typedef enum {
  RMM_VARIANT_AUTO = 0,
  RMM_VARIANT_GENERIC = 1,
  RMM_VARIANT_DECODE = 2,
  RMM_VARIANT_PREFILL = 3,
  RMM_VARIANT_STREAM = 4
} rmm_variant;

/* Y = RMSNorm(X; g, eps) W  (see the header comment for the definition).
 * X, g, W: inputs; Y: output, must not overlap any input.  eps is used as
 * given (fp32).  ws/ws_bytes: optional workspace (see above). */
rmm_status rmsnorm_matmul(const void* X, const void* g, const void* W, void* Y, float eps,
                          int64_t M, int64_t N, int64_t K, rmm_dtype dtype, void* ws,
                          size_t ws_bytes, hipStream_t stream);

/* rmsnorm_matmul for callers that cannot allocate: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments and result as rmsnorm_matmul without the workspace: the split-K
 * partial sums go to a fixed 16 MiB device array inside the library (one per
 * GPU, held until the process ends; its device address is looked up once per
 * device on the first call there).  Validation and errors as rmsnorm_matmul,
 * plus RMM_ERR_SCRATCH when the call would need more than 16 MiB of scratch
 * (never for M <= 32, nor for the stream variant's split form, nor for the
 * prefill split, whose count is chosen to fit the array); nothing is
 * allocated or freed.  Every call on one GPU shares that array: calls that
 * may overlap on one GPU (different streams or threads) race and must be
 * serialised by the caller.  A call leaves the array's counters zeroed for
 * the next, whatever its shape. */
rmm_status rmsnorm_matmul_noalloc(const void* X, const void* g, const void* W, void* Y, float eps,
                                  int64_t M, int64_t N, int64_t K, rmm_dtype dtype,
                                  hipStream_t stream);

/* Y = silu(RMSNorm(X) W1) * (RMSNorm(X) W3); W1 and W3 are both K x N and the
 * 1/RMS scale is applied to both products before the SiLU. */
rmm_status rmsnorm_gated_mlp(const void* X, const void* g, const void* W1, const void* W3,
                             void* Y, float eps, int64_t M, int64_t N, int64_t K,
                             rmm_dtype dtype, void* ws, size_t ws_bytes, hipStream_t stream);

/* As above with a forced variant.  splits: number of K chunks the DECODE
 * or PREFILL variant combines across workgroups (0 = chosen by the library,
 * 1 = no cross-workgroup combine, so no workspace is needed; PREFILL rounds
 * a forced count to whole, even ranges of 64-deep steps, so the count that
 * runs, reported by rmm_plan, may be lower; above ceil(K / 64) or with
 * partial sums above 2 GiB: RMM_ERR_VARIANT); must be 0 for the other
 * variants. */
rmm_status rmsnorm_matmul_ex(const void* X, const void* g, const void* W, void* Y, float eps,
                             int64_t M, int64_t N, int64_t K, rmm_dtype dtype,
                             rmm_variant variant, int splits, void* ws, size_t ws_bytes,
                             hipStream_t stream);
rmm_status rmsnorm_gated_mlp_ex(const void* X, const void* g, const void* W1, const void* W3,
                                void* Y, float eps, int64_t M, int64_t N, int64_t K,
                                rmm_dtype dtype, rmm_variant variant, int splits, void* ws,
                                size_t ws_bytes, hipStream_t stream);

/* The unfused program, for comparison.  The page that introduces the worked
 * example ("核心概念 / μGraph示例") contrasts the fused kernel with what
 * existing systems run: an RMSNorm kernel that writes the normalised
 * activations to device memory, then a MatMul kernel that reads them back.
 * These three calls are that program, built from the same kernels:
 *
 *   rmm_rmsnorm:      Xn = RMSNorm(X; g, eps), M x K, same dtype as X (bf16:
 *                     X*g*(1/RMS) formed in fp32, rounded once to nearest even).
 *   rmm_matmul:       Y = X W (no gain, no 1/RMS scale); the variants, split
 *                     counts and workspace rules of rmsnorm_matmul apply.
 *   rmm_gated_matmul: Y = silu(X W1) * (X W3).
 *
 * rmm_rmsnorm followed by rmm_matmul computes the same Y as rmsnorm_matmul up to
 * the extra rounding of Xn.  Validation order and error codes are those of
 * the fused calls (rmm_rmsnorm: RMM_ERR_NULL, RMM_ERR_SHAPE for M < 0 or
 * K <= 0, RMM_ERR_EPS, RMM_ERR_DTYPE, RMM_ERR_ALIAS when Xn overlaps X or
 * g; any alignment and K are accepted).  Xn may not be X: the kernel reads
 * each row twice. */
rmm_status rmm_rmsnorm(const void* X, const void* g, void* Xn, float eps, int64_t M, int64_t K,
                       rmm_dtype dtype, hipStream_t stream);
rmm_status rmm_matmul(const void* X, const void* W, void* Y, int64_t M, int64_t N, int64_t K,
                      rmm_dtype dtype, void* ws, size_t ws_bytes, hipStream_t stream);
rmm_status rmm_gated_matmul(const void* X, const void* W1, const void* W3, void* Y, int64_t M,
                            int64_t N, int64_t K, rmm_dtype dtype, void* ws, size_t ws_bytes,
                            hipStream_t stream);

/* Low-rank adapter (LoRA), the LoRA row of the same page's benchmark table
 * ("五、实验结果"; the page names the benchmark only, the reading is the usual
 * adapter): the frozen product plus a rank-R update applied as two thin
 * products,
 *
 *   rmsnorm_lora:    Y = Nrm W + (Nrm A^T) B,   Nrm = RMSNorm(X; g, eps)
 *   rmm_lora_matmul: Y = X W + (X A^T) B        (no gain, no 1/RMS scale)
 *
 * Layouts: A is R x K row-major (row r is the r-th down-projection vector,
 * A[r*K + k]; the layout of a torch Linear(K, R) weight), B is R x N
 * row-major (B[r*N + n]); both in the call's dtype, 1 <= R <= 64
 * (RMM_LORA_MAX_RANK, else RMM_ERR_SHAPE).  The down-projection T = Act A^T
 * is summed in fp32 from the same operand the weight product uses (bf16:
 * X*g carried exactly as two bf16 parts, see the top of this file), kept in
 * fp32 (never rounded to the storage type), and T B is added to the k-sum
 * before the 1/RMS scale, so one rounding produces Y.  Not combined with
 * the gate.  Variants: DECODE (bf16, M <= 128 as one launch per 32-row
 * block, R <= 32; the down-projection partials travel with the split-K
 * partials), PREFILL (bf16, any M, R <= 64, a workspace required: a first
 * kernel writes T to it, then a tile of 128 rows x 256 columns carries X g
 * as two bf16 parts and adds T B, T likewise in two parts, as one more
 * k-step of the same accumulators; with at most 128 tiles the K split of
 * the plain PREFILL variant, T B added by the last range; AUTO takes it
 * above 64 rows when a workspace is passed) and GENERIC (everything else); forcing STREAM
 * returns RMM_ERR_VARIANT.  NULL checks cover A and B; Y must not overlap
 * them.
 * Workspace rules are those of rmsnorm_matmul, sized by
 * rmm_lora_workspace_bytes (variant = RMM_VARIANT_AUTO, splits = 0 for the
 * plain entry points). */
#define RMM_LORA_MAX_RANK 64
rmm_status rmsnorm_lora(const void* X, const void* g, const void* W, const void* A, const void* B,
                        void* Y, float eps, int64_t M, int64_t N, int64_t K, int64_t R,
                        rmm_dtype dtype, void* ws, size_t ws_bytes, hipStream_t stream);
rmm_status rmsnorm_lora_ex(const void* X, const void* g, const void* W, const void* A,
                           const void* B, void* Y, float eps, int64_t M, int64_t N, int64_t K,
                           int64_t R, rmm_dtype dtype, rmm_variant variant, int splits, void* ws,
                           size_t ws_bytes, hipStream_t stream);
rmm_status rmm_lora_matmul(const void* X, const void* W, const void* A, const void* B, void* Y,
                           int64_t M, int64_t N, int64_t K, int64_t R, rmm_dtype dtype, void* ws,
                           size_t ws_bytes, hipStream_t stream);
size_t rmm_lora_workspace_bytes(rmm_dtype dtype, int64_t M, int64_t N, int64_t K, int64_t R,
                                rmm_variant variant, int splits);

/* QKNorm + attention, one query per batch-head (the QKNorm + Attention row of
 * the same page's benchmark table, "五、实验结果"; the page names the fusion
 * only, the reading is RMSNorm over the head dimension applied to the query
 * and to every cached key, then scaled dot-product attention, no mask):
 *
 *   qn = q / rms(q) * gq,  kn_s = k_s / rms(k_s) * gk,  rms(x) = sqrt(mean_d x^2 + eps)
 *   O  = sum_s softmax_s(qn . kn_s / sqrt(D)) v_s
 *
 * Layouts (row-major, packed, bf16 only): Q: BH x D (BH = batch x heads),
 * K and V: BH x S x D (key s of head h at (h*S + s)*D), gq, gk: D, O: BH x D.
 * The normalised keys are never formed: one pass over each key row
 * accumulates (q*gq*gk) . k_s and sum_d k_sd^2 in fp32, and the key's 1/RMS
 * scales the finished dot product; softmax in fp32 with a running maximum;
 * O rounded once to bf16.  D must be 64 or 128 and S >= 1 (RMM_ERR_SHAPE),
 * dtype RMM_DTYPE_BF16 (RMM_ERR_DTYPE), every pointer 16-byte aligned and
 * S*D*2 < 2^31 (RMM_ERR_VARIANT).  The keys of one batch-head are split
 * into chunks combined by the last workgroup to arrive (log-sum-exp merge of
 * (o, max, sum) partials); that needs a workspace (rules as above, sized by
 * rmm_attention_workspace_bytes); without one each batch-head runs in a
 * single workgroup.  splits (qknorm_attention_ex): chunks per batch-head,
 * 0 = chosen by the library, 1..S forced.  BH == 0 is a no-op. */
rmm_status qknorm_attention(const void* Q, const void* K, const void* V, const void* gq,
                            const void* gk, void* O, float eps, int64_t BH, int64_t S, int64_t D,
                            rmm_dtype dtype, void* ws, size_t ws_bytes, hipStream_t stream);
rmm_status qknorm_attention_ex(const void* Q, const void* K, const void* V, const void* gq,
                               const void* gk, void* O, float eps, int64_t BH, int64_t S,
                               int64_t D, rmm_dtype dtype, int splits, void* ws, size_t ws_bytes,
                               hipStream_t stream);
size_t rmm_attention_workspace_bytes(rmm_dtype dtype, int64_t BH, int64_t S, int64_t D,
                                     int splits);
/* Host-only: validates like qknorm_attention_ex and reports the chunk count
 * and keys per chunk that would run (either output may be NULL). */
rmm_status rmm_plan_attention(const void* Q, const void* K, const void* V, const void* gq,
                              const void* gk, const void* O, float eps, int64_t BH, int64_t S,
                              int64_t D, rmm_dtype dtype, int splits, const void* ws,
                              size_t ws_bytes, int* chunks_out, int64_t* keys_per_chunk_out);

/* Grouped-query form of qknorm_attention (several query heads per cached
 * key/value head, the layout of grouped-query attention; same reading of the
 * QKNorm + Attention row, "五、实验结果"): BH counts key/value heads, G in 1..16
 * query heads share each (RMM_ERR_SHAPE otherwise).  Q and O are (BH G) x D,
 * query row h G + g belonging to key/value head h; K and V are BH x S x D as
 * above.  One workgroup reads each key and value row once for the whole group
 * (every query's dot product, the key's sum of squares once); from G = 3 both
 * products run on the matrix cores, with q gq gk and the softmax weights each
 * carried as two bf16 parts (16 significant bits).  Other rules,
 * including the workspace (sized by rmm_attention_gqa_workspace_bytes) and
 * splits, are those of qknorm_attention_ex; G = 1 is qknorm_attention_ex. */
rmm_status qknorm_attention_gqa(const void* Q, const void* K, const void* V, const void* gq,
                                const void* gk, void* O, float eps, int64_t BH, int64_t G,
                                int64_t S, int64_t D, rmm_dtype dtype, int splits, void* ws,
                                size_t ws_bytes, hipStream_t stream);
size_t rmm_attention_gqa_workspace_bytes(rmm_dtype dtype, int64_t BH, int64_t G, int64_t S,
                                         int64_t D, int splits);
/* Host-only: validates like qknorm_attention_gqa and reports the chunk count
 * and keys per chunk that would run (either output may be NULL). */
rmm_status rmm_plan_attention_gqa(const void* Q, const void* K, const void* V, const void* gq,
                                  const void* gk, const void* O, float eps, int64_t BH, int64_t G,
                                  int64_t S, int64_t D, rmm_dtype dtype, int splits,
                                  const void* ws, size_t ws_bytes, int* chunks_out,
                                  int64_t* keys_per_chunk_out);

/* QKNorm + attention for many queries per head (prefill; same reading of the
 * QKNorm + Attention row, "五、实验结果"): every query row is normalised and
 * attends to its key/value head's normalised keys as in qknorm_attention.
 * Layouts (row-major, packed, bf16 only): Q and O: (BH G) x Sq x D (query
 * head h G + g, position i at ((h G + g) Sq + i) D), K and V: BH x Skv x D,
 * gq, gk: D.  causal != 0: query position i attends to keys 0 .. i + Skv -
 * Sq (the queries are the last Sq of the Skv positions; needs Skv >= Sq),
 * else to all Skv keys.  Both products run on the matrix cores, with q gq gk
 * and the softmax weights each carried as two bf16 parts (16 significant
 * bits); no workspace.  Errors: RMM_ERR_NULL, RMM_ERR_SHAPE (BH < 0, G < 1,
 * Sq or Skv < 1, D not 64 or 128, causal with Skv < Sq, element counts
 * overflowing), RMM_ERR_EPS, RMM_ERR_DTYPE (bf16 only), RMM_ERR_ALIAS (O
 * against any input), RMM_ERR_VARIANT (a pointer not 16-byte aligned, Skv D 2
 * >= 2^31).  BH == 0 is a no-op.  No split of the keys (see _ex). */
rmm_status qknorm_attention_prefill(const void* Q, const void* K, const void* V, const void* gq,
                                    const void* gk, void* O, float eps, int64_t BH, int64_t G,
                                    int64_t Sq, int64_t Skv, int64_t D, int causal,
                                    rmm_dtype dtype, hipStream_t stream);

/* As qknorm_attention_prefill with a split of the keys: splits spans of whole
 * 64-key tiles, each workgroup taking one span of one block of queries and
 * storing its raw (o, max, sum) in the workspace, a second kernel combining
 * the spans in order per query row (the log-sum-exp merge of the decode
 * form).  splits: 0 = chosen by the library (with a workspace: spans of at
 * least 512 keys, up to three workgroups per CU, when the query blocks alone
 * leave CUs idle; without one, no split), 1 = no split (no workspace), n > 1
 * forced (rounded to whole 64-key tiles, so the count that runs may be lower;
 * above ceil(Skv / 64): RMM_ERR_VARIANT; without a workspace:
 * RMM_ERR_WORKSPACE).  Workspace rules are those of rmsnorm_matmul, sized by
 * rmm_attention_prefill_workspace_bytes (same splits; 0 when no split runs);
 * O must not overlap it (RMM_ERR_ALIAS). */
rmm_status qknorm_attention_prefill_ex(const void* Q, const void* K, const void* V,
                                       const void* gq, const void* gk, void* O, float eps,
                                       int64_t BH, int64_t G, int64_t Sq, int64_t Skv, int64_t D,
                                       int causal, rmm_dtype dtype, int splits, void* ws,
                                       size_t ws_bytes, hipStream_t stream);
size_t rmm_attention_prefill_workspace_bytes(int64_t BH, int64_t G, int64_t Sq, int64_t Skv,
                                             int64_t D, int causal, int splits);

/* The attention step alone (the second kernel of the unfused QKNorm +
 * Attention program the same page's benchmark table compares against,
 * "五、实验结果"): Q and K arrive already normalised (rmsnorm over rows of
 * length D, one call for Q, one for K viewed as BH*S rows), and
 *
 *   O = sum_s softmax_s(q . k_s / sqrt(D)) v_s
 *
 * Layouts, dtype, alignment, size limits, workspace and error rules are
 * those of qknorm_attention (the chunk count is chosen by the library). */
rmm_status rmm_attention(const void* Q, const void* K, const void* V, void* O, int64_t BH,
                         int64_t S, int64_t D, rmm_dtype dtype, void* ws, size_t ws_bytes,
                         hipStream_t stream);

/* A chain of L fused layers in one persistent launch (the multi-layer
 * decode that the Mirage pages' persistent-kernel runtime, "Mirage
 * Persistent Kernel" on the first page, runs as one kernel):
 *   X_{l+1} = RMSNorm(X_l; g_l, eps) W_l,   l = 0 .. L-1,
 * each layer computed as rmsnorm_matmul computes it, the output of one
 * layer (rounded to bf16) being the input of the next.
 *   X0 : M x K          (layer-0 input)
 *   G  : L x K          (g_l = row l)
 *   W  : L x K x K      (W_l = W + l*K*K, K x K row-major: W_l[k*K + n])
 *   Xs : L x M x K      (output: Xs + l*M*K = X_{l+1}; every layer is kept)
 * bf16 only (else RMM_ERR_DTYPE); M <= 16, K a multiple of 128 small enough
 * that the decode tiling of a layer fits one resident workgroup per CU
 * (K <= 4096 on MI355X), 16-byte aligned pointers (else RMM_ERR_VARIANT).
 * One workgroup per CU at most (RMM_ERR_HIP with hipErrorInvalidConfiguration
 * if the device has fewer CUs than the tiling needs); every workgroup stays
 * resident and, before a layer, waits on device-side per-tile counters for
 * the tiles of the previous layer's output that its K chunk reads; half of
 * a layer's W loads are issued before that wait.  The call assumes no
 * other kernel holds CUs while it runs: a wait that gives up (bounded poll)
 * sets the flag word below and the results are then wrong.  A workspace is
 * required (RMM_ERR_WORKSPACE
 * if NULL or shorter than rmm_chain_workspace_bytes); zero-fill it before
 * first use; the kernel leaves its counters zeroed.  The 32-bit word at byte
 * offset ws + rmm_chain_flag_offset(M, K, L) becomes nonzero if a layer
 * wait ever gave up (a grid that was not resident); it is never cleared by
 * the library.  Xs must not overlap X0, G, W or the workspace.  M == 0 is a
 * no-op. */
rmm_status rmsnorm_matmul_chain(const void* X0, const void* G, const void* W, void* Xs, float eps,
                                int64_t M, int64_t K, int64_t L, rmm_dtype dtype, void* ws,
                                size_t ws_bytes, hipStream_t stream);
/* Workspace bytes of the chain call (0 for arguments it rejects). */
size_t rmm_chain_workspace_bytes(int64_t M, int64_t K, int64_t L);
/* Byte offset of the flag word in the chain workspace (0 for rejected arguments). */
size_t rmm_chain_flag_offset(int64_t M, int64_t K, int64_t L);

/* Workspace bytes the call with these arguments would use (0 if none).  The
 * plain entry points use variant = AUTO, splits = 0.  Returns 0 for
 * arguments that would fail validation. */
size_t rmm_workspace_bytes(rmm_dtype dtype, int64_t M, int64_t N, int64_t K, int gated);
size_t rmm_workspace_bytes_ex(rmm_dtype dtype, int64_t M, int64_t N, int64_t K, int gated,
                              rmm_variant variant, int splits);

/* Host-only planning, no HIP call: validates the arguments exactly as the
 * entry points do (pointer values are only compared, never dereferenced) and
 * reports the variant and split count that would run.  *variant_out and
 * *splits_out may be NULL. */
rmm_status rmm_plan(const void* X, const void* g, const void* W1, const void* W3, const void* Y,
                    float eps, int64_t M, int64_t N, int64_t K, rmm_dtype dtype, int gated,
                    rmm_variant variant, int splits, const void* ws, size_t ws_bytes,
                    rmm_variant* variant_out, int* splits_out);

/* rmm_plan for the adapter entry points (A, B, R as in rmsnorm_lora). */
rmm_status rmm_plan_lora(const void* X, const void* g, const void* W, const void* A,
                         const void* B, const void* Y, float eps, int64_t M, int64_t N, int64_t K,
                         int64_t R, rmm_dtype dtype, rmm_variant variant, int splits,
                         const void* ws, size_t ws_bytes, rmm_variant* variant_out,
                         int* splits_out);

/* Measurement probes (not part of the operation): the two ceilings this
 * part sustains, against which the kernels' roofline fractions are also
 * stated besides the published peaks.
 *   rmm_probe_hbm_read: reads `bytes` (a multiple of 16, > 0) from the device
 *     buffer `src` (16-byte aligned) once, linearly, with 16-byte loads; the
 *     4-byte device word `sink` is written only if the folded data hits one
 *     fixed pattern (in practice never).  Time it to get the achievable read
 *     bandwidth; pass a buffer far larger than the 256 MB last-level cache.
 *   rmm_probe_mfma_bf16: a dense loop of iters x 4 dependent-chain
 *     v_mfma_f32_32x32x16_bf16 per wave over two waves per SIMD of 256 CUs;
 *     rmm_probe_mfma_flops(iters) is the flop count of one launch (0 for
 *     iters outside 1..2^40).  `sink` as above (a 4-byte device word).
 * Errors: RMM_ERR_NULL, RMM_ERR_SHAPE (bytes or iters), RMM_ERR_VARIANT
 * (unaligned src), RMM_ERR_HIP.  Stream ordered, like every call here. */
rmm_status rmm_probe_hbm_read(const void* src, size_t bytes, void* sink, hipStream_t stream);
rmm_status rmm_probe_mfma_bf16(int64_t iters, void* sink, hipStream_t stream);
int64_t rmm_probe_mfma_flops(int64_t iters);

const char* rmm_status_string(rmm_status s);
int rmm_last_hip_error(void);
int rmm_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RMM_H */
