// C ABI of the fused RMSNorm+MatMul library: host-side validation, variant
// selection and launch.  Validation runs before any HIP call, so every error
// path can be exercised on a machine without a GPU.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "rmm.h"
#include "rmm_device.h"

namespace {

thread_local int g_last_hip_error = 0;

}  // namespace

void rmm_set_last_hip_error(int err) { g_last_hip_error = err; }

namespace {

struct Plan {
  rmm_variant variant;
  int splits;
  size_t ws_bytes;
  DecodePlan dec;
  Decode32Plan d32;
  PrefillPlan pre;
  StreamPlan st;
};

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool overlaps(const void* a, size_t an, const void* b, size_t bn) {
  if (!a || !b || an == 0 || bn == 0) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + bn && b0 < a0 + an;
}

// Decode: few rows.  The split count is the largest power of two that keeps
// the grid at one workgroup per CU (256 CUs): more splits add partial-sum
// traffic and lengthen the combine that the last arriving workgroup of each
// tile does alone, and measured fastest at this size.
constexpr int64_t kDecodeMaxM = 32;
// With the adapter (no other fast kernel takes it) up to 128 rows run as
// one decode launch per 32-row block.
constexpr int64_t kDecodeMaxMLora = 128;
constexpr int64_t kDecodeMaxMGated = 16;
// fp32 decode: plain calls only; 16 rows per launch, up to 32 rows as two
// launches (32 x 1024 x 1024: ~23 us against 40 us for the generic kernel;
// three launches for 48 rows no longer beat it at 4096 x 4096).
constexpr int64_t kDecodeRowsF32 = 16;
constexpr int64_t kDecodeMaxMF32 = 32;
constexpr int64_t kTargetWorkgroups = 256;
// Stream: up to 64 rows; auto-selected for plain calls only when there are
// enough 64-column strips to keep most CUs streaming.
// The stream kernel computes 64 rows; up to 128 rows (256 when N <= 4096)
// run as one launch per 64-row block, each reading W again, which still
// beats one row of 256 x 256 prefill tiles there (K = 4096, M = 256:
// N = 2048 69.6 us, N = 4096 85.0 us, against 111-112 us).
constexpr int64_t kStreamRows = 64;
constexpr int64_t kStreamMaxM = 128;
// Gated calls: 64-row stream launches up to 64 rows with a workspace (to
// 128 without one), the gated prefill tile above (with a workspace, its K
// split).  Measured, 96 and 128 rows: K = 4096, N = 14336 70-75 us against
// 98; N = 4096 34-39 against 55; K = 14336, N = 4096 69-75 against 121-127.
// At 32-64 rows the two are within a few percent, the stream kernel ahead at
// N = 14336 (55.5 against 68.5 us at 64 rows).
constexpr int64_t kGatedStreamMaxM = 128;
constexpr int64_t kGatedStreamMaxMWs = 64;
// Adapter calls with a workspace: the decode kernel (32-row launches) up to
// 64 rows, the prefill tile's K split above (6144 x 4096, R = 16: 96 rows
// 46 against 64 us, 128 rows 47 against 85; 64 rows 44.5 against 43).
constexpr int64_t kLoraDecodeMaxMWs = 64;
// Low-rank adapter: ranks 1..RMM_LORA_MAX_RANK; the decode kernel carries up
// to two 16-wide rank blocks, every other shape runs the generic kernel.
constexpr int64_t kLoraDecodeMaxRank = 32;

// fp32 decode: 128-column tiles, each K range at least 64 rows, about as
// many workgroups as fit at once (two per CU with 8-row blocks, one with
// 16: the accumulators of 16 rows leave room for one per SIMD).  Measured:
// 8 x 14336 x 4096 57 us with 4 ranges (448 workgroups) against 86 us with
// 2; 16 x 4096 x 4096 36 us with 8 ranges against 48 us with 16.
int auto_decode32_splits(int64_t M, int64_t N, int64_t K) {
  const int64_t tiles = (N + 127) / 128;
  const int64_t target = M <= 8 ? 2 * kTargetWorkgroups : kTargetWorkgroups;
  int64_t s = target / (tiles > 0 ? tiles : 1);
  const int64_t smax = (K + 63) / 64;
  if (s > smax) s = smax;
  return (int)(s < 1 ? 1 : s);
}

int auto_decode_splits(int64_t N, int64_t K) {
  const int64_t tiles = (N + 127) / 128;
  if (tiles < 1) return 1;
  const int64_t kgran = (K + 127) / 128;
  int64_t s = 1;
  while (2 * s * tiles <= kTargetWorkgroups && 2 * s <= kgran) s *= 2;
  return (int)s;
}

// Shape/variant part of the plan; `aligned` says whether every pointer is
// 16-byte aligned, `have_ws` whether a workspace was passed, `ws_avail` its
// size (SIZE_MAX when only sizes are asked for): the library's choice of a
// prefill split keeps its partial sums within it.
rmm_status plan_shape(int64_t M, int64_t N, int64_t K, rmm_dtype dtype, int gated,
                      rmm_variant variant, int splits, bool aligned, bool have_ws, Plan* out,
                      int64_t R = 0, size_t ws_avail = SIZE_MAX) {
  if (variant < RMM_VARIANT_AUTO || variant > RMM_VARIANT_STREAM) return RMM_ERR_VARIANT;
  if (splits < 0) return RMM_ERR_VARIANT;
  if (splits != 0 && variant != RMM_VARIANT_DECODE && variant != RMM_VARIANT_PREFILL)
    return RMM_ERR_VARIANT;
  if (M == 0 || N == 0) {  // nothing to compute, nothing launched
    out->variant = variant == RMM_VARIANT_AUTO ? RMM_VARIANT_GENERIC : variant;
    out->splits = 1;
    out->ws_bytes = 0;
    return RMM_OK;
  }
  // The fast variants address X and W with 32-bit buffer offsets.
  const bool fast_layout = dtype == RMM_DTYPE_BF16 && K % 8 == 0 && N % 8 == 0 && aligned &&
                           K * N * 2 <= (int64_t)INT32_MAX && M * K * 2 <= (int64_t)INT32_MAX;
  // With the adapter: 32-bit offsets into A as well (rank rows up to 32).
  const bool lora_ok = R == 0 || (R <= kLoraDecodeMaxRank && kLoraDecodeMaxRank * K * 2 <= (int64_t)INT32_MAX &&
                                  R * N * 2 <= (int64_t)INT32_MAX);
  const bool f32 = dtype == RMM_DTYPE_F32;
  const bool decode32_ok = f32 && aligned && N % 4 == 0 && !gated && R == 0 && M <= kDecodeMaxMF32;
  const bool decode_ok = (fast_layout && lora_ok &&
                          M <= (gated ? kDecodeMaxMGated : (R > 0 ? kDecodeMaxMLora : kDecodeMaxM))) ||
                         decode32_ok;
  // The adapter's prefill tile: T = (X g) A^T goes through the workspace;
  // A's and B's rows are addressed with 32-bit offsets.
  const bool lora_prefill_ok = R > 0 && !gated && R <= RMM_LORA_MAX_RANK &&
                               R * K * 2 <= (int64_t)INT32_MAX && R * N * 2 <= (int64_t)INT32_MAX;
  const bool prefill_ok = fast_layout && (R == 0 || lora_prefill_ok);
  const bool stream_ok = fast_layout && R == 0 &&
                         (gated || M <= kStreamMaxM || (M <= 256 && N <= 4096)) &&
                         rmm_stream_fits(M < kStreamRows ? M : kStreamRows, N, K);
  rmm_variant v = variant;
  if (v == RMM_VARIANT_AUTO) {
    if (R > 0)
      v = (decode_ok && (M <= kLoraDecodeMaxMWs || !have_ws)) ? RMM_VARIANT_DECODE
          : (prefill_ok && have_ws)                           ? RMM_VARIANT_PREFILL
          : decode_ok                                         ? RMM_VARIANT_DECODE
                                                              : RMM_VARIANT_GENERIC;
    else if (gated)  // decode (split-K over every CU) only with a workspace for its partials
      v = (decode_ok && have_ws) ? RMM_VARIANT_DECODE
          : (stream_ok && M <= (have_ws ? kGatedStreamMaxMWs : kGatedStreamMaxM))
              ? RMM_VARIANT_STREAM
          : prefill_ok ? RMM_VARIANT_PREFILL
          : stream_ok  ? RMM_VARIANT_STREAM
                       : RMM_VARIANT_GENERIC;
    else if (decode_ok)
      v = RMM_VARIANT_DECODE;
    else if (stream_ok && (M <= kStreamRows || !have_ws))
      v = RMM_VARIANT_STREAM;  // far faster than one row of unsplit 256 x 256 prefill tiles
    else if (prefill_ok)       // above 64 rows with a workspace: the prefill split
      v = RMM_VARIANT_PREFILL;
    else
      v = stream_ok ? RMM_VARIANT_STREAM : RMM_VARIANT_GENERIC;
  }
  if (v == RMM_VARIANT_DECODE && !decode_ok) return RMM_ERR_VARIANT;
  if (v == RMM_VARIANT_PREFILL && !prefill_ok) return RMM_ERR_VARIANT;
  if (v == RMM_VARIANT_STREAM && !stream_ok) return RMM_ERR_VARIANT;
  out->variant = v;
  out->splits = 1;
  out->ws_bytes = 0;
  if (v == RMM_VARIANT_DECODE && f32) {
    int s = splits;
    const int64_t rows = M < kDecodeRowsF32 ? M : kDecodeRowsF32;  // rows per launch
    if (s == 0) s = have_ws ? auto_decode32_splits(rows, N, K) : 1;
    if (s > (K + 63) / 64 && s > 1) return RMM_ERR_VARIANT;
    if (s > 1 && !have_ws) return RMM_ERR_WORKSPACE;  // a forced split count needs one
    rmm_decode32_plan(M, N, K, s, &out->d32);
    if (out->d32.ws_bytes > (size_t)INT32_MAX) return RMM_ERR_VARIANT;  // 32-bit offsets
    if (out->d32.splits > 1 && out->d32.tiles > kWsMaxCounters) return RMM_ERR_VARIANT;
    out->splits = out->d32.splits;
    out->ws_bytes = out->d32.ws_bytes;
  } else if (v == RMM_VARIANT_DECODE) {
    int s = splits;
    if (s == 0) s = have_ws ? auto_decode_splits(N, K) : 1;
    if (s > (K + 127) / 128) return RMM_ERR_VARIANT;
    if (s > 1 && !have_ws) return RMM_ERR_WORKSPACE;  // a forced split count needs one
    rmm_decode_plan(M < kDecodeMaxM ? M : kDecodeMaxM, N, K, gated, s, R, &out->dec);
    if (out->dec.ws_bytes > (size_t)INT32_MAX) return RMM_ERR_VARIANT;  // 32-bit offsets
    // one arrival counter per tile, all in the workspace's counter region
    if (out->dec.splits > 1 && out->dec.tiles > kWsMaxCounters) return RMM_ERR_VARIANT;
    out->splits = out->dec.splits;
    out->ws_bytes = out->dec.ws_bytes;
  } else if (v == RMM_VARIANT_PREFILL) {
    if (splits > (K + 63) / 64) return RMM_ERR_VARIANT;
    // a forced split count, and the adapter's T, need one
    if ((splits > 1 || R > 0) && !have_ws) return RMM_ERR_WORKSPACE;
    rmm_prefill_plan(M, N, K, gated, splits, have_ws ? ws_avail : 0, &out->pre, R);
    if (out->pre.ws_bytes > (size_t)INT32_MAX) return RMM_ERR_VARIANT;
    out->splits = out->pre.splits;
    out->ws_bytes = out->pre.ws_bytes;
  } else if (v == RMM_VARIANT_STREAM) {
    rmm_stream_plan(N, K, gated, (int)kTargetWorkgroups, have_ws, &out->st);
    if (out->st.ws_bytes > (size_t)INT32_MAX) return RMM_ERR_VARIANT;  // 32-bit offsets
    out->ws_bytes = out->st.split ? out->st.ws_bytes : 0;
  }
  return RMM_OK;
}

// R < 0: no adapter; R >= 0: the adapter entry points (R must be 1..max).
rmm_status plan_call(const void* X, const void* g, const void* W1, const void* W3, const void* Y,
                     float eps, int64_t M, int64_t N, int64_t K, rmm_dtype dtype, int gated,
                     rmm_variant variant, int splits, const void* ws, size_t ws_bytes, Plan* out,
                     const void* LA = nullptr, const void* LB = nullptr, int64_t R = -1) {
  const bool lora = R >= 0;
  // 1. pointers
  const bool empty = (M == 0 || N == 0);
  if (!empty && (!X || !g || !W1 || !Y || (gated && !W3) || (lora && (!LA || !LB))))
    return RMM_ERR_NULL;
  // 2. shape
  if (M < 0 || N < 0 || K <= 0) return RMM_ERR_SHAPE;
  if (lora && (R < 1 || R > RMM_LORA_MAX_RANK)) return RMM_ERR_SHAPE;
  int64_t mk, kn, mn, tmp;
  if (__builtin_mul_overflow(M, K, &mk) || __builtin_mul_overflow(K, N, &kn) ||
      __builtin_mul_overflow(M, N, &mn) || __builtin_mul_overflow(mk, (int64_t)4, &tmp) ||
      __builtin_mul_overflow(kn, (int64_t)4, &tmp) || __builtin_mul_overflow(mn, (int64_t)4, &tmp))
    return RMM_ERR_SHAPE;
  const int64_t rank = lora ? R : 0;  // R * K and R * N fit: R <= 64 and K * 4, N * 4 fit
  // 3. eps
  if (!isfinite(eps) || eps < 0.0f) return RMM_ERR_EPS;
  // 4. dtype
  if (dtype != RMM_DTYPE_F32 && dtype != RMM_DTYPE_BF16) return RMM_ERR_DTYPE;
  const size_t es = dtype == RMM_DTYPE_F32 ? 4 : 2;
  // 5. aliasing of the output with the inputs and the workspace
  if (!empty) {
    const size_t yb = (size_t)mn * es;
    if (overlaps(Y, yb, X, (size_t)mk * es) || overlaps(Y, yb, g, (size_t)K * es) ||
        overlaps(Y, yb, W1, (size_t)kn * es) || (gated && overlaps(Y, yb, W3, (size_t)kn * es)) ||
        overlaps(Y, yb, ws, ws ? ws_bytes : 0) ||
        (lora && (overlaps(Y, yb, LA, (size_t)(rank * K) * es) ||
                  overlaps(Y, yb, LB, (size_t)(rank * N) * es))))
      return RMM_ERR_ALIAS;
  }
  // 6. variant (and the split count it would use)
  const bool aligned = empty || (aligned16(X) && aligned16(g) && aligned16(W1) &&
                                 (!gated || aligned16(W3)) && aligned16(Y) &&
                                 (!lora || (aligned16(LA) && aligned16(LB))));
  rmm_status st =
      plan_shape(M, N, K, dtype, gated, variant, splits, aligned, ws != nullptr, out, rank,
                 ws ? ws_bytes : 0);
  if (st != RMM_OK) return st;
  // 7. workspace (its partial sums are read and written 16 bytes at a time)
  if (ws && (ws_bytes < out->ws_bytes || !aligned16(ws))) return RMM_ERR_WORKSPACE;
  return RMM_OK;
}

rmm_status run(const void* X, const void* g, const void* W1, const void* W3, void* Y, float eps,
               int64_t M, int64_t N, int64_t K, rmm_dtype dtype, int gated, rmm_variant variant,
               int splits, void* ws, size_t ws_bytes, hipStream_t stream, int norm = 1,
               const void* LA = nullptr, const void* LB = nullptr, int64_t R = -1) {
  Plan plan;
  rmm_status st = plan_call(X, g, W1, W3, Y, eps, M, N, K, dtype, gated, variant, splits, ws,
                            ws_bytes, &plan, LA, LB, R);
  if (st != RMM_OK) return st;
  if (M == 0 || N == 0) return RMM_OK;
  RmmArgs a{X, g, W1, gated ? W3 : nullptr, Y, eps, M, N, K, gated, norm, stream};
  if (R > 0) {
    a.LA = LA;
    a.LB = LB;
    a.R = R;
  }
  hipError_t err = hipSuccess;
  switch (plan.variant) {
    case RMM_VARIANT_GENERIC:
      err = rmm_launch_generic(a, dtype == RMM_DTYPE_BF16);
      break;
    case RMM_VARIANT_DECODE:
      if (dtype == RMM_DTYPE_F32)
        // Row blocks of 16, in order on the stream (each leaves the split
        // counters cleared for the next).
        for (int64_t r0 = 0; r0 < a.M && err == hipSuccess; r0 += kDecodeRowsF32) {
          RmmArgs b = a;
          b.X = (const float*)a.X + r0 * a.K;
          b.Y = (float*)a.Y + r0 * a.N;
          b.M = a.M - r0 < kDecodeRowsF32 ? a.M - r0 : kDecodeRowsF32;
          err = rmm_launch_decode32(b, plan.d32, plan.d32.splits > 1 ? ws : nullptr);
        }
      else
        // Row blocks of 32 (only calls with the adapter have more rows), in
        // order on the stream (each leaves the split counters cleared).
        for (int64_t r0 = 0; r0 < a.M && err == hipSuccess; r0 += kDecodeMaxM) {
          RmmArgs b = a;
          b.X = (const char*)a.X + r0 * a.K * 2;
          b.Y = (char*)a.Y + r0 * a.N * 2;
          b.M = a.M - r0 < kDecodeMaxM ? a.M - r0 : kDecodeMaxM;
          err = rmm_launch_decode(b, plan.dec, plan.dec.splits > 1 ? ws : nullptr);
        }
      break;
    case RMM_VARIANT_PREFILL:
      err = rmm_launch_prefill(a, plan.pre, plan.pre.ws_bytes > 0 ? ws : nullptr);
      break;
    case RMM_VARIANT_STREAM:
      // Row blocks of 64, in order on the stream (the split form's workspace
      // is left ready for the next launch by the one before).
      for (int64_t r0 = 0; r0 < a.M && err == hipSuccess; r0 += kStreamRows) {
        RmmArgs b = a;
        b.X = (const char*)a.X + r0 * a.K * 2;
        b.Y = (char*)a.Y + r0 * a.N * 2;
        b.M = a.M - r0 < kStreamRows ? a.M - r0 : kStreamRows;
        err = rmm_launch_stream(b, plan.st, plan.st.split ? ws : nullptr);
      }
      break;
    default:
      return RMM_ERR_VARIANT;
  }
  if (err != hipSuccess) {
    g_last_hip_error = (int)err;
    return RMM_ERR_HIP;
  }
  return RMM_OK;
}

// QKNorm + attention: validation in the documented order, then the plan.
// G: query heads per key/value head (BH counts key/value heads).
rmm_status attn_plan_call(const void* Q, const void* K, const void* V, const void* gq,
                          const void* gk, const void* O, float eps, int64_t BH, int64_t S,
                          int64_t D, rmm_dtype dtype, int splits, const void* ws, size_t ws_bytes,
                          AttnPlan* plan, int64_t G = 1) {
  // 1. pointers
  if (BH > 0 && (!Q || !K || !V || !gq || !gk || !O)) return RMM_ERR_NULL;
  // 2. shape: head dimension 64 or 128, at least one key, 1..16 queries per head
  if (BH < 0 || S < 1 || (D != 64 && D != 128) || G < 1 || G > 16) return RMM_ERR_SHAPE;
  int64_t sd, bhsd, tmp;
  if (__builtin_mul_overflow(S, D, &sd) || __builtin_mul_overflow(BH, sd, &bhsd) ||
      __builtin_mul_overflow(bhsd, (int64_t)2, &tmp) ||
      __builtin_mul_overflow(BH * G * D, (int64_t)2, &tmp))
    return RMM_ERR_SHAPE;
  // 3. eps
  if (!isfinite(eps) || eps < 0.0f) return RMM_ERR_EPS;
  // 4. dtype: this path stores bf16 only
  if (dtype != RMM_DTYPE_BF16) return RMM_ERR_DTYPE;
  if (BH == 0) {
    plan->chunks = 1;
    plan->kchunk = S;
    plan->ws_bytes = 0;
    return RMM_OK;
  }
  // 5. aliasing of the output
  const size_t ob = (size_t)(BH * G * D) * 2;
  if (overlaps(O, ob, Q, ob) || overlaps(O, ob, K, (size_t)bhsd * 2) ||
      overlaps(O, ob, V, (size_t)bhsd * 2) || overlaps(O, ob, gq, (size_t)D * 2) ||
      overlaps(O, ob, gk, (size_t)D * 2) || overlaps(O, ob, ws, ws ? ws_bytes : 0))
    return RMM_ERR_ALIAS;
  // 6. what the kernel can run: 16-byte aligned operands, 32-bit offsets
  // within one batch-head's keys, a split count between 1 and S
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(gq) || !aligned16(gk) ||
      !aligned16(O))
    return RMM_ERR_VARIANT;
  if (sd * 2 > (int64_t)INT32_MAX || splits < 0 || splits > S) return RMM_ERR_VARIANT;
  const int s = splits == 0 ? (ws ? 0 : 1) : splits;
  if (s > 1 && !ws) return RMM_ERR_WORKSPACE;
  rmm_attention_plan(BH, S, D, s, plan, G);
  if ((int64_t)plan->chunks * BH > (int64_t)INT32_MAX || plan->ws_bytes > (size_t)INT32_MAX)
    return RMM_ERR_VARIANT;
  // one arrival counter per batch-head, all in the workspace's counter region
  if (plan->chunks > 1 && BH > kWsMaxCounters) return RMM_ERR_VARIANT;
  // 7. workspace (its partial sums are read and written 16 bytes at a time)
  if (ws && (ws_bytes < plan->ws_bytes || !aligned16(ws))) return RMM_ERR_WORKSPACE;
  return RMM_OK;
}

// The adapter entry points pass their rank through this: internally R < 0
// means "no adapter", so a negative rank from a caller becomes 0, which
// fails the rank check like any other rank outside 1..64.
int64_t lora_rank_arg(int64_t R) { return R < 0 ? 0 : R; }

// Chain validation: NULL, shape, eps, dtype, alias, tiling, workspace.
rmm_status chain_plan_call(const void* X0, const void* G, const void* W, const void* Xs, float eps,
                           int64_t M, int64_t K, int64_t L, rmm_dtype dtype, const void* ws,
                           size_t ws_bytes, ChainPlan* plan) {
  if (M != 0 && (!X0 || !G || !W || !Xs)) return RMM_ERR_NULL;
  if (M < 0 || K <= 0 || L < 1) return RMM_ERR_SHAPE;
  int64_t mk, kk, lkk, lmk, lk, tmp;
  if (__builtin_mul_overflow(M, K, &mk) || __builtin_mul_overflow(K, K, &kk) ||
      __builtin_mul_overflow(L, kk, &lkk) || __builtin_mul_overflow(L, mk, &lmk) ||
      __builtin_mul_overflow(L, K, &lk) || __builtin_mul_overflow(lkk, (int64_t)2, &tmp) ||
      __builtin_mul_overflow(lmk, (int64_t)2, &tmp))
    return RMM_ERR_SHAPE;
  if (!isfinite(eps) || eps < 0.0f) return RMM_ERR_EPS;
  if (dtype != RMM_DTYPE_BF16) return RMM_ERR_DTYPE;
  if (M == 0) return RMM_OK;
  const size_t xsb = (size_t)lmk * 2;
  if (overlaps(Xs, xsb, X0, (size_t)mk * 2) || overlaps(Xs, xsb, G, (size_t)lk * 2) ||
      overlaps(Xs, xsb, W, (size_t)lkk * 2) || overlaps(Xs, xsb, ws, ws ? ws_bytes : 0))
    return RMM_ERR_ALIAS;
  if (M > 16 || K % 128 != 0 || kk * 2 > (int64_t)INT32_MAX ||
      !(aligned16(X0) && aligned16(G) && aligned16(W) && aligned16(Xs)))
    return RMM_ERR_VARIANT;
  if (rmm_chain_plan(M, K, L, plan) != 0) return RMM_ERR_VARIANT;  // not one workgroup per CU
  if (!ws || ws_bytes < plan->ws_bytes || !aligned16(ws)) return RMM_ERR_WORKSPACE;
  return RMM_OK;
}

// qknorm_attention_prefill(_ex): validation in the documented order, then
// the plan (query blocks per wave, key tiles, the split of the keys).
rmm_status prefill_attn_plan_call(const void* Q, const void* K, const void* V, const void* gq,
                                  const void* gk, const void* O, float eps, int64_t BH,
                                  int64_t G, int64_t Sq, int64_t Skv, int64_t D, int causal,
                                  rmm_dtype dtype, int splits, const void* ws, size_t ws_bytes,
                                  AttnPrefillPlan* plan) {
  // 1. pointers
  if (BH > 0 && (!Q || !K || !V || !gq || !gk || !O)) return RMM_ERR_NULL;
  // 2. shape
  if (BH < 0 || G < 1 || Sq < 1 || Skv < 1 || (D != 64 && D != 128) || (causal && Skv < Sq))
    return RMM_ERR_SHAPE;
  int64_t bhg, qn, kn, tmp;
  if (__builtin_mul_overflow(BH, G, &bhg) || __builtin_mul_overflow(bhg, Sq * D, &qn) ||
      __builtin_mul_overflow(Sq, D, &tmp) || __builtin_mul_overflow(BH, Skv * D, &kn) ||
      __builtin_mul_overflow(Skv, D, &tmp) || __builtin_mul_overflow(qn, (int64_t)2, &tmp) ||
      __builtin_mul_overflow(kn, (int64_t)2, &tmp))
    return RMM_ERR_SHAPE;
  // 3. eps
  if (!isfinite(eps) || eps < 0.0f) return RMM_ERR_EPS;
  // 4. dtype
  if (dtype != RMM_DTYPE_BF16) return RMM_ERR_DTYPE;
  if (BH == 0) return RMM_OK;
  // 5. aliasing of the output
  const size_t ob = (size_t)qn * 2;
  if (overlaps(O, ob, Q, ob) || overlaps(O, ob, K, (size_t)kn * 2) ||
      overlaps(O, ob, V, (size_t)kn * 2) || overlaps(O, ob, gq, (size_t)D * 2) ||
      overlaps(O, ob, gk, (size_t)D * 2) || overlaps(O, ob, ws, ws ? ws_bytes : 0))
    return RMM_ERR_ALIAS;
  // 6. what the kernel can run: 16-byte aligned operands, 32-bit offsets
  // within one head's keys, one workgroup per 64 positions of a query head
  // and key span, spans of whole 64-key tiles
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(gq) || !aligned16(gk) ||
      !aligned16(O))
    return RMM_ERR_VARIANT;
  if (Skv * D * 2 > (int64_t)INT32_MAX || G > (int64_t)INT32_MAX || splits < 0 ||
      splits > (Skv + 63) / 64)
    return RMM_ERR_VARIANT;
  rmm_attention_prefill_plan(bhg, Sq, Skv, D, causal ? 1 : 0, splits, ws != nullptr, plan);
  if (bhg * plan->nblk * plan->splits > (int64_t)INT32_MAX) return RMM_ERR_VARIANT;
  // 7. workspace
  if (plan->splits > 1 && !ws) return RMM_ERR_WORKSPACE;  // a forced split count needs one
  if (ws && (ws_bytes < plan->ws_bytes || !aligned16(ws))) return RMM_ERR_WORKSPACE;
  return RMM_OK;
}

}  // namespace

size_t rmm_workspace_bytes_within(int dtype, int64_t M, int64_t N, int64_t K, int gated,
                                  size_t cap) {
  if (M < 0 || N < 0 || K <= 0) return 0;
  if (dtype != RMM_DTYPE_F32 && dtype != RMM_DTYPE_BF16) return 0;
  Plan plan;
  if (plan_shape(M, N, K, (rmm_dtype)dtype, gated ? 1 : 0, RMM_VARIANT_AUTO, 0, true, true, &plan,
                 0, cap) !=
      RMM_OK)
    return 0;
  return plan.ws_bytes;
}

extern "C" {

rmm_status rmsnorm_matmul(const void* X, const void* g, const void* W, void* Y, float eps,
                          int64_t M, int64_t N, int64_t K, rmm_dtype dtype, void* ws,
                          size_t ws_bytes, hipStream_t stream) {
  return run(X, g, W, nullptr, Y, eps, M, N, K, dtype, 0, RMM_VARIANT_AUTO, 0, ws, ws_bytes,
             stream);
}

rmm_status rmsnorm_gated_mlp(const void* X, const void* g, const void* W1, const void* W3,
                             void* Y, float eps, int64_t M, int64_t N, int64_t K,
                             rmm_dtype dtype, void* ws, size_t ws_bytes, hipStream_t stream) {
  return run(X, g, W1, W3, Y, eps, M, N, K, dtype, 1, RMM_VARIANT_AUTO, 0, ws, ws_bytes, stream);
}

rmm_status rmsnorm_matmul_ex(const void* X, const void* g, const void* W, void* Y, float eps,
                             int64_t M, int64_t N, int64_t K, rmm_dtype dtype,
                             rmm_variant variant, int splits, void* ws, size_t ws_bytes,
                             hipStream_t stream) {
  return run(X, g, W, nullptr, Y, eps, M, N, K, dtype, 0, variant, splits, ws, ws_bytes, stream);
}

rmm_status rmsnorm_gated_mlp_ex(const void* X, const void* g, const void* W1, const void* W3,
                                void* Y, float eps, int64_t M, int64_t N, int64_t K,
                                rmm_dtype dtype, rmm_variant variant, int splits, void* ws,
                                size_t ws_bytes, hipStream_t stream) {
  return run(X, g, W1, W3, Y, eps, M, N, K, dtype, 1, variant, splits, ws, ws_bytes, stream);
}

rmm_status rmm_matmul(const void* X, const void* W, void* Y, int64_t M, int64_t N, int64_t K,
                      rmm_dtype dtype, void* ws, size_t ws_bytes, hipStream_t stream) {
  // The kernels take the gain from X's buffer and ignore it (norm = 0).
  return run(X, X, W, nullptr, Y, 0.0f, M, N, K, dtype, 0, RMM_VARIANT_AUTO, 0, ws, ws_bytes,
             stream, 0);
}

rmm_status rmm_gated_matmul(const void* X, const void* W1, const void* W3, void* Y, int64_t M,
                            int64_t N, int64_t K, rmm_dtype dtype, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
  return run(X, X, W1, W3, Y, 0.0f, M, N, K, dtype, 1, RMM_VARIANT_AUTO, 0, ws, ws_bytes, stream,
             0);
}

rmm_status rmsnorm_lora(const void* X, const void* g, const void* W, const void* A, const void* B,
                        void* Y, float eps, int64_t M, int64_t N, int64_t K, int64_t R,
                        rmm_dtype dtype, void* ws, size_t ws_bytes, hipStream_t stream) {
  return run(X, g, W, nullptr, Y, eps, M, N, K, dtype, 0, RMM_VARIANT_AUTO, 0, ws, ws_bytes,
             stream, 1, A, B, lora_rank_arg(R));
}

rmm_status rmsnorm_lora_ex(const void* X, const void* g, const void* W, const void* A,
                           const void* B, void* Y, float eps, int64_t M, int64_t N, int64_t K,
                           int64_t R, rmm_dtype dtype, rmm_variant variant, int splits, void* ws,
                           size_t ws_bytes, hipStream_t stream) {
  return run(X, g, W, nullptr, Y, eps, M, N, K, dtype, 0, variant, splits, ws, ws_bytes, stream, 1,
             A, B, lora_rank_arg(R));
}

rmm_status rmm_lora_matmul(const void* X, const void* W, const void* A, const void* B, void* Y,
                           int64_t M, int64_t N, int64_t K, int64_t R, rmm_dtype dtype, void* ws,
                           size_t ws_bytes, hipStream_t stream) {
  return run(X, X, W, nullptr, Y, 0.0f, M, N, K, dtype, 0, RMM_VARIANT_AUTO, 0, ws, ws_bytes,
             stream, 0, A, B, lora_rank_arg(R));
}

rmm_status qknorm_attention_ex(const void* Q, const void* K, const void* V, const void* gq,
                               const void* gk, void* O, float eps, int64_t BH, int64_t S,
                               int64_t D, rmm_dtype dtype, int splits, void* ws, size_t ws_bytes,
                               hipStream_t stream) {
  AttnPlan plan;
  const rmm_status st =
      attn_plan_call(Q, K, V, gq, gk, O, eps, BH, S, D, dtype, splits, ws, ws_bytes, &plan);
  if (st != RMM_OK || BH == 0) return st;
  const AttnArgs a{Q, K, V, gq, gk, O, eps, BH, S, D, stream, 1, 1};
  const hipError_t err = rmm_launch_attention(a, plan, plan.chunks > 1 ? ws : nullptr);
  if (err != hipSuccess) {
    g_last_hip_error = (int)err;
    return RMM_ERR_HIP;
  }
  return RMM_OK;
}

rmm_status qknorm_attention(const void* Q, const void* K, const void* V, const void* gq,
                            const void* gk, void* O, float eps, int64_t BH, int64_t S, int64_t D,
                            rmm_dtype dtype, void* ws, size_t ws_bytes, hipStream_t stream) {
  return qknorm_attention_ex(Q, K, V, gq, gk, O, eps, BH, S, D, dtype, 0, ws, ws_bytes, stream);
}

rmm_status rmm_attention(const void* Q, const void* K, const void* V, void* O, int64_t BH,
                         int64_t S, int64_t D, rmm_dtype dtype, void* ws, size_t ws_bytes,
                         hipStream_t stream) {
  // Validated as the fused call with Q standing in for both gains (the
  // kernel does not read them) and eps = 0.
  AttnPlan plan;
  const rmm_status st =
      attn_plan_call(Q, K, V, Q, Q, O, 0.0f, BH, S, D, dtype, 0, ws, ws_bytes, &plan);
  if (st != RMM_OK || BH == 0) return st;
  const AttnArgs a{Q, K, V, Q, Q, O, 0.0f, BH, S, D, stream, 0, 1};
  const hipError_t err = rmm_launch_attention(a, plan, plan.chunks > 1 ? ws : nullptr);
  if (err != hipSuccess) {
    g_last_hip_error = (int)err;
    return RMM_ERR_HIP;
  }
  return RMM_OK;
}

rmm_status qknorm_attention_gqa(const void* Q, const void* K, const void* V, const void* gq,
                                const void* gk, void* O, float eps, int64_t BH, int64_t G,
                                int64_t S, int64_t D, rmm_dtype dtype, int splits, void* ws,
                                size_t ws_bytes, hipStream_t stream) {
  AttnPlan plan;
  const rmm_status st =
      attn_plan_call(Q, K, V, gq, gk, O, eps, BH, S, D, dtype, splits, ws, ws_bytes, &plan, G);
  if (st != RMM_OK || BH == 0) return st;
  const AttnArgs a{Q, K, V, gq, gk, O, eps, BH, S, D, stream, 1, G};
  const hipError_t err = rmm_launch_attention(a, plan, plan.chunks > 1 ? ws : nullptr);
  if (err != hipSuccess) {
    g_last_hip_error = (int)err;
    return RMM_ERR_HIP;
  }
  return RMM_OK;
}

rmm_status qknorm_attention_prefill_ex(const void* Q, const void* K, const void* V,
                                       const void* gq, const void* gk, void* O, float eps,
                                       int64_t BH, int64_t G, int64_t Sq, int64_t Skv, int64_t D,
                                       int causal, rmm_dtype dtype, int splits, void* ws,
                                       size_t ws_bytes, hipStream_t stream) {
  AttnPrefillPlan plan;
  const rmm_status st = prefill_attn_plan_call(Q, K, V, gq, gk, O, eps, BH, G, Sq, Skv, D, causal,
                                               dtype, splits, ws, ws_bytes, &plan);
  if (st != RMM_OK || BH == 0) return st;
  AttnArgs a{Q, K, V, gq, gk, O, eps, BH, Skv, D, stream, 1, G};
  const hipError_t err = rmm_launch_attention_prefill(a, Sq, Skv, causal ? 1 : 0, plan, ws);
  if (err != hipSuccess) {
    g_last_hip_error = (int)err;
    return RMM_ERR_HIP;
  }
  return RMM_OK;
}

rmm_status qknorm_attention_prefill(const void* Q, const void* K, const void* V, const void* gq,
                                    const void* gk, void* O, float eps, int64_t BH, int64_t G,
                                    int64_t Sq, int64_t Skv, int64_t D, int causal,
                                    rmm_dtype dtype, hipStream_t stream) {
  return qknorm_attention_prefill_ex(Q, K, V, gq, gk, O, eps, BH, G, Sq, Skv, D, causal, dtype, 1,
                                     nullptr, 0, stream);
}

size_t rmm_attention_prefill_workspace_bytes(int64_t BH, int64_t G, int64_t Sq, int64_t Skv,
                                             int64_t D, int causal, int splits) {
  if (BH < 1 || G < 1 || Sq < 1 || Skv < 1 || (D != 64 && D != 128) || (causal && Skv < Sq) ||
      splits < 0 || splits > (Skv + 63) / 64)
    return 0;
  int64_t bhg;
  if (__builtin_mul_overflow(BH, G, &bhg)) return 0;
  AttnPrefillPlan plan;
  rmm_attention_prefill_plan(bhg, Sq, Skv, D, causal ? 1 : 0, splits, true, &plan);
  return plan.ws_bytes;
}

size_t rmm_attention_gqa_workspace_bytes(rmm_dtype dtype, int64_t BH, int64_t G, int64_t S,
                                         int64_t D, int splits) {
  if (dtype != RMM_DTYPE_BF16 || BH <= 0 || S < 1 || (D != 64 && D != 128) || splits < 0 ||
      splits > S || G < 1 || G > 16)
    return 0;
  AttnPlan plan;
  rmm_attention_plan(BH, S, D, splits, &plan, G);
  return plan.ws_bytes;
}

size_t rmm_attention_workspace_bytes(rmm_dtype dtype, int64_t BH, int64_t S, int64_t D,
                                     int splits) {
  if (dtype != RMM_DTYPE_BF16 || BH <= 0 || S < 1 || (D != 64 && D != 128) || splits < 0 ||
      splits > S)
    return 0;
  AttnPlan plan;
  rmm_attention_plan(BH, S, D, splits, &plan);
  return plan.ws_bytes;
}

rmm_status rmm_plan_attention_gqa(const void* Q, const void* K, const void* V, const void* gq,
                                  const void* gk, const void* O, float eps, int64_t BH, int64_t G,
                                  int64_t S, int64_t D, rmm_dtype dtype, int splits,
                                  const void* ws, size_t ws_bytes, int* chunks_out,
                                  int64_t* keys_per_chunk_out) {
  AttnPlan plan;
  const rmm_status st =
      attn_plan_call(Q, K, V, gq, gk, O, eps, BH, S, D, dtype, splits, ws, ws_bytes, &plan, G);
  if (st == RMM_OK) {
    if (chunks_out) *chunks_out = plan.chunks;
    if (keys_per_chunk_out) *keys_per_chunk_out = plan.kchunk;
  }
  return st;
}

rmm_status rmm_plan_attention(const void* Q, const void* K, const void* V, const void* gq,
                              const void* gk, const void* O, float eps, int64_t BH, int64_t S,
                              int64_t D, rmm_dtype dtype, int splits, const void* ws,
                              size_t ws_bytes, int* chunks_out, int64_t* keys_per_chunk_out) {
  AttnPlan plan;
  const rmm_status st =
      attn_plan_call(Q, K, V, gq, gk, O, eps, BH, S, D, dtype, splits, ws, ws_bytes, &plan);
  if (st == RMM_OK) {
    if (chunks_out) *chunks_out = plan.chunks;
    if (keys_per_chunk_out) *keys_per_chunk_out = plan.kchunk;
  }
  return st;
}

rmm_status rmm_rmsnorm(const void* X, const void* g, void* Xn, float eps, int64_t M, int64_t K,
                       rmm_dtype dtype, hipStream_t stream) {
  if (M != 0 && (!X || !g || !Xn)) return RMM_ERR_NULL;
  int64_t mk, tmp;
  if (M < 0 || K <= 0 || __builtin_mul_overflow(M, K, &mk) ||
      __builtin_mul_overflow(mk, (int64_t)4, &tmp))
    return RMM_ERR_SHAPE;
  if (!isfinite(eps) || eps < 0.0f) return RMM_ERR_EPS;
  if (dtype != RMM_DTYPE_F32 && dtype != RMM_DTYPE_BF16) return RMM_ERR_DTYPE;
  if (M == 0) return RMM_OK;
  const size_t es = dtype == RMM_DTYPE_F32 ? 4 : 2;
  if (overlaps(Xn, (size_t)mk * es, X, (size_t)mk * es) || overlaps(Xn, (size_t)mk * es, g, (size_t)K * es))
    return RMM_ERR_ALIAS;
  const hipError_t err = rmm_launch_rmsnorm(X, g, Xn, eps, M, K, dtype == RMM_DTYPE_BF16, stream);
  if (err != hipSuccess) {
    g_last_hip_error = (int)err;
    return RMM_ERR_HIP;
  }
  return RMM_OK;
}

size_t rmm_workspace_bytes_ex(rmm_dtype dtype, int64_t M, int64_t N, int64_t K, int gated,
                              rmm_variant variant, int splits) {
  // Sizes only: aligned pointers and a workspace are assumed to be present.
  if (M < 0 || N < 0 || K <= 0) return 0;
  if (dtype != RMM_DTYPE_F32 && dtype != RMM_DTYPE_BF16) return 0;
  Plan plan;
  if (plan_shape(M, N, K, dtype, gated ? 1 : 0, variant, splits, true, true, &plan) != RMM_OK)
    return 0;
  return plan.ws_bytes;
}

size_t rmm_workspace_bytes(rmm_dtype dtype, int64_t M, int64_t N, int64_t K, int gated) {
  return rmm_workspace_bytes_ex(dtype, M, N, K, gated, RMM_VARIANT_AUTO, 0);
}


size_t rmm_lora_workspace_bytes(rmm_dtype dtype, int64_t M, int64_t N, int64_t K, int64_t R,
                                rmm_variant variant, int splits) {
  if (M < 0 || N < 0 || K <= 0 || R < 1 || R > RMM_LORA_MAX_RANK) return 0;
  if (dtype != RMM_DTYPE_F32 && dtype != RMM_DTYPE_BF16) return 0;
  Plan plan;
  if (plan_shape(M, N, K, dtype, 0, variant, splits, true, true, &plan, R) != RMM_OK) return 0;
  return plan.ws_bytes;
}

rmm_status rmm_plan(const void* X, const void* g, const void* W1, const void* W3, const void* Y,
                    float eps, int64_t M, int64_t N, int64_t K, rmm_dtype dtype, int gated,
                    rmm_variant variant, int splits, const void* ws, size_t ws_bytes,
                    rmm_variant* variant_out, int* splits_out) {
  Plan plan;
  rmm_status st = plan_call(X, g, W1, W3, Y, eps, M, N, K, dtype, gated ? 1 : 0, variant, splits,
                            ws, ws_bytes, &plan);
  if (st == RMM_OK) {
    if (variant_out) *variant_out = plan.variant;
    if (splits_out) *splits_out = plan.splits;
  }
  return st;
}

rmm_status rmm_plan_lora(const void* X, const void* g, const void* W, const void* A,
                         const void* B, const void* Y, float eps, int64_t M, int64_t N, int64_t K,
                         int64_t R, rmm_dtype dtype, rmm_variant variant, int splits,
                         const void* ws, size_t ws_bytes, rmm_variant* variant_out,
                         int* splits_out) {
  Plan plan;
  rmm_status st = plan_call(X, g, W, nullptr, Y, eps, M, N, K, dtype, 0, variant, splits, ws,
                            ws_bytes, &plan, A, B, lora_rank_arg(R));
  if (st == RMM_OK) {
    if (variant_out) *variant_out = plan.variant;
    if (splits_out) *splits_out = plan.splits;
  }
  return st;
}

const char* rmm_status_string(rmm_status s) {
  switch (s) {
    case RMM_OK: return "RMM_OK";
    case RMM_ERR_NULL: return "RMM_ERR_NULL: a required pointer is NULL";
    case RMM_ERR_SHAPE: return "RMM_ERR_SHAPE: M < 0, N < 0, K <= 0, rank outside 1..64 or size overflow";
    case RMM_ERR_EPS: return "RMM_ERR_EPS: eps must be finite and >= 0";
    case RMM_ERR_DTYPE: return "RMM_ERR_DTYPE: unknown dtype";
    case RMM_ERR_ALIAS: return "RMM_ERR_ALIAS: Y overlaps an input or the workspace";
    case RMM_ERR_WORKSPACE: return "RMM_ERR_WORKSPACE: workspace too small or not 16-byte aligned";
    case RMM_ERR_HIP: return "RMM_ERR_HIP: kernel launch failed";
    case RMM_ERR_VARIANT: return "RMM_ERR_VARIANT: variant/splits cannot run this call";
    case RMM_ERR_SCRATCH:
      return "RMM_ERR_SCRATCH: the call needs more than the 16 MiB device scratch array of "
             "rmsnorm_matmul_noalloc (use rmsnorm_matmul with a workspace)";
  }
  return "unknown rmm_status";
}

int rmm_last_hip_error(void) { return g_last_hip_error; }

int rmm_abi_version(void) { return RMM_ABI_VERSION; }

rmm_status rmsnorm_matmul_chain(const void* X0, const void* G, const void* W, void* Xs, float eps,
                                int64_t M, int64_t K, int64_t L, rmm_dtype dtype, void* ws,
                                size_t ws_bytes, hipStream_t stream) {
  ChainPlan plan;
  const rmm_status st = chain_plan_call(X0, G, W, Xs, eps, M, K, L, dtype, ws, ws_bytes, &plan);
  if (st != RMM_OK || M == 0) return st;
  const hipError_t err = rmm_launch_chain(X0, G, W, Xs, eps, M, K, L, plan, ws, stream);
  if (err != hipSuccess) {
    g_last_hip_error = (int)err;
    return RMM_ERR_HIP;
  }
  return RMM_OK;
}

size_t rmm_chain_workspace_bytes(int64_t M, int64_t K, int64_t L) {
  if (M < 1 || M > 16 || K <= 0 || K % 128 != 0 || L < 1 || K * K * 2 > (int64_t)INT32_MAX) return 0;
  ChainPlan plan;
  if (rmm_chain_plan(M, K, L, &plan) != 0) return 0;
  return plan.ws_bytes;
}

rmm_status rmm_probe_hbm_read(const void* src, size_t bytes, void* sink, hipStream_t stream) {
  if (!src || !sink) return RMM_ERR_NULL;
  if (bytes == 0 || bytes % 16 != 0) return RMM_ERR_SHAPE;
  if (!aligned16(src)) return RMM_ERR_VARIANT;
  const hipError_t err = rmm_launch_probe_read(src, bytes, sink, stream);
  if (err != hipSuccess) {
    g_last_hip_error = (int)err;
    return RMM_ERR_HIP;
  }
  return RMM_OK;
}

rmm_status rmm_probe_mfma_bf16(int64_t iters, void* sink, hipStream_t stream) {
  if (!sink) return RMM_ERR_NULL;
  if (iters < 1 || iters > ((int64_t)1 << 40)) return RMM_ERR_SHAPE;
  const hipError_t err = rmm_launch_probe_mfma(iters, sink, stream);
  if (err != hipSuccess) {
    g_last_hip_error = (int)err;
    return RMM_ERR_HIP;
  }
  return RMM_OK;
}

int64_t rmm_probe_mfma_flops(int64_t iters) {
  return iters < 1 || iters > ((int64_t)1 << 40) ? 0 : rmm_probe_mfma_flops_per_launch(iters);
}

size_t rmm_chain_flag_offset(int64_t M, int64_t K, int64_t L) {
  if (rmm_chain_workspace_bytes(M, K, L) == 0) return 0;
  ChainPlan plan;
  rmm_chain_plan(M, K, L, &plan);
  return plan.ws_done_off + sizeof(unsigned);
}

}  // extern "C"
