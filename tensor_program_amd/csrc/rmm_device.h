// Device-side helpers shared by the gfx950 kernels of the RMSNorm+MatMul
// library: storage types, bf16 conversion, vector types, launcher prototypes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rmm {

typedef uint16_t bf16_t;  // bf16 storage (bit pattern)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// bf16 pair (1.0, 1.0): the gain when the call is a plain product.
constexpr uint32_t kBf16OnePair = 0x3f803f80u;

// bf16 bits -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(bf16_t h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16 bits, round to nearest even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(bf16_t, b);
}
// Two fp32 -> packed bf16 pair (lo, hi), round to nearest even (one
// v_cvt_pk_bf16_f32).
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const floatx2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// Two fp32 values that are each the exact product of two bf16 values (at
// most 16 significant bits) -> packed bf16 pairs hi and lo with
// hi + lo == the products exactly: hi is the nearest-even rounding, and the
// remainder (computed exactly in fp32) has at most 8 significant bits, so
// its own rounding to bf16 is exact.  The gated and adapter paths feed both
// parts to the matrix cores, so their k-sums see X*g without rounding.
// Returns {hi, lo}.
__device__ __forceinline__ u32x2 split_bf16x2(float p0, float p1) {
  const uint32_t hi = pack_bf16x2(p0, p1);
  return u32x2{hi, pack_bf16x2(p0 - __uint_as_float(hi << 16), p1 - __uint_as_float(hi & 0xffff0000u))};
}

// Load/store of one element of the storage type as fp32.
__device__ __forceinline__ float load_f32(const float* p) { return *p; }
__device__ __forceinline__ float load_f32(const bf16_t* p) { return bf16_to_f32(*p); }
__device__ __forceinline__ void store_f32(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_f32(bf16_t* p, float v) { *p = f32_to_bf16(v); }

// silu(z1) * z3 for the gated epilogue, silu(z) = z / (1 + e^-z), with the
// logistic factor taken as 1 / (1 + e^-|z|) for z >= 0 and e^-|z| / (1 + e^-|z|)
// for z < 0: e^-|z| never overflows, so below z = -88.7 (where e^-z is past
// the fp32 range) the result stays the small number it is instead of 0.
__device__ __forceinline__ float silu_gate(float z1, float z3) {
  const float e = expf(-fabsf(z1));
  return z1 * ((z1 >= 0.0f ? 1.0f : e) / (1.0f + e)) * z3;
}

// 1 / sqrt(ss / K + eps) with IEEE division and square root, so that
// exact inputs (ss = K * 4^j, eps = 0) give an exact power of two.
__device__ __forceinline__ float inv_rms(float ss, int64_t K, float eps) {
  return 1.0f / __fsqrt_rn(__fdiv_rn(ss, (float)K) + eps);
}

}  // namespace rmm

// Host-side launchers (return hipSuccess or the launch error).
struct RmmArgs {
  const void* X;
  const void* g;
  const void* W1;
  const void* W3;  // NULL unless gated
  void* Y;
  float eps;
  int64_t M, N, K;
  int gated;
  int norm;  // 1: fused RMSNorm (gain g, 1/RMS scale); 0: plain product (g = 1, no scale)
  hipStream_t stream;
  // Low-rank adapter (R = 0: none): Y += (Act A^T) B before the 1/RMS scale,
  // A: R x K (row r = down-projection vector r), B: R x N.  Not with gated.
  const void* LA = nullptr;
  const void* LB = nullptr;
  int64_t R = 0;
};

hipError_t rmm_launch_generic(const RmmArgs& a, bool bf16);

// Records the hipError_t behind an RMM_ERR_HIP (rmm_last_hip_error).
void rmm_set_last_hip_error(int err);

// Every workspace layout starts with the same 64 KiB counter region: the
// arrival counters of any call are its first words (at most
// kWsMaxCounters of them; a call that would need more runs without a
// cross-workgroup combine or is refused), the layer chain keeps its
// call-wide counts and flag word in the region's last 256 bytes, and the
// partial sums of every layout start after the region.  Each call leaves
// its counters at zero, so one zero-filled workspace serves any sequence of
// calls, whatever their shapes and variants.
constexpr size_t kWsCounterBytes = 64 * 1024;
constexpr int64_t kWsMaxCounters = (int64_t)((kWsCounterBytes - 256) / 4);
constexpr size_t kWsChainBlockOff = kWsCounterBytes - 256;

struct DecodePlan {
  int mb;          // 16-row blocks (1..2)
  int wv;          // waves per workgroup (4 or 8); a step covers 32 wv rows of K
  int splits;      // K chunks combined across workgroups
  int64_t kchunk;  // K per chunk (multiple of 128)
  int64_t tiles;   // 128-column tiles
  int lr;          // 16-wide blocks of the adapter rank (0: no adapter)
  size_t ws_cnt_off, ws_ssq_off, ws_part_off, ws_bytes;
};
void rmm_decode_plan(int64_t M, int64_t N, int64_t K, int gated, int splits, int64_t lora_rank,
                     DecodePlan* p);
hipError_t rmm_launch_decode(const RmmArgs& a, const DecodePlan& p, void* ws);

// fp32 decode (M <= 16, not gated, no adapter): 128-column tiles, K split
// into `splits` ranges of `krange` rows walked in chunks of `kc` (64) rows.
struct Decode32Plan {
  int mr;          // rows computed per workgroup (8 or 16)
  int splits;      // K ranges combined across workgroups
  int64_t kc;      // k rows per chunk (64)
  int64_t krange;  // K per range (multiple of kc)
  int64_t tiles;   // 128-column tiles
  size_t ws_cnt_off, ws_ssq_off, ws_part_off, ws_bytes;
};
void rmm_decode32_plan(int64_t M, int64_t N, int64_t K, int splits, Decode32Plan* p);
hipError_t rmm_launch_decode32(const RmmArgs& a, const Decode32Plan& p, void* ws);

// Layer chain (persistent decode over L square layers): the decode tiling
// with every workgroup resident (tiles * splits <= 256).
struct ChainPlan {
  int64_t tiles;   // 128-column tiles (N = K)
  int splits;      // K chunks per tile
  int64_t kchunk;  // rows per chunk (<= 1024, whole 128-row granules)
  size_t ws_cnt_off, ws_done_off, ws_ssq_off, ws_part_off, ws_bytes;
};
int rmm_chain_plan(int64_t M, int64_t K, int64_t L, ChainPlan* p);  // 0, or -1 if not co-resident
hipError_t rmm_launch_chain(const void* X0, const void* G, const void* W, void* Xs, float eps,
                            int64_t M, int64_t K, int64_t L, const ChainPlan& p, void* ws,
                            hipStream_t stream);

struct PrefillPlan {
  int tiles_m, tiles_n;  // output tiles: 256 x 256, gated 128 x 128 (of each weight)
  int group_m;           // tile-rows walked together (L2 reuse)
  int xcd_remap;         // contiguous tile ranges per XCD
  int splits;            // K ranges (plain tile only; > 1: partial sums + combine kernel)
  int ksteps;            // 64-deep k-steps per range (even when splits > 1)
  int rb;                // adapter: 16-wide rank blocks of T (0: no adapter)
  size_t ws_part_off, ws_t_off, ws_bytes;
};
// splits: 0 = chosen by the library (a split only if its partial sums fit
// in ws_avail bytes of workspace), else the requested count (the count that
// runs may be lower: whole, even ranges).
// R > 0: the adapter tile (plain product, T = (X g) A^T in the workspace).
void rmm_prefill_plan(int64_t M, int64_t N, int64_t K, int gated, int splits, size_t ws_avail,
                      PrefillPlan* p, int64_t R = 0);
// Workspace bytes of an AUTO plain or gated call given a workspace of `cap`
// bytes (the prefill split is chosen to fit), 0 for invalid arguments.
size_t rmm_workspace_bytes_within(int dtype, int64_t M, int64_t N, int64_t K, int gated,
                                  size_t cap);
hipError_t rmm_launch_prefill(const RmmArgs& a, const PrefillPlan& p, void* ws);

// Stream variant: one workgroup per 64-column strip, or (split form, with a
// workspace, when there are fewer strips than workgroups wanted) `grid`
// workgroups each taking an equal share of the strips' k-steps, partial
// sums combined in the workspace.
struct StreamPlan {
  int split;   // 1: split form
  int strips;  // 64-column strips
  int grid;    // workgroups launched
  size_t ws_cnt_off, ws_part_off, ws_ssq_off, ws_bytes;
};
void rmm_stream_plan(int64_t N, int64_t K, int gated, int target, bool have_ws, StreamPlan* p);
hipError_t rmm_launch_stream(const RmmArgs& a, const StreamPlan& p, void* ws);
// Whether a 64-row chunk of an M x K by K x N product fits the stream kernel's
// 32-bit buffer offsets.
bool rmm_stream_fits(int64_t M, int64_t N, int64_t K);

// QKNorm + attention, one query per query head (bf16, D = 64 or 128); G
// query heads share each key/value head.
struct AttnArgs {
  const void* Q;   // (BH G) x D
  const void* K;   // BH x S x D
  const void* V;   // BH x S x D
  const void* gq;  // D
  const void* gk;  // D
  void* O;         // (BH G) x D
  float eps;
  int64_t BH, S, D;
  hipStream_t stream;
  int norm;    // 1: QKNorm + attention; 0: attention on q and k as given (gains unused)
  int64_t G;   // query heads per key/value head (1..8); Q and O hold BH * G rows
};
struct AttnPlan {
  int64_t kchunk;  // keys per workgroup (a multiple of the workgroup's key round)
  int chunks;      // key chunks per key/value head, merged by the last arriving workgroup
  size_t ws_cnt_off, ws_part_off, ws_bytes;
};
// BH: key/value heads; G: query heads per key/value head.
void rmm_attention_plan(int64_t BH, int64_t S, int64_t D, int splits, AttnPlan* p,
                        int64_t G = 1);
hipError_t rmm_launch_attention(const AttnArgs& a, const AttnPlan& p, void* ws);
// Many queries per head: Q and O (BH G) x Sq x D, K and V BH x Skv x D (a.S
// unused); causal: query i sees keys 0 .. i + Skv - Sq.
// Many queries per head: query blocks per wave (qw), key-tile length (kt),
// blocks per query head, and the split of the keys into spans of kspan
// (splits > 1: partials in the workspace, a second kernel combines them).
struct AttnPrefillPlan {
  int qw, kt, splits;
  int64_t nblk, kspan;
  size_t ws_part_off, ws_bytes;
};
void rmm_attention_prefill_plan(int64_t BHG, int64_t Sq, int64_t Skv, int64_t D, int causal,
                                int splits, bool have_ws, AttnPrefillPlan* p);
hipError_t rmm_launch_attention_prefill(const AttnArgs& a, int64_t Sq, int64_t Skv, int causal,
                                        const AttnPrefillPlan& p, void* ws);

// Unfused baseline, first kernel: Xn = bf16/f32(X * g / RMS) written out.
hipError_t rmm_launch_rmsnorm(const void* X, const void* g, void* Xn, float eps, int64_t M,
                              int64_t K, bool bf16, hipStream_t stream);

// Achievable-peak probes (rmm_probe.hip).
hipError_t rmm_launch_probe_read(const void* src, size_t bytes, void* sink, hipStream_t stream);
hipError_t rmm_launch_probe_mfma(int64_t iters, void* sink, hipStream_t stream);
int64_t rmm_probe_mfma_flops_per_launch(int64_t iters);
