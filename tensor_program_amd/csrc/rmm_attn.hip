// QKNorm + attention for one query per batch-head (decode), bandwidth-bound.
//
// The QKNorm + Attention row of the Mirage paper review's benchmark table
// ("五、实验结果") names the fusion only; the reading is RMSNorm over the head
// dimension D (gains gq, gk) applied to the query and to every cached key,
// then scaled dot-product attention over the keys:
//
//   score_s = (q/rms(q)*gq) . (k_s/rms(k_s)*gk) / sqrt(D)
//           = (sum_d u_d k_sd) / (rms(q) rms(k_s) sqrt(D)),   u = q * gq * gk
//   o = sum_s softmax(score)_s v_s
//
// As in the fused RMSNorm+MatMul ("核心公式": the k-independent divisor moves
// out of the sum), the normalised keys are never formed: each key row is read
// once, and the same pass accumulates u . k_s and sum_d k_sd^2; the key's
// 1/RMS scales the finished dot product.  u is exact in fp32 (a product of
// three bf16 values has at most 24 significant bits).
//
// Work decomposition: a workgroup (4 waves) owns one batch-head and a chunk of
// its keys.  D/8 lanes cover one key row (16 bytes each); a wave loads 64/(D/8)
// keys per instruction and U instructions per block, K and V double-buffered
// in registers.  Every lane group keeps its own running (max, sum, o) and
// rescales once per block (online softmax); groups merge by shuffles, waves
// through LDS.  With several chunks the workgroup stores (o, max, sum) with
// device-scope coherence and the last one to arrive merges them (log-sum-exp)
// and writes o / sum.  Keys past S or past the chunk are range-checked loads
// that read zeros and get weight 0.
#include <type_traits>

#include "rmm_device.h"

namespace rmm {

constexpr int AT_THREADS = 256;
constexpr uint32_t kAtOutOfRange = 0x80000000u;  // past every buffer this path accepts
constexpr int kAtCoherentDevice = 16;            // SC1: device-scope coherence
constexpr float kAtNone = -1.0e30f;              // running max before any valid key
constexpr float kLog2e = 1.44269504088896341f;

// Max and sum over lanes l, l ^ 16, l ^ 32 and l ^ 48 of a wave, with
// gfx950's permlane swaps (VALU, no LDS round trip): with both operands v,
// the 16-lane swap returns rows (0, 0, 2, 2) and (1, 1, 3, 3) of v, the
// 32-lane swap halves (0, 0) and (1, 1); every lane gets the same bits.
__device__ __forceinline__ float max_xor16_32(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_xor16_32(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Sum over aligned groups of LPK (8 or 16) lanes with DPP moves: swaps
// within quads, then the mirrored half-row and row.  Every lane of a group
// ends with the same bits (each step adds two operands in either order),
// which the softmax relies on: all lanes of a key see one score.
template <int LPK>
__device__ __forceinline__ float group_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));  // xor 1
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));  // xor 2
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, true));  // half mirror
  if (LPK == 16)
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, true));  // mirror
  return v;
}

// NORM = false: plain scaled dot-product attention on q and k as given (the
// second kernel of the unfused program; the gains are not read).
//
// Grouped queries (GT > 1): G <= GT query heads share each cached key and
// value head (query row h G + g of Q and O belongs to key head h); a
// workgroup owns one key head and a chunk of its keys for all G queries, so
// every key and value row is read once for the group.  Each lane keeps
// u, o and the softmax state of every query; the key's sum of squares is
// formed once.  Queries g >= G (GT rounds G up) are neither read nor stored.
template <int GT>
struct AtCfg {
  static constexpr int U = GT >= 4 ? 2 : 4;  // key loads per block and lane
};

template <int D, bool NORM, int GT>
__global__ __launch_bounds__(AT_THREADS) void qknorm_attention_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ Kc, const bf16_t* __restrict__ Vc,
    const bf16_t* __restrict__ gq, const bf16_t* __restrict__ gk, bf16_t* __restrict__ O,
    float eps, int64_t S, int64_t kchunk, int C, int G, unsigned* __restrict__ cnt,
    float* __restrict__ part) {
  constexpr int LPK = D / 8;          // lanes per key row
  constexpr int KPI = 64 / LPK;       // keys per load instruction (per wave)
  constexpr int UU = AtCfg<GT>::U;
  constexpr int BLK = UU * KPI;       // keys per wave block
  constexpr int NWV = AT_THREADS / 64;
  __shared__ float sm_o[NWV][GT][D];
  __shared__ float sm_m[NWV][GT], sm_l[NWV][GT];
  __shared__ int last;

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int j = l / LPK, c = l % LPK;  // key slot in an instruction, 8-dim chunk
  const int64_t bh = blockIdx.x / C;
  const int chunk = (int)(blockIdx.x % C);
  const int64_t s_lo = (int64_t)chunk * kchunk;
  const int64_t s_hi = (s_lo + kchunk < S) ? (s_lo + kchunk) : S;

  // u = q * gq * gk for this lane's 8 dims; cq = 1 / (rms(q) sqrt(D)), IEEE
  // divide and square root (plain: 1 / sqrt(D)).
  float u[GT][8], cq[GT];
  {
    constexpr u32x4 ones{kBf16OnePair, kBf16OnePair, kBf16OnePair, kBf16OnePair};
    const u32x4 a = NORM ? *(const u32x4*)(gq + 8 * c) : ones;
    const u32x4 b = NORM ? *(const u32x4*)(gk + 8 * c) : ones;
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      const u32x4 qv = g < G ? *(const u32x4*)(Q + (bh * G + g) * D + 8 * c)
                             : u32x4{0u, 0u, 0u, 0u};
      float qss = 0.f;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const float q0 = bf16_lo(qv[d]), q1 = bf16_hi(qv[d]);
        u[g][2 * d] = q0 * bf16_lo(a[d]) * bf16_lo(b[d]);
        u[g][2 * d + 1] = q1 * bf16_hi(a[d]) * bf16_hi(b[d]);
        qss += q0 * q0 + q1 * q1;
      }
#pragma unroll
      for (int o = 1; o < LPK; o <<= 1) qss += __shfl_xor(qss, o);
      cq[g] = NORM ? 1.0f / (__fsqrt_rn(__fdiv_rn(qss, (float)D) + eps) * __fsqrt_rn((float)D))
                   : 1.0f / __fsqrt_rn((float)D);
    }
  }

  // Buffer resources over this head's S x D rows (the plan keeps S * D * 2
  // below 2^31), so offsets are 32-bit and past-the-end reads zero.
  const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(Kc + bh * S * D), 0, (int)(S * D * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(Vc + bh * S * D), 0, (int)(S * D * 2), 0x00020000);
  auto key_of = [&](int64_t blk, int uu) { return s_lo + blk * BLK + uu * KPI + j; };
  auto load = [&](int64_t blk, u32x4 (&kk)[UU], u32x4 (&vv)[UU]) {
#pragma unroll
    for (int uu = 0; uu < UU; ++uu) {
      const int64_t s = key_of(blk, uu);
      const uint32_t off = s < s_hi ? (uint32_t)((s * D + 8 * c) * 2) : kAtOutOfRange;
      kk[uu] = __builtin_amdgcn_raw_buffer_load_b128(kr, off, 0, 0);
      vv[uu] = __builtin_amdgcn_raw_buffer_load_b128(vr, off, 0, 0);
    }
  };

  float m[GT], lsum[GT], o[GT][8];
#pragma unroll
  for (int g = 0; g < GT; ++g) {
    m[g] = kAtNone;
    lsum[g] = 0.f;
#pragma unroll
    for (int d = 0; d < 8; ++d) o[g][d] = 0.f;
  }

  auto consume = [&](int64_t blk, const u32x4 (&kk)[UU], const u32x4 (&vv)[UU]) {
    float sc[UU][GT];
    bool ok[UU];
    float mb[GT];
#pragma unroll
    for (int g = 0; g < GT; ++g) mb[g] = kAtNone;
#pragma unroll
    for (int uu = 0; uu < UU; ++uu) {
      float ss = 0.f;
      if (NORM) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const float k0 = bf16_lo(kk[uu][d]), k1 = bf16_hi(kk[uu][d]);
          ss += k0 * k0 + k1 * k1;
        }
        ss = group_sum<LPK>(ss);
      }
      // 1/D is a power of two (exact); v_rsq_f32 for the key's 1/RMS.
      const float rk = NORM ? __builtin_amdgcn_rsqf(ss * (1.0f / D) + eps) : 1.0f;
      ok[uu] = key_of(blk, uu) < s_hi;
#pragma unroll
      for (int g = 0; g < GT; ++g) {
        float dot = 0.f;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const float k0 = bf16_lo(kk[uu][d]), k1 = bf16_hi(kk[uu][d]);
          dot += u[g][2 * d] * k0 + u[g][2 * d + 1] * k1;
        }
        dot = group_sum<LPK>(dot);
        sc[uu][g] = NORM ? dot * cq[g] * rk : dot * cq[g];
        if (ok[uu]) mb[g] = fmaxf(mb[g], sc[uu][g]);
      }
    }
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      const float mn = fmaxf(m[g], mb[g]);
      const float alpha = __expf(m[g] - mn);
      lsum[g] *= alpha;
#pragma unroll
      for (int d = 0; d < 8; ++d) o[g][d] *= alpha;
#pragma unroll
      for (int uu = 0; uu < UU; ++uu) {
        const float p = ok[uu] ? __expf(sc[uu][g] - mn) : 0.f;
        lsum[g] += p;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          o[g][2 * d] += p * bf16_lo(vv[uu][d]);
          o[g][2 * d + 1] += p * bf16_hi(vv[uu][d]);
        }
      }
      m[g] = mn;
    }
  };

  // Blocks w, w + NWV, ... of the chunk; two register stages.
  const int64_t nblk = (s_hi - s_lo + BLK - 1) / BLK;
  u32x4 ka[UU], va[UU], kb[UU], vb[UU];
  load(w, ka, va);
  load(w + NWV, kb, vb);
  int64_t blk = w;
  for (; blk + NWV < nblk; blk += 2 * NWV) {
    consume(blk, ka, va);
    load(blk + 2 * NWV, ka, va);
    consume(blk + NWV, kb, vb);
    load(blk + 3 * NWV, kb, vb);
  }
  if (blk < nblk) consume(blk, ka, va);

  // Merge the lane groups of a wave (same dims, different keys).
#pragma unroll
  for (int g = 0; g < GT; ++g) {
#pragma unroll
    for (int x = LPK; x < 64; x <<= 1) {
      const float mo = __shfl_xor(m[g], x), lo = __shfl_xor(lsum[g], x);
      const float mn = fmaxf(m[g], mo);
      const float a = __expf(m[g] - mn), b = __expf(mo - mn);
      lsum[g] = lsum[g] * a + lo * b;
#pragma unroll
      for (int d = 0; d < 8; ++d) o[g][d] = o[g][d] * a + __shfl_xor(o[g][d], x) * b;
      m[g] = mn;
    }
  }
  if (l < LPK) {
#pragma unroll
    for (int g = 0; g < GT; ++g) {
#pragma unroll
      for (int d = 0; d < 8; ++d) sm_o[w][g][8 * c + d] = o[g][d];
      if (l == 0) {
        sm_m[w][g] = m[g];
        sm_l[w][g] = lsum[g];
      }
    }
  }
  __syncthreads();

  // Thread t merges the waves for (query t / D, dim t % D), t < G D.
  constexpr int PER = (GT * D + AT_THREADS - 1) / AT_THREADS;
  float od[PER], ld[PER], md[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int t = tid + AT_THREADS * e, g = t / D, d = t % D;
    od[e] = 0.f;
    ld[e] = 0.f;
    md[e] = kAtNone;
    if (g < G) {
#pragma unroll
      for (int ww = 0; ww < NWV; ++ww) md[e] = fmaxf(md[e], sm_m[ww][g]);
#pragma unroll
      for (int ww = 0; ww < NWV; ++ww) {
        const float a = __expf(sm_m[ww][g] - md[e]);
        od[e] += sm_o[ww][g][d] * a;
        ld[e] += sm_l[ww][g] * a;
      }
    }
  }
  if (C > 1) {
    // Partial (o[D], max, sum) of each query of this chunk; device-scope
    // stores acknowledged before the arrival count, as in the split-K
    // combine of the decode path.
    const int64_t slot = bh * C + chunk;
    // The plan keeps the whole partial area below 2^31 bytes.
    const __amdgpu_buffer_rsrc_t pr =
        __builtin_amdgcn_make_buffer_rsrc(part, 0, 0x7fffffff, 0x00020000);
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int t = tid + AT_THREADS * e, g = t / D, d = t % D;
      if (g < G) {
        const int64_t base = (slot * G + g) * (D + 2);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(od[e]), pr, (int)((base + d) * 4),
                                              0, kAtCoherentDevice);
        if (d == 0) {
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(md[e]), pr,
                                                (int)((base + D) * 4), 0, kAtCoherentDevice);
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(ld[e]), pr,
                                                (int)((base + D + 1) * 4), 0, kAtCoherentDevice);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0)
      last = (__hip_atomic_fetch_add(&cnt[bh], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
              (unsigned)(C - 1));
    __syncthreads();
    if (!last) return;
    // The chunks' partials in chunk order, 8 chunks' loads in flight at a
    // time (each is a round trip to memory), merged with a running maximum.
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int t = tid + AT_THREADS * e, g = t / D, d = t % D;
      if (g < G) {
        md[e] = kAtNone;
        od[e] = 0.f;
        ld[e] = 0.f;
        for (int c0 = 0; c0 < C; c0 += 8) {
          float oc[8], mc[8], lc[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const int64_t base = ((bh * C + c0 + q) * G + g) * (D + 2);
            const bool in = c0 + q < C;
            oc[q] = in ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                             pr, (int)((base + d) * 4), 0, kAtCoherentDevice))
                       : 0.f;
            mc[q] = in ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                             pr, (int)((base + D) * 4), 0, kAtCoherentDevice))
                       : kAtNone;
            lc[q] = in ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                             pr, (int)((base + D + 1) * 4), 0, kAtCoherentDevice))
                       : 0.f;
          }
          float mn = md[e];
#pragma unroll
          for (int q = 0; q < 8; ++q) mn = fmaxf(mn, mc[q]);
          const float r = __expf(md[e] - mn);
          od[e] *= r;
          ld[e] *= r;
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const float a = __expf(mc[q] - mn);
            od[e] += oc[q] * a;
            ld[e] += lc[q] * a;
          }
          md[e] = mn;
        }
      }
    }
    // All arrivals are in: reset the counter for the next call.
    if (tid == 0) __hip_atomic_store(&cnt[bh], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int t = tid + AT_THREADS * e, g = t / D, d = t % D;
    if (g < G) O[(bh * G + g) * D + d] = f32_to_bf16(__fdiv_rn(od[e], ld[e]));
  }
}


// ---------------------------------------------------------------------------
// Grouped queries on the matrix cores (G = 3 .. 16 query heads per key/value
// head).  The VALU form above spends every query's dot product and value
// update on the vector ALUs, which for G >= 4 costs more than streaming the
// keys; here both products are 16 x 16 x 32 bf16 MFMAs over a block of up
// to 16 queries:
//   * scores, transposed: S^T (16 keys x 16 queries) = K (keys x 32 d) .
//     U^T, with U = q gq gk (fp32) carried as two bf16 parts (16 significant
//     bits of its 24: within 2^-17 of U); the K fragments are the key rows as
//     loaded (lane l: key l % 16, 8 dims);
//   * each lane then holds 4 keys of one query (column l % 16): the key's
//     1/RMS (its sum of squares from the same K fragments, reduced over the
//     4 lanes holding that key) and the query's scale give the score; the
//     online softmax runs per query column over 32 keys per tile (2 x 16);
//   * values: O (16 queries x 16 d) += P (queries x 32 keys) . V (keys x 16
//     d), P (in [0, 1]) as two bf16 parts; P's A fragments are the score
//     registers as they lie (lane l: query l % 16, keys 4 (l / 16) + i of
//     both halves), and the matching V fragments come from the wave's V tile
//     in LDS through two transposing reads (ds_read_b64_tr_b16: rows = keys
//     4 (l / 16) .. +3 and 16 + 4 (l / 16) .. +3, column = d).
// A workgroup (4 waves) owns one key/value head and a chunk of its keys;
// wave w takes 32-key tiles w, w + 4, ...; each wave's tile loads for the
// next tile are in flight while it multiplies the current one.  The waves'
// (o, max, sum) merge through LDS, the chunks through the workspace as in
// the VALU form.
constexpr int AQ_THREADS = 256;
typedef short at_i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) at_i16x4 at_lds_i16x4;
typedef __attribute__((address_space(3))) char at_lds_char;

template <int D>
__device__ __forceinline__ int aq_v_off(int key, int n) {
  // V tile row `key` (2 D bytes), 16-byte chunk c stored at c ^ f(key): a
  // half-wave's transposing reads (rows 8 i .. 8 i + 7, 32 bytes of each)
  // then cover all 16 bank groups.  D = 128 (256-byte rows): f = 2 (key & 7);
  // D = 64 (128-byte rows, odd rows on the other 8 groups): f = 2 ((key >> 1) & 3).
  const int f = D == 128 ? 2 * (key & 7) : 2 * ((key >> 1) & 3);
  return key * (2 * D) + (((n >> 3) ^ f) << 4) + ((n & 7) << 1);
}

template <int D, bool NORM>
__global__ __launch_bounds__(AQ_THREADS) void gqa_mfma_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ Kc, const bf16_t* __restrict__ Vc,
    const bf16_t* __restrict__ gq, const bf16_t* __restrict__ gk, bf16_t* __restrict__ O,
    float eps, int64_t S, int64_t kchunk, int C, int G, unsigned* __restrict__ cnt,
    float* __restrict__ part) {
  constexpr int NDB = D / 32;       // 32-deep d blocks of the score products
  constexpr int NOB = D / 16;       // 16-wide d blocks of O
  constexpr int CPR = D / 8;        // 16-byte chunks per key row
  constexpr int NV = 32 * CPR / 64; // V tile chunks per lane
  constexpr int NWV = AQ_THREADS / 64;
  __shared__ __attribute__((aligned(16))) char v_s[NWV][2][32 * 2 * D];
  __shared__ __attribute__((aligned(16))) float mo_s[NWV][16][D];
  __shared__ float mm_s[NWV][16], ml_s[NWV][16];
  __shared__ __attribute__((aligned(16))) float rk_w[NWV][2][16];  // keys' 1/RMS, per wave
  __shared__ int last;

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lq = l & 15, lg = l >> 4;
  const int64_t bh = blockIdx.x / C;
  const int chunk = (int)(blockIdx.x % C);
  const int64_t s_lo = (int64_t)chunk * kchunk;
  const int64_t s_hi = (s_lo + kchunk < S) ? (s_lo + kchunk) : S;

  u32x4 uh[NDB], ul[NDB];  // U^T fragments, formed below behind the first tile loads
  float cq;
  const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(Kc + bh * S * D), 0, (int)(S * D * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(Vc + bh * S * D), 0, (int)(S * D * 2), 0x00020000);
  const int64_t ntile = (s_hi - s_lo + 31) / 32;
  // Tile loads: K fragments (key 16 h + lq, dims 32 db + 8 lg) and the V
  // tile's chunks (key j (64 / CPR) + l / CPR, chunk l % CPR).
  auto load = [&](int64_t t, u32x4 (&kk)[2][NDB], u32x4 (&vv)[NV]) {
    const int64_t k0 = s_lo + 32 * t;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t key = k0 + 16 * h + lq;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        kk[h][db] = __builtin_amdgcn_raw_buffer_load_b128(
            kr, key < s_hi ? (uint32_t)((key * D + 32 * db + 8 * lg) * 2) : kAtOutOfRange, 0, 0);
    }
#pragma unroll
    for (int jv = 0; jv < NV; ++jv) {
      const int64_t key = k0 + jv * (64 / CPR) + l / CPR;
      vv[jv] = __builtin_amdgcn_raw_buffer_load_b128(
          vr, key < s_hi ? (uint32_t)((key * D + 8 * (l % CPR)) * 2) : kAtOutOfRange, 0, 0);
    }
  };

  float m = kAtNone, lpart = 0.f;
  floatx4 o[NOB];
#pragma unroll
  for (int ob = 0; ob < NOB; ++ob) o[ob] = floatx4{0.f, 0.f, 0.f, 0.f};

  auto consume = [&](int64_t t, int buf, const u32x4 (&kk)[2][NDB], const u32x4 (&vv)[NV]) {
    // V tile into this wave's LDS buffer (the wave's own LDS operations
    // complete in order, so its reads below see these writes).
    char* vt = v_s[w][buf];
#pragma unroll
    for (int jv = 0; jv < NV; ++jv)
      *(u32x4*)(vt + aq_v_off<D>(jv * (64 / CPR) + l / CPR, 8 * (l % CPR))) = vv[jv];
    // Scores S^T and the keys' sums of squares.
    floatx4 sc[2];
    float rk[2][4];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      sc[h] = floatx4{0.f, 0.f, 0.f, 0.f};
      float ss = 0.f;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        sc[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kk[h][db]),
                                                        __builtin_bit_cast(bf16x8, uh[db]), sc[h],
                                                        0, 0, 0);
        sc[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kk[h][db]),
                                                        __builtin_bit_cast(bf16x8, ul[db]), sc[h],
                                                        0, 0, 0);
        if (NORM) {
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            const float k0 = bf16_lo(kk[h][db][d]), k1 = bf16_hi(kk[h][db][d]);
            ss += k0 * k0 + k1 * k1;
          }
        }
      }
      if (NORM) {
        ss = sum_xor16_32(ss);
        // 1/D is a power of two (exact); v_rsq_f32 for the key's 1/RMS.
        const float r = __builtin_amdgcn_rsqf(ss * (1.0f / D) + eps);
        // this lane's score rows are keys 4 lg + i of the half: their 1/RMS
        // sits on the lanes whose key column lq is 4 lg + i; passed through
        // the wave's LDS slots (its own LDS operations complete in order)
        if (lg == 0) rk_w[w][h][lq] = r;
        const floatx4 r4 = *(const floatx4*)&rk_w[w][h][4 * lg];
#pragma unroll
        for (int i = 0; i < 4; ++i) rk[h][i] = r4[i];
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) rk[h][i] = 1.0f;
      }
    }
    // Online softmax per query column lq over the tile's 32 keys.
    const int64_t k0 = s_lo + 32 * t;
    float p[2][4];
    float mb = kAtNone;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[h][i] = sc[h][i] * cq * rk[h][i];
        if (k0 + 16 * h + 4 * lg + i < s_hi) mb = fmaxf(mb, p[h][i]);
      }
    mb = max_xor16_32(mb);
    const float mn = fmaxf(m, mb);
    const float alpha = __builtin_amdgcn_exp2f(m - mn);
    lpart *= alpha;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[h][i] = (k0 + 16 * h + 4 * lg + i < s_hi) ? __builtin_amdgcn_exp2f(p[h][i] - mn) : 0.f;
        lpart += p[h][i];
      }
    m = mn;
    u32x4 ph, pl;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; i += 2) {
        const uint32_t hi = pack_bf16x2(p[h][i], p[h][i + 1]);
        ph[2 * h + i / 2] = hi;
        pl[2 * h + i / 2] = pack_bf16x2(p[h][i] - bf16_lo(hi), p[h][i + 1] - bf16_hi(hi));
      }
    const at_lds_char* vl = (const at_lds_char*)vt;
    // Rescale O only when some query's maximum moved.  O rows are queries
    // 4 lg + i: their alpha sits on lanes lq = 4 lg + i.
    if (__any(alpha != 1.0f)) {
      float ar[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ar[i] = __shfl(alpha, 4 * lg + i);
#pragma unroll
      for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[ob][i] *= ar[i];
    }
#pragma unroll
    for (int ob = 0; ob < NOB; ++ob) {
      const int col = 16 * ob + 4 * (lq & 3), row = 4 * lg + (lq >> 2);
      const u32x2 v0 = __builtin_bit_cast(
          u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((at_lds_i16x4*)(vl + aq_v_off<D>(row, col))));
      const u32x2 v1 = __builtin_bit_cast(
          u32x2,
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((at_lds_i16x4*)(vl + aq_v_off<D>(row + 16, col))));
      const u32x4 vb = {v0[0], v0[1], v1[0], v1[1]};
      o[ob] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ph),
                                                      __builtin_bit_cast(bf16x8, vb), o[ob], 0, 0,
                                                      0);
      o[ob] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, pl),
                                                      __builtin_bit_cast(bf16x8, vb), o[ob], 0, 0,
                                                      0);
    }
  };

  // The query and the gains are loaded first, the first two tiles right
  // behind them, and U is formed while the tiles are in flight (HBM is
  // busy from the start; the wait for the query's loads does not cover the
  // tiles').
  constexpr u32x4 ones{kBf16OnePair, kBf16OnePair, kBf16OnePair, kBf16OnePair};
  u32x4 qv[NDB], ga[NDB], gb[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int d0 = 32 * db + 8 * lg;
    qv[db] = lq < G ? *(const u32x4*)(Q + (bh * G + lq) * D + d0) : u32x4{0u, 0u, 0u, 0u};
    ga[db] = NORM ? *(const u32x4*)(gq + d0) : ones;
    gb[db] = NORM ? *(const u32x4*)(gk + d0) : ones;
  }
  u32x4 ka[2][NDB], va[NV], kb[2][NDB], vb[NV];
  load(w, ka, va);
  load(w + NWV, kb, vb);

  // U^T fragments (query lq, dims 32 db + 8 lg .. +7) and the query's scale.
  {
    float qss = 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const float q0 = bf16_lo(qv[db][d]), q1 = bf16_hi(qv[db][d]);
        const float u0 = q0 * bf16_lo(ga[db][d]) * bf16_lo(gb[db][d]);
        const float u1 = q1 * bf16_hi(ga[db][d]) * bf16_hi(gb[db][d]);
        const uint32_t hi = pack_bf16x2(u0, u1);
        uh[db][d] = hi;
        ul[db][d] = pack_bf16x2(u0 - bf16_lo(hi), u1 - bf16_hi(hi));
        qss += q0 * q0 + q1 * q1;
      }
    }
    qss += __shfl_xor(qss, 16);
    qss += __shfl_xor(qss, 32);
    // log2(e) folded in: scores in base-2 units, one v_exp_f32 per weight
    cq = lq >= G ? 0.f
         : NORM ? kLog2e / (__fsqrt_rn(__fdiv_rn(qss, (float)D) + eps) * __fsqrt_rn((float)D))
                : kLog2e / __fsqrt_rn((float)D);
  }

  int64_t t = w;
  for (; t + NWV < ntile; t += 2 * NWV) {
    consume(t, 0, ka, va);
    load(t + 2 * NWV, ka, va);
    consume(t + NWV, 1, kb, vb);
    load(t + 3 * NWV, kb, vb);
  }
  if (t < ntile) consume(t, 0, ka, va);

  // This wave's (o, max, sum) per query into LDS.
  lpart += __shfl_xor(lpart, 16);
  lpart += __shfl_xor(lpart, 32);
  if (lg == 0) {
    mm_s[w][lq] = m;
    ml_s[w][lq] = lpart;
  }
#pragma unroll
  for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
    for (int i = 0; i < 4; ++i) mo_s[w][4 * lg + i][16 * ob + lq] = o[ob][i];
  __syncthreads();

  // Thread t merges the waves for (query p / (D/4), dims 4 (p % (D/4)) ..
  // +3), p = t + 256 e (float4 in LDS and in the workspace); the maxima are
  // in base-2 units.
  constexpr int D4 = D / 4;
  constexpr int PER = 16 * D4 / AQ_THREADS;
  floatx4 od[PER];
  float ld[PER], md[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int pp = tid + AQ_THREADS * e, g = pp / D4, d0 = 4 * (pp % D4);
    od[e] = floatx4{0.f, 0.f, 0.f, 0.f};
    ld[e] = 0.f;
    md[e] = kAtNone;
    if (g < G) {
#pragma unroll
      for (int ww = 0; ww < NWV; ++ww) md[e] = fmaxf(md[e], mm_s[ww][g]);
#pragma unroll
      for (int ww = 0; ww < NWV; ++ww) {
        const float a = __builtin_amdgcn_exp2f(mm_s[ww][g] - md[e]);
        const floatx4 v = *(const floatx4*)&mo_s[ww][g][d0];
#pragma unroll
        for (int i = 0; i < 4; ++i) od[e][i] += v[i] * a;
        ld[e] += ml_s[ww][g] * a;
      }
    }
  }
  if (C > 1) {
    // Workspace: o as [slot][query][D], then m and l as [slot][query]; slot =
    // key/value head * C + chunk.  Device-coherent (SC1) stores and loads:
    // the chunks of a head run on any XCD.
    const int64_t nslot = (int64_t)gridDim.x, slot = bh * C + chunk;
    const int64_t m_off = nslot * G * D, l_off = nslot * G * (D + 1);
    const __amdgpu_buffer_rsrc_t pr =
        __builtin_amdgcn_make_buffer_rsrc(part, 0, 0x7fffffff, 0x00020000);
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int pp = tid + AQ_THREADS * e, g = pp / D4, d0 = 4 * (pp % D4);
      if (g < G) {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, od[e]), pr,
                                               (int)(((slot * G + g) * D + d0) * 4), 0,
                                               kAtCoherentDevice);
        if (d0 == 0) {
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(md[e]), pr,
                                                (int)((m_off + slot * G + g) * 4), 0,
                                                kAtCoherentDevice);
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(ld[e]), pr,
                                                (int)((l_off + slot * G + g) * 4), 0,
                                                kAtCoherentDevice);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0)
      last = (__hip_atomic_fetch_add(&cnt[bh], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
              (unsigned)(C - 1));
    __syncthreads();
    if (!last) return;
    // The last arrival adds the chunks in order, 8 at a time, every load of
    // a batch issued before any is used.
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      md[e] = kAtNone;
      od[e] = floatx4{0.f, 0.f, 0.f, 0.f};
      ld[e] = 0.f;
    }
    for (int c0 = 0; c0 < C; c0 += 8) {
      floatx4 oc[PER][8];
      float mc[PER][8], lc[PER][8];
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        const int pp = tid + AQ_THREADS * e, g = pp / D4, d0 = 4 * (pp % D4);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int64_t sl = bh * C + c0 + q;
          const bool in = g < G && c0 + q < C;
          oc[e][q] = in ? __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(
                                                          pr, (int)(((sl * G + g) * D + d0) * 4), 0,
                                                          kAtCoherentDevice))
                        : floatx4{0.f, 0.f, 0.f, 0.f};
          mc[e][q] = in ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                              pr, (int)((m_off + sl * G + g) * 4), 0, kAtCoherentDevice))
                        : kAtNone;
          lc[e][q] = in ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                              pr, (int)((l_off + sl * G + g) * 4), 0, kAtCoherentDevice))
                        : 0.f;
        }
      }
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        float mn = md[e];
#pragma unroll
        for (int q = 0; q < 8; ++q) mn = fmaxf(mn, mc[e][q]);
        const float r = __builtin_amdgcn_exp2f(md[e] - mn);
#pragma unroll
        for (int i = 0; i < 4; ++i) od[e][i] *= r;
        ld[e] *= r;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const float a = __builtin_amdgcn_exp2f(mc[e][q] - mn);
#pragma unroll
          for (int i = 0; i < 4; ++i) od[e][i] += oc[e][q][i] * a;
          ld[e] += lc[e][q] * a;
        }
        md[e] = mn;
      }
    }
    if (tid == 0) __hip_atomic_store(&cnt[bh], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int pp = tid + AQ_THREADS * e, g = pp / D4, d0 = 4 * (pp % D4);
    if (g < G) {
      const uint32_t lo = pack_bf16x2(__fdiv_rn(od[e][0], ld[e]), __fdiv_rn(od[e][1], ld[e]));
      const uint32_t hi = pack_bf16x2(__fdiv_rn(od[e][2], ld[e]), __fdiv_rn(od[e][3], ld[e]));
      *(u32x2*)(O + (bh * G + g) * D + d0) = u32x2{lo, hi};
    }
  }
}


// ---------------------------------------------------------------------------
// Many queries per head (prefill): Q and O are (BH G) x Sq x D, K and V are
// BH x Skv x D (query head qh reads key/value head qh / G); with the causal
// mask query i sees keys 0 .. i + Skv - Sq.  The same two matrix-core
// products as gqa_mfma_kernel, on blocks of 16 query positions:
//   * a workgroup (4 waves) owns 64 QW consecutive positions of one query
//     head, wave w the 16 QW rows from 16 QW w (QW = 1 or 2 blocks of 16);
//     each tile of 32 or 64 keys of K and V is loaded once per workgroup into LDS
//     (double-buffered, one barrier per tile; the next tile travels in
//     registers meanwhile) and read by all four waves;
//   * K rows as the A fragments of the transposed scores come from LDS with
//     16-byte reads (chunk c of key row j stored at c ^ (j mod D/8), so the
//     16 keys of one read hit 16 different chunks); V as in gqa_mfma_kernel;
//   * every wave keeps its own queries' softmax state over all the keys its
//     block needs, so nothing is combined across workgroups: o / sum is
//     stored directly.  Causal workgroups are ordered by their number of
//     key tiles (see the kernel), the others so that an XCD takes a
//     contiguous range of (head, block) pairs.
constexpr int AP_THREADS = 256;
constexpr int AP_QB = 64;  // query positions per workgroup per 16-row block of each wave


template <int D>
__device__ __forceinline__ int ap_k_off(int key, int c) {
  return key * (2 * D) + ((c ^ (key & (D / 8 - 1))) << 4);
}

// QW: 16-row query blocks per wave (1 or 2); with two, each K and V
// fragment read from LDS feeds both blocks' MFMAs, halving the LDS reads
// per query.  The workgroup then owns 64 QW positions, wave w rows
// 16 QW w .. +16 QW - 1.  KT: keys per tile (32 or 64), NH blocks of 16 in
// the scores, NP steps of 32 in the value product.
template <int D, bool NORM, bool CAUSAL, int QW, int KT>
__global__ __launch_bounds__(AP_THREADS, 2) void attn_prefill_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ Kc, const bf16_t* __restrict__ Vc,
    const bf16_t* __restrict__ gq, const bf16_t* __restrict__ gk, bf16_t* __restrict__ O,
    float eps, int64_t Sq, int64_t Skv, int G, int nblk, int order, int splits, int kspan,
    float* __restrict__ part) {
  constexpr int NDB = D / 32;
  constexpr int NOB = D / 16;
  constexpr int CPR = D / 8;
  constexpr int NL = KT * CPR / AP_THREADS;  // K (and V) tile chunks per thread
  constexpr int QB = AP_QB * QW;             // query positions per workgroup
  constexpr int NH = KT / 16, NP = KT / 32;  // 16-key score blocks, 32-key value steps
  __shared__ __attribute__((aligned(16))) char k_s[2][KT * 2 * D];
  __shared__ __attribute__((aligned(16))) char v_s[2][KT * 2 * D];
  __shared__ __attribute__((aligned(16))) float rk_s[2][KT];  // the tile's keys' 1/RMS

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lq = l & 15, lg = l >> 4;
  // Order of the (query head, block) pairs.  order 1 (causal, blocks of
  // unequal length): by length, longest first, the second half of the grid
  // in the reverse order, so that a CU taking workgroups b and b + grid/2
  // gets about the same number of key tiles as every other CU.  Order 0:
  // an XCD (workgroups b % 8) takes a contiguous range of pairs, latest
  // blocks of a head first; 2: as 0 without the XCD remap.
  // With the keys split into `splits` spans of kspan keys, workgroup b takes
  // span b / (grid / splits) of pair b % (grid / splits).
  const int64_t total = (int64_t)gridDim.x / splits;
  const int split = (int)(blockIdx.x / total);
  const int64_t bidx = (int64_t)blockIdx.x - (int64_t)split * total;
  int64_t qh, blk;
  if (order == 1) {
    const int64_t half = (total + 1) / 2, b = bidx;
    const int64_t r = b < half ? b : total - 1 - (b - half);
    const int64_t nh = total / nblk;
    blk = nblk - 1 - r / nh;
    qh = r % nh;
  } else {
    int64_t t = bidx;
    if (order == 0) t = (t & 7) * (total >> 3) + (t >> 3);
    qh = t / nblk;
    blk = nblk - 1 - t % nblk;
  }
  const int64_t h = qh / G;
  const int64_t p0 = blk * QB + 16 * QW * w;  // this wave's first query position
  const int64_t off = Skv - Sq;                // causal horizon of position p: p + off

  // U^T fragments of this wave's queries (block b: positions p0 + 16 b ..):
  // u = q gq gk c, with the query's scale c = log2(e) / (rms(q) sqrt(D))
  // folded in (scores come out in base-2 units, so each softmax weight is
  // one v_exp_f32 of a difference), as two bf16 parts.
  u32x4 uh[QW][NDB], ul[QW][NDB];
#pragma unroll
  for (int b = 0; b < QW; ++b) {
    const int64_t p = p0 + 16 * b + lq;
    const bool qok = p < Sq;
    u32x4 qv[NDB];
    float qss = 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      qv[db] = qok ? *(const u32x4*)(Q + (qh * Sq + p) * D + 32 * db + 8 * lg) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const float q0 = bf16_lo(qv[db][d]), q1 = bf16_hi(qv[db][d]);
        qss += q0 * q0 + q1 * q1;
      }
    }
    qss += __shfl_xor(qss, 16);
    qss += __shfl_xor(qss, 32);
    const float cq = !qok ? 0.f
                     : NORM ? kLog2e / (__fsqrt_rn(__fdiv_rn(qss, (float)D) + eps) * __fsqrt_rn((float)D))
                            : kLog2e / __fsqrt_rn((float)D);
    constexpr u32x4 ones{kBf16OnePair, kBf16OnePair, kBf16OnePair, kBf16OnePair};
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int d0 = 32 * db + 8 * lg;
      const u32x4 ga = NORM ? *(const u32x4*)(gq + d0) : ones;
      const u32x4 gb = NORM ? *(const u32x4*)(gk + d0) : ones;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const float u0 = bf16_lo(qv[db][d]) * bf16_lo(ga[d]) * bf16_lo(gb[d]) * cq;
        const float u1 = bf16_hi(qv[db][d]) * bf16_hi(ga[d]) * bf16_hi(gb[d]) * cq;
        const uint32_t hi = pack_bf16x2(u0, u1);
        uh[b][db][d] = hi;
        ul[b][db][d] = pack_bf16x2(u0 - bf16_lo(hi), u1 - bf16_hi(hi));
      }
    }
  }

  // Keys the block needs: up to the horizon of its last position, within
  // this workgroup's span [kbeg, kbeg + kspan) (all of them without a split).
  int64_t kend = Skv;
  if (CAUSAL) {
    const int64_t last = (blk + 1) * QB - 1 < Sq - 1 ? (blk + 1) * QB - 1 : Sq - 1;
    kend = last + off + 1;
  }
  const int64_t kbeg = (int64_t)split * kspan;
  if (splits > 1 && kbeg + kspan < kend) kend = kbeg + kspan;
  const int64_t ntile = kend > kbeg ? (kend - kbeg + KT - 1) / KT : 0;
  const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(Kc + h * Skv * D), 0, (int)(Skv * D * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(Vc + h * Skv * D), 0, (int)(Skv * D * 2), 0x00020000);
  // Tile loads into registers: chunk e = tid + 256 j is key e / CPR, chunk e % CPR.
  auto load = [&](int64_t tt, u32x4 (&kk)[NL], u32x4 (&vv)[NL]) {
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      const int e = tid + AP_THREADS * j;
      const int64_t key = kbeg + KT * tt + e / CPR;
      const uint32_t o = (tt < ntile && key < kend) ? (uint32_t)((key * D + 8 * (e % CPR)) * 2)
                                                    : kAtOutOfRange;
      kk[j] = __builtin_amdgcn_raw_buffer_load_b128(kr, o, 0, 0);
      vv[j] = __builtin_amdgcn_raw_buffer_load_b128(vr, o, 0, 0);
    }
  };
  // Stores a tile into a stage; with the norm, the CPR threads holding a key
  // row (adjacent lanes) also add its squares and one of them stores the
  // key's 1/RMS (v_rsq_f32; 1/D is a power of two).
  auto store = [&](int stage, const u32x4 (&kk)[NL], const u32x4 (&vv)[NL]) {
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      const int e = tid + AP_THREADS * j, key = e / CPR, c = e % CPR;
      *(u32x4*)(k_s[stage] + ap_k_off<D>(key, c)) = kk[j];
      *(u32x4*)(v_s[stage] + aq_v_off<D>(key, 8 * c)) = vv[j];
      if (NORM) {
        float ss = 0.f;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const float a0 = bf16_lo(kk[j][d]), a1 = bf16_hi(kk[j][d]);
          ss += a0 * a0 + a1 * a1;
        }
        ss = group_sum<CPR>(ss);
        if (c == 0) rk_s[stage][key] = __builtin_amdgcn_rsqf(ss * (1.0f / D) + eps);
      }
    }
  };

  float m[QW], lpart[QW];
  floatx4 o[QW][NOB];
#pragma unroll
  for (int b = 0; b < QW; ++b) {
    m[b] = kAtNone;
    lpart[b] = 0.f;
#pragma unroll
    for (int ob = 0; ob < NOB; ++ob) o[b][ob] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  auto compute = [&](int64_t tt, int stage) {
    const char* ks = k_s[stage];
    const int64_t k0 = kbeg + KT * tt;
    floatx4 sc[QW][NH];
    float rk[NH][4];
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
#pragma unroll
      for (int b = 0; b < QW; ++b) sc[b][hh] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const bf16x8 kf = __builtin_bit_cast(
            bf16x8, *(const u32x4*)(ks + ap_k_off<D>(16 * hh + lq, 4 * db + lg)));
#pragma unroll
        for (int b = 0; b < QW; ++b) {
          sc[b][hh] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              kf, __builtin_bit_cast(bf16x8, uh[b][db]), sc[b][hh], 0, 0, 0);
          sc[b][hh] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              kf, __builtin_bit_cast(bf16x8, ul[b][db]), sc[b][hh], 0, 0, 0);
        }
      }
      // this lane's score rows are keys 16 hh + 4 lg + i
      const floatx4 r4 = NORM ? *(const floatx4*)(&rk_s[stage][16 * hh + 4 * lg])
                              : floatx4{1.f, 1.f, 1.f, 1.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) rk[hh][i] = r4[i];
    }
    // Every key of the tile visible to every query of the wave (the tile
    // ends before kend and, causal, at or before the wave's first horizon):
    // no mask.  Key and position indices fit in 32 bits (Skv D 2 < 2^31).
    const int kt = (int)k0;
    const bool full = kt + KT - 1 < (int)kend && (!CAUSAL || kt + KT - 1 <= (int)(p0 + off));
    u32x4 ph[QW][NP], pl[QW][NP];
#pragma unroll
    for (int b = 0; b < QW; ++b) {
      float p[NH][4];
      float mb = kAtNone;
      if (full) {
#pragma unroll
        for (int hh = 0; hh < NH; ++hh)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            p[hh][i] = sc[b][hh][i] * rk[hh][i];
            mb = fmaxf(mb, p[hh][i]);
          }
      } else {
        // Visible keys of query column lq: below kend and, causal, within its horizon.
        const int horizon = CAUSAL ? (int)(p0 + off) + 16 * b + lq : (int)kend - 1;
        const int kv = horizon < (int)kend - 1 ? horizon : (int)kend - 1;
#pragma unroll
        for (int hh = 0; hh < NH; ++hh)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float v = sc[b][hh][i] * rk[hh][i];
            p[hh][i] = kt + 16 * hh + 4 * lg + i <= kv ? v : -__builtin_inff();
            mb = fmaxf(mb, p[hh][i]);
          }
      }
      mb = max_xor16_32(mb);
      const float mn = fmaxf(m[b], mb);
      const float alpha = __builtin_amdgcn_exp2f(m[b] - mn);
      lpart[b] *= alpha;
      // A masked key's score is -inf: its weight 2^(-inf - mn) is 0.
#pragma unroll
      for (int hh = 0; hh < NH; ++hh)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[hh][i] = __builtin_amdgcn_exp2f(p[hh][i] - mn);
          lpart[b] += p[hh][i];
        }
      m[b] = mn;
      // P fragments of value step hp: keys 32 hp + 4 lg .. +3 and
      // 32 hp + 16 + 4 lg .. +3 of query column lq.
#pragma unroll
      for (int hh = 0; hh < NH; ++hh)
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
          const uint32_t hi = pack_bf16x2(p[hh][i], p[hh][i + 1]);
          ph[b][hh >> 1][2 * (hh & 1) + i / 2] = hi;
          pl[b][hh >> 1][2 * (hh & 1) + i / 2] =
              pack_bf16x2(p[hh][i] - bf16_lo(hi), p[hh][i + 1] - bf16_hi(hi));
        }
      // Rescale O only when some query's maximum moved (once the running
      // maxima settle, most tiles skip it).
      if (__any(alpha != 1.0f)) {
        float ar[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) ar[i] = __shfl(alpha, 4 * lg + i);
#pragma unroll
        for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
          for (int i = 0; i < 4; ++i) o[b][ob][i] *= ar[i];
      }
    }
    const at_lds_char* vl = (const at_lds_char*)v_s[stage];
#pragma unroll
    for (int hp = 0; hp < NP; ++hp)
#pragma unroll
      for (int ob = 0; ob < NOB; ++ob) {
        const int col = 16 * ob + 4 * (lq & 3), row = 32 * hp + 4 * lg + (lq >> 2);
        const u32x2 v0 = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((at_lds_i16x4*)(vl + aq_v_off<D>(row, col))));
        const u32x2 v1 = __builtin_bit_cast(
            u32x2,
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((at_lds_i16x4*)(vl + aq_v_off<D>(row + 16, col))));
        const u32x4 vb4 = {v0[0], v0[1], v1[0], v1[1]};
        const bf16x8 vb = __builtin_bit_cast(bf16x8, vb4);
#pragma unroll
        for (int b = 0; b < QW; ++b) {
          o[b][ob] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ph[b][hp]),
                                                             vb, o[b][ob], 0, 0, 0);
          o[b][ob] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, pl[b][hp]),
                                                             vb, o[b][ob], 0, 0, 0);
        }
      }
  };

  // Pipeline: at the top of iteration tt stage tt & 1 holds tile tt (the
  // barrier publishes it, and every wave is done with the other stage);
  // tile tt + 1 goes from registers into the other stage, tile tt + 2 is
  // loaded into registers, tile tt is multiplied.
  u32x4 kk[NL], vv[NL];
  load(0, kk, vv);
  store(0, kk, vv);
  load(1, kk, vv);
  for (int64_t tt = 0; tt < ntile; ++tt) {
    __syncthreads();
    if (tt + 1 < ntile) store((int)((tt + 1) & 1), kk, vv);
    load(tt + 2, kk, vv);
    compute(tt, (int)(tt & 1));
  }

  // A span of a split call: the raw (o, max, sum) of its keys per query to
  // the workspace -- o as [span][query head][position][D] fp32, then the
  // maxima (base 2) and the sums as [span][query head][position] -- for
  // the combine kernel.  A span past the block's keys stores (0, -1e30, 0).
  if (splits > 1) {
    const int64_t rows = (int64_t)splits * total / nblk * Sq;  // spans x query heads x Sq
    float* po = part;
    float* pm = part + rows * D;
    float* pl = pm + rows;
    const int64_t row0 = ((int64_t)split * (total / nblk) + qh) * Sq;
#pragma unroll
    for (int b = 0; b < QW; ++b) {
      float ls = lpart[b];
      ls += __shfl_xor(ls, 16);
      ls += __shfl_xor(ls, 32);
      const int64_t pc = p0 + 16 * b + lq;  // this lane's query column
      if (lg == 0 && pc < Sq) {
        pm[row0 + pc] = m[b];
        pl[row0 + pc] = ls;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t p = p0 + 16 * b + 4 * lg + i;
        if (p < Sq) {
#pragma unroll
          for (int ob = 0; ob < NOB; ++ob) po[(row0 + p) * D + 16 * ob + lq] = o[b][ob][i];
        }
      }
    }
    return;
  }

  // o / sum for this wave's rows (block b: queries 4 lg + i of its 16).
#pragma unroll
  for (int b = 0; b < QW; ++b) {
    float ls = lpart[b];
    ls += __shfl_xor(ls, 16);
    ls += __shfl_xor(ls, 32);
    float lr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) lr[i] = __shfl(ls, 4 * lg + i);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t p = p0 + 16 * b + 4 * lg + i;
      if (p < Sq) {
#pragma unroll
        for (int ob = 0; ob < NOB; ++ob)
          O[(qh * Sq + p) * D + 16 * ob + lq] = f32_to_bf16(__fdiv_rn(o[b][ob][i], lr[i]));
      }
    }
  }
}

// Spans of a split prefill call: per query row, O = sum_s o_s 2^(m_s - M) /
// sum_s l_s 2^(m_s - M), M = max_s m_s, the spans added in order; 4 dims per
// thread.
constexpr int AC_THREADS = 256;

template <int D>
__global__ __launch_bounds__(AC_THREADS) void attn_prefill_combine_kernel(
    const float* __restrict__ part, bf16_t* __restrict__ O, int64_t rows, int splits) {
  const int64_t idx = (int64_t)blockIdx.x * AC_THREADS + threadIdx.x;
  if (idx >= rows * (D / 4)) return;
  const int64_t r = idx / (D / 4);
  const int d0 = 4 * (int)(idx % (D / 4));
  const float* pm = part + (int64_t)splits * rows * D;
  const float* pl = pm + (int64_t)splits * rows;
  float mx = kAtNone;
  for (int sp = 0; sp < splits; ++sp) mx = fmaxf(mx, pm[(int64_t)sp * rows + r]);
  float l = 0.f, o[4] = {0.f, 0.f, 0.f, 0.f};
  for (int sp = 0; sp < splits; ++sp) {
    const int64_t rr = (int64_t)sp * rows + r;
    const float wgt = __builtin_amdgcn_exp2f(pm[rr] - mx);
    const floatx4 v = *(const floatx4*)(part + rr * D + d0);
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] += v[i] * wgt;
    l += pl[rr] * wgt;
  }
  const uint32_t lo = pack_bf16x2(__fdiv_rn(o[0], l), __fdiv_rn(o[1], l));
  const uint32_t hi = pack_bf16x2(__fdiv_rn(o[2], l), __fdiv_rn(o[3], l));
  *(u32x2*)(O + r * D + d0) = u32x2{lo, hi};
}

}  // namespace rmm

static size_t at_align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Chunks: about one workgroup per CU (256; measured fastest: with more,
// the combine costs more than the extra loads in flight buy), at least 256
// keys per chunk, a whole number of the workgroup's key rounds.
static int attn_group_template(int64_t G) { return G <= 1 ? 1 : G <= 2 ? 2 : G <= 4 ? 4 : 8; }
// Query groups from this size run on the matrix cores (gqa_mfma_kernel).
constexpr int64_t kAttnMfmaMinG = 3;

void rmm_attention_plan(int64_t BH, int64_t S, int64_t D, int splits, AttnPlan* p, int64_t G) {
  using namespace rmm;
  const int gt = attn_group_template(G);
  const int uu = gt == 1 ? AtCfg<1>::U : gt == 2 ? AtCfg<2>::U : gt == 4 ? AtCfg<4>::U : AtCfg<8>::U;
  // keys per workgroup round: the VALU form's blocks, or the MFMA form's
  // 32-key tiles over 4 waves
  const int64_t round = G >= kAttnMfmaMinG ? (int64_t)(AQ_THREADS / 64) * 32
                                          : (int64_t)(AT_THREADS / 64) * uu * (64 / (D / 8));
  int64_t C = splits;
  if (C <= 0) {
    const int64_t want = BH > 0 ? (256 + BH - 1) / BH : 1;
    const int64_t most = (S + 255) / 256;
    C = want < most ? want : most;
  }
  if (C < 1) C = 1;
  if (C > S) C = S;
  int64_t kc = (S + C - 1) / C;
  kc = (kc + round - 1) / round * round;
  p->kchunk = kc;
  p->chunks = (int)((S + kc - 1) / kc);
  p->ws_cnt_off = 0;
  p->ws_part_off = kWsCounterBytes;
  p->ws_bytes = p->chunks > 1 ? p->ws_part_off + at_align256(sizeof(float) * (size_t)BH *
                                                             p->chunks * G * (D + 2))
                              : 0;
}

hipError_t rmm_launch_attention(const AttnArgs& a, const AttnPlan& p, void* ws) {
  using namespace rmm;
  char* base = (char*)ws;
  unsigned* cnt = (ws && p.chunks > 1) ? (unsigned*)(base + p.ws_cnt_off) : nullptr;
  float* part = (ws && p.chunks > 1) ? (float*)(base + p.ws_part_off) : nullptr;
  const dim3 grid((unsigned)(a.BH * p.chunks)), block(AT_THREADS);
  auto launch = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, block, 0, a.stream, (const bf16_t*)a.Q, (const bf16_t*)a.K,
                       (const bf16_t*)a.V, (const bf16_t*)a.gq, (const bf16_t*)a.gk, (bf16_t*)a.O,
                       a.eps, a.S, p.kchunk, p.chunks, (int)a.G, cnt, part);
  };
  auto by_dim = [&](auto gt) {
    constexpr int GT = decltype(gt)::value;
    if (a.D == 128)
      a.norm ? launch(qknorm_attention_kernel<128, true, GT>)
             : launch(qknorm_attention_kernel<128, false, GT>);
    else
      a.norm ? launch(qknorm_attention_kernel<64, true, GT>)
             : launch(qknorm_attention_kernel<64, false, GT>);
  };
  if ((a.D != 64 && a.D != 128) || a.G < 1 || a.G > 16) return hipErrorInvalidValue;
  if (a.G >= kAttnMfmaMinG) {
    if (a.D == 128)
      a.norm ? launch(gqa_mfma_kernel<128, true>) : launch(gqa_mfma_kernel<128, false>);
    else
      a.norm ? launch(gqa_mfma_kernel<64, true>) : launch(gqa_mfma_kernel<64, false>);
    return hipGetLastError();
  }
  switch (attn_group_template(a.G)) {
    case 1: by_dim(std::integral_constant<int, 1>{}); break;
    case 2: by_dim(std::integral_constant<int, 2>{}); break;
    case 4: by_dim(std::integral_constant<int, 4>{}); break;
    default: by_dim(std::integral_constant<int, 8>{}); break;
  }
  return hipGetLastError();
}

void rmm_attention_prefill_plan(int64_t BHG, int64_t Sq, int64_t Skv, int64_t D, int causal,
                                int splits, bool have_ws, AttnPrefillPlan* p) {
  using namespace rmm;
  // Two 16-row query blocks per wave when the 128-position workgroups
  // number at least one per CU (blocks of equal length) or, causal, two
  // rounds of the two that fit on each CU: with fewer, the 64-position
  // blocks (three per CU) balance the unequal lengths better.  Measured,
  // causal, D = 128: 32 heads x 2048 129.6 us (one block per wave) against
  // 149.0 (two); 32 x 4096 426.1 against 415.6; non-causal 32 x 2048 218.8
  // against 167.3.
  const int64_t wg2 = BHG * ((Sq + 2 * AP_QB - 1) / (2 * AP_QB));
  p->qw = wg2 >= (causal ? 4 * 256 : 256) ? 2 : 1;
  p->nblk = (Sq + p->qw * AP_QB - 1) / (p->qw * AP_QB);
  const int64_t grid = BHG * p->nblk;
  // Split of the keys into spans (a whole number of 64-key tiles each),
  // combined by a second kernel: with a workspace and no forced count, when
  // the query blocks alone make one workgroup per CU or fewer, up to three
  // workgroups per CU with spans of at least 512 keys.  Measured (causal
  // unless noted, D = 128): 8 x 4 heads, 512 queries over 8192 keys 261 ->
  // 176 us (3 spans); 256 queries 231 -> 98 us (6); 128 over 16384 keys 450
  // -> 103 us (8); 16 x 4 heads, 512 over 8192, D = 64, non-causal 272 ->
  // 177 us (3).
  int64_t s = splits;
  if (s == 0) {
    s = 1;
    if (have_ws && grid <= 256) {
      s = 768 / (grid > 0 ? grid : 1);
      if (s > Skv / 512) s = Skv / 512;
      if (s > 8) s = 8;
      if (s < 1) s = 1;
    }
  }
  int64_t span = (Skv + s - 1) / s;
  span = (span + 63) / 64 * 64;
  p->kspan = span;
  p->splits = (int)((Skv + span - 1) / span);
  // 64-key tiles (half the barriers and softmax rounds per key; 221 VGPRs
  // and 64 KB of LDS: two workgroups per CU instead of three) when the grid
  // holds at most one workgroup per CU anyway.  Measured: 8 x 4 heads, 512
  // queries over 8192 keys 276.6 -> 237.5 us; 32 heads x 2048 causal
  // (1024 workgroups) 116.4 -> 120.6 us.
  p->kt = p->qw == 1 && grid * p->splits <= 256 ? 64 : 32;
  // Workspace (split calls): the counter region stays unused, then o
  // ([span][row][D]) and the spans' maxima and sums ([span][row]), fp32.
  p->ws_part_off = kWsCounterBytes;
  p->ws_bytes = p->splits > 1
                    ? kWsCounterBytes + (size_t)p->splits * (size_t)(BHG * Sq) * (size_t)(D + 2) * 4
                    : 0;
}

hipError_t rmm_launch_attention_prefill(const AttnArgs& a, int64_t Sq, int64_t Skv, int causal,
                                        const AttnPrefillPlan& p, void* ws) {
  using namespace rmm;
  const int qw = p.qw, kt = p.kt, splits = p.splits;
  const int64_t nblk = p.nblk;
  const int64_t grid = a.BH * a.G * nblk * splits;
  if (splits > 1 && !ws) return hipErrorInvalidValue;
  float* part = splits > 1 ? (float*)((char*)ws + p.ws_part_off) : nullptr;
  const int order = causal ? 1 : ((grid / splits) % 8 == 0 ? 0 : 2);
  auto launch = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(AP_THREADS), 0, a.stream,
                       (const bf16_t*)a.Q, (const bf16_t*)a.K, (const bf16_t*)a.V,
                       (const bf16_t*)a.gq, (const bf16_t*)a.gk, (bf16_t*)a.O, a.eps, Sq, Skv,
                       (int)a.G, (int)nblk, order, splits, (int)p.kspan, part);
  };
  auto by_qw = [&](auto d, auto norm, auto cz) {
    constexpr int D = decltype(d)::value;
    constexpr bool NORM = decltype(norm)::value, CAUSAL = decltype(cz)::value;
    if (qw == 2)
      launch(attn_prefill_kernel<D, NORM, CAUSAL, 2, 32>);
    else if (kt == 64)
      launch(attn_prefill_kernel<D, NORM, CAUSAL, 1, 64>);
    else
      launch(attn_prefill_kernel<D, NORM, CAUSAL, 1, 32>);
  };
  auto by_mask = [&](auto d, auto norm) {
    causal ? by_qw(d, norm, std::true_type{}) : by_qw(d, norm, std::false_type{});
  };
  auto by_norm = [&](auto d) {
    a.norm ? by_mask(d, std::true_type{}) : by_mask(d, std::false_type{});
  };
  if (a.D == 128)
    by_norm(std::integral_constant<int, 128>{});
  else if (a.D == 64)
    by_norm(std::integral_constant<int, 64>{});
  else
    return hipErrorInvalidValue;
  if (splits > 1) {
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int64_t rows = a.BH * a.G * Sq;
    const dim3 cgrid((unsigned)((rows * (a.D / 4) + AC_THREADS - 1) / AC_THREADS));
    if (a.D == 128)
      hipLaunchKernelGGL(attn_prefill_combine_kernel<128>, cgrid, dim3(AC_THREADS), 0, a.stream,
                         (const float*)part, (bf16_t*)a.O, rows, splits);
    else
      hipLaunchKernelGGL(attn_prefill_combine_kernel<64>, cgrid, dim3(AC_THREADS), 0, a.stream,
                         (const float*)part, (bf16_t*)a.O, rows, splits);
  }
  return hipGetLastError();
}
