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

}  // namespace rmm

static size_t at_align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Chunks: about one workgroup per CU (256; measured fastest: with more,
// the combine costs more than the extra loads in flight buy), at least 256
// keys per chunk, a whole number of the workgroup's key rounds.
static int attn_group_template(int64_t G) { return G <= 1 ? 1 : G <= 2 ? 2 : G <= 4 ? 4 : 8; }

void rmm_attention_plan(int64_t BH, int64_t S, int64_t D, int splits, AttnPlan* p, int64_t G) {
  using namespace rmm;
  const int gt = attn_group_template(G);
  const int uu = gt == 1 ? AtCfg<1>::U : gt == 2 ? AtCfg<2>::U : gt == 4 ? AtCfg<4>::U : AtCfg<8>::U;
  const int64_t round = (int64_t)(AT_THREADS / 64) * uu * (64 / (D / 8));  // keys per WG round
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
  if ((a.D != 64 && a.D != 128) || a.G < 1 || a.G > 8) return hipErrorInvalidValue;
  switch (attn_group_template(a.G)) {
    case 1: by_dim(std::integral_constant<int, 1>{}); break;
    case 2: by_dim(std::integral_constant<int, 2>{}); break;
    case 4: by_dim(std::integral_constant<int, 4>{}); break;
    default: by_dim(std::integral_constant<int, 8>{}); break;
  }
  return hipGetLastError();
}
