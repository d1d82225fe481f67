// Decode variant for fp32 storage: few rows (M <= 16), bandwidth-bound,
// fp32 arithmetic throughout (no bf16 rounding anywhere).
//
// Same decomposition as the bf16 decode kernel, on the vector ALUs: the two
// k-sums of the fused form -- sum_k (X g)[m,k] W[k,n] and sum_k X[m,k]^2 --
// are split along K across workgroups, the partial sums are added exactly
// as partial sums, and the division by the RMS happens once at the end (the
// abstract expression E(O) = sum(k, div(mul(I1,I2), I3)) of the Mirage paper
// review, "核心公式", with the k-independent divisor moved outside the sum).
//
//   * a workgroup (256 threads = 8 k-groups x 32 four-column chunks) owns a
//     128-column tile of Y and a range of K, walked in chunks of KC = 8 KPT
//     rows; a thread loads its KPT rows of W (4 columns, 16 bytes each: 32
//     threads read one 512-byte row segment), and the next chunk's loads are
//     issued before the current chunk is multiplied;
//   * the workgroup stages X g (fp32 product) for the chunk in LDS and adds
//     X^2 to the row sums of squares (16 threads per row);
//   * each thread keeps MR x 4 fp32 accumulators and adds (X g)[m,k] * W[k,n]
//     with fused multiply-adds; the X g values are LDS broadcasts (the 32
//     threads of a k-group read the same word);
//   * the 8 k-groups' sums are added through LDS in a fixed order; with
//     several K ranges the partials go to the workspace and the last
//     workgroup to arrive at a tile (arrival counter) adds them in split
//     order, so the result does not depend on arrival order;
//   * epilogue: Y = acc / sqrt(ss / K + eps), stored as fp32.
#include "rmm_device.h"

namespace rmm {

constexpr int D32_COLS = 128;
constexpr int D32_THREADS = 256;
constexpr int D32_KG = 8;  // k-groups
constexpr int D32_MAXR = 16;
// Workspace accesses of the split-K combine: device-scope coherent (SC1),
// as in the bf16 decode kernel (the XCDs do not share an L2).
constexpr int kD32Coherent = 16;

template <int MR, int KPT>
struct D32Smem {
  float xg[2][MR][D32_KG * KPT];  // X g of a chunk, double-buffered
  float red[D32_KG][MR][D32_COLS];
  float ss[MR];
  float inv[MR];
  int last;
};

template <int MR, int KPT>
__global__ __launch_bounds__(D32_THREADS) void decode32_kernel(
    const float* __restrict__ X, const float* __restrict__ g, const float* __restrict__ W,
    float* __restrict__ Y, float eps, int M, int64_t N, int64_t K, int64_t krange, int S,
    int tiles, unsigned* __restrict__ cnt, float* __restrict__ ssq_ws, float* __restrict__ part_ws,
    int norm) {
  constexpr int KC = D32_KG * KPT;  // k rows per chunk
  __shared__ D32Smem<MR, KPT> sm;
  const int tid = threadIdx.x, kg = tid >> 5, c = tid & 31;
  const int tile = blockIdx.x / S, split = blockIdx.x % S;
  const int64_t n = (int64_t)tile * D32_COLS + 4 * c;
  const bool col_ok = n < N;  // N % 4 == 0: a 4-column chunk is all in or all out
  const int64_t k_lo = (int64_t)split * krange;
  const int64_t k_hi = (k_lo + krange < K) ? (k_lo + krange) : K;
  // Staging: thread -> row sr = tid / 16, k offsets (tid % 16) + 16 j.
  const int sr = tid >> 4, sk = tid & 15;

  float acc[MR][4];
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[m][q] = 0.f;
  float ssl = 0.f;

  auto load = [&](int64_t kb, float4 (&wv)[KPT]) {
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int64_t k = kb + kg * KPT + j;
      wv[j] = (k < k_hi && col_ok) ? *(const float4*)(W + k * N + n)
                                   : float4{0.f, 0.f, 0.f, 0.f};
    }
  };
  auto stage = [&](int64_t kb, int buf) {
    if (sr < MR) {
#pragma unroll
      for (int j = 0; j < KC / 16; ++j) {
        const int kk = sk + 16 * j;
        const int64_t k = kb + kk;
        const bool in = k < k_hi;
        const float x = (in && sr < M) ? X[(int64_t)sr * K + k] : 0.f;
        const float gv = in ? (norm ? g[k] : 1.0f) : 0.f;
        sm.xg[buf][sr][kk] = x * gv;
        ssl = fmaf(x, x, ssl);
      }
    }
  };
  auto multiply = [&](int buf, const float4 (&wv)[KPT]) {
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int kk = kg * KPT + j;
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        const float xv = sm.xg[buf][m][kk];
        acc[m][0] = fmaf(xv, wv[j].x, acc[m][0]);
        acc[m][1] = fmaf(xv, wv[j].y, acc[m][1]);
        acc[m][2] = fmaf(xv, wv[j].z, acc[m][2]);
        acc[m][3] = fmaf(xv, wv[j].w, acc[m][3]);
      }
    }
  };

  // Pairs of chunks with two register stages: the loads of the next chunk
  // are in flight while the current one is multiplied; the X g buffers
  // alternate, so one barrier per chunk publishes the staging (the barrier
  // of the next chunk orders its overwrite after this chunk's reads).
  float4 wa[KPT], wb[KPT];
  load(k_lo, wa);
  for (int64_t kb = k_lo; kb < k_hi; kb += 2 * KC) {
    load(kb + KC, wb);
    stage(kb, 0);
    __syncthreads();
    multiply(0, wa);
    if (kb + KC >= k_hi) break;
    load(kb + 2 * KC, wa);
    stage(kb + KC, 1);
    __syncthreads();
    multiply(1, wb);
  }

  // Row sums of squares: the 16 staging threads of a row are adjacent lanes.
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) ssl += __shfl_xor(ssl, o);
  __syncthreads();  // every thread is done with the staging buffers
  if (sk == 0 && sr < MR) sm.ss[sr] = ssl;
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int q = 0; q < 4; ++q) sm.red[kg][m][4 * c + q] = acc[m][q];
  __syncthreads();

  // Sum of the k-groups in a fixed order: thread -> entries e = tid + 256 u,
  // row e / 128, column e % 128 (MR * 128 entries, PER per thread).
  constexpr int PER = MR * D32_COLS / D32_THREADS;
  static_assert(PER * D32_THREADS == MR * D32_COLS, "whole entries per thread");
  float v[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int e = tid + D32_THREADS * u, er = e / D32_COLS, ec = e % D32_COLS;
    v[u] = 0.f;
#pragma unroll
    for (int q = 0; q < D32_KG; ++q) v[u] += sm.red[q][er][ec];
  }
  float ssw = tid < MR ? sm.ss[tid] : 0.f;

  if (S > 1) {
    const int64_t slot = (int64_t)split * tiles + tile;
    const int64_t nslots = (int64_t)S * tiles;
    const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
        part_ws, 0, (int)(nslots * MR * D32_COLS * 4), 0x00020000);
#pragma unroll
    for (int u = 0; u < PER; ++u)
      __builtin_amdgcn_raw_buffer_store_b32(
          __float_as_uint(v[u]), prs, (int)((slot * MR * D32_COLS + tid + D32_THREADS * u) * 4), 0,
          kD32Coherent);
    if (tid < MR)
      __hip_atomic_store(&ssq_ws[slot * MR + tid], ssw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0)
      sm.last = (__hip_atomic_fetch_add(&cnt[tile], 1u, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT) == (unsigned)(S - 1));
    __syncthreads();
    if (!sm.last) return;
    // Last arrival: add the S partials in split order (deterministic), with
    // the loads of up to 4 splits in flight at once.
#pragma unroll
    for (int u = 0; u < PER; ++u) v[u] = 0.f;
    ssw = 0.f;
    for (int s0 = 0; s0 < S; s0 += 4) {
      float buf[4][PER], sb[4];
#pragma unroll
      for (int uu = 0; uu < 4; ++uu) {
        const int64_t sl = (int64_t)(s0 + uu) * tiles + tile;
        const bool ok = s0 + uu < S;
#pragma unroll
        for (int u = 0; u < PER; ++u)
          buf[uu][u] = ok ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                                prs, (int)((sl * MR * D32_COLS + tid + D32_THREADS * u) * 4), 0,
                                kD32Coherent))
                          : 0.f;
        sb[uu] = (ok && tid < MR) ? __hip_atomic_load(&ssq_ws[sl * MR + tid], __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT)
                                  : 0.f;
      }
#pragma unroll
      for (int uu = 0; uu < 4; ++uu) {
#pragma unroll
        for (int u = 0; u < PER; ++u) v[u] += buf[uu][u];
        ssw += sb[uu];
      }
    }
    if (tid == 0) __hip_atomic_store(&cnt[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (tid < MR) sm.inv[tid] = norm ? inv_rms(ssw, K, eps) : 1.0f;
  __syncthreads();
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int e = tid + D32_THREADS * u, er = e / D32_COLS, ec = e % D32_COLS;
    const int64_t col = (int64_t)tile * D32_COLS + ec;
    if (er < M && col < N) Y[(int64_t)er * N + col] = v[u] * sm.inv[er];
  }
}

}  // namespace rmm

static size_t align256_32(size_t x) { return (x + 255) & ~(size_t)255; }

// K per workgroup: a multiple of the chunk; the split count puts about one
// workgroup on each CU, the chunk is the smallest of 64/128/256 rows that
// covers K in that many splits.
void rmm_decode32_plan(int64_t M, int64_t N, int64_t K, int splits, Decode32Plan* p) {
  using namespace rmm;
  p->mr = M <= 8 ? 8 : 16;
  p->tiles = (N + D32_COLS - 1) / D32_COLS;
  int64_t s = splits < 1 ? 1 : splits;
  const int64_t per = (K + s - 1) / s;
  // chunks of 64 rows (8 per k-group; two chunks of 16-byte loads in flight)
  p->kc = 64;
  p->krange = ((per + p->kc - 1) / p->kc) * p->kc;
  p->splits = (int)((K + p->krange - 1) / p->krange);
  p->ws_cnt_off = 0;
  p->ws_ssq_off = kWsCounterBytes;
  p->ws_part_off = p->ws_ssq_off + align256_32(sizeof(float) * (size_t)p->splits * p->tiles * p->mr);
  p->ws_bytes = p->splits > 1
                    ? p->ws_part_off + align256_32(sizeof(float) * (size_t)p->splits * p->tiles *
                                                   p->mr * D32_COLS)
                    : 0;
}

template <int MR, int KPT>
static void launch_decode32_t(const RmmArgs& a, const Decode32Plan& p, void* ws) {
  using namespace rmm;
  char* base = (char*)ws;
  unsigned* cnt = ws ? (unsigned*)(base + p.ws_cnt_off) : nullptr;
  float* ssq = ws ? (float*)(base + p.ws_ssq_off) : nullptr;
  float* part = ws ? (float*)(base + p.ws_part_off) : nullptr;
  const unsigned grid = (unsigned)(p.tiles * p.splits);
  hipLaunchKernelGGL((decode32_kernel<MR, KPT>), dim3(grid), dim3(D32_THREADS), 0, a.stream,
                     (const float*)a.X, (const float*)a.g, (const float*)a.W1, (float*)a.Y, a.eps,
                     (int)a.M, a.N, a.K, p.krange, p.splits, (int)p.tiles, cnt, ssq, part, a.norm);
}

hipError_t rmm_launch_decode32(const RmmArgs& a, const Decode32Plan& p, void* ws) {
  if (a.gated || a.R > 0 || a.M > 16) return hipErrorInvalidValue;
  if (p.splits > 1 && !ws) return hipErrorInvalidValue;
  if (p.kc != 64) return hipErrorInvalidValue;
  if (p.mr == 8)
    launch_decode32_t<8, 8>(a, p, ws);
  else
    launch_decode32_t<16, 8>(a, p, ws);
  return hipGetLastError();
}
