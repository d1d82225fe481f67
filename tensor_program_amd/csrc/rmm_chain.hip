// A chain of fused RMSNorm+MatMul layers in one persistent launch:
//
//   X_{l+1} = RMSNorm(X_l; g_l, eps) W_l,   l = 0 .. L-1,   W_l: K x K,
//
// the multi-layer decode that the Mirage pages' persistent runtime (the
// "Mirage Persistent Kernel" section of the first page) turns into one
// kernel: instead of one launch per layer, every workgroup stays resident
// and moves from layer to layer, waiting on a device-side counter for the
// layer before to finish.  The weights do not depend on the activations, so
// each workgroup issues half of its next layer's W loads before it waits
// (the other half behind that layer's X loads, once the wait is over): the
// W stream of layer l+1 overlaps the tail (split-K combine, epilogue) of
// layer l that a chain of separate launches would expose, without flooding
// the memory system while that latency-bound combine runs.
//
// Per layer the work is the decode kernel's: a workgroup (8 waves) owns a
// 128-column tile and a K chunk of at most 1024 rows (one staged segment),
// stages bf16(X_l g_l) in LDS while adding X_l^2 to the row sums of squares,
// streams its W rows through registers into v_mfma_f32_16x16x32_bf16, and
// the last workgroup to arrive at a tile adds the fp32 partials of all
// chunks and divides by the RMS (the abstract expression
// E(O) = sum(k, div(mul(I1,I2), I3)) of the paper review's "核心公式", with
// the k-independent divisor moved outside the sum).  That workgroup writes
// the tile of X_{l+1} with device-coherent stores and then counts the tile
// as done (a per-tile count of finished layers).  A workgroup starts layer
// l+1 once the tiles of X_{l+1} its K chunk reads (kchunk / 128 of them)
// have finished layer l: it never waits on tiles it does not read.
//
// The grid has at most one workgroup per CU (the launcher checks the
// device's CU count) and each workgroup needs a whole CU's LDS share, so on
// an otherwise idle GPU every workgroup is resident at once and a workgroup
// waiting on the counter never blocks one that has not started.  (A
// cooperative launch, which guarantees residency, cost ~20 us per call on
// this stack.)  The wait is bounded anyway: after kChainSpinMax polls it sets
// the flag word of the workspace and goes on -- wrong results, never a hang
// -- which is what happens if other kernels hold CUs during the call.
#include <hip/hip_runtime.h>

#include "rmm_decode_core.h"

namespace rmm {

constexpr int CH_WV = 8;
constexpr int CH_NT = CH_WV * 64;
constexpr int CH_SEG = 1024;  // k rows staged per chunk: the whole chunk
constexpr int kChainSpinMax = 1 << 20;

struct ChainSmem {
  floatx4 red[CH_WV][8][64];    // per-wave accumulators [wave][c][lane]
  u32x4 xg[CH_SEG / 8][16];     // A operand, [k/8][row]
  float ssr[16];
  float inv[16];
  int last;
  int reset;
};

__global__ __launch_bounds__(CH_NT) void chain_kernel(
    const bf16_t* __restrict__ X0, const bf16_t* __restrict__ G, const bf16_t* __restrict__ W,
    bf16_t* __restrict__ Xs, float eps, int M, int64_t K, int L, int64_t kchunk, int S, int tiles,
    int xcd_remap, unsigned* __restrict__ cnt, unsigned* __restrict__ done,
    unsigned* __restrict__ flag, float* __restrict__ ssq_ws, float* __restrict__ part_ws) {
  constexpr int ROWS = 16, STEP = 32 * CH_WV, TPR = CH_NT / ROWS, NU = CH_SEG / 8 / TPR;
  __shared__ ChainSmem sm;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, q = l >> 4, p = l & 15;
  // Per-tile counts of finished layers follow the call-wide count and the
  // flag word.
  unsigned* done_t = done + 2;
  if (tid == 0) sm.reset = 0;
  int tile, split;
  {
    const int bid = blockIdx.x;
    if (xcd_remap) {
      const int xcd = bid & 7, j = bid >> 3;
      tile = (j / S) * 8 + xcd;
      split = j % S;
    } else {
      tile = bid / S;
      split = bid % S;
    }
  }
  const int64_t N = K;
  const int64_t col = (int64_t)tile * DEC_COLS + 8 * p;
  const bool col_ok = col < N;
  const int64_t k_lo = (int64_t)split * kchunk;
  const int64_t k_hi = (k_lo + kchunk < K) ? (k_lo + kchunk) : K;
  const int nsteps = (int)((k_hi - k_lo + STEP - 1) / STEP);
  const int srow = tid / TPR, sj = tid % TPR;
  const int64_t slot = (int64_t)split * tiles + tile;
  constexpr int E4 = 8 * 64;  // floatx4 per partial: one per thread
  const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
      part_ws, 0, (int)((int64_t)S * tiles * E4 * 16), 0x00020000);
  floatx4* red0 = &sm.red[0][0][0];

  // Sources of a layer: W_l, X_l (the previous layer's output), g_l.
  auto sources = [&](int layer) {
    DecodeSrc src;
    const bf16_t* Xl = layer == 0 ? X0 : Xs + (int64_t)(layer - 1) * M * K;
    src.w1 = __builtin_amdgcn_make_buffer_rsrc((void*)(W + (int64_t)layer * K * K), 0, (int)(K * K * 2),
                                               0x00020000);
    src.w3 = src.w1;
    src.x = __builtin_amdgcn_make_buffer_rsrc((void*)Xl, 0, (int)((int64_t)M * K * 2), 0x00020000);
    src.g = __builtin_amdgcn_make_buffer_rsrc((void*)(G + (int64_t)layer * K), 0, (int)(K * 2), 0x00020000);
    return src;
  };
  // The W stages of a layer do not depend on its input.  Every workgroup
  // issues the first one as soon as its part of the layer before is counted
  // (a combining workgroup: right behind its tile stores), and the second
  // after the wait, behind the layer's X loads.  Issuing both before the
  // wait was slower (8 layers of 4096 x 4096: 110.1 vs 103.1 us): 33 MB of
  // W requests in flight queue the latency-bound combine, count and reload
  // of x behind them.
  u32x4 wa[1][8], wb[1][8];
  {
    const DecodeSrc src0 = sources(0);
    decode_load<1>(wa, src0, N, k_lo + 32 * w + 8 * q, k_hi, col, col_ok);
    decode_load<1>(wb, src0, N, k_lo + STEP + 32 * w + 8 * q, k_hi, col, col_ok);
  }

  for (int layer = 0; layer < L; ++layer) {
    bf16_t* Yl = Xs + (int64_t)layer * M * K;
    const DecodeSrc src = sources(layer);

    if (layer > 0) {
      // Thread j polls the count of tile j0 + j of X_l (columns k_lo ..
      // k_hi of the layer before's output).
      const int j0 = (int)(k_lo / DEC_COLS), nj = (int)((k_hi - k_lo + DEC_COLS - 1) / DEC_COLS);
      if (tid < nj) {
        for (int it = 0;; ++it) {
          if (__hip_atomic_load(&done_t[j0 + tid], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >=
              (unsigned)layer)
            break;
          if (it >= kChainSpinMax) {
            __hip_atomic_store(flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
          }
          __builtin_amdgcn_s_sleep(16);
        }
      }
      __syncthreads();
    }

    // Stage bf16(X_l g_l) for the chunk.  X_l (l > 0) was written during this
    // call on other XCDs: device-coherent loads.
    float ssl = 0.f;
    {
      u32x4 xs[NU], gs[NU];
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int64_t k = k_lo + 8 * (sj + TPR * u);
        const bool ok = k < k_hi;
        xs[u] = __builtin_amdgcn_raw_buffer_load_b128(
            src.x, (ok && srow < M) ? (uint32_t)(((int64_t)srow * K + k) * 2) : kOutOfRange, 0,
            kCoherentDevice);
        gs[u] = __builtin_amdgcn_raw_buffer_load_b128(src.g, ok ? (uint32_t)(k * 2) : kOutOfRange, 0, 0);
      }
      if (layer > 0) decode_load<1>(wb, src, N, k_lo + STEP + 32 * w + 8 * q, k_hi, col, col_ok);
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        u32x4 av;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const float x0 = bf16_lo(xs[u][d]), x1 = bf16_hi(xs[u][d]);
          const float g0 = bf16_lo(gs[u][d]), g1 = bf16_hi(gs[u][d]);
          ssl += x0 * x0 + x1 * x1;
          av[d] = pack_bf16x2(x0 * g0, x1 * g1);
        }
        sm.xg[sj + TPR * u][srow] = av;
      }
    }
    __syncthreads();

    floatx4 acc[1][1][8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[0][0][c] = floatx4{0.f, 0.f, 0.f, 0.f};
    int s = 0;
    for (; s + 2 <= nsteps; s += 2) {
      u32x4 a[1];
      a[0] = sm.xg[(s * STEP + 32 * w + 8 * q) >> 3][p];
      decode_mma<1, 1>(wa, a, acc);
      decode_load<1>(wa, src, N, k_lo + (int64_t)(s + 2) * STEP + 32 * w + 8 * q, k_hi, col, col_ok);
      a[0] = sm.xg[((s + 1) * STEP + 32 * w + 8 * q) >> 3][p];
      decode_mma<1, 1>(wb, a, acc);
      decode_load<1>(wb, src, N, k_lo + (int64_t)(s + 3) * STEP + 32 * w + 8 * q, k_hi, col, col_ok);
    }
    if (s < nsteps) {
      u32x4 a[1];
      a[0] = sm.xg[(s * STEP + 32 * w + 8 * q) >> 3][p];
      decode_mma<1, 1>(wa, a, acc);
    }

    // Row sums of squares: the TPR staging threads of a row are adjacent lanes.
#pragma unroll
    for (int o = 1; o < TPR; o <<= 1) ssl += __shfl_xor(ssl, o);
    if (sj == 0) sm.ssr[srow] = ssl;
#pragma unroll
    for (int c = 0; c < 8; ++c) sm.red[w][c][l] = acc[0][0][c];
    __syncthreads();
    floatx4 v = red0[tid];
#pragma unroll
    for (int ww = 1; ww < CH_WV; ++ww) v += red0[ww * E4 + tid];
    float ssw = tid < ROWS ? sm.ssr[tid] : 0.f;

    bool last = true;
    if (S > 1) {
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), prs,
                                             (int)((slot * E4 + tid) * 16), 0, kCoherentDevice);
      if (tid < ROWS)
        __hip_atomic_store(&ssq_ws[slot * ROWS + tid], ssw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (tid == 0)
        sm.last = (__hip_atomic_fetch_add(&cnt[tile], 1u, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT) == (unsigned)(S - 1));
      __syncthreads();
      last = sm.last;
      if (last) {
        v = floatx4{0.f, 0.f, 0.f, 0.f};
        ssw = 0.f;
        for (int s0 = 0; s0 < S; s0 += 8) {
          u32x4 buf[8];
          float sb[8];
#pragma unroll
          for (int uu = 0; uu < 8; ++uu) {
            const int64_t sl = (int64_t)(s0 + uu) * tiles + tile;
            const bool ok = s0 + uu < S;
            buf[uu] = ok ? __builtin_amdgcn_raw_buffer_load_b128(prs, (int)((sl * E4 + tid) * 16), 0,
                                                                 kCoherentDevice)
                         : u32x4{0u, 0u, 0u, 0u};
            sb[uu] = (ok && tid < ROWS) ? __hip_atomic_load(&ssq_ws[sl * ROWS + tid], __ATOMIC_RELAXED,
                                                            __HIP_MEMORY_SCOPE_AGENT)
                                        : 0.f;
          }
#pragma unroll
          for (int uu = 0; uu < 8; ++uu) {
            v += __builtin_bit_cast(floatx4, buf[uu]);
            ssw += sb[uu];
          }
        }
        if (tid == 0) __hip_atomic_store(&cnt[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    auto prefetch_next = [&] {
      const DecodeSrc nsrc = sources(layer + 1);
      decode_load<1>(wa, nsrc, N, k_lo + 32 * w + 8 * q, k_hi, col, col_ok);
    };
    if (layer + 1 < L && !last) prefetch_next();
    if (last) {
      __syncthreads();  // every thread is done reading sm.red
      red0[tid] = v;
      if (tid < ROWS) sm.inv[tid] = inv_rms(ssw, K, eps);
      __syncthreads();
      // Epilogue: thread -> row 4 (lane/16) + r, columns 8 (lane%16) .. +7 of
      // the tile (element (c, lane, r) is float (c*64 + lane)*4 + r).
      const float* redf = (const float*)red0;
      const __amdgpu_buffer_rsrc_t yrs =
          __builtin_amdgcn_make_buffer_rsrc((void*)Yl, 0, (int)((int64_t)M * K * 2), 0x00020000);
      if (tid < 256) {
        const int ln = tid & 63, r = tid >> 6;
        const int row = 4 * (ln >> 4) + r;
        const int64_t cc = (int64_t)tile * DEC_COLS + 8 * (ln & 15);
        if (row < M && cc < N) {
          const float inv = sm.inv[row];
          u32x4 out;
#pragma unroll
          for (int c = 0; c < 8; c += 2)
            out[c >> 1] = pack_bf16x2(redf[((c * 64) + ln) * 4 + r] * inv,
                                      redf[(((c + 1) * 64) + ln) * 4 + r] * inv);
          __builtin_amdgcn_raw_buffer_store_b128(out, yrs, (int)((row * K + cc) * 2), 0, kCoherentDevice);
        }
      }
      // The tile is visible device-wide before it is counted as done.  The
      // next layer's first W loads go out behind the tile's stores; vector
      // memory operations complete in issue order, so waiting until only
      // those 8 loads may be outstanding waits for the stores alone.
      if (layer + 1 < L) {
        prefetch_next();
        __builtin_amdgcn_s_waitcnt(0x8 | (7 << 4) | (15 << 8));  // vmcnt(8)
      } else {
        __builtin_amdgcn_s_waitcnt(0);
      }
      __builtin_amdgcn_s_barrier();
      if (tid == 0) {
        __hip_atomic_fetch_add(&done_t[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const unsigned prev =
            __hip_atomic_fetch_add(done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // Every tile of every layer counted: every workgroup has passed its
        // last wait, so this workgroup clears the counts for the next call.
        if (prev + 1 == (unsigned)tiles * (unsigned)L) sm.reset = 1;
      }
    }
    __syncthreads();  // LDS is reused by the next layer
  }
  if (sm.reset) {
    // A tile count may still be on its way (it is a separate atomic from the
    // call-wide one): wait until it reads L before clearing it.
    for (int j = tid; j < tiles; j += CH_NT) {
      for (int it = 0;; ++it) {
        if (__hip_atomic_load(&done_t[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= (unsigned)L)
          break;
        if (it >= kChainSpinMax) {
          __hip_atomic_store(flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      __hip_atomic_store(&done_t[j], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (tid == 0) __hip_atomic_store(done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace rmm

static size_t chain_align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Split count: the largest power of two that keeps the grid at one
// workgroup per CU (every workgroup must be resident), with chunks of at
// most 1024 rows (one staged segment) in whole 128-row granules.
int rmm_chain_plan(int64_t M, int64_t K, int64_t L, ChainPlan* p) {
  (void)M;
  (void)L;
  p->tiles = (K + 127) / 128;
  const int64_t kgran = (K + 127) / 128;
  int64_t s = 1;
  while (2 * s * p->tiles <= 256 && 2 * s <= kgran) s *= 2;
  while ((kgran + s - 1) / s * 128 > rmm::CH_SEG && s < kgran) s *= 2;
  p->kchunk = (kgran + s - 1) / s * 128;
  p->splits = (int)((K + p->kchunk - 1) / p->kchunk);
  p->ws_cnt_off = 0;
  p->ws_done_off = kWsChainBlockOff;
  p->ws_ssq_off = kWsCounterBytes;
  p->ws_part_off = p->ws_ssq_off + chain_align256(sizeof(float) * (size_t)p->splits * p->tiles * 16);
  p->ws_bytes = p->ws_part_off + chain_align256((size_t)p->splits * p->tiles * 8 * 64 * 16);
  // The 256-byte counter block holds the call-wide count, the flag and one
  // count per tile.
  if (4 * (2 + p->tiles) > 256) return -1;
  return p->tiles * p->splits <= 256 ? 0 : -1;
}

hipError_t rmm_launch_chain(const void* X0, const void* G, const void* W, void* Xs, float eps,
                            int64_t M, int64_t K, int64_t L, const ChainPlan& p, void* ws,
                            hipStream_t stream) {
  using namespace rmm;
  char* base = (char*)ws;
  unsigned* cnt = (unsigned*)(base + p.ws_cnt_off);
  unsigned* done = (unsigned*)(base + p.ws_done_off);
  unsigned* flag = done + 1;
  float* ssq = (float*)(base + p.ws_ssq_off);
  float* part = (float*)(base + p.ws_part_off);
  const bf16_t* x0 = (const bf16_t*)X0;
  const bf16_t* g = (const bf16_t*)G;
  const bf16_t* w = (const bf16_t*)W;
  bf16_t* xs = (bf16_t*)Xs;
  int m = (int)M, l = (int)L, s = p.splits, t = (int)p.tiles;
  int xcd_remap = (p.tiles % 8) == 0;
  int64_t k = K, kc = p.kchunk;
  void* args[] = {&x0, &g, &w, &xs, &eps, &m, &k, &l, &kc, &s, &t, &xcd_remap,
                  &cnt, &done, &flag, &ssq, &part};
  // Every workgroup must be resident at once (one per CU: the LDS use
  // allows no second), so the grid may not exceed the device's CUs.
  int dev = 0, cus = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err == hipSuccess) err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (err != hipSuccess) return err;
  if ((int64_t)p.tiles * p.splits > cus) return hipErrorInvalidConfiguration;
  return hipLaunchKernel((const void*)chain_kernel, dim3((unsigned)(p.tiles * p.splits)), dim3(CH_NT),
                         args, 0, stream);
}
