// Decode variant of fused RMSNorm+MatMul: few rows (M <= 32), bandwidth-bound.
//
// The weight matrix dominates the traffic, so the kernel streams each byte
// of W exactly once from HBM, split along K across workgroups so that the
// whole chip is streaming.  Both k-sums the fused form needs -- the
// numerator sum_k (X g)[m,k] W[k,n] and the row sum of squares sum_k X[m,k]^2
// -- are linear in their k-chunks, so partial sums from different chunks are
// added exactly as partial sums, and the division by the RMS happens once at
// the end.  This is the abstract expression E(O) = sum(k, div(mul(I1,I2),I3))
// of the Mirage paper review ("核心公式") with the k-independent divisor I3
// moved outside the sum.
//
// Work decomposition (one workgroup = 4 waves of 64 lanes):
//   * a workgroup owns a 128-column tile of Y and a chunk of K;
//   * its 4 waves take interleaved 32-deep k-blocks of the chunk;
//   * per k-block, lane (q = lane/16, p = lane%16) loads rows kb+8q .. kb+8q+7
//     of W at columns 8p .. 8p+7 of the tile (eight 16-byte loads; each load
//     instruction reads four 256-byte row segments), transposes the 8x8 block
//     in registers, and feeds it as the B operand of eight
//     v_mfma_f32_16x16x32_bf16 (one per column 8p+c).  The A operand is
//     (X g) for rows 16*mb + p, k = kb+8q .. +7, formed in fp32 and rounded
//     once to bf16; the same lanes accumulate X^2 in fp32 for the row RMS.
//   * the 4 waves' accumulators are summed through LDS; with several K chunks
//     the workgroup stores its fp32 partial to the workspace, and the last
//     workgroup to arrive at a tile (arrival counter) adds the partials and
//     runs the epilogue  Y = acc / RMS  (gated: silu(acc1/RMS) * acc3/RMS).
//   * the partials cross XCDs (each XCD has its own L2), so they are written
//     and read with device-scope coherent accesses, ordered by waiting for the
//     stores' acknowledgements before the arrival count.  A device-wide fence
//     per workgroup (an L2 write-back plus invalidate on gfx950) would also be
//     correct but costs several microseconds per call at this size.
//   * the block index is remapped so that all chunks of a tile are dispatched
//     to the same XCD (workgroups go round-robin over the 8 XCDs); this only
//     affects locality, never correctness.
#include "rmm_device.h"

namespace rmm {

constexpr int DEC_THREADS = 256;
constexpr int DEC_COLS = 128;  // columns per workgroup tile
constexpr int DEC_KWG = 128;   // k per workgroup step (4 waves x 32)

template <int MB, int NW>
struct DecodeSmem {
  alignas(16) float red[4][NW * MB * 32][64];  // per-wave accumulators, [wave][element][lane]
  float ss[4][MB * 16];
  float inv[MB * 16];
  int last;
};

// Column c (0..7) of an 8x8 bf16 block held as 8 rows of 4 dwords (row j,
// dword e = columns 2e, 2e+1) -> 8 consecutive-k values of that column.
__device__ __forceinline__ u32x4 column_of(const u32x4 (&rows)[8], int c) {
  u32x4 out;
  const int e = c >> 1;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t lo = rows[2 * d][e], hi = rows[2 * d + 1][e];
    out[d] = (c & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
  }
  return out;
}

// Registers of one pipeline stage: NBW k-blocks of W (and W3), X and g.
template <int MB, int NBW, int NW>
struct DecodeStage {
  u32x4 w[NW][NBW][8];
  u32x4 x[NBW][MB];
  u32x4 g[NBW];
};

// Buffer resources (base, size) of the operands.  Loads go through them
// with a 32-bit byte offset per lane; an offset past the end returns zeros
// (hardware range check), which is how rows beyond K and M, and columns
// beyond N, read as zero without a branch.
struct DecodeSrc {
  __amdgpu_buffer_rsrc_t w1, w3, x, g;
};
constexpr uint32_t kOutOfRange = 0x80000000u;  // > every buffer the variant accepts

template <int MB, int NBW, int NW>
__device__ __forceinline__ void decode_load(DecodeStage<MB, NBW, NW>& st, const DecodeSrc& src,
                                            int M, int64_t N, int64_t K, int64_t k0,
                                            int64_t k_hi, int64_t col, bool col_ok, int w, int q,
                                            int p) {
  const uint32_t row_bytes = (uint32_t)(N * 2);
#pragma unroll
  for (int i = 0; i < NBW; ++i) {
    const int64_t krow = k0 + 32 * (w + 4 * i) + 8 * q;
    const bool k_ok = krow < k_hi;  // K % 8 == 0: the 8 rows are all in or all out
    const uint32_t wo = (k_ok && col_ok) ? (uint32_t)((krow * N + col) * 2) : kOutOfRange;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      st.w[0][i][j] = __builtin_amdgcn_raw_buffer_load_b128(src.w1, wo, j * row_bytes, 0);
      if (NW == 2)
        st.w[NW - 1][i][j] = __builtin_amdgcn_raw_buffer_load_b128(src.w3, wo, j * row_bytes, 0);
    }
    const uint32_t go = k_ok ? (uint32_t)(krow * 2) : kOutOfRange;
    st.g[i] = __builtin_amdgcn_raw_buffer_load_b128(src.g, go, 0, 0);
#pragma unroll
    for (int b = 0; b < MB; ++b) {
      const int row = 16 * b + p;
      const uint32_t xo = (k_ok && row < M) ? (uint32_t)(((int64_t)row * K + krow) * 2) : kOutOfRange;
      st.x[i][b] = __builtin_amdgcn_raw_buffer_load_b128(src.x, xo, 0, 0);
    }
  }
}

template <int MB, int NBW, int NW>
__device__ __forceinline__ void decode_compute(const DecodeStage<MB, NBW, NW>& st,
                                               floatx4 (&acc)[NW][MB][8], float (&ss)[MB]) {
#pragma unroll
  for (int i = 0; i < NBW; ++i) {
    bf16x8 a[MB];
#pragma unroll
    for (int b = 0; b < MB; ++b) {
      u32x4 av;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const float x0 = bf16_lo(st.x[i][b][d]), x1 = bf16_hi(st.x[i][b][d]);
        const float g0 = bf16_lo(st.g[i][d]), g1 = bf16_hi(st.g[i][d]);
        ss[b] += x0 * x0 + x1 * x1;
        av[d] = pack_bf16x2(x0 * g0, x1 * g1);
      }
      a[b] = __builtin_bit_cast(bf16x8, av);
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
#pragma unroll
      for (int wi = 0; wi < NW; ++wi) {
        const bf16x8 bop = __builtin_bit_cast(bf16x8, column_of(st.w[wi][i], c));
#pragma unroll
        for (int b = 0; b < MB; ++b)
          acc[wi][b][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[b], bop, acc[wi][b][c], 0, 0, 0);
      }
    }
  }
}

// Workspace accesses of the split-K combine: 16-byte buffer loads/stores
// with device (agent) scope coherence (the SC1 cache-policy bit), so the
// partials written on one XCD are read correctly on any other without a
// cache-wide write-back or invalidate.
constexpr int kCoherentDevice = 16;  // SC1

template <int MB, int NBW, bool GATED>
__global__ __launch_bounds__(DEC_THREADS) void decode_kernel(
    const bf16_t* __restrict__ X, const bf16_t* __restrict__ g, const bf16_t* __restrict__ W1,
    const bf16_t* __restrict__ W3, bf16_t* __restrict__ Y, float eps, int M, int64_t N,
    int64_t K, int64_t kchunk, int S, int tiles, int xcd_remap, unsigned* __restrict__ cnt,
    float* __restrict__ ssq_ws, float* __restrict__ part_ws) {
  constexpr int NW = GATED ? 2 : 1;
  constexpr int E = NW * MB * 32 * 64;  // accumulator floats per workgroup
  constexpr int PER = E / DEC_THREADS;  // floats per thread in the combine (8 NW MB)
  __shared__ DecodeSmem<MB, NW> sm;

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, q = l >> 4, p = l & 15;
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
  const int64_t col = (int64_t)tile * DEC_COLS + 8 * p;
  const bool col_ok = col < N;
  const int64_t k_lo = (int64_t)split * kchunk;
  const int64_t k_hi = (k_lo + kchunk < K) ? (k_lo + kchunk) : K;

  floatx4 acc[NW][MB][8];
#pragma unroll
  for (int a = 0; a < NW; ++a)
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[a][b][c] = floatx4{0.f, 0.f, 0.f, 0.f};
  float ss[MB];
#pragma unroll
  for (int b = 0; b < MB; ++b) ss[b] = 0.f;

  // Two register stages: the loads of step s+1 are in flight while step s
  // is multiplied.
  const int64_t step = (int64_t)DEC_KWG * NBW;
  const int nsteps = (int)((k_hi - k_lo + step - 1) / step);
  DecodeSrc src;
  src.w1 = __builtin_amdgcn_make_buffer_rsrc((void*)W1, 0, (int)(K * N * 2), 0x00020000);
  src.w3 = __builtin_amdgcn_make_buffer_rsrc((void*)(GATED ? W3 : W1), 0, (int)(K * N * 2), 0x00020000);
  src.x = __builtin_amdgcn_make_buffer_rsrc((void*)X, 0, (int)((int64_t)M * K * 2), 0x00020000);
  src.g = __builtin_amdgcn_make_buffer_rsrc((void*)g, 0, (int)(K * 2), 0x00020000);
  DecodeStage<MB, NBW, NW> sa, sb;
  decode_load(sa, src, M, N, K, k_lo, k_hi, col, col_ok, w, q, p);
  int s = 0;
  for (; s + 2 <= nsteps; s += 2) {
    decode_load(sb, src, M, N, K, k_lo + (s + 1) * step, k_hi, col, col_ok, w, q, p);
    decode_compute(sa, acc, ss);
    if (s + 2 < nsteps) decode_load(sa, src, M, N, K, k_lo + (s + 2) * step, k_hi, col, col_ok, w, q, p);
    decode_compute(sb, acc, ss);
  }
  if (s < nsteps) decode_compute(sa, acc, ss);

  // Row sums of squares: lanes p, p+16, p+32, p+48 hold the four k-groups.
#pragma unroll
  for (int b = 0; b < MB; ++b) {
    ss[b] += __shfl_xor(ss[b], 16);
    ss[b] += __shfl_xor(ss[b], 32);
    if (q == 0) sm.ss[w][16 * b + p] = ss[b];
  }
  // Per-wave accumulators to LDS: element e = (wi*MB + b)*32 + c*4 + r.
#pragma unroll
  for (int wi = 0; wi < NW; ++wi)
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
      for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) sm.red[w][(wi * MB + b) * 32 + c * 4 + r][l] = acc[wi][b][c][r];
  __syncthreads();

  // Workgroup sum of the four waves; thread owns flat floats [PER*tid, PER*tid + PER).
  float* red0 = &sm.red[0][0][0];
  floatx4 v[PER / 4];
#pragma unroll
  for (int t = 0; t < PER / 4; ++t) {
    const int f = PER * tid + 4 * t;
    v[t] = *(const floatx4*)(&sm.red[0][0][0] + f) + *(const floatx4*)(&sm.red[1][0][0] + f) +
           *(const floatx4*)(&sm.red[2][0][0] + f) + *(const floatx4*)(&sm.red[3][0][0] + f);
  }
  float ssw = 0.f;
  if (tid < MB * 16) ssw = sm.ss[0][tid] + sm.ss[1][tid] + sm.ss[2][tid] + sm.ss[3][tid];

  if (S > 1) {
    const int64_t slot = (int64_t)split * tiles + tile;
    const int64_t nslots = (int64_t)S * tiles;
    const __amdgpu_buffer_rsrc_t prs =
        __builtin_amdgcn_make_buffer_rsrc(part_ws, 0, (int)(nslots * E * 4), 0x00020000);
    // Partials go out with device-scope coherence; waiting for every store's
    // acknowledgement before the arrival count makes them visible to
    // whichever workgroup arrives last.
#pragma unroll
    for (int t = 0; t < PER / 4; ++t)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v[t]), prs,
                                             (int)((slot * E + PER * tid + 4 * t) * 4), 0,
                                             kCoherentDevice);
    if (tid < MB * 16)
      __hip_atomic_store(&ssq_ws[slot * (MB * 16) + tid], ssw, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0)
      sm.last = (__hip_atomic_fetch_add(&cnt[tile], 1u, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT) == (unsigned)(S - 1));
    __syncthreads();
    if (!sm.last) return;
    // Last arrival: add the S partials, four splits' loads in flight at a time.
#pragma unroll
    for (int t = 0; t < PER / 4; ++t) v[t] = floatx4{0.f, 0.f, 0.f, 0.f};
    ssw = 0.f;
    for (int s0 = 0; s0 < S; s0 += 4) {
      u32x4 buf[4][PER / 4];
      float sbuf[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t sl = (int64_t)(s0 + u) * tiles + tile;
        const bool ok = s0 + u < S;
#pragma unroll
        for (int t = 0; t < PER / 4; ++t)
          buf[u][t] = ok ? __builtin_amdgcn_raw_buffer_load_b128(
                               prs, (int)((sl * E + PER * tid + 4 * t) * 4), 0, kCoherentDevice)
                         : u32x4{0u, 0u, 0u, 0u};
        sbuf[u] = (ok && tid < MB * 16)
                      ? __hip_atomic_load(&ssq_ws[sl * (MB * 16) + tid], __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT)
                      : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int t = 0; t < PER / 4; ++t) v[t] += __builtin_bit_cast(floatx4, buf[u][t]);
        ssw += sbuf[u];
      }
    }
    // Leave the workspace zeroed for the next call (all arrivals are in).
    if (tid == 0) __hip_atomic_store(&cnt[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();  // everyone is done reading sm.red before it is overwritten
#pragma unroll
  for (int t = 0; t < PER / 4; ++t) *(floatx4*)(red0 + PER * tid + 4 * t) = v[t];
  if (tid < MB * 16) sm.inv[tid] = inv_rms(ssw, K, eps);
  __syncthreads();

  // Epilogue: group (b, r, lane) -> row 16b + 4(lane/16) + r, 8 columns.
#pragma unroll
  for (int t = 0; t < MB; ++t) {
    const int grp = tid + DEC_THREADS * t;
    const int ln = grp & 63, br = grp >> 6, b = br >> 2, r = br & 3;
    const int row = 16 * b + 4 * (ln >> 4) + r;
    const int64_t cc = (int64_t)tile * DEC_COLS + 8 * (ln & 15);
    if (row >= M || cc >= N) continue;
    const float inv = sm.inv[row];
    u32x4 out;
#pragma unroll
    for (int c = 0; c < 8; c += 2) {
      float y0 = red0[((0 * MB + b) * 32 + c * 4 + r) * 64 + ln] * inv;
      float y1 = red0[((0 * MB + b) * 32 + (c + 1) * 4 + r) * 64 + ln] * inv;
      if (GATED) {
        const float z0 = red0[((1 * MB + b) * 32 + c * 4 + r) * 64 + ln] * inv;
        const float z1 = red0[((1 * MB + b) * 32 + (c + 1) * 4 + r) * 64 + ln] * inv;
        y0 = silu_gate(y0, z0);
        y1 = silu_gate(y1, z1);
      }
      out[c >> 1] = pack_bf16x2(y0, y1);
    }
    *(u32x4*)(Y + (int64_t)row * N + cc) = out;
  }
}

}  // namespace rmm

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

void rmm_decode_plan(int64_t M, int64_t N, int64_t K, int gated, int splits, int nbw,
                     DecodePlan* p) {
  using namespace rmm;
  p->mb = (int)((M + 15) / 16);
  p->nbw = nbw;
  p->tiles = (N + DEC_COLS - 1) / DEC_COLS;
  const int64_t kgran = (K + DEC_KWG - 1) / DEC_KWG;  // 128-deep granules
  int64_t s = splits;
  if (s < 1) s = 1;
  if (s > kgran) s = kgran;
  const int64_t gran_per = (kgran + s - 1) / s;
  p->kchunk = gran_per * DEC_KWG;
  p->splits = (int)((K + p->kchunk - 1) / p->kchunk);
  const int nw = gated ? 2 : 1;
  const size_t E = (size_t)nw * p->mb * 32 * 64;
  p->ws_cnt_off = 0;
  p->ws_ssq_off = align256(sizeof(unsigned) * (size_t)p->tiles);
  p->ws_part_off = p->ws_ssq_off + align256(sizeof(float) * (size_t)p->splits * p->tiles * p->mb * 16);
  p->ws_bytes = p->splits > 1 ? p->ws_part_off + align256(sizeof(float) * (size_t)p->splits * p->tiles * E) : 0;
}

template <int MB, int NBW, bool GATED>
static void launch_decode_t(const RmmArgs& a, const DecodePlan& p, void* ws) {
  using namespace rmm;
  const int xcd_remap = (p.tiles % 8) == 0;
  char* base = (char*)ws;
  unsigned* cnt = ws ? (unsigned*)(base + p.ws_cnt_off) : nullptr;
  float* ssq = ws ? (float*)(base + p.ws_ssq_off) : nullptr;
  float* part = ws ? (float*)(base + p.ws_part_off) : nullptr;
  const unsigned grid = (unsigned)(p.tiles * p.splits);
  hipLaunchKernelGGL((decode_kernel<MB, NBW, GATED>), dim3(grid), dim3(DEC_THREADS), 0, a.stream,
                     (const bf16_t*)a.X, (const bf16_t*)a.g, (const bf16_t*)a.W1,
                     (const bf16_t*)a.W3, (bf16_t*)a.Y, a.eps, (int)a.M, a.N, a.K, p.kchunk,
                     p.splits, (int)p.tiles, xcd_remap, cnt, ssq, part);
}

hipError_t rmm_launch_decode(const RmmArgs& a, const DecodePlan& p, void* ws) {
  const bool gd = a.gated != 0;
  if (p.nbw == 2) {
    if (!gd && p.mb == 1) launch_decode_t<1, 2, false>(a, p, ws);
    else if (!gd && p.mb == 2) launch_decode_t<2, 2, false>(a, p, ws);
    else if (gd && p.mb == 1) launch_decode_t<1, 2, true>(a, p, ws);
    else return hipErrorInvalidValue;
  } else if (p.nbw == 1) {
    if (!gd && p.mb == 1) launch_decode_t<1, 1, false>(a, p, ws);
    else if (!gd && p.mb == 2) launch_decode_t<2, 1, false>(a, p, ws);
    else if (gd && p.mb == 1) launch_decode_t<1, 1, true>(a, p, ws);
    else return hipErrorInvalidValue;
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
