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
//   * the block index is remapped so that all chunks of a tile run on the
//     same XCD (workgroups are dispatched round-robin over the 8 XCDs), so
//     the partials of a tile meet in one L2.
#include "rmm_device.h"

namespace rmm {

constexpr int DEC_THREADS = 256;
constexpr int DEC_COLS = 128;  // columns per workgroup tile
constexpr int DEC_KWG = 128;   // k per workgroup step (4 waves x 32)

template <int MB, int NW>
struct DecodeSmem {
  float red[4][NW * MB * 32][64];  // per-wave accumulators, [wave][element][lane]
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

template <int MB, int NBW, bool GATED>
__global__ __launch_bounds__(DEC_THREADS) void decode_kernel(
    const bf16_t* __restrict__ X, const bf16_t* __restrict__ g, const bf16_t* __restrict__ W1,
    const bf16_t* __restrict__ W3, bf16_t* __restrict__ Y, float eps, int M, int64_t N,
    int64_t K, int64_t kchunk, int S, int tiles, int xcd_remap, unsigned* __restrict__ cnt,
    float* __restrict__ ssq_ws, float* __restrict__ part_ws) {
  constexpr int NW = GATED ? 2 : 1;
  constexpr int E = NW * MB * 32 * 64;  // accumulator floats per workgroup
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

  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  for (int64_t k0 = k_lo; k0 < k_hi; k0 += (int64_t)DEC_KWG * NBW) {
    u32x4 wv[NW][NBW][8];
    u32x4 xv[NBW][MB];
    u32x4 gv[NBW];
    // Issue every load of this step before any arithmetic.
#pragma unroll
    for (int i = 0; i < NBW; ++i) {
      const int64_t krow = k0 + 32 * (w + 4 * i) + 8 * q;
      const bool k_ok = krow < k_hi;  // K % 8 == 0: the 8 rows are all in or all out
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int64_t off = (krow + j) * N + col;
        wv[0][i][j] = (k_ok && col_ok) ? *(const u32x4*)(W1 + off) : zero4;
        if (GATED) wv[NW - 1][i][j] = (k_ok && col_ok) ? *(const u32x4*)(W3 + off) : zero4;
      }
      gv[i] = k_ok ? *(const u32x4*)(g + krow) : zero4;
#pragma unroll
      for (int b = 0; b < MB; ++b) {
        const int row = 16 * b + p;
        xv[i][b] = (k_ok && row < M) ? *(const u32x4*)(X + (int64_t)row * K + krow) : zero4;
      }
    }
#pragma unroll
    for (int i = 0; i < NBW; ++i) {
      bf16x8 a[MB];
#pragma unroll
      for (int b = 0; b < MB; ++b) {
        u32x4 av;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const float x0 = bf16_lo(xv[i][b][d]), x1 = bf16_hi(xv[i][b][d]);
          const float g0 = bf16_lo(gv[i][d]), g1 = bf16_hi(gv[i][d]);
          ss[b] += x0 * x0 + x1 * x1;
          av[d] = pack_bf16x2(x0 * g0, x1 * g1);
        }
        a[b] = __builtin_bit_cast(bf16x8, av);
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) {
#pragma unroll
        for (int wi = 0; wi < NW; ++wi) {
          const bf16x8 bop = __builtin_bit_cast(bf16x8, column_of(wv[wi][i], c));
#pragma unroll
          for (int b = 0; b < MB; ++b)
            acc[wi][b][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[b], bop, acc[wi][b][c], 0, 0, 0);
        }
      }
    }
  }

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

  // Workgroup sum of the four waves; thread owns flat indices tid + 256 t.
  float v[E / DEC_THREADS];
  float* red0 = &sm.red[0][0][0];
#pragma unroll
  for (int t = 0; t < E / DEC_THREADS; ++t) {
    const int f = tid + DEC_THREADS * t;
    v[t] = (&sm.red[0][0][0])[f] + (&sm.red[1][0][0])[f] + (&sm.red[2][0][0])[f] +
           (&sm.red[3][0][0])[f];
  }
  float ssw = 0.f;
  if (tid < MB * 16) ssw = sm.ss[0][tid] + sm.ss[1][tid] + sm.ss[2][tid] + sm.ss[3][tid];

  if (S > 1) {
    const int64_t slot = (int64_t)split * tiles + tile;
    float* part = part_ws + slot * E;
#pragma unroll
    for (int t = 0; t < E / DEC_THREADS; ++t) part[tid + DEC_THREADS * t] = v[t];
    if (tid < MB * 16) ssq_ws[slot * (MB * 16) + tid] = ssw;
    // Release the partial, count arrivals; the last arrival combines.
    __threadfence();
    __syncthreads();
    if (tid == 0) sm.last = (atomicAdd(&cnt[tile], 1u) == (unsigned)(S - 1));
    __syncthreads();
    if (!sm.last) return;
    __threadfence();
#pragma unroll
    for (int t = 0; t < E / DEC_THREADS; ++t) v[t] = 0.f;
    ssw = 0.f;
    for (int s = 0; s < S; ++s) {
      const int64_t sl = (int64_t)s * tiles + tile;
      const float* ps = part_ws + sl * E;
#pragma unroll
      for (int t = 0; t < E / DEC_THREADS; ++t) v[t] += ps[tid + DEC_THREADS * t];
      if (tid < MB * 16) ssw += ssq_ws[sl * (MB * 16) + tid];
    }
    if (tid == 0) cnt[tile] = 0u;  // leave the workspace zeroed for the next call
  }
  __syncthreads();  // everyone is done reading sm.red before it is overwritten
#pragma unroll
  for (int t = 0; t < E / DEC_THREADS; ++t) red0[tid + DEC_THREADS * t] = v[t];
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
