// Prefill variant of fused RMSNorm+MatMul: many rows, matrix-core bound.
//
// An LDS-tiled bf16 MFMA GEMM whose k-loop also produces the two other
// pieces of the fused form (Mirage paper review, "核心公式": the abstract
// expression E(O) = sum(k, div(mul(I1,I2), I3)) with the k-independent I3
// taken outside the sum):
//   * while a tile of X is staged into LDS it is multiplied by g in fp32 and
//     rounded once to bf16 -- the A operand is (X g), so g never has to be
//     applied to W;
//   * the same registers give the row sums of squares of raw X, kept in fp32;
//   * after the k-loop the accumulators are scaled by 1/sqrt(ss/K + eps) and
//     stored: the normalised X is never written anywhere.
//
// Tiling: workgroup tile 256 (M) x 256 (N) x 64 (K), 4 waves in a 2x2 grid,
// each wave owning a 128x128 block = 4x4 v_mfma_f32_32x32x16_bf16 tiles
// (256 fp32 accumulators per lane).  Two LDS stages of (A 32 KB + B 32 KB);
// the global loads of step k+1 are issued before the MFMAs of step k.
//
// W is K x N with n contiguous, but an MFMA operand wants 8 consecutive k per
// lane.  Each thread loads an 8 (k) x 8 (n) block of W with eight 16-byte
// loads (coalesced: 32 lanes cover a 512-byte row segment), transposes it in
// registers and writes eight k-contiguous 16-byte chunks to LDS.
//
// LDS layout: both tiles are [256 rows][64 k] bf16 with 128-byte rows; the
// 16-byte chunk kc of row r is stored at chunk kc ^ ((r ^ r>>3) & 7).  Eight
// consecutive lanes then hit eight different 16-byte bank groups both when
// MFMA fragments are read (consecutive rows, same chunk) and when staging
// writes land (A: same row, consecutive chunks; B: rows 8 apart, same chunk).
#include "rmm_device.h"

namespace rmm {

constexpr int PF_BM = 256, PF_BN = 256, PF_BK = 64, PF_THREADS = 256;
constexpr int PF_TILE_BYTES = 256 * 128;  // one [256][64] bf16 tile
constexpr uint32_t kPfOutOfRange = 0x80000000u;

__device__ __forceinline__ int pf_lds_off(int r, int kc) {
  return r * 128 + ((kc ^ ((r ^ (r >> 3)) & 7)) << 4);
}

// Column c (0..7) of an 8x8 bf16 block held as 8 rows of 4 dwords.
__device__ __forceinline__ u32x4 pf_column(const u32x4 (&rows)[8], int c) {
  u32x4 out;
  const int e = c >> 1;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t lo = rows[2 * d][e], hi = rows[2 * d + 1][e];
    out[d] = (c & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
  }
  return out;
}

struct PfStage {
  u32x4 a[8];  // X rows (t>>3) + 32 i, chunk t&7
  u32x4 g;     // g for chunk t&7
  u32x4 b[8];  // W rows 8 (t>>5) + j, columns 8 (t&31) .. +7
};

__device__ __forceinline__ void pf_load(PfStage& st, __amdgpu_buffer_rsrc_t xr,
                                        __amdgpu_buffer_rsrc_t gr, __amdgpu_buffer_rsrc_t wr,
                                        int64_t m0, int64_t n0, int64_t k0, int64_t M, int64_t N,
                                        int64_t K, int tid) {
  const int ca = tid & 7;
  const int64_t ka = k0 + 8 * ca;
  const bool ka_ok = ka < K;  // K % 8 == 0: a chunk is all in or all out
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t m = m0 + (tid >> 3) + 32 * i;
    const uint32_t off = (ka_ok && m < M) ? (uint32_t)((m * K + ka) * 2) : kPfOutOfRange;
    st.a[i] = __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0);
  }
  st.g = __builtin_amdgcn_raw_buffer_load_b128(gr, ka_ok ? (uint32_t)(ka * 2) : kPfOutOfRange, 0, 0);
  const int64_t kb = k0 + 8 * (tid >> 5);
  const int64_t nb = n0 + 8 * (tid & 31);
  const uint32_t row_bytes = (uint32_t)(N * 2);
  const uint32_t wo = (kb < K && nb < N) ? (uint32_t)((kb * N + nb) * 2) : kPfOutOfRange;
#pragma unroll
  for (int j = 0; j < 8; ++j) st.b[j] = __builtin_amdgcn_raw_buffer_load_b128(wr, wo, j * row_bytes, 0);
}

// Stage registers -> LDS (A: X*g rounded to bf16; B: transposed W), and the
// row sums of squares of raw X.
__device__ __forceinline__ void pf_store(const PfStage& st, char* a_lds, char* b_lds, float (&ss)[8],
                                         int tid) {
  const int ca = tid & 7;
  float gf[8];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    gf[2 * d] = bf16_lo(st.g[d]);
    gf[2 * d + 1] = bf16_hi(st.g[d]);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    u32x4 v;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const float x0 = bf16_lo(st.a[i][d]), x1 = bf16_hi(st.a[i][d]);
      ss[i] += x0 * x0 + x1 * x1;
      v[d] = pack_bf16x2(x0 * gf[2 * d], x1 * gf[2 * d + 1]);
    }
    *(u32x4*)(a_lds + pf_lds_off((tid >> 3) + 32 * i, ca)) = v;
  }
  const int kc = tid >> 5, nc = 8 * (tid & 31);
#pragma unroll
  for (int c = 0; c < 8; ++c) *(u32x4*)(b_lds + pf_lds_off(nc + c, kc)) = pf_column(st.b, c);
}

template <bool GATED>
__global__ __launch_bounds__(PF_THREADS, 1) void prefill_kernel(
    const bf16_t* __restrict__ X, const bf16_t* __restrict__ g, const bf16_t* __restrict__ W1,
    const bf16_t* __restrict__ W3, bf16_t* __restrict__ Y, float eps, int64_t M, int64_t N,
    int64_t K, int tiles_m, int tiles_n, int group_m, int xcd_remap) {
  static_assert(!GATED, "gated prefill tiles are not built");
  __shared__ __attribute__((aligned(16))) char smem[2][2][PF_TILE_BYTES];  // [stage][A|B]
  __shared__ float inv_s[PF_BM];

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  // Tile order: with xcd_remap, XCD x (workgroups bid % 8 == x) takes a
  // contiguous range of the tile sequence; the sequence walks groups of
  // group_m tile-rows column by column, so concurrently resident workgroups
  // of one XCD share A and B tiles in its L2.
  const int ntiles = tiles_m * tiles_n;
  int t = blockIdx.x;
  if (xcd_remap) t = (t & 7) * (ntiles >> 3) + (t >> 3);
  const int group = group_m * tiles_n;
  const int gid = t / group, first_m = gid * group_m;
  const int gm = (tiles_m - first_m < group_m) ? (tiles_m - first_m) : group_m;
  const int tm = first_m + (t % group) % gm;
  const int tn = (t % group) / gm;
  const int64_t m0 = (int64_t)tm * PF_BM, n0 = (int64_t)tn * PF_BN;

  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc((void*)X, 0, (int)(M * K * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t gr = __builtin_amdgcn_make_buffer_rsrc((void*)g, 0, (int)(K * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc((void*)W1, 0, (int)(K * N * 2), 0x00020000);

  floatx16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  float ss[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) ss[i] = 0.f;

  const int wm = w >> 1, wn = w & 1;
  const int nk = (int)((K + PF_BK - 1) / PF_BK);
  PfStage st;
  pf_load(st, xr, gr, wr, m0, n0, 0, M, N, K, tid);
  pf_store(st, smem[0][0], smem[0][1], ss, tid);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) pf_load(st, xr, gr, wr, m0, n0, (int64_t)(kt + 1) * PF_BK, M, N, K, tid);
    const char* a_lds = smem[cur][0];
    const char* b_lds = smem[cur][1];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int kc = 2 * s + (l >> 5);
      bf16x8 af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *(const bf16x8*)(a_lds + pf_lds_off(wm * 128 + 32 * i + (l & 31), kc));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bfr[j] = *(const bf16x8*)(b_lds + pf_lds_off(wn * 128 + 32 * j + (l & 31), kc));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) pf_store(st, smem[cur ^ 1][0], smem[cur ^ 1][1], ss, tid);
    __syncthreads();
  }

  // Row sums of squares: the 8 lanes tid&7 = 0..7 share rows (tid>>3) + 32 i.
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float v = ss[i];
    v += __shfl_xor(v, 1);
    v += __shfl_xor(v, 2);
    v += __shfl_xor(v, 4);
    if ((tid & 7) == 0) inv_s[(tid >> 3) + 32 * i] = inv_rms(v, K, eps);
  }
  __syncthreads();

  // Epilogue.  32x32 accumulator layout: lane l holds column l%32 and, for
  // register 4 jj + r, row 8 jj + 4 (l/32) + r.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t n = n0 + wn * 128 + 32 * j + (l & 31);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int lr = wm * 128 + 32 * i + 8 * jj + 4 * (l >> 5) + r;
          const int64_t m = m0 + lr;
          if (m < M && n < N) Y[m * N + n] = f32_to_bf16(acc[i][j][4 * jj + r] * inv_s[lr]);
        }
      }
    }
  }
}

}  // namespace rmm

void rmm_prefill_plan(int64_t M, int64_t N, int64_t K, PrefillPlan* p) {
  using namespace rmm;
  p->tiles_m = (int)((M + PF_BM - 1) / PF_BM);
  p->tiles_n = (int)((N + PF_BN - 1) / PF_BN);
  p->group_m = 4;
  p->xcd_remap = ((int64_t)p->tiles_m * p->tiles_n) % 8 == 0;
}

hipError_t rmm_launch_prefill(const RmmArgs& a, const PrefillPlan& p) {
  using namespace rmm;
  if (a.gated) return hipErrorInvalidValue;
  const unsigned grid = (unsigned)((int64_t)p.tiles_m * p.tiles_n);
  hipLaunchKernelGGL((prefill_kernel<false>), dim3(grid), dim3(PF_THREADS), 0, a.stream,
                     (const bf16_t*)a.X, (const bf16_t*)a.g, (const bf16_t*)a.W1,
                     (const bf16_t*)a.W3, (bf16_t*)a.Y, a.eps, a.M, a.N, a.K, p.tiles_m,
                     p.tiles_n, p.group_m, p.xcd_remap);
  return hipGetLastError();
}
