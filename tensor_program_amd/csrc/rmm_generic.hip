// Generic fused RMSNorm+MatMul kernel: any M, N, K, any alignment, fp32 or
// bf16 storage.  fp32 products on the vector ALUs.
//
// Fusion as in the Mirage example (paper review, "μGraph示例" and the
// abstract expression E(O) = sum(k, div(mul(I1,I2), I3)) of "核心公式"): the
// k-sum of X*g*W and the row sum of squares are accumulated separately, and
// the division by the row RMS is applied once to the finished sum.
//
// Workgroup tile: 64 columns x 8 rows, 256 threads = 64 columns x 4 k-slices.
// Thread (c, s) owns column c of the tile and k = s, s+4, s+8, ... of each
// 64-deep chunk; the four k-slices are summed through LDS at the end.  A
// chunk of X*g (8 x 64, fp32) is staged in LDS and read as broadcasts.
//
// Low-rank adapter (R = 1..64 ranks, not with the gate): thread (c, s) also
// accumulates T[i][c] = sum_k (X g)[i,k] A[c,k] over its k-slice for c < R;
// the epilogue adds sum_r T[i][r] B[r][n] to the k-sum before the 1/RMS scale.
#include "rmm_device.h"

namespace rmm {

constexpr int GEN_COLS = 64;
constexpr int GEN_ROWS = 8;
constexpr int GEN_KC = 64;
constexpr int GEN_THREADS = 256;

template <typename T, bool GATED>
__global__ __launch_bounds__(GEN_THREADS) void generic_kernel(
    const T* __restrict__ X, const T* __restrict__ g, const T* __restrict__ W1,
    const T* __restrict__ W3, T* __restrict__ Y, float eps, int64_t M, int64_t N, int64_t K,
    int norm, const T* __restrict__ LA, const T* __restrict__ LB, int R) {
  __shared__ float a_s[GEN_ROWS][GEN_KC];
  __shared__ float red[GATED ? 2 : 1][4][GEN_ROWS][GEN_COLS];
  __shared__ float t_s[GATED ? 1 : 4][GEN_ROWS][GEN_COLS];  // adapter partials [slice][row][rank]
  __shared__ float ss_s[GEN_ROWS][32];
  __shared__ float inv_s[GEN_ROWS];

  const int tid = threadIdx.x;
  const int64_t n0 = (int64_t)blockIdx.x * GEN_COLS;
  const int64_t m0 = (int64_t)blockIdx.y * GEN_ROWS;

  // Row sums of squares of raw X (32 threads per row, 8 loads in flight).
  {
    const int r = tid / 32, j = tid % 32;
    float ss = 0.0f;
    if (m0 + r < M) {
      const T* xr = X + (m0 + r) * K;
      for (int64_t k = j; k < K; k += 256) {
        float x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) x[u] = (k + 32 * u < K) ? load_f32(xr + k + 32 * u) : 0.0f;
#pragma unroll
        for (int u = 0; u < 8; ++u) ss += x[u] * x[u];
      }
    }
    ss_s[r][j] = ss;
  }
  __syncthreads();
  if (tid < GEN_ROWS) {
    float ss = 0.0f;
    for (int j = 0; j < 32; ++j) ss += ss_s[tid][j];
    inv_s[tid] = norm ? inv_rms(ss, K, eps) : 1.0f;
  }

  const int c = tid % GEN_COLS, s = tid / GEN_COLS;
  const int64_t n = n0 + c;
  const bool col_ok = n < N;
  float acc1[GEN_ROWS], acc3[GEN_ROWS], tl[GEN_ROWS];
#pragma unroll
  for (int i = 0; i < GEN_ROWS; ++i) acc1[i] = acc3[i] = tl[i] = 0.0f;
  const bool lora_c = !GATED && c < R;  // this thread's rank column

  // W of a chunk: thread (c, s) loads k = s, s+4, ..., s+60 of column c,
  // all at once; the next chunk's loads are in flight while this one is
  // multiplied.
  constexpr int NU = GEN_KC / 4;
  auto load_w = [&](int64_t k0, float (&w1)[NU], float (&w3)[NU]) {
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int64_t k = k0 + s + 4 * u;
      const bool ok = col_ok && k < K;
      w1[u] = ok ? load_f32(W1 + k * N + n) : 0.0f;
      w3[u] = (GATED && ok) ? load_f32(W3 + k * N + n) : 0.0f;
    }
  };
  float w1c[NU], w3c[NU];
  load_w(0, w1c, w3c);
  for (int64_t k0 = 0; k0 < K; k0 += GEN_KC) {
    __syncthreads();
    // Stage X*g for the chunk (fp32, no rounding).
    for (int e = tid; e < GEN_ROWS * GEN_KC; e += GEN_THREADS) {
      const int r = e / GEN_KC, kk = e % GEN_KC;
      const int64_t m = m0 + r, k = k0 + kk;
      a_s[r][kk] = (m < M && k < K) ? load_f32(X + m * K + k) * (norm ? load_f32(g + k) : 1.0f) : 0.0f;
    }
    __syncthreads();
    float w1n[NU], w3n[NU];
    load_w(k0 + GEN_KC, w1n, w3n);
#pragma unroll
    for (int u = 0; u < NU; ++u) {
#pragma unroll
      for (int i = 0; i < GEN_ROWS; ++i) {
        acc1[i] += a_s[i][s + 4 * u] * w1c[u];
        if (GATED) acc3[i] += a_s[i][s + 4 * u] * w3c[u];
      }
    }
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      w1c[u] = w1n[u];
      w3c[u] = w3n[u];
    }
    if (lora_c) {
      for (int u = 0; u < NU; ++u) {
        const int64_t k = k0 + s + 4 * u;
        const float av = k < K ? load_f32(LA + (int64_t)c * K + k) : 0.0f;
#pragma unroll
        for (int i = 0; i < GEN_ROWS; ++i) tl[i] += a_s[i][s + 4 * u] * av;
      }
    }
  }

  // Sum the four k-slices, then scale by 1/RMS (after the k-sum) and store.
#pragma unroll
  for (int i = 0; i < GEN_ROWS; ++i) {
    red[0][s][i][c] = acc1[i];
    if (GATED) red[GATED ? 1 : 0][s][i][c] = acc3[i];
    if (!GATED) t_s[GATED ? 0 : s][i][c] = tl[i];
  }
  __syncthreads();
  // Adapter: the four k-slices of T summed into slice 0.
  if (!GATED && R > 0) {
    for (int e = tid; e < GEN_ROWS * GEN_COLS; e += GEN_THREADS) {
      const int r = e / GEN_COLS, j = e % GEN_COLS;
      float t = 0.0f;
#pragma unroll
      for (int sl = 0; sl < (GATED ? 1 : 4); ++sl) t += t_s[sl][r][j];
      a_s[r][j] = t;  // a_s is free after the k-loop
    }
    __syncthreads();
  }
  for (int e = tid; e < GEN_ROWS * GEN_COLS; e += GEN_THREADS) {
    const int r = e / GEN_COLS, cc = e % GEN_COLS;
    const int64_t m = m0 + r, nn = n0 + cc;
    if (m >= M || nn >= N) continue;
    const float inv = inv_s[r];
    float lo = 0.0f;
    if (!GATED)
      for (int j = 0; j < R; ++j) lo += a_s[r][j] * load_f32(LB + (int64_t)j * N + nn);
    const float z1 =
        (red[0][0][r][cc] + red[0][1][r][cc] + red[0][2][r][cc] + red[0][3][r][cc] + lo) * inv;
    float y = z1;
    if (GATED) {
      const int b = GATED ? 1 : 0;
      const float z3 = (red[b][0][r][cc] + red[b][1][r][cc] + red[b][2][r][cc] + red[b][3][r][cc]) * inv;
      y = silu_gate(z1, z3);
    }
    store_f32(Y + m * N + nn, y);
  }
}

}  // namespace rmm

hipError_t rmm_launch_generic(const RmmArgs& a, bool bf16) {
  using namespace rmm;
  dim3 grid((unsigned)((a.N + GEN_COLS - 1) / GEN_COLS), (unsigned)((a.M + GEN_ROWS - 1) / GEN_ROWS));
  dim3 block(GEN_THREADS);
  const int R = (int)a.R;
  if (bf16) {
    auto X = (const bf16_t*)a.X, g = (const bf16_t*)a.g, W1 = (const bf16_t*)a.W1,
         W3 = (const bf16_t*)a.W3;
    auto LA = (const bf16_t*)a.LA, LB = (const bf16_t*)a.LB;
    auto Y = (bf16_t*)a.Y;
    if (a.gated)
      hipLaunchKernelGGL((generic_kernel<bf16_t, true>), grid, block, 0, a.stream, X, g, W1, W3,
                         Y, a.eps, a.M, a.N, a.K, a.norm, LA, LB, R);
    else
      hipLaunchKernelGGL((generic_kernel<bf16_t, false>), grid, block, 0, a.stream, X, g, W1,
                         W3, Y, a.eps, a.M, a.N, a.K, a.norm, LA, LB, R);
  } else {
    auto X = (const float*)a.X, g = (const float*)a.g, W1 = (const float*)a.W1,
         W3 = (const float*)a.W3;
    auto LA = (const float*)a.LA, LB = (const float*)a.LB;
    auto Y = (float*)a.Y;
    if (a.gated)
      hipLaunchKernelGGL((generic_kernel<float, true>), grid, block, 0, a.stream, X, g, W1, W3, Y,
                         a.eps, a.M, a.N, a.K, a.norm, LA, LB, R);
    else
      hipLaunchKernelGGL((generic_kernel<float, false>), grid, block, 0, a.stream, X, g, W1, W3,
                         Y, a.eps, a.M, a.N, a.K, a.norm, LA, LB, R);
  }
  return hipGetLastError();
}
