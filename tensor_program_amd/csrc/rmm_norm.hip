// Standalone RMSNorm: the first of the two kernels of the unfused program
// that the Mirage paper review's worked example ("核心概念 / μGraph示例")
// compares against -- existing systems normalise X into a buffer in device
// memory, then run the MatMul on that buffer.  The fused variants never
// write this tensor; this kernel exists to measure what that costs.
//
//   Xn[m,k] = X[m,k] * g[k] / sqrt(sum_k X[m,k]^2 / K + eps)
//
// One workgroup per row: the row's sum of squares (fp32) is reduced across
// the workgroup, then the row is scaled and stored (bf16: the fp32 value
// X*g*(1/RMS) rounded once to nearest even).  Rows of bf16 with K % 8 == 0
// and 16-byte-aligned pointers move 16 bytes per lane; anything else goes
// element by element.  Short aligned bf16 rows (K = 64 .. 512, at most 2^24
// rows) take a group of lanes per row instead, many rows per workgroup.
#include "rmm_device.h"

namespace rmm {

constexpr int NORM_THREADS = 256;

__device__ __forceinline__ float norm_block_sum(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  if (l == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < NORM_THREADS / 64; ++i) t += red[i];
  return t;
}

template <typename T, bool VEC>
__global__ __launch_bounds__(NORM_THREADS) void rmsnorm_kernel(const T* __restrict__ X,
                                                               const T* __restrict__ g,
                                                               T* __restrict__ Xn, float eps,
                                                               int64_t M, int64_t K) {
  __shared__ float red[NORM_THREADS / 64];
  const int tid = threadIdx.x;
  for (int64_t m = blockIdx.x; m < M; m += gridDim.x) {
    const T* x = X + m * K;
    T* y = Xn + m * K;
    float ss = 0.f;
    if (VEC) {  // bf16, K % 8 == 0, 16-byte aligned rows
      for (int64_t k = 8 * (int64_t)tid; k < K; k += 8 * NORM_THREADS) {
        const u32x4 v = *(const u32x4*)(x + k);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const float a = bf16_lo(v[d]), b = bf16_hi(v[d]);
          ss += a * a + b * b;
        }
      }
    } else {
      for (int64_t k = tid; k < K; k += NORM_THREADS) {
        const float a = load_f32(x + k);
        ss += a * a;
      }
    }
    const float inv = inv_rms(norm_block_sum(ss, red), K, eps);
    if (VEC) {
      for (int64_t k = 8 * (int64_t)tid; k < K; k += 8 * NORM_THREADS) {
        const u32x4 v = *(const u32x4*)(x + k);
        const u32x4 gv = *(const u32x4*)(g + k);
        u32x4 o;
#pragma unroll
        for (int d = 0; d < 4; ++d)
          o[d] = pack_bf16x2(bf16_lo(v[d]) * bf16_lo(gv[d]) * inv,
                             bf16_hi(v[d]) * bf16_hi(gv[d]) * inv);
        *(u32x4*)(y + k) = o;
      }
    } else {
      for (int64_t k = tid; k < K; k += NORM_THREADS)
        store_f32(y + k, load_f32(x + k) * load_f32(g + k) * inv);
    }
    __syncthreads();  // red is rewritten for the next row
  }
}

// Short bf16 rows (K = 8 LPR, LPR a power of two up to 64; 16-byte aligned):
// a group of LPR lanes per row, NORM_THREADS / LPR rows per workgroup, the
// sum of squares reduced within the group by lane shuffles.  Same arithmetic
// as rmsnorm_kernel.  (The unfused QKNorm program normalises every cached
// key, rows of 64 or 128.)
template <int LPR>
__global__ __launch_bounds__(NORM_THREADS) void rmsnorm_rows_kernel(const bf16_t* __restrict__ X,
                                                                    const bf16_t* __restrict__ g,
                                                                    bf16_t* __restrict__ Xn,
                                                                    float eps, int64_t M) {
  constexpr int K = 8 * LPR, RPB = NORM_THREADS / LPR;
  const int tid = threadIdx.x, c = tid % LPR;
  const int64_t m = (int64_t)blockIdx.x * RPB + tid / LPR;
  const bool ok = m < M;  // the whole group agrees
  const u32x4 v = ok ? *(const u32x4*)(X + m * K + 8 * c) : u32x4{0u, 0u, 0u, 0u};
  float ss = 0.f;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const float a = bf16_lo(v[d]), b = bf16_hi(v[d]);
    ss += a * a + b * b;
  }
#pragma unroll
  for (int o = 1; o < LPR; o <<= 1) ss += __shfl_xor(ss, o);
  const float inv = inv_rms(ss, K, eps);
  const u32x4 gv = *(const u32x4*)(g + 8 * c);
  u32x4 o;
#pragma unroll
  for (int d = 0; d < 4; ++d)
    o[d] = pack_bf16x2(bf16_lo(v[d]) * bf16_lo(gv[d]) * inv, bf16_hi(v[d]) * bf16_hi(gv[d]) * inv);
  if (ok) *(u32x4*)(Xn + m * K + 8 * c) = o;
}

}  // namespace rmm

hipError_t rmm_launch_rmsnorm(const void* X, const void* g, void* Xn, float eps, int64_t M,
                              int64_t K, bool bf16, hipStream_t stream) {
  using namespace rmm;
  const dim3 grid((unsigned)(M < (1 << 20) ? M : (1 << 20))), block(NORM_THREADS);
  if (bf16) {
    const bool vec = K % 8 == 0 && (((uintptr_t)X | (uintptr_t)g | (uintptr_t)Xn) & 15u) == 0;
    if (vec && (K == 64 || K == 128 || K == 256 || K == 512) && M <= (1 << 24)) {
      auto rows = [&](auto kernel, int lpr) {
        const int64_t rpb = NORM_THREADS / lpr;
        hipLaunchKernelGGL(kernel, dim3((unsigned)((M + rpb - 1) / rpb)), block, 0, stream,
                           (const bf16_t*)X, (const bf16_t*)g, (bf16_t*)Xn, eps, M);
      };
      if (K == 64) rows(rmsnorm_rows_kernel<8>, 8);
      else if (K == 128) rows(rmsnorm_rows_kernel<16>, 16);
      else if (K == 256) rows(rmsnorm_rows_kernel<32>, 32);
      else rows(rmsnorm_rows_kernel<64>, 64);
    } else if (vec)
      hipLaunchKernelGGL((rmsnorm_kernel<bf16_t, true>), grid, block, 0, stream,
                         (const bf16_t*)X, (const bf16_t*)g, (bf16_t*)Xn, eps, M, K);
    else
      hipLaunchKernelGGL((rmsnorm_kernel<bf16_t, false>), grid, block, 0, stream,
                         (const bf16_t*)X, (const bf16_t*)g, (bf16_t*)Xn, eps, M, K);
  } else {
    hipLaunchKernelGGL((rmsnorm_kernel<float, false>), grid, block, 0, stream, (const float*)X,
                       (const float*)g, (float*)Xn, eps, M, K);
  }
  return hipGetLastError();
}
