// Device pieces shared by the decode kernels (single call and layer chain):
// tile constants, the W stream loads and the register-transposed MFMA step.
// Included by rmm_decode.hip and rmm_chain.hip.
#pragma once

#include "rmm_device.h"

namespace rmm {

constexpr int DEC_COLS = 128;             // columns per workgroup tile
constexpr uint32_t kOutOfRange = 0x80000000u;  // > every buffer the variant accepts
// Workspace accesses of the split-K combine: device (agent) scope coherence
// (the SC1 cache-policy bit), so partials written on one XCD are read
// correctly on any other without a cache-wide write-back or invalidate.
constexpr int kCoherentDevice = 16;

struct DecodeSrc {
  __amdgpu_buffer_rsrc_t w1, w3, x, g;
};

// W rows krow .. krow+7 (krow = k0 + 32 w + 8 q) at columns col .. col+7 of
// one or two weights.  An offset past the end returns zeros (range check).
template <int NW>
__device__ __forceinline__ void decode_load(u32x4 (&wv)[NW][8], const DecodeSrc& src, int64_t N,
                                            int64_t krow, int64_t k_hi, int64_t col,
                                            bool col_ok) {
  const uint32_t row_bytes = (uint32_t)(N * 2);
  const uint32_t wo = (krow < k_hi && col_ok) ? (uint32_t)((krow * N + col) * 2) : kOutOfRange;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    wv[0][j] = __builtin_amdgcn_raw_buffer_load_b128(src.w1, wo, j * row_bytes, 0);
    if (NW == 2) wv[NW - 1][j] = __builtin_amdgcn_raw_buffer_load_b128(src.w3, wo, j * row_bytes, 0);
  }
}

// Column c of the 8x8 block (row j, dword e = columns 2e, 2e+1) -> 8
// consecutive-k values; one byte permute per output dword.
template <int MB, int NW>
__device__ __forceinline__ void decode_mma(const u32x4 (&wv)[NW][8], const u32x4 (&a)[MB],
                                           floatx4 (&acc)[NW][MB][8]) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
#pragma unroll
    for (int wi = 0; wi < NW; ++wi) {
      u32x4 bop;
#pragma unroll
      for (int d = 0; d < 4; ++d)
        bop[d] = __builtin_amdgcn_perm(wv[wi][2 * d + 1][c >> 1], wv[wi][2 * d][c >> 1],
                                       (c & 1) ? 0x07060302u : 0x05040100u);
#pragma unroll
      for (int b = 0; b < MB; ++b)
        acc[wi][b][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, a[b]), __builtin_bit_cast(bf16x8, bop), acc[wi][b][c], 0, 0,
            0);
    }
  }
}

// As decode_mma, for an operand carried exactly as two bf16 parts: the
// k-sum takes a_hi + a_lo against each transposed W column.
template <int MB, int NW>
__device__ __forceinline__ void decode_mma2(const u32x4 (&wv)[NW][8], const u32x4 (&a)[MB],
                                            const u32x4 (&al)[MB], floatx4 (&acc)[NW][MB][8]) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
#pragma unroll
    for (int wi = 0; wi < NW; ++wi) {
      u32x4 bop;
#pragma unroll
      for (int d = 0; d < 4; ++d)
        bop[d] = __builtin_amdgcn_perm(wv[wi][2 * d + 1][c >> 1], wv[wi][2 * d][c >> 1],
                                       (c & 1) ? 0x07060302u : 0x05040100u);
#pragma unroll
      for (int b = 0; b < MB; ++b) {
        acc[wi][b][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, a[b]), __builtin_bit_cast(bf16x8, bop), acc[wi][b][c], 0, 0,
            0);
        acc[wi][b][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, al[b]), __builtin_bit_cast(bf16x8, bop), acc[wi][b][c], 0, 0,
            0);
      }
    }
  }
}

}  // namespace rmm
