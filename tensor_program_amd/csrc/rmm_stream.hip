// Stream variant of fused RMSNorm+MatMul: up to 64 rows, one or two weights
// (the gated MLP of the Mirage paper review's benchmark table, "五、实验结果",
// read as silu(norm(X) W1) * (norm(X) W3)), bandwidth-bound.
//
// Each workgroup owns a 64-column strip of Y and streams the matching
// 64-column strips of W1 (and W3) over all of K, so no cross-workgroup
// combine is needed: the k-sum of X g W and the row sum of squares of X are
// finished inside the workgroup and the division by the RMS is applied once
// at the end (the abstract expression E(O) = sum(k, div(mul(I1,I2), I3)) of
// "核心公式", with the k-independent divisor moved outside the sum).
//
// Pipeline (8 waves, k-steps of 64): every operand byte goes straight from
// memory into an LDS ring (buffer loads with the LDS-direct bit) several
// k-steps ahead -- the W strips, the X rows and the g slice of a step.
// Vector-memory loads complete in issue order, so keeping every load in this
// one stream lets each iteration wait only for the steps it needs.
//   * W slot layout [64 k][64 n] bf16, 128-byte rows, 16-byte chunk c of row
//     k at chunk c ^ 2(k & 3): the transposing LDS reads are conflict-free.
//   * X slot layout [64 rows][64 k] bf16, 128-byte rows, chunk c of row r at
//     chunk c ^ ((r >> 1) & 7): the 16 rows one quarter-wave reads in a
//     fragment load fall on 16 distinct 16-byte bank groups (a plain
//     c ^ (r & 7) puts rows r and r + 8 on the same banks).
//   * one step ahead of its use, the workgroup turns the X slot into the
//     matrix operand in place: each thread takes 8 consecutive k of one row,
//     forms X*g in fp32 (bf16 dot2 with one lane of g zeroed: an exact
//     product) rounded once to bf16, and adds X^2 to its row's sum of squares.
//   * each wave multiplies a 64-row x 32-column block of one weight over a
//     k-half (gated) or a k-quarter (plain) of every step with
//     v_mfma_f32_32x32x16_bf16; B fragments come from ds_read_b64_tr_b16
//     (gfx950's transposing LDS read): lane i of each 16-lane group receives
//     4 consecutive k of column i.  Each W element is read from LDS once.
//   * epilogue through LDS: the partial k-sums are added, Y = acc / RMS,
//     gated Y = silu(acc1/RMS) * acc3/RMS.
#include "rmm_device.h"

namespace rmm {

constexpr int ST_THREADS = 512;
constexpr int ST_BN = 64;                        // columns per workgroup
constexpr int ST_BM = 64;                        // rows (M <= 64)
constexpr int ST_BK = 64;                        // k per step
constexpr int ST_W_BYTES = ST_BK * ST_BN * 2;    // 8 KB per weight per slot
constexpr int ST_X_BYTES = ST_BM * ST_BK * 2;    // 8 KB per slot
constexpr int ST_G_BYTES = 128;                  // the g slice of a step
constexpr uint32_t kStOutOfRange = 0x80000000u;

// Ring depth per weight count.  The load latency is covered with 2 steps
// ahead already (what bounds the kernel is the bytes each CU takes in); with
// two weights 3 steps ahead (5 slots) measured ~1% faster than 4 or 2.
template <int NW>
struct StCfg {
  static constexpr int RING = NW == 2 ? 5 : 8;
  static constexpr int AHEAD = RING - 2;  // steps issued ahead of the one multiplied
  static constexpr int SUBS = NW == 2 ? 2 : 1;  // 16-deep sub-steps per wave per step
};

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ bf16x2 st_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2, v); }

// X slot swizzle: physical 16-byte chunk of logical chunk c in row r is
// c ^ st_xswz(r).  Rows 32 apart share it (fragment row blocks).
__device__ __forceinline__ int st_xswz(int r) { return (r >> 1) & 7; }

// Raw buffer resource (stride 0, 32-bit data format) for [base, base+bytes).
__device__ __forceinline__ i32x4 st_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = 0x00020000;
  return r;
}

// 16 bytes per active lane from memory straight into LDS (lane l at
// lds_addr + 16 l).  Inline asm keeps the compiler from serialising it
// against the other loads in flight; the k-loop waits with explicit vmcnt.
__device__ __forceinline__ void st_lds_load16(uint32_t lds_addr, uint32_t voff, i32x4 rsrc) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(rsrc)
               : "memory");
}

#define ST_WAIT_VMCNT(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14))

template <int NW>
struct StSmem {
  char w[StCfg<NW>::RING][NW][ST_W_BYTES];
  char x[StCfg<NW>::RING][ST_X_BYTES];
  char g[StCfg<NW>::RING][ST_G_BYTES];
  float ss[ST_BM];
  float inv[ST_BM];
};
// The epilogue reuses the W and X rings (contiguous) for 4 fp32 partial
// blocks of 64 x 64.
constexpr int ST_RED_BYTES = 4 * ST_BM * ST_BN * 4;
static_assert(sizeof(StSmem<1>::w) + sizeof(StSmem<1>::x) >= ST_RED_BYTES, "ring too small");
static_assert(sizeof(StSmem<2>::w) + sizeof(StSmem<2>::x) >= ST_RED_BYTES, "ring too small");
static_assert(sizeof(StSmem<2>) <= 160 * 1024 && sizeof(StSmem<1>) <= 160 * 1024, "LDS");

template <int NW>
__global__ __launch_bounds__(ST_THREADS, 1) void stream_kernel(
    const bf16_t* __restrict__ X, const bf16_t* __restrict__ g, const bf16_t* __restrict__ W1,
    const bf16_t* __restrict__ W3, bf16_t* __restrict__ Y, float eps, int M, int64_t N,
    int64_t K, int norm) {
  constexpr int RING = StCfg<NW>::RING, AHEAD = StCfg<NW>::AHEAD, SUBS = StCfg<NW>::SUBS;
  __shared__ __attribute__((aligned(1024))) StSmem<NW> sm;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int64_t n0 = (int64_t)blockIdx.x * ST_BN;
  const int nk = (int)((K + ST_BK - 1) / ST_BK);

  // Per-lane source offsets of one step (relative to the step's resource).
  // W: wave w fills rows 8w .. 8w+7 of a slot; lane l lands at byte 16 l.
  uint32_t w_off;
  {
    const int kl = 8 * w + (l >> 3);
    const int c = (l & 7) ^ (2 * (kl & 3));
    const int64_t nn = n0 + 8 * c;
    w_off = nn < N ? (uint32_t)((kl * N + nn) * 2) : kStOutOfRange;
  }
  // X: wave w fills rows 8w .. 8w+7; lane l -> row 8w + l/8, chunk
  // (l&7) ^ st_xswz(row); the k-range check happens per step.
  const int x_row = 8 * w + (l >> 3);
  const int x_kc = (l & 7) ^ st_xswz(x_row);
  const uint32_t x_off = x_row < M ? (uint32_t)(((int64_t)x_row * K + 8 * x_kc) * 2) : kStOutOfRange;
  const uint32_t lds_w = (uint32_t)(uintptr_t)(lds_char*)&sm.w[0][0][0] + w * 1024;
  const uint32_t lds_x = (uint32_t)(uintptr_t)(lds_char*)&sm.x[0][0] + w * 1024;
  const uint32_t lds_g = (uint32_t)(uintptr_t)(lds_char*)&sm.g[0][0];
  const bf16_t* Wp[2] = {W1, NW == 2 ? W3 : W1};

  // Issue every transfer of one step: NW W blocks, one X block and, from
  // lanes 0..7 of wave 0 only, the step's g slice (every wave reads it after
  // the barrier) -- NW + 1 vector-memory instructions per wave, NW + 2 for
  // wave 0.
  auto issue_step = [&](int step) {
    const int64_t k0 = (int64_t)step * ST_BK;
    const int64_t rows = K - k0 > 0 ? K - k0 : 0;
    const int slot = step % RING;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      const i32x4 rs = st_rsrc(Wp[v] + k0 * N, (uint32_t)(rows * N * 2));
      st_lds_load16(lds_w + (uint32_t)((slot * NW + v) * ST_W_BYTES), w_off, rs);
    }
    const i32x4 xs = st_rsrc(X + k0, (uint32_t)(((int64_t)M * K - (k0 < (int64_t)M * K ? k0 : 0)) * 2));
    st_lds_load16(lds_x + (uint32_t)(slot * ST_X_BYTES), k0 + 8 * x_kc < K ? x_off : kStOutOfRange, xs);
    const i32x4 gs = st_rsrc(g + k0, (uint32_t)(rows * 2));
    if (w == 0 && l < 8) st_lds_load16(lds_g + (uint32_t)(slot * ST_G_BYTES), (uint32_t)(16 * l), gs);
  };

  // Operand forming: thread -> row tid/8, logical k-chunk tid%8 of a step.
  // The X slot is overwritten in place with bf16(X * g); the row's sum of
  // squares accumulates in the thread (its row never changes).
  const int f_row = tid >> 3, f_c = tid & 7;
  const int f_off = f_row * 128 + ((f_c ^ st_xswz(f_row)) << 4);
  float ss = 0.f;
  auto form = [&](int step) {
    const int slot = step % RING;
    char* xp = &sm.x[slot][f_off];
    const u32x4 xv = *(const u32x4*)xp;
    const u32x4 gl = *(const u32x4*)&sm.g[slot][16 * f_c];
    const u32x4 gv = norm ? gl : u32x4{kBf16OnePair, kBf16OnePair, kBf16OnePair, kBf16OnePair};
    u32x4 av;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const bf16x2 x = st_bf16x2(xv[d]);
      av[d] = pack_bf16x2(__builtin_amdgcn_fdot2_f32_bf16(x, st_bf16x2(gv[d] & 0xffffu), 0.0f, false),
                          __builtin_amdgcn_fdot2_f32_bf16(x, st_bf16x2(gv[d] & 0xffff0000u), 0.0f, false));
      ss = __builtin_amdgcn_fdot2_f32_bf16(x, x, ss, false);
    }
    *(u32x4*)xp = av;
  };

  // Wave roles: partial set w>>1 (gated: weight set>>1, k-half set&1;
  // plain: k-quarter set), column block w&1, both 32-row blocks.
  const int set = w >> 1, cb = w & 1;
  const int wsel = NW == 2 ? (set >> 1) : 0;
  const int s_first = NW == 2 ? 2 * (set & 1) : set;
  const int a_lo = l & 31;  // fragment row within a 32-row block
  const int bG = l >> 4, bi = l & 15;
  const int b_k = 8 * (bG >> 1) + (bi >> 2), b_n = cb * 32 + 16 * (bG & 1) + 4 * (bi & 3);
  const int b_off = b_k * 128 + (((b_n >> 3) ^ (2 * (b_k & 3))) << 4) + ((b_n & 7) << 1);
  floatx16 acc[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[rb][e] = 0.f;

  // Steps 0 .. AHEAD-1 in flight, step 0 formed, before the loop.
  // Iteration kt issues step kt+AHEAD into the slot last read in iteration
  // kt-2 (the barrier of iteration kt-1 orders that), waits until only the
  // AHEAD-1 newest steps may be outstanding (step kt+1 has landed for this
  // wave); after the barrier (every wave's part of step kt+1 has landed and
  // iteration kt-1 is finished everywhere) it reads the operands of step kt
  // (formed in iteration kt-1), forms step kt+1 and multiplies step kt.
  // Steps past the last one read zeros (range checks).
  // Wait until this wave's part of the step AHEAD-1 issues back has landed.
  auto wait_landed = [&] {
    if (w == 0)
      ST_WAIT_VMCNT((AHEAD - 1) * (NW + 2));
    else
      ST_WAIT_VMCNT((AHEAD - 1) * (NW + 1));
  };
  for (int st = 0; st < AHEAD; ++st) issue_step(st);
  wait_landed();
  __syncthreads();
  form(0);
  for (int kt = 0; kt < nk; ++kt) {
    issue_step(kt + AHEAD);
    wait_landed();
    __syncthreads();
    const int slot = kt % RING;
    const char* x_lds = &sm.x[slot][0];
    const lds_char* b_lds = (const lds_char*)&sm.w[slot][wsel][0];
    u32x4 av[SUBS][2], bv[SUBS];
#pragma unroll
    for (int i = 0; i < SUBS; ++i) {
      const int s = s_first + i;
      const int kc = 2 * s + (l >> 5);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
        av[i][rb] = *(const u32x4*)(x_lds + (rb * 32 + a_lo) * 128 + ((kc ^ st_xswz(a_lo)) << 4));
      const u32x2 lo = __builtin_bit_cast(
          u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(b_lds + b_off + 16 * s * 128)));
      const u32x2 hi = __builtin_bit_cast(
          u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(b_lds + b_off + (16 * s + 4) * 128)));
      bv[i] = u32x4{lo[0], lo[1], hi[0], hi[1]};
    }
    if (kt + 1 < nk) form(kt + 1);
#pragma unroll
    for (int i = 0; i < SUBS; ++i)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
        acc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[i][rb]),
                                                          __builtin_bit_cast(bf16x8, bv[i]),
                                                          acc[rb], 0, 0, 0);
  }
  ST_WAIT_VMCNT(0);

  // Row sums of squares: the 8 threads of a row hold disjoint k-chunks.
  ss += __shfl_xor(ss, 1);
  ss += __shfl_xor(ss, 2);
  ss += __shfl_xor(ss, 4);
  if (f_c == 0) sm.ss[f_row] = ss;
  __syncthreads();  // every wave is done with the rings before they are reused
  // Partial blocks to LDS as [set][row][col] fp32.  32x32 layout: lane l
  // holds column l%32 and, for register 4 jj + r, row 8 jj + 4 (l/32) + r.
  float* red = (float*)&sm.w[0][0][0];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = rb * 32 + 8 * jj + 4 * (l >> 5) + r, col = cb * 32 + (l & 31);
        red[(set * ST_BM + row) * ST_BN + col] = acc[rb][4 * jj + r];
      }
  if (tid < ST_BM) sm.inv[tid] = norm ? inv_rms(sm.ss[tid], K, eps) : 1.0f;
  __syncthreads();

  // Epilogue: thread -> row tid>>3, columns 8 (tid&7) .. +7.
  const int orow = tid >> 3, oc = 8 * (tid & 7);
  const int64_t n = n0 + oc;
  if (orow < M && n < N) {
    const float inv = sm.inv[orow];
    float p[4][8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const floatx4* src = (const floatx4*)(red + (q * ST_BM + orow) * ST_BN + oc);
      const floatx4 u = src[0], v = src[1];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        p[q][e] = u[e];
        p[q][4 + e] = v[e];
      }
    }
    u32x4 out;
#pragma unroll
    for (int c = 0; c < 8; c += 2) {
      float y[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        if (NW == 2)
          y[e] = silu_gate((p[0][c + e] + p[1][c + e]) * inv, (p[2][c + e] + p[3][c + e]) * inv);
        else
          y[e] = ((p[0][c + e] + p[1][c + e]) + (p[2][c + e] + p[3][c + e])) * inv;
      }
      out[c >> 1] = pack_bf16x2(y[0], y[1]);
    }
    *(u32x4*)(Y + (int64_t)orow * N + n) = out;
  }
}

}  // namespace rmm

hipError_t rmm_launch_stream(const RmmArgs& a) {
  using namespace rmm;
  const unsigned grid = (unsigned)((a.N + ST_BN - 1) / ST_BN);
  if (a.gated)
    hipLaunchKernelGGL((stream_kernel<2>), dim3(grid), dim3(ST_THREADS), 0, a.stream,
                       (const bf16_t*)a.X, (const bf16_t*)a.g, (const bf16_t*)a.W1,
                       (const bf16_t*)a.W3, (bf16_t*)a.Y, a.eps, (int)a.M, a.N, a.K, a.norm);
  else
    hipLaunchKernelGGL((stream_kernel<1>), dim3(grid), dim3(ST_THREADS), 0, a.stream,
                       (const bf16_t*)a.X, (const bf16_t*)a.g, (const bf16_t*)a.W1,
                       (const bf16_t*)a.W3, (bf16_t*)a.Y, a.eps, (int)a.M, a.N, a.K, a.norm);
  return hipGetLastError();
}
