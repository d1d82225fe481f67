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
// Split-form partial sums: device-scope coherent (SC1) accesses, since the
// workgroups sharing a strip run on different XCDs (no shared L2).
constexpr int kStCoherent = 16;

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

// The gated form carries the operand X*g exactly as two bf16 parts
// (split_bf16x2): the gate multiplies one product's error by the other
// product, so a single rounding of X*g would not keep every output within
// the elementwise bound the plain product meets.  The high part replaces X
// in its ring slot; the low part goes to a two-slot ring of its own (the
// step being multiplied and the step being formed).
template <int NW>
struct StSplitOp {
  static constexpr bool value = NW == 2;
};

template <int NW>
struct StSmem {
  char w[StCfg<NW>::RING][NW][ST_W_BYTES];
  char x[StCfg<NW>::RING][ST_X_BYTES];
  char xl[StSplitOp<NW>::value ? 2 : 1][StSplitOp<NW>::value ? ST_X_BYTES : 16];
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

// Workspace of the split (stream-K) form: which global steps a workgroup
// takes, and where a segment's partial sums go.  Global step s is k-step
// s % nk of strip s / nk; workgroup b of P takes steps [b T / P, (b+1) T / P)
// of the T = strips * nk, so a range covers at most two strips (fewer
// strips than workgroups) and a strip is shared by consecutive workgroups.
struct StSplit {
  int strips;            // 64-column strips (< P)
  unsigned* cnt;         // per strip: segments counted so far
  float* part;           // [P][2 segments][NW][64 rows][64 cols] fp32
  float* ssq;            // [P][2 segments][64 rows] fp32
};

__device__ __forceinline__ int64_t st_first_step(int64_t b, int64_t T, int64_t P) { return b * T / P; }
// The workgroup whose range holds global step s.
__device__ __forceinline__ int st_owner(int64_t s, int64_t T, int64_t P) {
  return (int)(((s + 1) * P - 1) / T);
}

template <int NW, bool SK>
__global__ __launch_bounds__(ST_THREADS, 1) void stream_kernel(
    const bf16_t* __restrict__ X, const bf16_t* __restrict__ g, const bf16_t* __restrict__ W1,
    const bf16_t* __restrict__ W3, bf16_t* __restrict__ Y, float eps, int M, int64_t N,
    int64_t K, int norm, StSplit sp) {
  constexpr int RING = StCfg<NW>::RING, AHEAD = StCfg<NW>::AHEAD, SUBS = StCfg<NW>::SUBS;
  constexpr bool SPLIT = StSplitOp<NW>::value;
  __shared__ __attribute__((aligned(1024))) StSmem<NW> sm;
  __shared__ int last2[2];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int nk = (int)((K + ST_BK - 1) / ST_BK);
  // Local steps 0 .. n-1 of this workgroup: strip strip0 from k-step kt0
  // on, continuing into strip strip0 + 1 past its last k-step.
  const int64_t P = gridDim.x, T = SK ? (int64_t)sp.strips * nk : 0;
  const int64_t s_lo = SK ? st_first_step(blockIdx.x, T, P) : 0;
  const int n = SK ? (int)(st_first_step(blockIdx.x + 1, T, P) - s_lo) : nk;
  const int strip0 = SK ? (int)(s_lo / nk) : (int)blockIdx.x;
  const int kt0 = SK ? (int)(s_lo % nk) : 0;
  // A range that reaches into the next strip takes that strip's first nb
  // k-steps first, then strip0's from kt0: every workgroup then sweeps K
  // within a few steps of the others, as the unsplit form does, so the
  // weight rows read at one time stay close together in memory (in global
  // order, plain 16 x 4096 x 6144 took 31.4 -> 29.3 us with this order and
  // a batched combine).
  const int nb = kt0 + n > nk ? kt0 + n - nk : 0;

  // Per-lane source offsets of one step (relative to the step's resource).
  // W: wave w fills rows 8w .. 8w+7 of a slot; lane l lands at byte 16 l;
  // the strip's column offset is added per step.
  uint32_t w_lane;
  int w_col;
  {
    const int kl = 8 * w + (l >> 3);
    const int c = (l & 7) ^ (2 * (kl & 3));
    w_col = 8 * c;
    w_lane = (uint32_t)((kl * N + w_col) * 2);
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
    // Local step -> (strip, k-step); past the range: k-step nk (zeros).
    const int strip = step < nb ? strip0 + 1 : strip0;
    const int kt = step < nb ? step : (step < n ? kt0 + step - nb : nk);
    const int64_t k0 = (int64_t)kt * ST_BK;
    const int64_t rows = K - k0 > 0 ? K - k0 : 0;
    const int slot = step % RING;
    const int64_t ns = (int64_t)strip * ST_BN;
    const uint32_t w_off = ns + w_col < N ? w_lane + (uint32_t)(ns * 2) : kStOutOfRange;
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
    u32x4 av, al;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const bf16x2 x = st_bf16x2(xv[d]);
      const float p0 = __builtin_amdgcn_fdot2_f32_bf16(x, st_bf16x2(gv[d] & 0xffffu), 0.0f, false);
      const float p1 = __builtin_amdgcn_fdot2_f32_bf16(x, st_bf16x2(gv[d] & 0xffff0000u), 0.0f, false);
      if (SPLIT) {
        const u32x2 hl = split_bf16x2(p0, p1);
        av[d] = hl[0];
        al[d] = hl[1];
      } else
        av[d] = pack_bf16x2(p0, p1);
      ss = __builtin_amdgcn_fdot2_f32_bf16(x, x, ss, false);
    }
    *(u32x4*)xp = av;
    if (SPLIT) *(u32x4*)&sm.xl[step & 1][f_off] = al;
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
  floatx16 acc[2], acc0[2], accl[2];
  float ss0 = 0.f;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[rb][e] = acc0[rb][e] = accl[rb][e] = 0.f;

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
  for (int kt = 0; kt < n; ++kt) {
    issue_step(kt + AHEAD);
    wait_landed();
    __syncthreads();
    const int slot = kt % RING;
    // Split form: local step kt+1 starts the range's second strip.
    const bool seg_end = SK && kt + 1 == nb;
    const char* x_lds = &sm.x[slot][0];
    const char* xl_lds = &sm.xl[SPLIT ? (kt & 1) : 0][0];
    const lds_char* b_lds = (const lds_char*)&sm.w[slot][wsel][0];
    u32x4 av[SUBS][2], avl[SUBS][2], bv[SUBS];
#pragma unroll
    for (int i = 0; i < SUBS; ++i) {
      const int s = s_first + i;
      const int kc = 2 * s + (l >> 5);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const int ao = (rb * 32 + a_lo) * 128 + ((kc ^ st_xswz(a_lo)) << 4);
        av[i][rb] = *(const u32x4*)(x_lds + ao);
        if (SPLIT) avl[i][rb] = *(const u32x4*)(xl_lds + ao);
      }
      const u32x2 lo = __builtin_bit_cast(
          u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(b_lds + b_off + 16 * s * 128)));
      const u32x2 hi = __builtin_bit_cast(
          u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(b_lds + b_off + (16 * s + 4) * 128)));
      bv[i] = u32x4{lo[0], lo[1], hi[0], hi[1]};
    }
    // The MFMAs go out first, the forming of the next step (VALU and LDS)
    // runs in their shadow.  The low parts accumulate separately (two more
    // independent accumulator chains per wave).
#pragma unroll
    for (int i = 0; i < SUBS; ++i)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
        acc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[i][rb]),
                                                          __builtin_bit_cast(bf16x8, bv[i]),
                                                          acc[rb], 0, 0, 0);
    if (SPLIT) {
#pragma unroll
      for (int i = 0; i < SUBS; ++i)
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
          accl[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, avl[i][rb]),
                                                             __builtin_bit_cast(bf16x8, bv[i]),
                                                             accl[rb], 0, 0, 0);
    }
    if (seg_end) {
      ss0 = ss;
      ss = 0.f;
    }
    if (kt + 1 < n) form(kt + 1);
    if (seg_end) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        acc0[rb] = SPLIT ? acc[rb] + accl[rb] : acc[rb];
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[rb][e] = accl[rb][e] = 0.f;
      }
    }
  }
  if (SPLIT) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) acc[rb] += accl[rb];
  }
  ST_WAIT_VMCNT(0);

  // Tail, per segment (one, or two in the split form): the waves' partial
  // sets to LDS as [set][row][col] fp32 (the rings are free now), then for
  // thread -> row tid>>3, columns 8 (tid&7) .. +7 the sums of the sets: the
  // two k-halves of each weight (gated) or the four k-quarters (plain).
  float* red = (float*)&sm.w[0][0][0];
  const int orow = tid >> 3, oc = 8 * (tid & 7);
  auto stage_sets = [&](const floatx16 (&a)[2], float ssv) {
    // Row sums of squares: the 8 threads of a row hold disjoint k-chunks.
    ssv += __shfl_xor(ssv, 1);
    ssv += __shfl_xor(ssv, 2);
    ssv += __shfl_xor(ssv, 4);
    __syncthreads();  // the rings (or the previous segment's sets) are no longer read
    if (f_c == 0) sm.ss[f_row] = ssv;
    // 32x32 layout: lane l holds column l%32 and, for register 4 jj + r,
    // row 8 jj + 4 (l/32) + r.
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = rb * 32 + 8 * jj + 4 * (l >> 5) + r, col = cb * 32 + (l & 31);
          red[(set * ST_BM + row) * ST_BN + col] = a[rb][4 * jj + r];
        }
    __syncthreads();
  };
  auto sum_sets = [&](float (&z)[NW][8]) {
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
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      if (NW == 2) {
        z[0][c] = p[0][c] + p[1][c];
        z[NW - 1][c] = p[2][c] + p[3][c];
      } else {
        z[0][c] = (p[0][c] + p[1][c]) + (p[2][c] + p[3][c]);
      }
    }
  };
  // Y = z / RMS (gated: silu(z1 / RMS) * z3 / RMS), 16 bytes per thread.
  auto store_y = [&](const float (&z)[NW][8], float ssr, int strip) {
    const int64_t n = (int64_t)strip * ST_BN + oc;
    if (orow < M && n < N) {
      const float inv = norm ? inv_rms(ssr, K, eps) : 1.0f;
      u32x4 out;
#pragma unroll
      for (int c = 0; c < 8; c += 2) {
        float y[2];
#pragma unroll
        for (int e = 0; e < 2; ++e)
          y[e] = NW == 2 ? silu_gate(z[0][c + e] * inv, z[NW - 1][c + e] * inv) : z[0][c + e] * inv;
        out[c >> 1] = pack_bf16x2(y[0], y[1]);
      }
      *(u32x4*)(Y + (int64_t)orow * N + n) = out;
    }
  };

  if (!SK) {
    stage_sets(acc, ss);
    float z[NW][8];
    sum_sets(z);
    store_y(z, sm.ss[orow], strip0);
    return;
  }

  // Split form: a segment that covers its whole strip is finished here; any
  // other stores its sums (fp32, device-coherent) and counts itself at the
  // strip; the strip's last segment to be counted adds every segment's sums
  // in k order (so the result does not depend on arrival order) and stores Y.
  // Segments in the order they were computed: strip0 + 1's first nb
  // k-steps (acc0), then strip0's from kt0 (acc).  A segment's sums go to
  // slot 2 b + (strip != strip0).  Both segments are stored before one wait
  // for the stores and one round of counting.
  const int nseg = nb > 0 ? 2 : 1;
  const int64_t slots = 2 * P;
  const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
      sp.part, 0, (int)(slots * NW * ST_BM * ST_BN * 4), 0x00020000);
  const __amdgpu_buffer_rsrc_t srs =
      __builtin_amdgcn_make_buffer_rsrc(sp.ssq, 0, (int)(slots * ST_BM * 4), 0x00020000);
  auto part_off = [&](int64_t sl, int v, int h) {
    return (int)((((sl * NW + v) * ST_BM + orow) * ST_BN + oc + 4 * h) * 4);
  };
  bool partial[2] = {false, false};
  for (int seg = 0; seg < nseg; ++seg) {
    const bool next = nseg == 2 && seg == 0;
    const int strip = next ? strip0 + 1 : strip0;
    const int kt_lo = next ? 0 : kt0;
    const int kt_hi = next ? nb : (kt0 + n - nb);
    if (next)
      stage_sets(acc0, ss0);
    else
      stage_sets(acc, ss);
    float z[NW][8];
    sum_sets(z);
    if (kt_lo == 0 && kt_hi == nk) {
      store_y(z, sm.ss[orow], strip);
      continue;
    }
    partial[seg] = true;
    const int64_t sl = 2 * (int64_t)blockIdx.x + (next ? 1 : 0);
#pragma unroll
    for (int v = 0; v < NW; ++v)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const floatx4 q4 = {z[v][4 * h], z[v][4 * h + 1], z[v][4 * h + 2], z[v][4 * h + 3]};
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, q4), prs, part_off(sl, v, h), 0,
                                               kStCoherent);
      }
    if (tid < ST_BM)
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sm.ss[tid]), srs, (int)((sl * ST_BM + tid) * 4),
                                            0, kStCoherent);
  }
  __builtin_amdgcn_s_waitcnt(0);  // the sums are visible device-wide before they are counted
  __syncthreads();
  // Thread seg counts segment seg at its strip.
  if (tid < nseg && partial[tid]) {
    const bool next = nseg == 2 && tid == 0;
    const int strip = next ? strip0 + 1 : strip0;
    const int b_lo = st_owner((int64_t)strip * nk, T, P), b_hi = st_owner((int64_t)strip * nk + nk - 1, T, P);
    last2[tid] = __hip_atomic_fetch_add(&sp.cnt[strip], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                 (unsigned)(b_hi - b_lo);
  }
  __syncthreads();
  for (int seg = 0; seg < nseg; ++seg) {
    if (!partial[seg] || !last2[seg]) continue;
    const bool next = nseg == 2 && seg == 0;
    const int strip = next ? strip0 + 1 : strip0;
    const int b_lo = st_owner((int64_t)strip * nk, T, P), b_hi = st_owner((int64_t)strip * nk + nk - 1, T, P);
    float zs[NW][8], ssr = 0.f;
#pragma unroll
    for (int v = 0; v < NW; ++v)
#pragma unroll
      for (int c = 0; c < 8; ++c) zs[v][c] = 0.f;
    // Up to 4 contributors' loads in flight at once, added in k order.
    for (int b0 = b_lo; b0 <= b_hi; b0 += 4) {
      floatx4 q[4][NW][2];
      float sv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int b = b0 + u;
        const bool ok = b <= b_hi;
        // Workgroup b's segment on this strip: its first, unless its range
        // starts in the strip before.
        const int64_t sb = 2 * (int64_t)b + (st_first_step(b, T, P) / nk == strip ? 0 : 1);
#pragma unroll
        for (int v = 0; v < NW; ++v)
#pragma unroll
          for (int h = 0; h < 2; ++h)
            q[u][v][h] = __builtin_bit_cast(
                floatx4, __builtin_amdgcn_raw_buffer_load_b128(
                             prs, ok ? (uint32_t)part_off(sb, v, h) : kStOutOfRange, 0, kStCoherent));
        sv[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
            srs, ok ? (uint32_t)((sb * ST_BM + orow) * 4) : kStOutOfRange, 0, kStCoherent));
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int v = 0; v < NW; ++v)
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int e = 0; e < 4; ++e) zs[v][4 * h + e] += q[u][v][h][e];
        ssr += sv[u];
      }
    }
    store_y(zs, ssr, strip);
    if (tid == 0) __hip_atomic_store(&sp.cnt[strip], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace rmm

static size_t st_align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Split form when there are at most half as many 64-column strips as
// `target` workgroups (one per CU): every CU then takes an equal share of
// all the k-steps.  With more strips the unsplit form is faster: at 224
// strips (the gated 64 x 4096 x 14336 shape) the split form took 62 us
// against 52 us, while at 96 strips (plain 16 x 4096 x 6144) it took 29 us
// against 34 us.  Spreading the workgroups' k-steps apart costs the unsplit
// form's lockstep sweep over the weight rows, and the partial sums add a
// combine; only a large gain in CUs pays for that.
void rmm_stream_plan(int64_t N, int64_t K, int gated, int target, bool have_ws, StreamPlan* p) {
  using namespace rmm;
  const int64_t strips = (N + ST_BN - 1) / ST_BN, nk = (K + ST_BK - 1) / ST_BK;
  const int64_t T = strips * nk;
  const int nw = gated ? 2 : 1;
  p->strips = (int)strips;
  p->split = have_ws && 2 * strips <= target;
  p->grid = p->split ? (int)(T < target ? T : target) : (int)strips;
  p->ws_cnt_off = 0;
  p->ws_part_off = kWsCounterBytes;
  p->ws_ssq_off = p->ws_part_off + (size_t)2 * target * nw * ST_BM * ST_BN * sizeof(float);
  // Sized for `target` workgroups whatever the grid, so the size depends on
  // the shape and the weight count only.
  p->ws_bytes = 2 * strips <= target ? p->ws_ssq_off + st_align256((size_t)2 * target * ST_BM * sizeof(float)) : 0;
}

hipError_t rmm_launch_stream(const RmmArgs& a, const StreamPlan& p, void* ws) {
  using namespace rmm;
  if (p.split && !ws) return hipErrorInvalidValue;
  StSplit sp{p.strips, nullptr, nullptr, nullptr};
  if (p.split) {
    char* base = (char*)ws;
    sp.cnt = (unsigned*)(base + p.ws_cnt_off);
    sp.part = (float*)(base + p.ws_part_off);
    sp.ssq = (float*)(base + p.ws_ssq_off);
  }
  const dim3 grid((unsigned)p.grid), block(ST_THREADS);
  const bf16_t *x = (const bf16_t*)a.X, *g = (const bf16_t*)a.g, *w1 = (const bf16_t*)a.W1,
               *w3 = (const bf16_t*)a.W3;
  bf16_t* y = (bf16_t*)a.Y;
  const int m = (int)a.M;
  if (a.gated && p.split)
    hipLaunchKernelGGL((stream_kernel<2, true>), grid, block, 0, a.stream, x, g, w1, w3, y, a.eps, m, a.N,
                       a.K, a.norm, sp);
  else if (a.gated)
    hipLaunchKernelGGL((stream_kernel<2, false>), grid, block, 0, a.stream, x, g, w1, w3, y, a.eps, m,
                       a.N, a.K, a.norm, sp);
  else if (p.split)
    hipLaunchKernelGGL((stream_kernel<1, true>), grid, block, 0, a.stream, x, g, w1, w3, y, a.eps, m, a.N,
                       a.K, a.norm, sp);
  else
    hipLaunchKernelGGL((stream_kernel<1, false>), grid, block, 0, a.stream, x, g, w1, w3, y, a.eps, m,
                       a.N, a.K, a.norm, sp);
  return hipGetLastError();
}
