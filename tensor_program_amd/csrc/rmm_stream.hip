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
//   * wave w takes row block w & 1 (32 rows) over k-quarter w >> 1 of every
//     step, for every 32-column block of the strip (2 per weight), with
//     v_mfma_f32_32x32x16_bf16.  Each X element of a step is read by one
//     lane, which forms the matrix operand in registers: X*g in fp32 (bf16
//     dot2 with one lane of g zeroed: an exact product) rounded once to bf16
//     -- for two weights split into two exact bf16 parts, both multiplied --
//     and X^2 added to its row's partial sum of squares.  B fragments come
//     from ds_read_b64_tr_b16 (gfx950's transposing LDS read): lane i of each
//     16-lane group receives 4 consecutive k of column i.  Each W element is
//     read from LDS by the two row-block waves of its k-quarter.
//   * epilogue through LDS: the k-quarters' partial sums are added, Y =
//     acc / RMS, gated Y = silu(acc1/RMS) * acc3/RMS.
#include "rmm_device.h"

namespace rmm {

constexpr int ST_THREADS = 512;
constexpr int ST_BN = 64;                        // columns per workgroup
constexpr int ST_BM = 64;                        // rows (M <= 64)
constexpr int ST_BK = 64;                        // k per step
constexpr int ST_W_BYTES = ST_BK * ST_BN * 2;    // 8 KB per weight per slot
constexpr int ST_X_BYTES = ST_BM * ST_BK * 2;    // 8 KB per slot
constexpr int ST_G_BYTES = 128;                  // the g slice of a step
// Out-of-range lane offset and the scalar offset of the steps past a range.
// Every buffer is at most 2^30 bytes and a W step at most 2^25 bytes
// (checked by the launcher), so a lane offset plus a scalar offset never
// wraps 32 bits, and either constant in the sum puts it past the buffer.
constexpr uint32_t kStOutOfRange = 0x40000000u;
constexpr uint32_t kStPastRange = 0x40000000u;
// Split-form partial sums: device-scope coherent (SC1) accesses, since the
// workgroups sharing a strip run on different XCDs (no shared L2).
constexpr int kStCoherent = 16;

// Ring depth per weight count: RING - 1 steps are in flight while one is
// multiplied.
template <int NW>
struct StCfg {
  static constexpr int RING = NW == 2 ? 6 : 8;
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
// lds_addr + 16 l), from byte voff + soff of the buffer; the range check
// covers voff + soff, so an offset at or past the buffer's size reads
// zeros.  Inline asm keeps the compiler from serialising it against the
// other loads in flight; the k-loop waits with explicit vmcnt.
__device__ __forceinline__ void st_lds_load16(uint32_t lds_addr, uint32_t voff, i32x4 rsrc, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(rsrc), "s"(soff)
               : "memory", "m0");
}
// The same from lanes 0..7 only (128 bytes): the exec mask is narrowed and
// restored inside the statement.
__device__ __forceinline__ void st_lds_load16_x8(uint32_t lds_addr, uint32_t voff, i32x4 rsrc, uint32_t soff) {
  uint64_t saved;
  asm volatile(
      "s_mov_b64 %0, exec\n\ts_mov_b64 exec, 0xff\n\ts_mov_b32 m0, %1\n\t"
      "buffer_load_dwordx4 %2, %3, %4 offen lds\n\ts_mov_b64 exec, %0"
      : "=&s"(saved)
      : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(rsrc), "s"(soff)
      : "memory", "m0");
}

#define ST_WAIT_VMCNT(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14))

// The gated form carries the operand X*g exactly as two bf16 parts
// (split_bf16x2): the gate multiplies one product's error by the other
// product, so a single rounding of X*g would not keep every output within
// the elementwise bound the plain product meets.  Both parts multiply the
// same W fragment into the same accumulator.
template <int NW>
struct StSplitOp {
  static constexpr bool value = NW == 2;
};

template <int NW>
struct StSmem {
  char w[StCfg<NW>::RING][NW][ST_W_BYTES];
  char x[StCfg<NW>::RING][ST_X_BYTES];
  char g[StCfg<NW>::RING][8][ST_G_BYTES];  // one copy of the g slice per wave
  float ssp[4][ST_BM];  // row sums of squares per k-quarter
  float ss[ST_BM];
};
// The epilogue reuses the W and X rings (contiguous) for 2 fp32 partial
// sets of NW blocks of 64 x 64.
template <int NW>
constexpr int st_red_bytes() { return 2 * NW * ST_BM * ST_BN * 4; }
static_assert(sizeof(StSmem<1>::w) + sizeof(StSmem<1>::x) >= st_red_bytes<1>(), "ring too small");
static_assert(sizeof(StSmem<2>::w) + sizeof(StSmem<2>::x) >= st_red_bytes<2>(), "ring too small");
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

template <int NW, bool SK, bool NORM>
__global__ __launch_bounds__(ST_THREADS, 1) void stream_kernel(
    const bf16_t* __restrict__ X, const bf16_t* __restrict__ g, const bf16_t* __restrict__ W1,
    const bf16_t* __restrict__ W3, bf16_t* __restrict__ Y, float eps, int M, int64_t N,
    int64_t K, StSplit sp) {
  constexpr int RING = StCfg<NW>::RING;
  // Without the gain the operand is X itself: one exact part.
  constexpr bool SPLIT = StSplitOp<NW>::value && NORM;
  __shared__ __attribute__((aligned(1024))) StSmem<NW> sm;
  __shared__ int last2[2];
  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
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

  // Buffer resources (fixed) and per-lane offsets; the step's position is a
  // scalar byte offset (soffset) added to every lane's.
  //   W (K x N): soffset (k0 N + n0) 2 for the step's first row and the
  //   strip's first column n0; wave w fills rows 8w .. 8w+7 of a slot, lane
  //   l lands at byte 16 l.  Rows past K fall past the buffer (zeros);
  //   columns past N get an out-of-range lane offset, checked once for each
  //   of the (at most two) strips of the range.
  //   X (M x K) and g (K): soffset 2 k0.  Lanes whose k is past K, or whose
  //   row is past M, get an out-of-range lane offset (a row's k past K
  //   would otherwise read the next row).
  // Past the last step of the range the offsets are moved out of range, so
  // the steps issued there read zeros.
  uint32_t w_off0, w_off1;
  {
    const int kl = 8 * w + (l >> 3);
    const int c = (l & 7) ^ (2 * (kl & 3));
    const uint32_t lane = (uint32_t)((kl * N + 8 * c) * 2);
    w_off0 = (int64_t)strip0 * ST_BN + 8 * c < N ? lane : kStOutOfRange;
    w_off1 = (int64_t)(strip0 + 1) * ST_BN + 8 * c < N ? lane : kStOutOfRange;
  }
  const int x_row = 8 * w + (l >> 3);
  const int x_k = 8 * ((l & 7) ^ st_xswz(x_row));
  const uint32_t x_off = x_row < M ? (uint32_t)((x_row * K + x_k) * 2) : kStOutOfRange;
  const uint32_t lds_w = (uint32_t)(uintptr_t)(lds_char*)&sm.w[0][0][0] + w * 1024;
  const uint32_t lds_x = (uint32_t)(uintptr_t)(lds_char*)&sm.x[0][0] + w * 1024;
  const uint32_t lds_g = (uint32_t)(uintptr_t)(lds_char*)&sm.g[0][w][0];
  const i32x4 rs_w[2] = {st_rsrc(W1, (uint32_t)(K * N * 2)), st_rsrc(NW == 2 ? W3 : W1, (uint32_t)(K * N * 2))};
  const i32x4 rs_x = st_rsrc(X, (uint32_t)(M * K * 2));
  const i32x4 rs_g = st_rsrc(g, (uint32_t)(K * 2));
  const uint32_t w_step = (uint32_t)(ST_BK * N * 2);
  // Issue state of the next step: W and X/g scalar offsets, K - k0.
  uint32_t so_w, so_x;
  int krem;
  auto seg_start = [&](int strip, int kt) {
    so_w = (uint32_t)(((int64_t)kt * ST_BK * N + (int64_t)strip * ST_BN) * 2);
    so_x = (uint32_t)(kt * ST_BK * 2);
    krem = (int)(K - (int64_t)kt * ST_BK);
  };
  seg_start(nb > 0 ? strip0 + 1 : strip0, nb > 0 ? 0 : kt0);

  // Issue every transfer of one step into ring slot `slot`: NW W blocks,
  // one X block and the step's g slice (lanes 0..7, one copy per wave) --
  // NW + 2 vector-memory instructions per wave (NW + 1 without the gain).
  // The steps are issued in order; the split form's range moves to strip0
  // at local step nb.
  auto issue_step = [&](int step, int slot) {
    if (SK && step == nb && nb > 0) seg_start(strip0, kt0);
    if (step == n) {
      so_w = so_x = kStPastRange;
      krem = 0;
    }
    const uint32_t w_off = SK && step < nb ? w_off1 : w_off0;
#pragma unroll
    for (int v = 0; v < NW; ++v)
      st_lds_load16(lds_w + (uint32_t)((slot * NW + v) * ST_W_BYTES), w_off, rs_w[v], so_w);
    st_lds_load16(lds_x + (uint32_t)(slot * ST_X_BYTES), x_k < krem ? x_off : kStOutOfRange, rs_x, so_x);
    if (NORM) st_lds_load16_x8(lds_g + (uint32_t)(slot * 8 * ST_G_BYTES), (uint32_t)(16 * l), rs_g, so_x);
    so_w += w_step;
    so_x += ST_BK * 2;
    krem -= ST_BK;
  };

  // Wave roles: wave w multiplies row block rb = w & 1 (32 rows) over
  // k-quarter kq = w >> 1 of every step (16 k), for all 64 columns of each
  // weight (2 NW column blocks of 32).  Every X element of a step is thus
  // read by exactly one lane, which forms its operand in registers: lane l
  // holds row 32 rb + l % 32, k 16 kq + 8 (l / 32) .. +7 of the step, the
  // A-fragment layout of v_mfma_f32_32x32x16_bf16; it multiplies by g in
  // fp32 (bf16 dot2 with one lane of g zeroed: an exact product), rounds once
  // to bf16 (gated: splits into two exact parts) and adds X^2 to its row's
  // partial sum of squares.
  const int rb = w & 1, kq = w >> 1;
  const int a_row = rb * 32 + (l & 31);
  const int a_kc = 2 * kq + (l >> 5);
  const int a_off = a_row * 128 + ((a_kc ^ st_xswz(a_row)) << 4);
  const int g_off = 16 * a_kc;
  // B fragments: lane i of each 16-lane group receives 4 consecutive k of
  // one column (ds_read_b64_tr_b16); column half h of a weight's 64.
  const int bG = l >> 4, bi = l & 15;
  const int b_k = 8 * (bG >> 1) + (bi >> 2) + 16 * kq;
  int b_off[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int b_n = h * 32 + 16 * (bG & 1) + 4 * (bi & 3);
    b_off[h] = b_k * 128 + (((b_n >> 3) ^ (2 * (b_k & 3))) << 4) + ((b_n & 7) << 1);
  }
  constexpr int NB = 2 * NW;  // column blocks per wave
  floatx16 acc[NB], acc0[NB];
  float ss = 0.f, ss0 = 0.f;
#pragma unroll
  for (int c = 0; c < NB; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[c][e] = acc0[c][e] = 0.f;

  // The operands of one step in registers: the W fragments of every column
  // block, and X*g formed from the raw X chunk and g slice.  Slot offsets
  // are compile-time constants in the unrolled loop below (immediate LDS
  // offsets), so reading a step costs no address arithmetic.
  auto read_b = [&](int slot, u32x4 (&bv)[NB]) {
#pragma unroll
    for (int c = 0; c < NB; ++c) {
      const lds_char* bp = (const lds_char*)&sm.w[slot][c >> 1][b_off[c & 1]];
      const u32x2 lo = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)bp));
      const u32x2 hi =
          __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(bp + 4 * 128)));
      bv[c] = u32x4{lo[0], lo[1], hi[0], hi[1]};
    }
  };
  auto read_xg = [&](int slot, u32x4& xv, u32x4& gl) {
    xv = *(const u32x4*)&sm.x[slot][a_off];
    if (NORM) gl = *(const u32x4*)&sm.g[slot][w][g_off];
  };
  // Forming works on fp32 values (bf16 -> fp32 is a shift; a product of two
  // bf16 is exact in fp32) with plain multiplies and FMAs: on gfx950 the
  // bf16 dot-product instructions occupy the matrix pipe and would not
  // overlap with the MFMAs they are interleaved with.
  auto form_regs = [&](const u32x4& xv, const u32x4& gl, u32x4& ah, u32x4& al) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      if (NORM) {
        const float x0 = __uint_as_float(xv[d] << 16), x1 = __uint_as_float(xv[d] & 0xffff0000u);
        const float p0 = x0 * __uint_as_float(gl[d] << 16), p1 = x1 * __uint_as_float(gl[d] & 0xffff0000u);
        if (SPLIT) {
          const u32x2 hl = split_bf16x2(p0, p1);
          ah[d] = hl[0];
          al[d] = hl[1];
        } else {
          ah[d] = pack_bf16x2(p0, p1);
        }
        ss = __builtin_fmaf(x1, x1, __builtin_fmaf(x0, x0, ss));
      } else {
        ah[d] = xv[d];  // without the gain no sums of squares are needed
      }
    }
  };

  // Software pipeline over a ring of RING slots, all of them filled before
  // the loop.  Iteration kt holds step kt's operands in registers; it waits
  // until only the RING-2 newest steps may be outstanding (step kt+1 has
  // landed for this wave); after the barrier every wave's part of step kt+1
  // has landed and iteration kt-1 -- which read step kt into registers --
  // is finished everywhere, so step kt's slot is free.  The wave then reads
  // step kt+1's W fragments and raw X chunk and g slice, issues step
  // kt+RING into step kt's slot, and multiplies step kt while it forms step
  // kt+1: the MFMAs need nothing the new reads bring, and the forming
  // arithmetic is placed between them (a wave issues in order).  Steps past
  // the last one read zeros (range checks).
  constexpr int PER_STEP = NW + (NORM ? 2 : 1);  // loads per wave and step
  for (int st = 0; st < RING; ++st) issue_step(st, st);
  ST_WAIT_VMCNT((RING - 1) * PER_STEP);
  __syncthreads();
  u32x4 ah, al, bv[NB];
  {
    u32x4 xv, gl;
    read_xg(0, xv, gl);
    read_b(0, bv);
    form_regs(xv, gl, ah, al);
  }
  constexpr int NMFMA = NB * (SPLIT ? 2 : 1);
  for (int kb = 0; kb < n; kb += RING) {
#pragma unroll
    for (int u = 0; u < RING; ++u) {
      const int kt = kb + u;
      if (kt >= n) break;
      ST_WAIT_VMCNT((RING - 2) * PER_STEP);
      __syncthreads();
      const int s1 = u + 1 < RING ? u + 1 : 0;
      u32x4 xv, gl, bn[NB];
      read_xg(s1, xv, gl);
      read_b(s1, bn);
      issue_step(kt + RING, u);
      // Split form: local step kt+1 starts the range's second strip.
      const bool seg_end = SK && kt + 1 == nb;
      if (SK) {
        ss0 = seg_end ? ss : ss0;
        ss = seg_end ? 0.f : ss;
      }
#pragma unroll
      for (int c = 0; c < NB; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ah),
                                                         __builtin_bit_cast(bf16x8, bv[c]), acc[c], 0, 0, 0);
      if (SPLIT) {
#pragma unroll
        for (int c = 0; c < NB; ++c)
          acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, al),
                                                           __builtin_bit_cast(bf16x8, bv[c]), acc[c], 0, 0, 0);
      }
      form_regs(xv, gl, ah, al);
#pragma unroll
      for (int c = 0; c < NB; ++c) bv[c] = bn[c];
      // Each MFMA followed by a share of the forming arithmetic.
#pragma unroll
      for (int q = 0; q < NMFMA; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, (48 + NMFMA - 1) / NMFMA, 0);
      }
      if (seg_end) {
#pragma unroll
        for (int c = 0; c < NB; ++c) {
          acc0[c] = acc[c];
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;
        }
      }
    }
  }
  ST_WAIT_VMCNT(0);

  // Tail, per segment (one, or two in the split form): the row sums of
  // squares and the waves' partial sums to LDS (the rings are free now),
  // k-quarters 0 and 1 as two sets [set][weight][row][col] fp32, then
  // k-quarters 2 and 3 added into them; thread -> row tid>>3, columns
  // 8 (tid&7) .. +7 then adds the two sets.
  float* red = (float*)&sm.w[0][0][0];
  const int orow = tid >> 3, oc = 8 * (tid & 7);
  auto stage_sets = [&](const floatx16 (&a)[NB], float ssv) {
    ssv += __shfl_xor(ssv, 32);  // the two k-chunks of the row in this wave
    __syncthreads();  // the rings (or the previous segment's sets) are no longer read
    if (l < 32) sm.ssp[kq][a_row] = ssv;
    // 32x32 layout: lane l holds column l%32 and, for register 4 jj + r,
    // row 8 jj + 4 (l/32) + r of the block.
    auto red_at = [&](int c, int jj, int r) -> float& {
      const int row = rb * 32 + 8 * jj + 4 * (l >> 5) + r, col = (c & 1) * 32 + (l & 31);
      return red[(((kq & 1) * NW + (c >> 1)) * ST_BM + row) * ST_BN + col];
    };
    if (kq < 2) {
#pragma unroll
      for (int c = 0; c < NB; ++c)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
          for (int r = 0; r < 4; ++r) red_at(c, jj, r) = a[c][4 * jj + r];
    }
    __syncthreads();
    if (kq >= 2) {
#pragma unroll
      for (int c = 0; c < NB; ++c)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
          for (int r = 0; r < 4; ++r) red_at(c, jj, r) += a[c][4 * jj + r];
    }
    if (tid < ST_BM) sm.ss[tid] = (sm.ssp[0][tid] + sm.ssp[1][tid]) + (sm.ssp[2][tid] + sm.ssp[3][tid]);
    __syncthreads();
  };
  auto sum_sets = [&](float (&z)[NW][8]) {
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      const floatx4* s0 = (const floatx4*)(red + ((0 * NW + v) * ST_BM + orow) * ST_BN + oc);
      const floatx4* s1 = (const floatx4*)(red + ((1 * NW + v) * ST_BM + orow) * ST_BN + oc);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const floatx4 u = s0[h], q = s1[h];
#pragma unroll
        for (int e = 0; e < 4; ++e) z[v][4 * h + e] = u[e] + q[e];
      }
    }
  };
  // Y = z / RMS (gated: silu(z1 / RMS) * z3 / RMS), 16 bytes per thread.
  auto store_y = [&](const float (&z)[NW][8], float ssr, int strip) {
    const int64_t n = (int64_t)strip * ST_BN + oc;
    if (orow < M && n < N) {
      const float inv = NORM ? inv_rms(ssr, K, eps) : 1.0f;
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

// The stream kernel's buffer offsets are 32-bit: each operand at most 2^30
// bytes, one W step (64 rows) at most 2^25 bytes.
bool rmm_stream_fits(int64_t M, int64_t N, int64_t K) {
  const int64_t lim = (int64_t)1 << 30;
  return M >= 0 && M <= 64 && K * N * 2 <= lim && M * K * 2 <= lim && 64 * N * 2 <= ((int64_t)1 << 25);
}

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
  if (!rmm_stream_fits(a.M, a.N, a.K)) return hipErrorInvalidValue;
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
  auto launch = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, block, 0, a.stream, x, g, w1, w3, y, a.eps, m, a.N, a.K, sp);
  };
  if (a.norm) {
    if (a.gated)
      p.split ? launch(stream_kernel<2, true, true>) : launch(stream_kernel<2, false, true>);
    else
      p.split ? launch(stream_kernel<1, true, true>) : launch(stream_kernel<1, false, true>);
  } else {
    if (a.gated)
      p.split ? launch(stream_kernel<2, true, false>) : launch(stream_kernel<2, false, false>);
    else
      p.split ? launch(stream_kernel<1, true, false>) : launch(stream_kernel<1, false, false>);
  }
  return hipGetLastError();
}
