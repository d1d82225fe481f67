// Prefill variant of fused RMSNorm+MatMul: many rows, matrix-core bound.
//
// An LDS-tiled bf16 MFMA GEMM whose k-loop also produces the two other
// pieces of the fused form (Mirage paper review, "核心公式": the abstract
// expression E(O) = sum(k, div(mul(I1,I2), I3)) with the k-independent I3
// taken outside the sum):
//   * while a tile of X is staged into LDS it is multiplied by g and rounded
//     once to bf16 -- the A operand is (X g), so g never touches W;
//   * the same registers give the row sums of squares of raw X, in fp32;
//   * after the k-loop the accumulators are scaled by 1/sqrt(ss/K + eps) and
//     stored: the normalised X is never written anywhere.
//
// Tiling: workgroup tile 256 (M) x 256 (N) x 64 (K), 8 waves in a 2x4 grid,
// each wave owning a 128x64 block = 4x2 v_mfma_f32_32x32x16_bf16 tiles (128
// fp32 accumulators per lane).  Two waves per SIMD let one wave's MFMAs run
// while the other waits on LDS, memory or the barrier.
//
// Operand paths:
//   * W (B operand) goes straight from memory into LDS (buffer loads with
//     the LDS-direct bit), one k-step ahead, as the raw K x N block with n
//     contiguous.  MFMA wants 8 consecutive k per lane; ds_read_b64_tr_b16
//     (gfx950's transposing LDS read) delivers exactly that: each 16-lane
//     group reads 4 rows x 16 columns and lane i receives column i.
//   * X (A operand) is loaded into registers two k-steps ahead, scaled by g
//     and written to LDS with 144-byte rows (128 + 16 padding), which makes
//     both the staging writes and the fragment reads bank-conflict-free.
// W tile layout: [64 k][256 n] bf16, 512-byte rows; 16-byte chunk c of row k
// sits at chunk c ^ 4(k & 3), so the 4 rows x 64 bytes that the two 16-lane
// groups of a half-wave read (columns 32 j .. +31 of rows k .. k+3) land on
// 16 different bank groups (with c ^ 2(k & 3) the two groups' reads fell on
// the same 8: two cycles of bank conflict per transposing read).
#include "rmm_device.h"

namespace rmm {

constexpr int PF_BM = 256, PF_BN = 256, PF_BK = 64, PF_THREADS = 512;
constexpr int PF_A_ROW = 144;                   // 64 bf16 + 16 bytes of padding
constexpr int PF_A_BYTES = PF_BM * PF_A_ROW;    // one A stage
constexpr int PF_B_BYTES = PF_BK * PF_BN * 2;   // one W stage, 32 KB
constexpr uint32_t kPfOutOfRange = 0x80000000u;

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2, v); }

// Byte offset of element n (a multiple of 4) of row k in a W stage.
__device__ __forceinline__ int pf_b_off(int k, int n) {
  return k * 512 + (((n >> 3) ^ (4 * (k & 3))) << 4) + ((n & 7) << 1);
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer resource (stride 0, 32-bit data format) for [base, base+bytes).
__device__ __forceinline__ i32x4 pf_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = 0x00020000;
  return r;
}

// X of one k-step for this thread: rows (t>>3) + 64 i, chunk t&7, and g.
struct PfA {
  u32x4 a[4];
  u32x4 g;
};

// 16 bytes per lane into registers.  Issued as inline asm, like the W
// transfers, so that the compiler does not place its own (too strict) wait
// for these registers: pf_wait_a below waits for exactly the loads that
// must have landed and is the only producer the compiler sees for them.
__device__ __forceinline__ u32x4 pf_load16(uint32_t voff, i32x4 rsrc) {
  u32x4 v;
  asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen" : "=v"(v) : "v"(voff), "s"(rsrc));
  return v;
}

// Columns at or past klim (K, or the end of this workgroup's K range) read
// as zeros.
template <bool GL>
__device__ __forceinline__ void pf_load_a(PfA& st, i32x4 xr, i32x4 gr, int64_t m0, int64_t k0,
                                          int64_t M, int64_t K, int64_t klim, int tid) {
  const int64_t ka = k0 + 8 * (tid & 7);
  const bool ka_ok = ka < klim;  // klim % 8 == 0: a chunk is all in or all out
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + (tid >> 3) + 64 * i;
    const uint32_t off = (ka_ok && m < M) ? (uint32_t)((m * K + ka) * 2) : kPfOutOfRange;
    st.a[i] = pf_load16(off, xr);
  }
  // With the gain held in LDS (GL) it is not loaded per step: every wave of
  // every workgroup reading the same 128 bytes of g at the same k-step
  // queues those requests on one L2 channel.
  if (!GL) st.g = pf_load16(ka_ok ? (uint32_t)(ka * 2) : kPfOutOfRange, gr);
}

// Wait until at most N vector-memory loads are outstanding; the registers
// of st are in/out operands, so no use of them moves above the wait.
// With the gain in LDS (GL) its register is not loaded and not tied here.
template <int N, bool GL>
__device__ __forceinline__ void pf_wait_a(PfA& st) {
  if (GL)
    asm volatile("s_waitcnt vmcnt(%4)"
                 : "+v"(st.a[0]), "+v"(st.a[1]), "+v"(st.a[2]), "+v"(st.a[3])
                 : "n"(N));
  else
    asm volatile("s_waitcnt vmcnt(%5)"
                 : "+v"(st.a[0]), "+v"(st.a[1]), "+v"(st.a[2]), "+v"(st.a[3]), "+v"(st.g)
                 : "n"(N));
}

// One 16-byte-per-lane load straight into LDS: lane l's data lands at
// lds_addr + 16 l.  Issued as inline asm so that the compiler does not
// serialise it against the other loads in flight; the k-loop waits for it
// explicitly (vmcnt) before the barrier that publishes the stage.
__device__ __forceinline__ void pf_lds_load16(uint32_t lds_addr, uint32_t voff, i32x4 rsrc) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(rsrc)
               : "memory");
}

// W block of step k0 into an LDS stage: wave w fills the four 1-KB blocks
// 4w .. 4w+3 (two k-rows each); lane l of a block lands at byte 16 l of the
// block, so it fetches the logical chunk the swizzle maps there.  The
// resource spans rows k0 .. klim - 1, so rows at or past klim (K, or the
// end of this workgroup's K range) read as zeros; columns past N are given
// an out-of-range offset.
struct PfDma {
  uint32_t off[4];  // per-lane byte offsets from row k0 (step independent)
};

__device__ __forceinline__ void pf_dma_setup(PfDma& d, int64_t n0, int64_t N, int w, int l) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int blk = 4 * w + q;
    const int kl = 2 * blk + (l >> 5);
    const int c = (l & 31) ^ (4 * (kl & 3));
    const int64_t nn = n0 + 8 * c;
    d.off[q] = nn < N ? (uint32_t)((kl * N + nn) * 2) : kPfOutOfRange;
  }
}

__device__ __forceinline__ void pf_dma_b(uint32_t b_lds, const PfDma& d, const bf16_t* W,
                                         int64_t k0, int64_t N, int64_t klim, int w) {
  const int64_t rows = klim - k0 > 0 ? klim - k0 : 0;
  const i32x4 rsrc = pf_rsrc(W + k0 * N, (uint32_t)(rows * N * 2));
#pragma unroll
  for (int q = 0; q < 4; ++q) pf_lds_load16(b_lds + (4 * w + q) * 1024, d.off[q], rsrc);
}

// Rows i0, i0+1 of a register stage -> A stage (the first step; the k-loop
// interleaves the same arithmetic with its MFMAs): X*g, each product formed
// exactly in fp32 (bf16 -> fp32 is a shift, and a product of two bf16 is
// exact in fp32), then rounded once to bf16; fp32 FMAs accumulate the row
// sums of squares of raw X.
template <bool GL>
__device__ __forceinline__ void pf_store_a(const PfA& st, char* a_lds, float (&ss)[4], int tid,
                                           int i0, int norm, const char* g_lds, int64_t k0) {
  const u32x4 gsrc = GL ? *(const u32x4*)(g_lds + 2 * (k0 + 8 * (tid & 7))) : st.g;
#pragma unroll
  for (int i = i0; i < i0 + 2; ++i) {
    u32x4 v;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t gd = (GL || norm) ? gsrc[d] : kBf16OnePair;
      const float x0 = __uint_as_float(st.a[i][d] << 16), x1 = __uint_as_float(st.a[i][d] & 0xffff0000u);
      v[d] = pack_bf16x2(x0 * __uint_as_float(gd << 16), x1 * __uint_as_float(gd & 0xffff0000u));
      ss[i] = __builtin_fmaf(x1, x1, __builtin_fmaf(x0, x0, ss[i]));
    }
    *(u32x4*)(a_lds + ((tid >> 3) + 64 * i) * PF_A_ROW + 16 * (tid & 7)) = v;
  }
}

// MFMA operand fragments of one 16-deep sub-step of the 128x64 wave tile.
struct PfFrag {
  bf16x8 a[4], b[2];
};

// a_base: this lane's A row (wm*128 + lane%32) and chunk (lane/32) in a stage;
// b_off0/1: this lane's transpose-read addresses for B fragments j = 0, 1.
__device__ __forceinline__ void pf_read_frags(PfFrag& f, const char* a_lds, const lds_char* b_lds,
                                              int a_base, int b_off0, int b_off1, int s) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    f.a[i] = *(const bf16x8*)(a_lds + a_base + 32 * i * PF_A_ROW + 32 * s);
  const int bo[2] = {b_off0, b_off1};
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const u32x2 lo = __builtin_bit_cast(
        u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(b_lds + bo[j] + 16 * s * 512)));
    const u32x2 hi = __builtin_bit_cast(
        u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(b_lds + bo[j] + (16 * s + 4) * 512)));
    const u32x4 v = {lo[0], lo[1], hi[0], hi[1]};
    f.b[j] = __builtin_bit_cast(bf16x8, v);
  }
}

__device__ __forceinline__ void pf_mfma(const PfFrag& f, floatx16 (&acc)[4][2]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
}

// s_waitcnt with only the vector-memory counter limited (gfx9 encoding:
// vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14).
#define PF_WAIT_VMCNT(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14))

// One k-step as 32 issue slots, one per MFMA: the wave issues in order, so
// every MFMA is followed by a small share of the step's other work, which
// then issues while the matrix pipe works (both waves of a SIMD reach the
// step together after the barrier, so batching the other work would leave
// the pipe idle).  Sub-step s (16 k) is 8 MFMAs over the 128 x 64 wave
// tile, operands from fragment set s & 1:
//   s = 0: + the fragment reads of sub-step 1, and `issue` (the W transfer
//          and the X loads of later steps);
//   s = 1, 2: + the fragment reads of sub-step s + 1, and the scaling of X
//          of the next step into a_nxt (16 units of one 16-byte chunk each,
//          a row written once its 4 chunks are formed);
//   s = 3: + the last scaling units.
// sched_barrier(0) between slots keeps this order.
template <int VM, bool GL, typename Issue>
__device__ __forceinline__ void pf_step(const char* a_cur, const lds_char* b_cur, char* a_nxt,
                                        PfA& st, floatx16 (&acc)[4][2], float (&ss)[4],
                                        int a_base, int b0, int b1, int tid, int norm,
                                        const char* g_lds, int64_t k_nxt, Issue issue) {
  // Fragment sets, B fragments as the two halves of the transposing reads.
  bf16x8 fa[2][4];
  u32x2 fb[2][2][2];
  const int bo[2] = {b0, b1};
  // Read q (0..7) of sub-step s into set s & 1, in the order the MFMAs use them.
  auto read_q = [&](int s, int q) {
    const int f = s & 1;
    // a0, b0lo, b0hi, a1, b1lo, b1hi, a2, a3
    if (q == 0 || q == 3 || q >= 6) {
      const int i = q == 0 ? 0 : (q == 3 ? 1 : q - 4);
      fa[f][i] = *(const bf16x8*)(a_cur + a_base + 32 * i * PF_A_ROW + 32 * s);
    } else {
      const int j = q < 3 ? 0 : 1, h = (q == 2 || q == 5);
      fb[f][j][h] = __builtin_bit_cast(
          u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                     (lds_i16x4*)(b_cur + bo[j] + (16 * s + 4 * h) * 512)));
    }
  };
  auto mfma_q = [&](int s, int q) {
    const int f = s & 1, i = q >> 1, j = q & 1;
    const u32x4 bv = {fb[f][j][0][0], fb[f][j][0][1], fb[f][j][1][0], fb[f][j][1][1]};
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[f][i], __builtin_bit_cast(bf16x8, bv),
                                                        acc[i][j], 0, 0, 0);
  };
  // Scaling: the gain of this thread's k-chunk as fp32 (bf16 -> fp32 is a
  // shift), once per step; unit u = 4 i + d forms chunk d of row i with
  // plain fp32 multiplies (a product of two bf16 is exact in fp32) and adds
  // the squares of X to the row's sum with fp32 FMAs.  No dot-product
  // instructions here: on gfx950 they occupy the matrix pipe and would not
  // overlap with the MFMAs.
  float g_f[8];
  u32x4 row_v, gsrc;
  auto gain = [&] {
    if (!GL) gsrc = st.g;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t gd = (GL || norm) ? gsrc[d] : kBf16OnePair;
      g_f[2 * d] = __uint_as_float(gd << 16);
      g_f[2 * d + 1] = __uint_as_float(gd & 0xffff0000u);
    }
  };
  auto unit = [&](int u) {
    const int i = u >> 2, d = u & 3;
    const float x0 = __uint_as_float(st.a[i][d] << 16), x1 = __uint_as_float(st.a[i][d] & 0xffff0000u);
    row_v[d] = pack_bf16x2(x0 * g_f[2 * d], x1 * g_f[2 * d + 1]);
    ss[i] = __builtin_fmaf(x1, x1, __builtin_fmaf(x0, x0, ss[i]));
    if (d == 3) *(u32x4*)(a_nxt + ((tid >> 3) + 64 * i) * PF_A_ROW + 16 * (tid & 7)) = row_v;
  };
#define PF_SLOT_END __builtin_amdgcn_sched_barrier(0)
  // Sub-step 0's fragments, then the transfers of later steps.
#pragma unroll
  for (int q = 0; q < 8; ++q) read_q(0, q);
  if (GL) gsrc = *(const u32x4*)(g_lds + 2 * (k_nxt + 8 * (tid & 7)));
  issue();
  PF_SLOT_END;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    mfma_q(0, q);
    read_q(1, q);
    PF_SLOT_END;
  }
  pf_wait_a<VM, GL>(st);
  gain();
  PF_SLOT_END;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    mfma_q(1, q);
    read_q(2, q);
    if (q < 6) unit(q);
    PF_SLOT_END;
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    mfma_q(2, q);
    read_q(3, q);
    if (q < 6) unit(6 + q);
    PF_SLOT_END;
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    mfma_q(3, q);
    if (q < 4) unit(12 + q);
    PF_SLOT_END;
  }
#undef PF_SLOT_END
}

// Largest K whose gain vector is held in LDS for the whole call (20 KB, the
// room left beside the A and W stages); the k-steps past K (up to one more
// step) read zeros from the padding.  Without the norm the LDS copy holds
// ones, so the k-loop forms X g with no select on the norm flag.
constexpr int PF_G_LDS_MAX = 10240;

template <bool GATED, bool GL>
__global__ __launch_bounds__(PF_THREADS, 2) void prefill_kernel(
    const bf16_t* __restrict__ X, const bf16_t* __restrict__ g, const bf16_t* __restrict__ W1,
    const bf16_t* __restrict__ W3, bf16_t* __restrict__ Y, float eps, int64_t M, int64_t N,
    int64_t K, int tiles_m, int tiles_n, int group_m, int xcd_remap, int norm, int splits,
    int ksteps, float* __restrict__ part) {
  static_assert(!GATED, "the gated tile is prefill_gated_kernel");
  // Loads per thread per k-step outside the W transfers: 4 rows of X, and
  // the gain unless it sits in LDS.
  constexpr int XL = GL ? 4 : 5;
  // Separate objects per stage, so the compiler can tell the W stage being
  // filled by direct loads from the one being read.
  __shared__ __attribute__((aligned(16))) char a_s0[PF_A_BYTES];
  __shared__ __attribute__((aligned(16))) char a_s1[PF_A_BYTES];
  __shared__ __attribute__((aligned(1024))) char b_s0[PF_B_BYTES];
  __shared__ __attribute__((aligned(1024))) char b_s1[PF_B_BYTES];
  __shared__ float inv_s[PF_BM];
  __shared__ __attribute__((aligned(16))) char g_s[GL ? 2 * (PF_G_LDS_MAX + 2 * PF_BK) : 16];

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  // Tile order: with xcd_remap, XCD x (workgroups bid % 8 == x) takes a
  // contiguous range of the sequence of (K range, tile) pairs, K range
  // major; the tiles of one K range are walked in groups of group_m
  // tile-rows, column by column, so concurrently resident workgroups of one
  // XCD share A and B tiles in its L2.
  const int ntiles = tiles_m * tiles_n;
  int t = blockIdx.x;
  if (xcd_remap) t = (t & 7) * ((ntiles * splits) >> 3) + (t >> 3);
  const int split = t / ntiles;
  t -= split * ntiles;
  const int group = group_m * tiles_n;
  const int gid = t / group, first_m = gid * group_m;
  const int gm = (tiles_m - first_m < group_m) ? (tiles_m - first_m) : group_m;
  const int tm = first_m + (t % group) % gm;
  const int tn = (t % group) / gm;
  const int64_t m0 = (int64_t)tm * PF_BM, n0 = (int64_t)tn * PF_BN;

  const i32x4 xr = pf_rsrc(X, (uint32_t)(M * K * 2));
  const i32x4 gr = pf_rsrc(g, (uint32_t)(K * 2));
  lds_char* b0s = (lds_char*)b_s0;
  lds_char* b1s = (lds_char*)b_s1;
  const uint32_t b0a = (uint32_t)(uintptr_t)b0s, b1a = (uint32_t)(uintptr_t)b1s;
  PfDma dma;
  pf_dma_setup(dma, n0, N, w, l);

  floatx16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  float ss[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) ss[i] = 0.f;

  const int wm = w >> 2, wn = w & 3;
  const int a_base = (wm * 128 + (l & 31)) * PF_A_ROW + 16 * (l >> 5);
  const int bG = l >> 4, bi = l & 15;
  const int bk = 8 * (bG >> 1) + (bi >> 2);
  const int bn = wn * 64 + 16 * (bG & 1) + 4 * (bi & 3);
  const int bo0 = pf_b_off(bk, bn), bo1 = pf_b_off(bk, bn + 32);
  // This workgroup's k-steps kt0 .. kt1 - 1 (all of K without a split; a
  // split's ksteps is even, so only the last range can end on an odd step);
  // every load at or past klim reads zeros.
  const int nk = (int)((K + PF_BK - 1) / PF_BK);
  const int kt0 = split * ksteps;
  const int kt1 = kt0 + ksteps < nk ? kt0 + ksteps : nk;
  const int64_t klim = (int64_t)kt1 * PF_BK < K ? (int64_t)kt1 * PF_BK : K;

  // Pipeline, with LDS stage kt&1 holding step kt at the top of iteration kt:
  // W of step kt+1 streams into the other W stage, X of step kt+1 (in
  // registers since the previous iteration) is scaled into the other A
  // stage, X of step kt+2 is in flight, and step kt is multiplied.  Loads
  // past the last step read zeros (buffer range check), so the loop body has
  // no branches; it is unrolled by two so each register stage is static.
  // The XL X (and g) loads of a step are issued after its W transfers, so
  // vmcnt <= XL means those transfers have landed; before X of the next step
  // is scaled, vmcnt <= XL + 4 (this iteration's 4 W and XL X loads may
  // still be in flight) means it has.  Both waits are explicit: the compiler
  // sees none of these loads.
  if (GL) {  // the whole gain vector, zero past K
    for (int c = tid; c < (PF_G_LDS_MAX + 2 * PF_BK) / 8; c += PF_THREADS)
      *(u32x4*)(g_s + 16 * c) = 8 * c >= K ? u32x4{0u, 0u, 0u, 0u}
                                : norm     ? *(const u32x4*)(g + 8 * c)
                                           : u32x4{kBf16OnePair, kBf16OnePair, kBf16OnePair, kBf16OnePair};
    __syncthreads();
  }

  const int64_t kb0 = (int64_t)kt0 * PF_BK;
  PfA sa, sb;
  pf_dma_b(b0a, dma, W1, kb0, N, klim, w);
  pf_load_a<GL>(sa, xr, gr, m0, kb0, M, K, klim, tid);
  pf_load_a<GL>(sb, xr, gr, m0, kb0 + PF_BK, M, K, klim, tid);
  pf_wait_a<XL, GL>(sa);
  pf_store_a<GL>(sa, a_s0, ss, tid, 0, norm, g_s, kb0);
  pf_store_a<GL>(sa, a_s0, ss, tid, 2, norm, g_s, kb0);
  PF_WAIT_VMCNT(0);
  __syncthreads();

  // Whole pairs of steps: with an odd step count the last one multiplies
  // zeros (every operand past klim reads as zero), which leaves the sums as
  // they are and keeps the accumulators in one place.
  for (int kt = kt0; kt < kt1; kt += 2) {
    pf_step<XL + 4, GL>(a_s0, b0s, a_s1, sb, acc, ss, a_base, bo0, bo1, tid, norm, g_s,
                        (int64_t)(kt + 1) * PF_BK, [&] {
                          pf_dma_b(b1a, dma, W1, (int64_t)(kt + 1) * PF_BK, N, klim, w);
                          pf_load_a<GL>(sa, xr, gr, m0, (int64_t)(kt + 2) * PF_BK, M, K, klim,
                                        tid);
                        });
    PF_WAIT_VMCNT(XL);
    __syncthreads();
    pf_step<XL + 4, GL>(a_s1, b1s, a_s0, sa, acc, ss, a_base, bo0, bo1, tid, norm, g_s,
                        (int64_t)(kt + 2) * PF_BK, [&] {
                          pf_dma_b(b0a, dma, W1, (int64_t)(kt + 2) * PF_BK, N, klim, w);
                          pf_load_a<GL>(sb, xr, gr, m0, (int64_t)(kt + 3) * PF_BK, M, K, klim,
                                        tid);
                        });
    PF_WAIT_VMCNT(XL);
    __syncthreads();
  }
  // The last iteration's X loads (past K: zeros) are still in flight and
  // their registers are dead to the compiler; the tied waits keep those
  // registers reserved until the loads have landed, so nothing after the
  // loop can be placed in them and then overwritten.
  pf_wait_a<0, GL>(sa);
  pf_wait_a<0, GL>(sb);
  PF_WAIT_VMCNT(0);

  // Row sums of squares: the 8 lanes tid&7 = 0..7 share rows (tid>>3) + 64 i.
  if (splits > 1) {
    // A K range of a split call: the raw sums go to the workspace, [split]
    // [M][N] fp32, then the row sums of squares, [split][M] (written by the
    // first tile-column; every tile-column computes the same values); the
    // combine kernel adds the ranges in order and applies 1/RMS.
    float* ssp = part + (int64_t)splits * M * N;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = ss[i];
      v += __shfl_xor(v, 1);
      v += __shfl_xor(v, 2);
      v += __shfl_xor(v, 4);
      const int64_t m = m0 + (tid >> 3) + 64 * i;
      if (tn == 0 && (tid & 7) == 0 && m < M) ssp[(int64_t)split * M + m] = v;
    }
    float* pp = part + (int64_t)split * M * N;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t n = n0 + wn * 64 + 32 * j + (l & 31);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int64_t m = m0 + wm * 128 + 32 * i + 8 * jj + 4 * (l >> 5) + r;
            if (m < M && n < N) pp[m * N + n] = acc[i][j][4 * jj + r];
          }
      }
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float v = ss[i];
    v += __shfl_xor(v, 1);
    v += __shfl_xor(v, 2);
    v += __shfl_xor(v, 4);
    if ((tid & 7) == 0) inv_s[(tid >> 3) + 64 * i] = norm ? inv_rms(v, K, eps) : 1.0f;
  }
  __syncthreads();

  // Epilogue.  32x32 accumulator layout: lane l holds column l%32 and, for
  // register 4 jj + r, row 8 jj + 4 (l/32) + r.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t n = n0 + wn * 64 + 32 * j + (l & 31);
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

// ---------------------------------------------------------------------------
// Gated tile: Y = silu(norm(X) W1) * (norm(X) W3) for many rows (the gated
// MLP row of the Mirage paper review's benchmark table, "五、实验结果").
//
// The gate multiplies one product's error by the other product, so, as in
// the decode and stream kernels, the operand X*g is carried exactly as two
// bf16 parts (hi = bf16(X g), lo = bf16(X g - hi)), both multiplied into the
// same accumulator.  Tile 128 rows x 128 columns of each weight x 64 k:
//   * A: two stages (hi, lo), double-buffered, 144-byte rows as above;
//   * W: one stage holds the 64 x 128 blocks of W1 and W3 ([weight][k][n],
//     256-byte rows, chunk c of row k at c ^ 4(k & 3)); each 1 KB
//     LDS-direct transfer reads 4 rows of one weight;
//   * wave w: rows 64 (w >> 2) .. +63, weight (w >> 1) & 1, columns
//     64 (w & 1) .. +63 of that weight: 2 x 2 v_mfma_f32_32x32x16_bf16
//     tiles, hi and lo MFMAs per sub-step (32 per k-step, as in the plain
//     tile);
//   * epilogue: the W3 waves hand their sums to the W1 waves through LDS,
//     which apply 1/RMS and the gate and store Y.
constexpr int PG_BM = 128, PG_BNW = 128;              // rows, columns per weight
constexpr int PG_A_BYTES = PG_BM * PF_A_ROW;          // one A stage (hi or lo)
constexpr int PG_B_BYTES = 2 * PF_BK * PG_BNW * 2;    // one W stage, 32 KB
constexpr int PG_W_BYTES = PF_BK * PG_BNW * 2;        // one weight's block, 16 KB

// Byte offset of element n (a multiple of 4) of row k in one weight's block.
__device__ __forceinline__ int pg_b_off(int k, int n) {
  return k * 256 + (((n >> 3) ^ (4 * (k & 3))) << 4) + ((n & 7) << 1);
}

// X of one k-step for this thread: rows (t>>3) and (t>>3) + 64, chunk t&7.
struct PgA {
  u32x4 a[2];
  u32x4 g;
};

// Columns at or past klim (K, or the end of this workgroup's K range) read
// as zeros.
template <bool GL>
__device__ __forceinline__ void pg_load_a(PgA& st, i32x4 xr, i32x4 gr, int64_t m0, int64_t k0,
                                          int64_t M, int64_t K, int64_t klim, int tid) {
  const int64_t ka = k0 + 8 * (tid & 7);
  const bool ka_ok = ka < klim;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int64_t m = m0 + (tid >> 3) + 64 * i;
    st.a[i] = pf_load16((ka_ok && m < M) ? (uint32_t)((m * K + ka) * 2) : kPfOutOfRange, xr);
  }
  if (!GL) st.g = pf_load16(ka_ok ? (uint32_t)(ka * 2) : kPfOutOfRange, gr);
}

template <int N, bool GL>
__device__ __forceinline__ void pg_wait_a(PgA& st) {
  if (GL)
    asm volatile("s_waitcnt vmcnt(%2)" : "+v"(st.a[0]), "+v"(st.a[1]) : "n"(N));
  else
    asm volatile("s_waitcnt vmcnt(%3)" : "+v"(st.a[0]), "+v"(st.a[1]), "+v"(st.g) : "n"(N));
}

// W of step k0 into a stage: wave w fills the 1-KB blocks 4w .. 4w+3 of
// weight w >> 2 (4 rows each); lane l lands at byte 16 l of its block.
struct PgDma {
  uint32_t off[4];
};

__device__ __forceinline__ void pg_dma_setup(PgDma& d, int64_t n0, int64_t N, int w, int l) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int blk = (4 * w + q) & 15;
    const int kl = 4 * blk + (l >> 4);
    const int c = (l & 15) ^ (4 * (kl & 3));
    const int64_t nn = n0 + 8 * c;
    d.off[q] = nn < N ? (uint32_t)((kl * N + nn) * 2) : kPfOutOfRange;
  }
}

__device__ __forceinline__ void pg_dma_b(uint32_t b_lds, const PgDma& d, const bf16_t* W1,
                                         const bf16_t* W3, int64_t k0, int64_t N, int64_t klim,
                                         int w) {
  const int64_t rows = klim - k0 > 0 ? klim - k0 : 0;
  const bf16_t* Wv = (w >> 2) ? W3 : W1;
  const i32x4 rsrc = pf_rsrc(Wv + k0 * N, (uint32_t)(rows * N * 2));
#pragma unroll
  for (int q = 0; q < 4; ++q) pf_lds_load16(b_lds + (4 * w + q) * 1024, d.off[q], rsrc);
}

// Rows of a register stage -> A stages (hi, lo): X*g formed exactly in fp32,
// split into two bf16 parts; fp32 FMAs accumulate the row sums of squares.
template <bool GL>
__device__ __forceinline__ void pg_form_unit(const PgA& st, const float (&g_f)[8], u32x4& hv, u32x4& lv,
                                             float (&ss)[2], int i, int d) {
  const float x0 = __uint_as_float(st.a[i][d] << 16), x1 = __uint_as_float(st.a[i][d] & 0xffff0000u);
  const u32x2 hl = split_bf16x2(x0 * g_f[2 * d], x1 * g_f[2 * d + 1]);
  hv[d] = hl[0];
  lv[d] = hl[1];
  ss[i] = __builtin_fmaf(x1, x1, __builtin_fmaf(x0, x0, ss[i]));
}

template <bool GL>
__device__ __forceinline__ void pg_gain(float (&g_f)[8], const u32x4& gsrc, int norm) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t gd = (GL || norm) ? gsrc[d] : kBf16OnePair;
    g_f[2 * d] = __uint_as_float(gd << 16);
    g_f[2 * d + 1] = __uint_as_float(gd & 0xffff0000u);
  }
}

// One k-step in 32 issue slots (as pf_step): sub-step s is 4 hi then 4 lo
// MFMAs over the 64 x 64 wave tile, fragments from set s & 1, each followed
// by a fragment read of sub-step s + 1 and, in sub-steps 1 and 2, a share
// of the forming of the next step's A stages.
template <int VM, bool GL, typename Issue, bool STAGE = true>
__device__ __forceinline__ void pg_step(const char* ah_cur, const char* al_cur, const lds_char* b_cur,
                                        char* ah_nxt, char* al_nxt, PgA& st, floatx16 (&acc)[2][2],
                                        float (&ss)[2], int a_base, int b0, int b1, int tid, int norm,
                                        const char* g_lds, int64_t k_nxt, Issue issue) {
  bf16x8 fh[2][2], fl[2][2];
  u32x2 fb[2][2][2];
  const int bo[2] = {b0, b1};
  // q: 0 hi0, 1 b0lo, 2 b0hi, 3 hi1, 4 b1lo, 5 b1hi, 6 lo0, 7 lo1
  auto read_q = [&](int s, int q) {
    const int f = s & 1;
    if (q == 0 || q == 3) {
      const int i = q == 0 ? 0 : 1;
      fh[f][i] = *(const bf16x8*)(ah_cur + a_base + 32 * i * PF_A_ROW + 32 * s);
    } else if (q >= 6) {
      const int i = q - 6;
      fl[f][i] = *(const bf16x8*)(al_cur + a_base + 32 * i * PF_A_ROW + 32 * s);
    } else {
      const int j = q < 3 ? 0 : 1, h = (q == 2 || q == 5);
      fb[f][j][h] = __builtin_bit_cast(
          u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(b_cur + bo[j] + (16 * s + 4 * h) * 256)));
    }
  };
  auto mfma_q = [&](int s, int q) {
    const int f = s & 1, i = (q & 3) >> 1, j = q & 1;
    const u32x4 bv = {fb[f][j][0][0], fb[f][j][0][1], fb[f][j][1][0], fb[f][j][1][1]};
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(q < 4 ? fh[f][i] : fl[f][i],
                                                        __builtin_bit_cast(bf16x8, bv), acc[i][j], 0, 0, 0);
  };
  float g_f[8];
  u32x4 hv, lv, gsrc;
  auto unit = [&](int u) {
    const int i = u >> 2, d = u & 3;
    pg_form_unit<GL>(st, g_f, hv, lv, ss, i, d);
    if (d == 3) {
      const int off = ((tid >> 3) + 64 * i) * PF_A_ROW + 16 * (tid & 7);
      *(u32x4*)(ah_nxt + off) = hv;
      *(u32x4*)(al_nxt + off) = lv;
    }
  };
#define PG_SLOT_END __builtin_amdgcn_sched_barrier(0)
#pragma unroll
  for (int q = 0; q < 8; ++q) read_q(0, q);
  if (STAGE && GL) gsrc = *(const u32x4*)(g_lds + 2 * (k_nxt + 8 * (tid & 7)));
  issue();
  PG_SLOT_END;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    mfma_q(0, q);
    read_q(1, q);
    PG_SLOT_END;
  }
  if (STAGE) {
    pg_wait_a<VM, GL>(st);
    if (!GL) gsrc = st.g;
    pg_gain<GL>(g_f, gsrc, norm);
  }
  PG_SLOT_END;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    mfma_q(1, q);
    read_q(2, q);
    if (STAGE && q < 4) unit(q);
    PG_SLOT_END;
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    mfma_q(2, q);
    read_q(3, q);
    if (STAGE && q < 4) unit(4 + q);
    PG_SLOT_END;
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    mfma_q(3, q);
    PG_SLOT_END;
  }
#undef PG_SLOT_END
}

// LORA: the same two-part tile for the plain product with the low-rank
// adapter (Y = Nrm W + (Nrm A^T) B, the LoRA row of the same benchmark
// table): the two weight slots are the two 128-column halves of a 256-column
// tile of W, and after the k-loop one more k-step multiplies T = (X g) A^T
// (fp32, from lora_down_kernel, split into two bf16 parts like X g) by the
// tile's columns of B (R <= 64 rows, zero past R), into the same
// accumulators, before 1/RMS: no rounding between the two products.
template <bool GL, bool LORA>
__global__ __launch_bounds__(PF_THREADS, 1) void prefill_gated_kernel(
    const bf16_t* __restrict__ X, const bf16_t* __restrict__ g, const bf16_t* __restrict__ W1,
    const bf16_t* __restrict__ W3, bf16_t* __restrict__ Y, float eps, int64_t M, int64_t N,
    int64_t K, int tiles_m, int tiles_n, int group_m, int xcd_remap, int norm,
    const float* __restrict__ T, int rp, const bf16_t* __restrict__ LB, int R, int splits,
    int ksteps, float* __restrict__ part) {
  constexpr int XL = GL ? 2 : 3;  // X (and g) loads per thread per k-step
  __shared__ __attribute__((aligned(16))) char ah_s0[PG_A_BYTES];
  __shared__ __attribute__((aligned(16))) char ah_s1[PG_A_BYTES];
  __shared__ __attribute__((aligned(16))) char al_s0[PG_A_BYTES];
  __shared__ __attribute__((aligned(16))) char al_s1[PG_A_BYTES];
  __shared__ __attribute__((aligned(1024))) char b_s0[PG_B_BYTES];
  __shared__ __attribute__((aligned(1024))) char b_s1[PG_B_BYTES];
  __shared__ float inv_s[PG_BM];
  __shared__ __attribute__((aligned(16))) char g_s[GL ? 2 * (PF_G_LDS_MAX + 2 * PF_BK) : 16];

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int ntiles = tiles_m * tiles_n;
  // (K range, tile) pairs, K range major, as in prefill_kernel.
  int t = blockIdx.x;
  if (xcd_remap) t = (t & 7) * ((ntiles * splits) >> 3) + (t >> 3);
  const int split = t / ntiles;
  t -= split * ntiles;
  const int group = group_m * tiles_n;
  const int gid = t / group, first_m = gid * group_m;
  const int gm = (tiles_m - first_m < group_m) ? (tiles_m - first_m) : group_m;
  const int tm = first_m + (t % group) % gm;
  const int tn = (t % group) / gm;
  // Gated: 128 columns of each weight; LORA: 256 columns of W, the upper
  // half in the second weight slot.
  const int64_t m0 = (int64_t)tm * PG_BM, n0 = (int64_t)tn * (LORA ? 2 * PG_BNW : PG_BNW);

  const i32x4 xr = pf_rsrc(X, (uint32_t)(M * K * 2));
  const i32x4 gr = pf_rsrc(g, (uint32_t)(K * 2));
  lds_char* b0s = (lds_char*)b_s0;
  lds_char* b1s = (lds_char*)b_s1;
  const uint32_t b0a = (uint32_t)(uintptr_t)b0s, b1a = (uint32_t)(uintptr_t)b1s;
  PgDma dma;
  pg_dma_setup(dma, n0 + (LORA && (w >> 2) ? PG_BNW : 0), N, w, l);

  floatx16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  float ss[2] = {0.f, 0.f};

  const int wm = w >> 2, wv = (w >> 1) & 1, wh = w & 1;
  const int a_base = (wm * 64 + (l & 31)) * PF_A_ROW + 16 * (l >> 5);
  const int bG = l >> 4, bi = l & 15;
  const int bk = 8 * (bG >> 1) + (bi >> 2);
  const int bn = wh * 64 + 16 * (bG & 1) + 4 * (bi & 3);
  const int bo0 = wv * PG_W_BYTES + pg_b_off(bk, bn), bo1 = wv * PG_W_BYTES + pg_b_off(bk, bn + 32);
  // This workgroup's k-steps kt0 .. kt1 - 1, as in prefill_kernel.
  const int nk = (int)((K + PF_BK - 1) / PF_BK);
  const int kt0 = split * ksteps;
  const int kt1 = kt0 + ksteps < nk ? kt0 + ksteps : nk;
  const int64_t klim = (int64_t)kt1 * PF_BK < K ? (int64_t)kt1 * PF_BK : K;
  const int64_t kb0 = (int64_t)kt0 * PF_BK;

  if (GL) {
    for (int c = tid; c < (PF_G_LDS_MAX + 2 * PF_BK) / 8; c += PF_THREADS)
      *(u32x4*)(g_s + 16 * c) = 8 * c >= K ? u32x4{0u, 0u, 0u, 0u}
                                : norm     ? *(const u32x4*)(g + 8 * c)
                                           : u32x4{kBf16OnePair, kBf16OnePair, kBf16OnePair, kBf16OnePair};
    __syncthreads();
  }

  // Pipeline as in prefill_kernel: stage kt&1 holds step kt at the top of
  // iteration kt, W of step kt+1 streams into the other stage, X of step
  // kt+1 is formed into the other A stages, X of step kt+2 is in flight.
  PgA sa, sb;
  pg_dma_b(b0a, dma, W1, W3, kb0, N, klim, w);
  pg_load_a<GL>(sa, xr, gr, m0, kb0, M, K, klim, tid);
  pg_load_a<GL>(sb, xr, gr, m0, kb0 + PF_BK, M, K, klim, tid);
  pg_wait_a<XL, GL>(sa);
  {
    float g_f[8];
    const u32x4 gsrc = GL ? *(const u32x4*)(g_s + 2 * kb0 + 16 * (tid & 7)) : sa.g;
    pg_gain<GL>(g_f, gsrc, norm);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      u32x4 hv, lv;
#pragma unroll
      for (int d = 0; d < 4; ++d) pg_form_unit<GL>(sa, g_f, hv, lv, ss, i, d);
      const int off = ((tid >> 3) + 64 * i) * PF_A_ROW + 16 * (tid & 7);
      *(u32x4*)(ah_s0 + off) = hv;
      *(u32x4*)(al_s0 + off) = lv;
    }
  }
  PF_WAIT_VMCNT(0);
  __syncthreads();

  for (int kt = kt0; kt < kt1; kt += 2) {
    pg_step<XL + 4, GL>(ah_s0, al_s0, b0s, ah_s1, al_s1, sb, acc, ss, a_base, bo0, bo1, tid, norm, g_s,
                        (int64_t)(kt + 1) * PF_BK, [&] {
                          pg_dma_b(b1a, dma, W1, W3, (int64_t)(kt + 1) * PF_BK, N, klim, w);
                          pg_load_a<GL>(sa, xr, gr, m0, (int64_t)(kt + 2) * PF_BK, M, K, klim, tid);
                        });
    PF_WAIT_VMCNT(XL);
    __syncthreads();
    pg_step<XL + 4, GL>(ah_s1, al_s1, b1s, ah_s0, al_s0, sa, acc, ss, a_base, bo0, bo1, tid, norm, g_s,
                        (int64_t)(kt + 2) * PF_BK, [&] {
                          pg_dma_b(b0a, dma, W1, W3, (int64_t)(kt + 2) * PF_BK, N, klim, w);
                          pg_load_a<GL>(sb, xr, gr, m0, (int64_t)(kt + 3) * PF_BK, M, K, klim, tid);
                        });
    PF_WAIT_VMCNT(XL);
    __syncthreads();
  }
  // The last X loads (past K: zeros) keep their registers reserved until
  // they have landed.
  pg_wait_a<0, GL>(sa);
  pg_wait_a<0, GL>(sb);
  PF_WAIT_VMCNT(0);

  // Row sums of squares: the 8 lanes tid&7 share rows (tid>>3) and +64.
  // A K range of a split call stores them raw ([split][M], from the first
  // tile-column) and applies no scale; the combine kernel does.
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    float v = ss[i];
    v += __shfl_xor(v, 1);
    v += __shfl_xor(v, 2);
    v += __shfl_xor(v, 4);
    const int row = (tid >> 3) + 64 * i;
    if (splits > 1) {
      float* ssp = part + (int64_t)splits * (LORA ? 1 : 2) * M * N;
      if (tn == 0 && (tid & 7) == 0 && m0 + row < M) ssp[(int64_t)split * M + m0 + row] = v;
      if ((tid & 7) == 0) inv_s[row] = 1.0f;
    } else if ((tid & 7) == 0) {
      inv_s[row] = norm ? inv_rms(v, K, eps) : 1.0f;
    }
  }
  __syncthreads();
  // A split call's gated tile stores both products' raw sums,
  // [split][weight][M][N]; the adapter's go on below (its last range adds
  // T B first).
  if (!LORA && splits > 1) {
    float* pp = part + ((int64_t)split * 2 + wv) * M * N;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t n = n0 + wh * 64 + 32 * j + (l & 31);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int64_t m = m0 + wm * 64 + 32 * i + 8 * jj + 4 * (l >> 5) + rr;
            if (m < M && n < N) pp[m * N + n] = acc[i][j][4 * jj + rr];
          }
      }
    return;
  }

  if (LORA) {
    // The adapter step (in a split call, by the last K range only): T rows
    // m0 .. m0 + 127 (rp columns, zero past R) as hi and lo A stages, B rows
    // 0 .. R - 1 of the tile's columns in a W stage (rows past R read as
    // zeros), then one k-step of MFMAs.
    if (split == splits - 1) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = (tid >> 3) + 64 * i, c = tid & 7;
      const int64_t m = m0 + row;
      u32x4 hv = {0u, 0u, 0u, 0u}, lv = {0u, 0u, 0u, 0u};
      if (m < M && 8 * c < rp) {
        const float4* tp = (const float4*)(T + m * rp + 8 * c);
        const float4 t0 = tp[0], t1 = tp[1];
        const float tv[8] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z, t1.w};
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const u32x2 hl = split_bf16x2(tv[2 * d], tv[2 * d + 1]);
          hv[d] = hl[0];
          lv[d] = hl[1];
        }
      }
      const int off = row * PF_A_ROW + 16 * c;
      *(u32x4*)(ah_s0 + off) = hv;
      *(u32x4*)(al_s0 + off) = lv;
    }
    pg_dma_b(b0a, dma, LB, LB, 0, N, R, w);
    PF_WAIT_VMCNT(0);
    __syncthreads();
    auto no_issue = [] {};
    pg_step<0, GL, decltype(no_issue), false>(ah_s0, al_s0, b0s, ah_s1, al_s1, sa, acc, ss, a_base,
                                              bo0, bo1, tid, norm, g_s, 0, no_issue);
    }
    // Y (or, in a split call, the range's raw sums [split][M][N]): each wave
    // stores its own 64 x 64 block.
    float* pp = splits > 1 ? part + (int64_t)split * M * N : nullptr;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t n = n0 + wv * PG_BNW + wh * 64 + 32 * j + (l & 31);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int lr = wm * 64 + 32 * i + 8 * jj + 4 * (l >> 5) + rr;
            const int64_t m = m0 + lr;
            if (m < M && n < N) {
              if (splits > 1)
                pp[m * N + n] = acc[i][j][4 * jj + rr];
              else
                Y[m * N + n] = f32_to_bf16(acc[i][j][4 * jj + rr] * inv_s[lr]);
            }
          }
      }
    return;
  }

  // Epilogue, one 64-row half at a time: the W3 waves of rows 64 r .. +63
  // put their sums in a W stage as [column half][row][col] fp32, the W1
  // waves of those rows read them back at the positions of their own sums.
  // 32x32 accumulator layout: lane l holds column l%32 and, for register
  // 4 jj + rr, row 8 jj + 4 (l/32) + rr.
  float* ex = (float*)b_s0;
  auto ex_at = [&](int i, int j, int jj, int rr) -> float& {
    const int row = 32 * i + 8 * jj + 4 * (l >> 5) + rr, col = 32 * j + (l & 31);
    return ex[(wh * 64 + row) * 64 + col];
  };
  for (int r = 0; r < 2; ++r) {
    if (wm == r && wv == 1) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) ex_at(i, j, jj, rr) = acc[i][j][4 * jj + rr];
    }
    __syncthreads();
    if (wm == r && wv == 0) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int64_t n = n0 + wh * 64 + 32 * j + (l & 31);
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
              const int lr = wm * 64 + 32 * i + 8 * jj + 4 * (l >> 5) + rr;
              const int64_t m = m0 + lr;
              const float inv = inv_s[lr];
              const float y = silu_gate(acc[i][j][4 * jj + rr] * inv, ex_at(i, j, jj, rr) * inv);
              if (m < M && n < N) Y[m * N + n] = f32_to_bf16(y);
            }
        }
    }
    __syncthreads();
  }
}

// Down-projection of the adapter for the prefill tile: T = (X g) A^T, M x R
// in fp32, row stride rp = 16 RB (columns R .. rp - 1 are zero).  As in the
// decode kernel's adapter, X g is formed exactly in fp32 and split into two
// bf16 parts, both multiplied into the sum, and A's R x K layout gives the
// k-contiguous B fragments of v_mfma_f32_16x16x32_bf16 directly: lane l
// holds row (rank) l % 16 and k chunk l / 16 of a 32-deep block for both
// operands.  A workgroup takes 16 rows; its 4 waves take every 4th 32-deep
// block of K and their sums are added in wave order.
constexpr int LD_THREADS = 256;

template <int RB>
__global__ __launch_bounds__(LD_THREADS) void lora_down_kernel(
    const bf16_t* __restrict__ X, const bf16_t* __restrict__ g, const bf16_t* __restrict__ A,
    float* __restrict__ T, int64_t M, int64_t K, int R, int norm) {
  __shared__ floatx4 red[4][RB][64];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int64_t m0 = (int64_t)blockIdx.x * 16;
  const int r16 = l & 15, kc = l >> 4;
  const int64_t m = m0 + r16;
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc((void*)X, 0, (int)(M * K * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t gr = __builtin_amdgcn_make_buffer_rsrc((void*)g, 0, (int)(K * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t ar = __builtin_amdgcn_make_buffer_rsrc((void*)A, 0, (int)(R * K * 2), 0x00020000);
  floatx4 acc[RB];
#pragma unroll
  for (int b = 0; b < RB; ++b) acc[b] = floatx4{0.f, 0.f, 0.f, 0.f};
  for (int64_t kb = 32 * w; kb < K; kb += 128) {
    const int64_t k = kb + 8 * kc;
    const bool kok = k < K;  // K % 8 == 0: a chunk is all in or all out
    const u32x4 xv = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                   xr,
                   (kok && m < M) ? (uint32_t)((m * K + k) * 2) : kPfOutOfRange, 0, 0));
    const u32x4 gv = norm ? __builtin_bit_cast(
                                u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                           gr,
                                           kok ? (uint32_t)(k * 2) : kPfOutOfRange, 0, 0))
                          : u32x4{kBf16OnePair, kBf16OnePair, kBf16OnePair, kBf16OnePair};
    u32x4 hi, lo;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const u32x2 hl = split_bf16x2(bf16_lo(xv[d]) * bf16_lo(gv[d]), bf16_hi(xv[d]) * bf16_hi(gv[d]));
      hi[d] = hl[0];
      lo[d] = hl[1];
    }
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      const int r = 16 * b + r16;
      const u32x4 av = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                     ar,
                     (kok && r < R) ? (uint32_t)(((int64_t)r * K + k) * 2) : kPfOutOfRange, 0, 0));
      acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, hi),
                                                       __builtin_bit_cast(bf16x8, av), acc[b], 0, 0, 0);
      acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, lo),
                                                       __builtin_bit_cast(bf16x8, av), acc[b], 0, 0, 0);
    }
  }
#pragma unroll
  for (int b = 0; b < RB; ++b) red[w][b][l] = acc[b];
  __syncthreads();
  // 16 x 16 accumulator layout: lane l holds column l % 16, rows 4 (l / 16) + i.
  if (w == 0) {
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      floatx4 v = red[0][b][l];
#pragma unroll
      for (int q = 1; q < 4; ++q) v += red[q][b][l];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t mm = m0 + 4 * (l >> 4) + i;
        if (mm < M) T[mm * (16 * RB) + 16 * b + (l & 15)] = v[i];
      }
    }
  }
}

// Second kernel of a split call (a split of K over workgroups, for shapes
// with too few output tiles to fill the chip): Y = (sum of the K ranges' raw
// sums) / RMS, the row's sum of squares likewise added over the ranges; both
// sums in range order, so the result does not depend on which workgroup
// finished first.  8 consecutive columns per thread (N % 8 == 0).
constexpr int PC_THREADS = 256;

__global__ __launch_bounds__(PC_THREADS) void prefill_combine_kernel(
    const float* __restrict__ part, bf16_t* __restrict__ Y, float eps, int64_t M, int64_t N,
    int64_t K, int splits, int norm) {
  const int64_t n8 = N >> 3;
  const int64_t idx = (int64_t)blockIdx.x * PC_THREADS + threadIdx.x;
  if (idx >= M * n8) return;
  const int64_t m = idx / n8, n = (idx - m * n8) * 8;
  const float* ssp = part + (int64_t)splits * M * N;
  float ss = 0.f, y[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) y[c] = 0.f;
  for (int s = 0; s < splits; ++s) {
    ss += ssp[(int64_t)s * M + m];
    const float4* p = (const float4*)(part + ((int64_t)s * M + m) * N + n);
    const float4 a = p[0], b = p[1];
    y[0] += a.x; y[1] += a.y; y[2] += a.z; y[3] += a.w;
    y[4] += b.x; y[5] += b.y; y[6] += b.z; y[7] += b.w;
  }
  const float inv = norm ? inv_rms(ss, K, eps) : 1.0f;
  u32x4 o;
#pragma unroll
  for (int d = 0; d < 4; ++d) o[d] = pack_bf16x2(y[2 * d] * inv, y[2 * d + 1] * inv);
  *(u32x4*)(Y + m * N + n) = o;
}

// The gated form: both products' ranges, [split][weight][M][N], then the
// gate on the scaled sums (1/RMS before the SiLU).
__global__ __launch_bounds__(PC_THREADS) void prefill_gated_combine_kernel(
    const float* __restrict__ part, bf16_t* __restrict__ Y, float eps, int64_t M, int64_t N,
    int64_t K, int splits, int norm) {
  const int64_t n8 = N >> 3;
  const int64_t idx = (int64_t)blockIdx.x * PC_THREADS + threadIdx.x;
  if (idx >= M * n8) return;
  const int64_t m = idx / n8, n = (idx - m * n8) * 8;
  const float* ssp = part + (int64_t)splits * 2 * M * N;
  float ss = 0.f, z[2][8];
#pragma unroll
  for (int v = 0; v < 2; ++v)
#pragma unroll
    for (int c = 0; c < 8; ++c) z[v][c] = 0.f;
  for (int s = 0; s < splits; ++s) {
    ss += ssp[(int64_t)s * M + m];
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const float4* p = (const float4*)(part + (((int64_t)s * 2 + v) * M + m) * N + n);
      const float4 a = p[0], b = p[1];
      z[v][0] += a.x; z[v][1] += a.y; z[v][2] += a.z; z[v][3] += a.w;
      z[v][4] += b.x; z[v][5] += b.y; z[v][6] += b.z; z[v][7] += b.w;
    }
  }
  const float inv = norm ? inv_rms(ss, K, eps) : 1.0f;
  u32x4 o;
#pragma unroll
  for (int d = 0; d < 4; ++d)
    o[d] = pack_bf16x2(silu_gate(z[0][2 * d] * inv, z[1][2 * d] * inv),
                       silu_gate(z[0][2 * d + 1] * inv, z[1][2 * d + 1] * inv));
  *(u32x4*)(Y + m * N + n) = o;
}

}  // namespace rmm

// Split of K for the plain tile.  Without a forced count, with a workspace
// and at most 128 output tiles (half the CUs), the count minimises a model
// fitted to timings on this part (M = 129 .. 2048, N = 4096 and 14336,
// K = 4096 and 14336): about 1.5 us per 64-deep k-step of a range, plus
// about 0.4 us per MB of fp32 partial sums (written once, read back by the
// combine kernel), with at most one workgroup per CU; ranges are whole,
// even numbers of steps.  The partial sums must fit in ws_avail.
namespace {
struct SplitShape {
  int64_t splits, ksteps;
};
SplitShape prefill_split_shape(int64_t nk, int64_t s) {
  int64_t q = (nk + s - 1) / s;
  q += q & 1;
  return {(nk + q - 1) / q, q};
}
// [split][product][M][N] sums, then [split][M] sums of squares
size_t prefill_part_bytes(int64_t M, int64_t N, int64_t S, int64_t nsum) {
  return (size_t)(S * (nsum * M * N + M)) * 4;
}
}  // namespace

void rmm_prefill_plan(int64_t M, int64_t N, int64_t K, int gated, int splits, size_t ws_avail,
                      PrefillPlan* p, int64_t R) {
  using namespace rmm;
  // Tiles: plain 256 x 256; gated 128 rows x 128 columns of each weight;
  // with the adapter 128 x 256 (the two-part tile over two column halves).
  const bool two = gated || R > 0;
  const int bm = two ? PG_BM : PF_BM, bn = (gated ? PG_BNW : PF_BN);
  p->tiles_m = (int)((M + bm - 1) / bm);
  p->tiles_n = (int)((N + bn - 1) / bn);
  p->group_m = 4;
  const int64_t nk = (K + PF_BK - 1) / PF_BK;
  const int64_t tiles = (int64_t)p->tiles_m * p->tiles_n;
  p->splits = 1;
  p->ksteps = (int)nk;
  p->rb = R > 0 ? (int)((R + 15) / 16) : 0;
  // Workspace: the counter region, the adapter's T (M x 16 rb fp32), then
  // the partial sums of a split call.
  p->ws_t_off = kWsCounterBytes;
  const size_t t_bytes = R > 0 ? (size_t)(M * 16 * p->rb) * 4 : 0;
  p->ws_part_off = kWsCounterBytes + ((t_bytes + 255) & ~(size_t)255);
  const size_t fixed = R > 0 ? p->ws_part_off : 0;
  const int64_t nsum = gated ? 2 : 1;  // products summed per output
  p->ws_bytes = fixed;
  SplitShape best{1, nk};
  if (splits > 1) {
    best = prefill_split_shape(nk, splits);
  } else if (splits == 0 && ws_avail > fixed && 2 * tiles <= 256 && nk >= 4) {
    double best_us = 1.5 * nk;
    for (int64_t s = 2; s * tiles <= 256 && s <= nk / 2; ++s) {
      const SplitShape c = prefill_split_shape(nk, s);
      if (p->ws_part_off + prefill_part_bytes(M, N, c.splits, nsum) > ws_avail) break;
      const double us = 1.5 * c.ksteps + 0.4e-6 * (double)(c.splits * nsum * M * N * 4);
      if (us < best_us) {
        best_us = us;
        best = c;
      }
    }
  }
  if (best.splits > 1) {
    p->splits = (int)best.splits;
    p->ksteps = (int)best.ksteps;
    p->ws_bytes = p->ws_part_off + prefill_part_bytes(M, N, best.splits, nsum);
  }
  p->xcd_remap = (tiles * p->splits) % 8 == 0;
}

hipError_t rmm_launch_prefill(const RmmArgs& a, const PrefillPlan& p, void* ws) {
  using namespace rmm;
  const unsigned grid = (unsigned)((int64_t)p.tiles_m * p.tiles_n * p.splits);
  float* part = p.splits > 1 ? (float*)((char*)ws + p.ws_part_off) : nullptr;
  if (p.splits > 1 && !ws) return hipErrorInvalidValue;
  auto launch = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(PF_THREADS), 0, a.stream, (const bf16_t*)a.X,
                       (const bf16_t*)a.g, (const bf16_t*)a.W1, (const bf16_t*)a.W3, (bf16_t*)a.Y, a.eps,
                       a.M, a.N, a.K, p.tiles_m, p.tiles_n, p.group_m, p.xcd_remap, a.norm,
                       (const float*)nullptr, 0, (const bf16_t*)nullptr, 0, p.splits, p.ksteps, part);
  };
  auto launch_plain = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(PF_THREADS), 0, a.stream, (const bf16_t*)a.X,
                       (const bf16_t*)a.g, (const bf16_t*)a.W1, (const bf16_t*)a.W3, (bf16_t*)a.Y, a.eps,
                       a.M, a.N, a.K, p.tiles_m, p.tiles_n, p.group_m, p.xcd_remap, a.norm,
                       p.splits, p.ksteps, part);
  };
  const bool gl = a.K <= PF_G_LDS_MAX;
  if (a.R > 0) {
    if (!ws || p.rb < 1 || p.rb > 4) return hipErrorInvalidValue;
    float* T = (float*)((char*)ws + p.ws_t_off);
    const dim3 dgrid((unsigned)((a.M + 15) / 16)), dblock(LD_THREADS);
    auto down = [&](auto kernel) {
      hipLaunchKernelGGL(kernel, dgrid, dblock, 0, a.stream, (const bf16_t*)a.X, (const bf16_t*)a.g,
                         (const bf16_t*)a.LA, T, a.M, a.K, (int)a.R, a.norm);
    };
    if (p.rb == 1) down(lora_down_kernel<1>);
    else if (p.rb == 2) down(lora_down_kernel<2>);
    else if (p.rb == 3) down(lora_down_kernel<3>);
    else down(lora_down_kernel<4>);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    auto tile = [&](auto kernel) {
      hipLaunchKernelGGL(kernel, dim3(grid), dim3(PF_THREADS), 0, a.stream, (const bf16_t*)a.X,
                         (const bf16_t*)a.g, (const bf16_t*)a.W1, (const bf16_t*)a.W1, (bf16_t*)a.Y,
                         a.eps, a.M, a.N, a.K, p.tiles_m, p.tiles_n, p.group_m, p.xcd_remap, a.norm,
                         (const float*)T, 16 * p.rb, (const bf16_t*)a.LB, (int)a.R, p.splits,
                         p.ksteps, part);
    };
    gl ? tile(prefill_gated_kernel<true, true>) : tile(prefill_gated_kernel<false, true>);
  } else if (a.gated) {
    gl ? launch(prefill_gated_kernel<true, false>) : launch(prefill_gated_kernel<false, false>);
  } else {
    gl ? launch_plain(prefill_kernel<false, true>) : launch_plain(prefill_kernel<false, false>);
  }
  if (p.splits > 1) {
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int64_t threads = a.M * (a.N >> 3);
    const dim3 cgrid((unsigned)((threads + PC_THREADS - 1) / PC_THREADS));
    if (a.gated && a.R == 0)
      hipLaunchKernelGGL(prefill_gated_combine_kernel, cgrid, dim3(PC_THREADS), 0, a.stream,
                         (const float*)part, (bf16_t*)a.Y, a.eps, a.M, a.N, a.K, p.splits, a.norm);
    else
      hipLaunchKernelGGL(prefill_combine_kernel, cgrid, dim3(PC_THREADS), 0, a.stream,
                         (const float*)part, (bf16_t*)a.Y, a.eps, a.M, a.N, a.K, p.splits, a.norm);
  }
  return hipGetLastError();
}
