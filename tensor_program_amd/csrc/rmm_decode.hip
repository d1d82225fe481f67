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
// Work decomposition (one workgroup = WV waves of 64 lanes):
//   * a workgroup owns a 128-column tile of Y and a chunk of K;
//   * first it stages A = bf16(X g) for (a segment of) its chunk in LDS,
//     laid out [k/8][row] in 16-byte units, and accumulates the row sums of
//     squares while doing so; these loads are issued before any W load, so
//     the W stream starts at once behind them;
//   * the waves take interleaved 32-deep k-blocks; per k-block, lane
//     (q = lane/16, p = lane%16) holds rows kb+8q .. kb+8q+7 of W at columns
//     8p .. 8p+7 of the tile (eight 16-byte loads, each load instruction
//     reading four 256-byte row segments), transposes the 8x8 block in
//     registers with byte permutes, and feeds column c as the B operand of
//     v_mfma_f32_16x16x32_bf16 number c; the A operand is one 16-byte LDS
//     read.  W is double-buffered in registers: the loads of the next k-block
//     are in flight while one is multiplied.  Loads past the chunk are issued
//     anyway (their range check returns zeros without a memory access), so
//     the compiler's wait counters track a fixed pattern;
//   * the waves' accumulators are summed through LDS; with several K chunks
//     the workgroup stores its fp32 partial to the workspace, and the last
//     workgroup to arrive at a tile (arrival counter) adds the partials and
//     runs the epilogue  Y = acc / RMS  (gated: silu(acc1/RMS) * acc3/RMS).
//   * the partials cross XCDs (each XCD has its own L2), so they are written
//     and read with device-scope coherent accesses, ordered by waiting for the
//     stores' acknowledgements before the arrival count.
//   * the block index is remapped so that all chunks of a tile are dispatched
//     to the same XCD (workgroups go round-robin over the 8 XCDs); this only
//     affects locality, never correctness.
#include "rmm_decode_core.h"

namespace rmm {

constexpr int DEC_STAGE_BYTES = 32768;    // LDS for the staged A operand

// The gated and adapter calls carry the operand X*g exactly as two bf16
// parts (split_bf16x2): the gate multiplies one product's error by the other
// product, and the adapter's two terms can cancel, so a single rounding of
// X*g would not keep those outputs within the elementwise bound the plain
// product meets.  The extra matrix-core work is free here (bandwidth-bound).
template <int NW, int LR>
struct DecSplit {
  static constexpr bool value = NW == 2 || LR > 0;
};

template <int MB, int NW, int WV, int LR>
struct DecodeSmem {
  static constexpr bool SPLIT = DecSplit<NW, LR>::value;
  // per-wave accumulators [wave][slot][lane]: slots (wi,b,c) of the weight
  // products, then (b,lb) of the adapter's down-projection
  floatx4 red[WV][NW * MB * 8 + MB * LR][64];
  u32x4 xg[DEC_STAGE_BYTES / (16 * 16 * MB)][16 * MB];  // A operand, [k/8][row]
  // low part of the split operand, same layout
  u32x4 xl[SPLIT ? DEC_STAGE_BYTES / (16 * 16 * MB) : 1][16 * MB];
  u32x4 lb[LR > 0 ? 16 * LR : 1][16];  // adapter: the tile's B rows, [rank][8-column chunk]
  float ssr[16 * MB];
  float inv[16 * MB];
  int last;
};

template <int MB, bool GATED, int WV, int LR>
__global__ __launch_bounds__(WV * 64) void decode_kernel(
    const bf16_t* __restrict__ X, const bf16_t* __restrict__ g, const bf16_t* __restrict__ W1,
    const bf16_t* __restrict__ W3, bf16_t* __restrict__ Y, float eps, int M, int64_t N,
    int64_t K, int64_t kchunk, int S, int tiles, int xcd_remap, unsigned* __restrict__ cnt,
    float* __restrict__ ssq_ws, float* __restrict__ part_ws, int norm,
    const bf16_t* __restrict__ LA, const bf16_t* __restrict__ LB, int R) {
  constexpr int NW = GATED ? 2 : 1;
  constexpr bool SPLIT = DecSplit<NW, LR>::value;
  static_assert(!(GATED && LR), "the adapter is not combined with the gate");
  static_assert(sizeof(DecodeSmem<MB, NW, WV, LR>) <= 160 * 1024, "LDS");
  constexpr int NT = WV * 64;
  constexpr int EW = NW * MB * 8;                 // weight-product slots
  constexpr int E4 = (EW + MB * LR) * 64;         // floatx4 per partial
  constexpr int PER4 = (E4 + NT - 1) / NT;        // floatx4 per thread in the combine
  constexpr bool E4_FULL = E4 % NT == 0;          // every thread owns PER4 of them
  constexpr int ROWS = 16 * MB;
  constexpr int SEG = DEC_STAGE_BYTES / (16 * ROWS) * 8;  // k rows staged at a time
  constexpr int TPR = NT / ROWS;                          // staging threads per row
  constexpr int NU = SEG / 8 / TPR;                       // 16-byte chunks per staging thread
  constexpr int STEP = 32 * WV;                           // k rows per pipeline step
  constexpr int SPS = SEG / STEP;                         // steps per staged segment
  static_assert(SPS % 2 == 0 && NU >= 1, "segment must hold an even number of steps");
  __shared__ DecodeSmem<MB, NW, WV, LR> sm;

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
  const int nsteps = (int)((k_hi - k_lo + STEP - 1) / STEP);

  DecodeSrc src;
  src.w1 = __builtin_amdgcn_make_buffer_rsrc((void*)W1, 0, (int)(K * N * 2), 0x00020000);
  src.w3 = __builtin_amdgcn_make_buffer_rsrc((void*)(GATED ? W3 : W1), 0, (int)(K * N * 2), 0x00020000);
  src.x = __builtin_amdgcn_make_buffer_rsrc((void*)X, 0, (int)((int64_t)M * K * 2), 0x00020000);
  src.g = __builtin_amdgcn_make_buffer_rsrc((void*)g, 0, (int)(K * 2), 0x00020000);
  // Adapter: lane (q, p) of block lb reads A[16 lb + p][krow .. krow+7], the
  // B fragment of one v_mfma_f32_16x16x32_bf16 as stored; rows past R fall
  // outside the buffer and read zeros.
  const __amdgpu_buffer_rsrc_t lar =
      __builtin_amdgcn_make_buffer_rsrc((void*)(LR ? LA : W1), 0, LR ? (int)(R * K * 2) : 0, 0x00020000);
  auto lora_load = [&](u32x4 (&lv)[LR > 0 ? LR : 1], int64_t krow) {
#pragma unroll
    for (int lb = 0; lb < LR; ++lb)
      lv[lb] = __builtin_amdgcn_raw_buffer_load_b128(
          lar, krow < k_hi ? (uint32_t)(((int64_t)(16 * lb + p) * K + krow) * 2) : kOutOfRange, 0, 0);
  };

  // Staging: thread -> row srow, 16-byte k-chunks sj + TPR u of the segment.
  const int srow = tid / TPR, sj = tid % TPR;
  float ssl = 0.f;
  auto stage_load = [&](int64_t seg_lo, u32x4 (&xs)[NU], u32x4 (&gs)[NU]) {
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int64_t k = seg_lo + 8 * (sj + TPR * u);
      const bool ok = k < k_hi && k < seg_lo + SEG;
      xs[u] = __builtin_amdgcn_raw_buffer_load_b128(
          src.x, (ok && srow < M) ? (uint32_t)(((int64_t)srow * K + k) * 2) : kOutOfRange, 0, 0);
      gs[u] = __builtin_amdgcn_raw_buffer_load_b128(src.g, ok ? (uint32_t)(k * 2) : kOutOfRange, 0, 0);
    }
  };
  auto stage_form = [&](const u32x4 (&xs)[NU], const u32x4 (&gs)[NU]) {
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      u32x4 av, al;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const float x0 = bf16_lo(xs[u][d]), x1 = bf16_hi(xs[u][d]);
        const uint32_t gd = norm ? gs[u][d] : kBf16OnePair;
        const float g0 = bf16_lo(gd), g1 = bf16_hi(gd);
        ssl += x0 * x0 + x1 * x1;
        if (SPLIT) {
          const u32x2 hl = split_bf16x2(x0 * g0, x1 * g1);
          av[d] = hl[0];
          al[d] = hl[1];
        } else
          av[d] = pack_bf16x2(x0 * g0, x1 * g1);
      }
      sm.xg[sj + TPR * u][srow] = av;
      if (SPLIT) sm.xl[sj + TPR * u][srow] = al;
    }
  };

  // Segment 0 staging loads, then both W stages (with the adapter: then this
  // tile's rows of B, which only the workgroup combining the tile uses but
  // which would otherwise be fetched on its critical path; they are parked in
  // LDS after the k-loop), then the A operand.
  u32x4 wa[NW][8], wb[NW][8];
  u32x4 la[LR > 0 ? LR : 1], lb[LR > 0 ? LR : 1];
  constexpr int BCH = LR > 0 ? (256 * LR + NT - 1) / NT : 1;  // B chunks per thread
  u32x4 bv[BCH];
  {
    u32x4 xs[NU], gs[NU];
    stage_load(k_lo, xs, gs);
    decode_load<NW>(wa, src, N, k_lo + 32 * w + 8 * q, k_hi, col, col_ok);
    lora_load(la, k_lo + 32 * w + 8 * q);
    decode_load<NW>(wb, src, N, k_lo + STEP + 32 * w + 8 * q, k_hi, col, col_ok);
    lora_load(lb, k_lo + STEP + 32 * w + 8 * q);
    if (LR > 0) {
      const __amdgpu_buffer_rsrc_t lbr =
          __builtin_amdgcn_make_buffer_rsrc((void*)LB, 0, (int)(R * N * 2), 0x00020000);
#pragma unroll
      for (int i = 0; i < BCH; ++i) {
        const int e = tid + NT * i, r = e >> 4;
        const int64_t bc = (int64_t)tile * DEC_COLS + 8 * (e & 15);
        bv[i] = __builtin_amdgcn_raw_buffer_load_b128(
            lbr, (r < R && e < 256 * LR && bc < N) ? (uint32_t)(((int64_t)r * N + bc) * 2) : kOutOfRange,
            0, 0);
      }
    }
    stage_form(xs, gs);
  }
  __syncthreads();

  floatx4 acc[NW][MB][8];
#pragma unroll
  for (int a = 0; a < NW; ++a)
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[a][b][c] = floatx4{0.f, 0.f, 0.f, 0.f};
  // Adapter down-projection T = (X g) A^T: lane element (row 16b + 4q + r,
  // rank 16 lb + p) of block (b, lb).
  floatx4 lacc[MB][LR > 0 ? LR : 1];
#pragma unroll
  for (int b = 0; b < MB; ++b)
#pragma unroll
    for (int i = 0; i < LR; ++i) lacc[b][i] = floatx4{0.f, 0.f, 0.f, 0.f};
  auto lora_mma = [&](const u32x4 (&lv)[LR > 0 ? LR : 1], const u32x4 (&a)[MB],
                      const u32x4 (&al)[MB]) {
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
      for (int i = 0; i < LR; ++i) {
        lacc[b][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, a[b]), __builtin_bit_cast(bf16x8, lv[i]), lacc[b][i], 0, 0, 0);
        lacc[b][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, al[b]), __builtin_bit_cast(bf16x8, lv[i]), lacc[b][i], 0, 0, 0);
      }
  };
  auto mma = [&](const u32x4 (&wv)[NW][8], const u32x4 (&a)[MB], const u32x4 (&al)[MB]) {
    if (SPLIT)
      decode_mma2<MB, NW>(wv, a, al, acc);
    else
      decode_mma<MB, NW>(wv, a, acc);
  };

  auto fetch_a = [&](int s, u32x4 (&a)[MB], u32x4 (&al)[MB]) {
    const int kc = ((s % SPS) * STEP + 32 * w + 8 * q) >> 3;
#pragma unroll
    for (int b = 0; b < MB; ++b) {
      a[b] = sm.xg[kc][16 * b + p];
      if (SPLIT) al[b] = sm.xl[kc][16 * b + p];
    }
  };
  // A new segment: everyone is done with the old one, stage, publish.
  auto restage = [&](int s) {
    __syncthreads();
    u32x4 xs[NU], gs[NU];
    stage_load(k_lo + (int64_t)s * STEP, xs, gs);
    stage_form(xs, gs);
    __syncthreads();
  };
  int s = 0;
  for (; s + 2 <= nsteps; s += 2) {
    if (s > 0 && s % SPS == 0) restage(s);
    u32x4 a[MB], al[MB];
    fetch_a(s, a, al);
    mma(wa, a, al);
    lora_mma(la, a, al);
    decode_load<NW>(wa, src, N, k_lo + (int64_t)(s + 2) * STEP + 32 * w + 8 * q, k_hi, col, col_ok);
    lora_load(la, k_lo + (int64_t)(s + 2) * STEP + 32 * w + 8 * q);
    fetch_a(s + 1, a, al);
    mma(wb, a, al);
    lora_mma(lb, a, al);
    decode_load<NW>(wb, src, N, k_lo + (int64_t)(s + 3) * STEP + 32 * w + 8 * q, k_hi, col, col_ok);
    lora_load(lb, k_lo + (int64_t)(s + 3) * STEP + 32 * w + 8 * q);
  }
  if (s < nsteps) {
    if (s > 0 && s % SPS == 0) restage(s);
    u32x4 a[MB], al[MB];
    fetch_a(s, a, al);
    mma(wa, a, al);
    lora_mma(la, a, al);
  }

  if (LR > 0) {
#pragma unroll
    for (int i = 0; i < BCH; ++i) {
      const int e = tid + NT * i;
      if ((256 * LR) % NT == 0 || e < 256 * LR) sm.lb[e >> 4][e & 15] = bv[i];
    }
  }
  // Row sums of squares: the TPR staging threads of a row are adjacent lanes.
#pragma unroll
  for (int o = 1; o < TPR; o <<= 1) ssl += __shfl_xor(ssl, o);
  if (sj == 0) sm.ssr[srow] = ssl;
  // Per-wave accumulators to LDS as floatx4: e = (wi*MB + b)*8 + c.
#pragma unroll
  for (int wi = 0; wi < NW; ++wi)
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
      for (int c = 0; c < 8; ++c) sm.red[w][(wi * MB + b) * 8 + c][l] = acc[wi][b][c];
#pragma unroll
  for (int b = 0; b < MB; ++b)
#pragma unroll
    for (int i = 0; i < LR; ++i) sm.red[w][EW + b * LR + i][l] = lacc[b][i];
  __syncthreads();

  // Workgroup sum of the waves; thread owns floatx4 tid + NT u (E4 is a
  // multiple of 64, so the bound is uniform per wave).
  floatx4* red0 = &sm.red[0][0][0];
  floatx4 v[PER4];
#pragma unroll
  for (int u = 0; u < PER4; ++u) {
    const int f = tid + NT * u;
    floatx4 t4 = floatx4{0.f, 0.f, 0.f, 0.f};
    if (E4_FULL || f < E4) {
      t4 = red0[f];
#pragma unroll
      for (int ww = 1; ww < WV; ++ww) t4 += red0[ww * E4 + f];
    }
    v[u] = t4;
  }
  float ssw = tid < ROWS ? sm.ssr[tid] : 0.f;


  if (S > 1) {
    const int64_t slot = (int64_t)split * tiles + tile;
    const int64_t nslots = (int64_t)S * tiles;
    const __amdgpu_buffer_rsrc_t prs =
        __builtin_amdgcn_make_buffer_rsrc(part_ws, 0, (int)(nslots * E4 * 16), 0x00020000);
    // Partials go out with device-scope coherence; waiting for every store's
    // acknowledgement before the arrival count makes them visible to
    // whichever workgroup arrives last.
#pragma unroll
    for (int u = 0; u < PER4; ++u)
      if (E4_FULL || tid + NT * u < E4)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v[u]), prs,
                                               (int)((slot * E4 + tid + NT * u) * 16), 0,
                                               kCoherentDevice);
    if (tid < ROWS)
      __hip_atomic_store(&ssq_ws[slot * ROWS + tid], ssw, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0)
      sm.last = (__hip_atomic_fetch_add(&cnt[tile], 1u, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT) == (unsigned)(S - 1));
    __syncthreads();
    if (!sm.last) return;
    // Last arrival: add the S partials, up to 8 splits' loads in flight.
    constexpr int RS = 8 / PER4 > 0 ? 8 / PER4 : 1;
#pragma unroll
    for (int u = 0; u < PER4; ++u) v[u] = floatx4{0.f, 0.f, 0.f, 0.f};
    ssw = 0.f;
    for (int s0 = 0; s0 < S; s0 += RS) {
      u32x4 buf[RS][PER4];
      float sb[RS];
#pragma unroll
      for (int uu = 0; uu < RS; ++uu) {
        const int64_t sl = (int64_t)(s0 + uu) * tiles + tile;
        const bool ok = s0 + uu < S;
#pragma unroll
        for (int u = 0; u < PER4; ++u)
          buf[uu][u] = (ok && (E4_FULL || tid + NT * u < E4)) ? __builtin_amdgcn_raw_buffer_load_b128(
                                prs, (int)((sl * E4 + tid + NT * u) * 16), 0, kCoherentDevice)
                          : u32x4{0u, 0u, 0u, 0u};
        sb[uu] = (ok && tid < ROWS) ? __hip_atomic_load(&ssq_ws[sl * ROWS + tid], __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_AGENT)
                                    : 0.f;
      }
#pragma unroll
      for (int uu = 0; uu < RS; ++uu) {
#pragma unroll
        for (int u = 0; u < PER4; ++u) v[u] += __builtin_bit_cast(floatx4, buf[uu][u]);
        ssw += sb[uu];
      }
    }
    // Reset the tile's arrival counter for the next call (all arrivals are
    // in); the partial slots are overwritten by the next call before use.
    if (tid == 0) __hip_atomic_store(&cnt[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();  // everyone is done reading sm.red before it is overwritten
#pragma unroll
  for (int u = 0; u < PER4; ++u)
    if (E4_FULL || tid + NT * u < E4) red0[tid + NT * u] = v[u];
  if (tid < ROWS) sm.inv[tid] = norm ? inv_rms(ssw, K, eps) : 1.0f;
  __syncthreads();

  // Epilogue: group (b, r, lane) -> row 16b + 4(lane/16) + r, 8 columns
  // 8(lane%16) .. +7; element (wi, b, c, lane, r) is float
  // (((wi*MB + b)*8 + c)*64 + lane)*4 + r of the summed block.
  const float* redf = (const float*)red0;
#pragma unroll
  for (int t = 0; t < (MB * 256 + NT - 1) / NT; ++t) {
    const int grp = tid + NT * t;
    if (grp >= MB * 256) break;
    const int ln = grp & 63, br = grp >> 6, b = br >> 2, r = br & 3;
    const int row = 16 * b + 4 * (ln >> 4) + r;
    const int64_t cc = (int64_t)tile * DEC_COLS + 8 * (ln & 15);
    if (row >= M || cc >= N) continue;
    const float inv = sm.inv[row];
    // Adapter: y += sum_r T[row][r] B[r][cc + c], T from slot (b, r / 16),
    // lane 16 (ln / 16) + r % 16, component r of the summed block.
    float ya[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int rr = 0; rr < 16 * LR; ++rr) {
      const float t = redf[((EW + b * LR + rr / 16) * 64 + 16 * (ln >> 4) + rr % 16) * 4 + r];
      const u32x4 bq = sm.lb[rr][ln & 15];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        ya[2 * d] += t * bf16_lo(bq[d]);
        ya[2 * d + 1] += t * bf16_hi(bq[d]);
      }
    }
    u32x4 out;
#pragma unroll
    for (int c = 0; c < 8; c += 2) {
      float y0 = redf[(((0 * MB + b) * 8 + c) * 64 + ln) * 4 + r];
      float y1 = redf[(((0 * MB + b) * 8 + c + 1) * 64 + ln) * 4 + r];
      if (LR > 0) {
        y0 += ya[c];
        y1 += ya[c + 1];
      }
      y0 *= inv;
      y1 *= inv;
      if (GATED) {
        const float z0 = redf[(((1 * MB + b) * 8 + c) * 64 + ln) * 4 + r] * inv;
        const float z1 = redf[(((1 * MB + b) * 8 + c + 1) * 64 + ln) * 4 + r] * inv;
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

// Chunks are whole 128-deep granules; eight waves (256-deep steps) when the
// grid has at most one workgroup per CU and the per-wave accumulators fit.
void rmm_decode_plan(int64_t M, int64_t N, int64_t K, int gated, int splits, int64_t lora_rank,
                     DecodePlan* p) {
  using namespace rmm;
  p->mb = (int)((M + 15) / 16);
  p->lr = (int)((lora_rank + 15) / 16);
  p->tiles = (N + DEC_COLS - 1) / DEC_COLS;
  const int64_t kgran = (K + 127) / 128;
  int64_t s = splits;
  if (s < 1) s = 1;
  if (s > kgran) s = kgran;
  const int64_t gran_per = (kgran + s - 1) / s;
  p->kchunk = gran_per * 128;
  p->splits = (int)((K + p->kchunk - 1) / p->kchunk);
  const int nw = gated ? 2 : 1;
  p->wv = (nw * p->mb == 1 && p->tiles * p->splits <= 256) ? 8 : 4;
  const size_t E = ((size_t)nw * p->mb * 8 + (size_t)p->mb * p->lr) * 64 * 4;  // floats per partial
  p->ws_cnt_off = 0;
  p->ws_ssq_off = kWsCounterBytes;
  p->ws_part_off = p->ws_ssq_off + align256(sizeof(float) * (size_t)p->splits * p->tiles * p->mb * 16);
  p->ws_bytes = p->splits > 1 ? p->ws_part_off + align256(sizeof(float) * (size_t)p->splits * p->tiles * E) : 0;
}

template <int MB, bool GATED, int WV, int LR>
static void launch_decode_t(const RmmArgs& a, const DecodePlan& p, void* ws) {
  using namespace rmm;
  const int xcd_remap = (p.tiles % 8) == 0;
  char* base = (char*)ws;
  unsigned* cnt = ws ? (unsigned*)(base + p.ws_cnt_off) : nullptr;
  float* ssq = ws ? (float*)(base + p.ws_ssq_off) : nullptr;
  float* part = ws ? (float*)(base + p.ws_part_off) : nullptr;
  const unsigned grid = (unsigned)(p.tiles * p.splits);
  hipLaunchKernelGGL((decode_kernel<MB, GATED, WV, LR>), dim3(grid), dim3(WV * 64), 0, a.stream,
                     (const bf16_t*)a.X, (const bf16_t*)a.g, (const bf16_t*)a.W1,
                     (const bf16_t*)a.W3, (bf16_t*)a.Y, a.eps, (int)a.M, a.N, a.K, p.kchunk,
                     p.splits, (int)p.tiles, xcd_remap, cnt, ssq, part, a.norm,
                     (const bf16_t*)a.LA, (const bf16_t*)a.LB, (int)a.R);
}

hipError_t rmm_launch_decode(const RmmArgs& a, const DecodePlan& p, void* ws) {
  const bool gd = a.gated != 0;
  const int lr = a.R > 0 ? p.lr : 0;
  if (lr != p.lr) return hipErrorInvalidValue;
  if (!gd && lr == 0 && p.mb == 1 && p.wv == 8) launch_decode_t<1, false, 8, 0>(a, p, ws);
  else if (!gd && lr == 0 && p.mb == 1 && p.wv == 4) launch_decode_t<1, false, 4, 0>(a, p, ws);
  else if (!gd && lr == 0 && p.mb == 2 && p.wv == 4) launch_decode_t<2, false, 4, 0>(a, p, ws);
  else if (gd && lr == 0 && p.mb == 1 && p.wv == 4) launch_decode_t<1, true, 4, 0>(a, p, ws);
  else if (!gd && lr == 1 && p.mb == 1 && p.wv == 8) launch_decode_t<1, false, 8, 1>(a, p, ws);
  else if (!gd && lr == 1 && p.mb == 1 && p.wv == 4) launch_decode_t<1, false, 4, 1>(a, p, ws);
  else if (!gd && lr == 1 && p.mb == 2 && p.wv == 4) launch_decode_t<2, false, 4, 1>(a, p, ws);
  else if (!gd && lr == 2 && p.mb == 1 && p.wv == 8) launch_decode_t<1, false, 8, 2>(a, p, ws);
  else if (!gd && lr == 2 && p.mb == 1 && p.wv == 4) launch_decode_t<1, false, 4, 2>(a, p, ws);
  else if (!gd && lr == 2 && p.mb == 2 && p.wv == 4) launch_decode_t<2, false, 4, 2>(a, p, ws);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}
