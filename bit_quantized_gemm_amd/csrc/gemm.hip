// W4A4 grouped GEMM for gfx950 on the matrix cores.
//
// Y[m,n] = sum over 128-channel groups g of acc_g[m,n] * sx[g,m] * sw[g,n], with
// acc_g = exact integer dot product of the codes of group g.  The method runs this product
// on integer operators (index page of "Atom: Low-bit Quantization for Efficient and Accurate
// LLM Serving", Abstract; quantization record, "notes": an integer-operator path, not FP4).
//
// INT4 groups.  gfx950 has no 4-bit integer MFMA.  An INT4 code q in [-7, 7] is exactly the
// fp6 e2m3 subnormal with bits (q < 0) << 5 | |q| (value q / 8), and the packed layout (a unit
// of 16 codes = the 96 bits of their fp6 fields with the third word folded into the always-zero
// exponent bits of the first two, see atom_internal.h) turns 8 bytes into 12 operand bytes
// with four bit operations.  v_mfma_scale_f32_32x32x64_f8f6f4 on fp6 operands with scales
// 2^3 * 2^3 then returns the group's integer dot product exactly in fp32: every product and
// partial sum is an integer of magnitude below 2^24.  The INT4 groups thus run at the dense
// fp6 rate, twice the int8 / fp8 rate, and their accumulators are already fp32.
//
// INT8 outlier group (record, "notes": a 128-channel high-precision group): int8 codes feed
// v_mfma_i32_32x32x32_i8 directly; its int32 accumulators are converted once.
//
// Scales.  The rank-one product sx[g,:] (x) sw[g,:] of a 32x32 output tile comes from one
// v_mfma_f32_32x32x8_f16 whose only nonzero K slots (0 and 4) hold the fp16 scales: fp16 x
// fp16 is exact in fp32, the two equal products sum exactly to 2 * sx * sw, and the result
// lands in the accumulator layout.  The epilogue per output element and group is then a
// single fp32 FMA; the factor 2 is removed once at the store.  Each thread stores its fp16
// scale in LDS as a ready 8-byte operand (scale, 0, 0, 0), read with one ds_read_b64.
//
// Pipeline.  A packed row is a sequence of 64-byte stages: stage s < G-1 is INT4 group s,
// stages G-1 and G are the two 64-byte halves of the INT8 outlier group.  Each wave copies
// 16-row slabs of a stage of the A (activation) and B (weight) tiles straight into LDS with
// LDS-DMA buffer loads (16 bytes per lane, the stage offset in a scalar), still packed, so
// LDS carries 64 bytes per row and group and no registers or VALU work go into staging.
// Three stage buffers form a ring: while group s is multiplied its operands are in
// registers, stage s+1 has landed and is read into registers as they free up, and stages
// s+2 and s+3 are in flight.  One barrier per group.  Every wave decodes the packed bytes of
// its own operands in registers just before the MFMAs that use them.
//
// LDS layout.  A staged row is 64 bytes = four 16-byte chunks; chunk c of row r is stored at
// position c ^ ((r >> 2) & 3), so the 16 lanes of a ds_read_b128 group (16 consecutive rows,
// one chunk) cover all 16 bank groups of 16 bytes.  A copy writes 16 consecutive bytes per
// lane, so the swizzle is applied to the global address each lane copies from.
//
// Waves.  A workgroup of WAVES_M x WAVES_N waves computes a BM x BN tile of Y; each wave
// owns a (BM/WAVES_M) x (BN/WAVES_N) sub-tile held as 32x32 MFMA tiles.  Lane l supplies row
// (A) / column (B) l & 31 of a tile and the K half l >> 5 of each operand.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include <mutex>

#include "atom_internal.h"
#include "lds_ring.h"
#include "row_quant.h"

namespace atom {
namespace {

typedef int32_t v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef int32_t v8i __attribute__((ext_vector_type(8)));
typedef int32_t v4i __attribute__((ext_vector_type(4)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));

constexpr int kStageBytes = 64;          // bytes of one stage of a packed row
constexpr int kLdsRow = 64;              // bytes of one staged (packed) row in LDS
constexpr int kXcds = 8;                 // accelerator complex dies (each with its own L2)
constexpr int kScaleE8M0 = 127 + 3;      // 2^3: the e2m3 subnormal q / 8 counts as q
constexpr int kFairBit = 9;              // real-time clock bit (100 MHz: 5.12 us period) of the turns

// Issue priority 1 if bit 0 of b is set, else 0 (s_setprio takes only an immediate).  One asm
// statement with its own skip, so the compiler's control flow and register allocation around
// the main loop are untouched.
__device__ __forceinline__ void set_priority_from_bit0(uint32_t b) {
  asm volatile(
      "s_bitcmp1_b32 %0, 0\n\t"
      "s_cbranch_scc0 1f\n\t"
      "s_setprio 1\n\t"
      "s_branch 2f\n"
      "1:\n\t"
      "s_setprio 0\n"
      "2:"
      :
      : "s"(b)
      : "scc");
}

// Issue priority v (0, 1 or 2), the same way.
__device__ __forceinline__ void set_priority_0_to_2(uint32_t v) {
  asm volatile(
      "s_cmp_eq_u32 %0, 0\n\t"
      "s_cbranch_scc0 1f\n\t"
      "s_setprio 0\n\t"
      "s_branch 3f\n"
      "1:\n\t"
      "s_cmp_eq_u32 %0, 1\n\t"
      "s_cbranch_scc0 2f\n\t"
      "s_setprio 1\n\t"
      "s_branch 3f\n"
      "2:\n\t"
      "s_setprio 2\n"
      "3:"
      :
      : "s"(v)
      : "scc");
}

// fp6 operand (32 codes, six words) of the two packed units in words 4h .. 4h+3 of w: unit
// words (w0, w1) -> fields T0 = w0 & ~kFp6Exp0, T1 = w1 & ~kFp6Exp1,
// T2 = (w0 & kFp6Exp0) | (w1 & kFp6Exp1).  The last two words are not read by the fp6 MFMA.
__device__ __forceinline__ v8i fp6_operand(v8i w, int h) {
  v8i r;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const uint32_t w0 = (uint32_t)w[4 * h + 2 * u], w1 = (uint32_t)w[4 * h + 2 * u + 1];
    r[3 * u] = (int)(w0 & ~kFp6Exp0);
    r[3 * u + 1] = (int)(w1 & ~kFp6Exp1);
    r[3 * u + 2] = (int)((w0 & kFp6Exp0) | (w1 & kFp6Exp1));
  }
  r[6] = 0;
  r[7] = 0;
  return r;
}

// The matrix-core calls below take the weight operand b as their first source and the
// activation operand a as their second, so a 32x32 accumulator holds the output tile
// transposed: lane l owns output row l & 31, and its element r is column
// (r >> 2) * 8 + (l >> 5) * 4 + (r & 3), i.e. four runs of four consecutive columns that
// the epilogue stores as vectors.
__device__ __forceinline__ v16f mma_fp6(v8i a, v8i b, v16f c) {
  // cbsz = blgp = 2: both operands fp6 e2m3; opsel 0 and E8M0 scale 2^3 on both sides
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c, 2, 2, 0, kScaleE8M0, 0, kScaleE8M0);
}

// One issue slot of the INT4 main loop: the scheduling region's MFMA first, then up to NV
// vector ALU operations, then up to NDS LDS reads; the region ends here.
#define ATOM_SLOT(NV, NDS)                                  \
  do {                                                      \
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      \
    __builtin_amdgcn_sched_group_barrier(0x002, (NV), 0);   \
    __builtin_amdgcn_sched_group_barrier(0x100, (NDS), 0);  \
    __builtin_amdgcn_sched_barrier(0);                      \
  } while (0)

__device__ __forceinline__ v16i mma_i8(v4i a, v4i b, v16i c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(b, a, c, 0, 0, 0);
}

// Output row (within a 32x32 tile) and first of four consecutive columns held by element
// group q (elements 4q .. 4q+3) of a lane's accumulator.
__device__ __forceinline__ int acc_row(int lane) { return lane & 31; }
__device__ __forceinline__ int acc_col(int lane, int q) { return q * 8 + (lane >> 5) * 4; }

// Chunk position swizzle of LDS row r (rows are 64 bytes)
__device__ __forceinline__ int chunk_swz(int r) { return (r >> 2) & 3; }



template <int BM, int BN, int WAVES_M, int WAVES_N>
struct Tile {
  static constexpr int kThreads = WAVES_M * WAVES_N * 64;
  static constexpr int kWTM = BM / WAVES_M;            // wave tile rows
  static constexpr int kWTN = BN / WAVES_N;            // wave tile columns
  static constexpr int kTM = kWTM / 32;                // MFMA tiles per wave (rows)
  static constexpr int kTN = kWTN / 32;                // MFMA tiles per wave (columns)
  static constexpr int kWaves = WAVES_M * WAVES_N;
  static constexpr int kDma = BM / kWaves / 16;        // LDS-DMA instructions per wave per stage and tile
  static constexpr int kSPT = (BM + BN) / kThreads;    // scales per thread per stage
  static_assert(kWTM % 32 == 0 && kWTN % 32 == 0, "wave tile must be a multiple of 32");
  static_assert(kSPT * kThreads == BM + BN && kSPT >= 1 && kSPT <= 2, "one or two scales per thread per stage");
  static_assert(BM == BN && kDma * kWaves * 16 == BM, "each wave copies whole 16-row slabs of A and B");
};

// Per-thread addressing of the stage copy, fixed for the whole K loop.  Wave w copies tile
// rows [w * BM / W, (w + 1) * BM / W) of A and the same rows of B (W waves), 16 rows per
// LDS-DMA instruction: lane i of instruction h lands at LDS row r = w * BM / W + 16h + i / 4,
// position i % 4, so it loads chunk (i % 4) ^ chunk_swz(r) of that row.  Rows past M / N
// repeat the last valid row.  Scale slot t < BM carries the activation scale of tile row t,
// slot BM + u the weight scale of tile column u; thread t holds slots t, t + threads, ...
template <int NDMA, int NS>
struct StageAddr {
  __amdgpu_buffer_rsrc_t a_rsrc, b_rsrc;  // the workgroup's rows of Xq / Wq
  int a_voff[NDMA], b_voff[NDMA];          // byte offset of this lane's chunk in stage 0
  int lds_row0;                            // first LDS row of this wave's copy (wave-uniform)
  const uint16_t* s_src[NS];               // this thread's scales in group 0
  bool s_is_x[NS];                         // activation (stride M) or weight (stride N) scale
};


// Copy stage s of this wave's rows into LDS (asynchronous; tracked by vmcnt).
template <int NDMA, int NS>
__device__ __forceinline__ void dma_stage(const StageAddr<NDMA, NS>& ad, uint8_t* la, uint8_t* lb, int s) {
  const int soff = s * kStageBytes;
#pragma unroll
  for (int h = 0; h < NDMA; ++h) {
    lds_dma16(ad.a_rsrc, la + (ad.lds_row0 + 16 * h) * kLdsRow, ad.a_voff[h], soff);
    lds_dma16(ad.b_rsrc, lb + (ad.lds_row0 + 16 * h) * kLdsRow, ad.b_voff[h], soff);
  }
}

// This thread's scale u of stage s (group min(s, G-1): the INT8 group fills two stages).
template <int NDMA, int NS>
__device__ __forceinline__ uint16_t load_scale(const StageAddr<NDMA, NS>& ad, int s, int G, int M, int N, int u) {
  const int g = min(s, G - 1);
  const size_t ox = (size_t)g * M, ow = (size_t)g * N;   // uniform
  return ad.s_src[u][ad.s_is_x[u] ? ox : ow];
}

// kAcc = false: Y output.  kAcc = true: write the per-group integer accumulators instead.
// Split-K (Y output only): the first `full` tiles run whole; the INT4 groups of each of the
// last `rem` tiles are divided among `splits` pieces (the last piece also takes the INT8
// group), each writing its fp32 tile sum, still carrying the factor 2 of the scale
// products, tile-major to part[(piece split * rem + tile - full) * BM * BN].
// One output tile (or one split-K piece of it) of the tiled GEMM: tile `lin` in tile order, K piece
// `split` of `nsplit`.  NBUF stage buffers (3 .. 8) form the ring: NBUF - 1 stages of copies are
// in flight ahead of the group being multiplied.  The LDS is declared here, once per kernel that
// calls this; a kernel that calls it for several tiles puts a workgroup barrier between them.
// SUB > 1: the workgroup is SUB parts of WAVES_M x WAVES_N waves; part k takes the k-th 1/SUB
// of the tile's INT4 groups (the last part also the INT8 group), each part with a ring of
// stage buffers of its own.  Parts of one wave need no barrier in the loop; parts of several
// share the workgroup barrier, and a part with one group fewer passes one extra barrier so
// that every wave passes the same number.  The SUB partial tiles are then added through LDS
// in part order: the wave of part t adds up and stores MFMA tile t of its wave tile (parts past
// the wave tile's MFMA tile count only hand in partials).
template <int BM, int BN, int WAVES_M, int WAVES_N, int NBUF, bool kAcc, int SUB = 1, bool kFair = false>
__device__ __forceinline__ void gemm_tile(const uint8_t* __restrict__ Xq, const uint16_t* __restrict__ sx,
                                          const uint8_t* __restrict__ Wq, const uint16_t* __restrict__ sw, int M, int N,
                                          int K, uint16_t* __restrict__ Y, int32_t* __restrict__ acc_out, int lin,
                                          int split, int nsplit, int full, int rem, float* __restrict__ part,
                                          int fair_cus = 0) {
  using T = Tile<BM, BN, WAVES_M, WAVES_N>;
  static_assert(NBUF >= 3 && NBUF <= 8, "ring of 3 to 8 stage buffers");
  static_assert(SUB == 1 || (!kAcc && T::kTM * T::kTN <= SUB && SUB * T::kWaves <= 2 * NBUF),
                "K parts: at most one output MFMA tile per wave, partials fit the stage buffers");
  // The stage buffers, each its own object: the compiler then knows that a copy into one does
  // not write what is read from another, and waits only where a buffer is really shared.
  // Buffers past NBUF are never referenced and take no LDS.
  // (SUB parts side by side in each buffer)
  __shared__ __attribute__((aligned(16))) uint8_t la0[SUB * BM * kLdsRow], la1[SUB * BM * kLdsRow],
      la2[SUB * BM * kLdsRow], la3[SUB * BM * kLdsRow], la4[SUB * BM * kLdsRow], la5[SUB * BM * kLdsRow],
      la6[SUB * BM * kLdsRow], la7[SUB * BM * kLdsRow];
  __shared__ __attribute__((aligned(16))) uint8_t lb0[SUB * BN * kLdsRow], lb1[SUB * BN * kLdsRow],
      lb2[SUB * BN * kLdsRow], lb3[SUB * BN * kLdsRow], lb4[SUB * BN * kLdsRow], lb5[SUB * BN * kLdsRow],
      lb6[SUB * BN * kLdsRow], lb7[SUB * BN * kLdsRow];
  // sx rows, then sw columns, each as a ready scale operand
  __shared__ __attribute__((aligned(16))) h4 ls0[SUB * (BM + BN)], ls1[SUB * (BM + BN)], ls2[SUB * (BM + BN)],
      ls3[SUB * (BM + BN)], ls4[SUB * (BM + BN)], ls5[SUB * (BM + BN)], ls6[SUB * (BM + BN)], ls7[SUB * (BM + BN)];
  const int tid = threadIdx.x;
  const int sub = SUB > 1 ? __builtin_amdgcn_readfirstlane(tid / T::kThreads) : 0;   // this wave's K part
  const int vtid = SUB > 1 ? tid % T::kThreads : tid;                                 // thread within the part
  auto LA0 = [&](int p) -> uint8_t* {
    switch (p) {
      case 0: return la0; case 1: return la1; case 2: return la2; case 3: return la3;
      case 4: return la4; case 5: return la5; case 6: return la6; default: return la7;
    }
  };
  auto LB0 = [&](int p) -> uint8_t* {
    switch (p) {
      case 0: return lb0; case 1: return lb1; case 2: return lb2; case 3: return lb3;
      case 4: return lb4; case 5: return lb5; case 6: return lb6; default: return lb7;
    }
  };
  auto LS0 = [&](int p) -> h4* {
    switch (p) {
      case 0: return ls0; case 1: return ls1; case 2: return ls2; case 3: return ls3;
      case 4: return ls4; case 5: return ls5; case 6: return ls6; default: return ls7;
    }
  };
  auto LA = [&](int p) { return LA0(p) + sub * (BM * kLdsRow); };
  auto LB = [&](int p) { return LB0(p) + sub * (BN * kLdsRow); };
  auto LS = [&](int p) { return LS0(p) + sub * (BM + BN); };
  // One barrier per group orders a stage's copies and reads among the waves sharing it; a
  // one-wave K part has its stages to itself, and its own waits order them.
  auto ring_barrier = [&]() {
    if constexpr (SUB == 1 || T::kWaves > 1) wg_barrier();
  };

  const int lane = tid & 63;
  const int wave = vtid >> 6;
  const int wm = wave / WAVES_N;
  const int wn = wave % WAVES_N;
  const bool is_piece = SUB == 1 && nsplit > 1;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const int2 tc = tile_coords(lin, tiles_m, tiles_n);
  const int m0 = tc.x * BM, n0 = tc.y * BN;
  const int G = K / ATOM_GROUP;
  // this workgroup's INT4 groups [ga, gb); the last piece also takes the INT8 group
  const int kpart = SUB > 1 ? sub : split, nparts = SUB > 1 ? SUB : nsplit;
  const int ga = kpart * (G - 1) / nparts, gb = (kpart + 1) * (G - 1) / nparts;
  const bool last_split = kpart == nparts - 1;
  const int S = G + 1;                                  // stages per row
  const size_t rbytes = (size_t)S * kStageBytes;        // = (K-128)/2 + 128
  const int l32 = lane & 31;                            // row (A) / column (B) inside a 32x32 tile
  const int kh = lane >> 5;                             // which K half of an operand this lane supplies

  // ---- per-lane stage-copy addresses
  StageAddr<T::kDma, T::kSPT> ad;
  {
    const int rows_a = min(BM, M - m0), rows_b = min(BN, N - n0);
    ad.a_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)(Xq + (size_t)m0 * rbytes), (short)0,
                                                  (int)(rows_a * rbytes), 0x00020000);
    ad.b_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)(Wq + (size_t)n0 * rbytes), (short)0,
                                                  (int)(rows_b * rbytes), 0x00020000);
    ad.lds_row0 = __builtin_amdgcn_readfirstlane(wave) * (BM / T::kWaves);
#pragma unroll
    for (int h = 0; h < T::kDma; ++h) {
      const int r = ad.lds_row0 + 16 * h + lane / 4, c = ((lane & 3) ^ chunk_swz(r)) * 16;
      ad.a_voff[h] = min(r, rows_a - 1) * (int)rbytes + c;
      ad.b_voff[h] = min(r, rows_b - 1) * (int)rbytes + c;
    }
#pragma unroll
    for (int u = 0; u < T::kSPT; ++u) {
      const int t = vtid + u * T::kThreads;
      ad.s_is_x[u] = t < BM;
      ad.s_src[u] = kAcc ? nullptr : t < BM ? sx + min(m0 + t, M - 1) : sw + min(n0 + t - BM, N - 1);
    }
  }

  v16f yacc[T::kTM][T::kTN];
#pragma unroll
  for (int i = 0; i < T::kTM; ++i)
#pragma unroll
    for (int j = 0; j < T::kTN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) yacc[i][j][r] = 0.0f;
  // 16-byte LDS chunk c of the row supplying this lane in tile i (A) / j (B).  The swizzle
  // term depends only on l32 (tile rows start at multiples of 32).
  const int lane_swz = chunk_swz(l32);
  const int a_row = (wm * T::kWTM + l32) * kLdsRow, b_row = (wn * T::kWTN + l32) * kLdsRow;
  auto lds_chunk = [&](const uint8_t* buf, int row, int t, int c) {
    return *reinterpret_cast<const v4i*>(buf + row + t * 32 * kLdsRow + ((c ^ lane_swz) << 4));
  };
  auto cat = [](v4i lo, v4i hi) { return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]}; };

  // Rank-one fp16 scale operands of a group: every lane puts its row's sx (A) / column's sw
  // (B) in K slot 0 of its half, so the f16 MFMA returns 2 * sx * sw exactly (two equal
  // exact products).  Every term of the Y accumulators thus carries the factor 2, which the
  // final store removes; a power of two changes no rounding.  LDS holds each scale already
  // as its operand (scale, 0, 0, 0).
  auto scale_operand = [](uint16_t v) {
    return h4{__builtin_bit_cast(_Float16, v), (_Float16)0, (_Float16)0, (_Float16)0};
  };
  auto read_scales = [&](const h4* ls, h4 (&sa)[T::kTM], h4 (&sb)[T::kTN]) {
#pragma unroll
    for (int i = 0; i < T::kTM; ++i) sa[i] = ls[wm * T::kWTM + i * 32 + l32];
#pragma unroll
    for (int j = 0; j < T::kTN; ++j) sb[j] = ls[BM + wn * T::kWTN + j * 32 + l32];
  };

  // Rank-one scale product 2 * sx (x) sw of tile (i, j), in the accumulator layout.
  auto scale_product = [&](h4 sai, h4 sbj) {
    return kAcc ? v16f{} : __builtin_amdgcn_mfma_f32_32x32x8f16(sbj, sai, v16f{}, 0, 0, 0);
  };
  // Group sum of tile (i, j) -> Y accumulators (or, kAcc, to acc_out for group g).
  auto apply_element = [&](int i, int j, const v16f& acc, const v16f& sp, int g, int r) {
    if (kAcc) {
      const int m = m0 + wm * T::kWTM + i * 32 + acc_row(lane);
      const int n = n0 + wn * T::kWTN + j * 32 + acc_col(lane, r >> 2) + (r & 3);
      if (m < M && n < N) acc_out[((size_t)g * M + m) * N + n] = (int32_t)acc[r];   // exact integers
    } else {
      yacc[i][j][r] = __builtin_fmaf(acc[r], sp[r], yacc[i][j][r]);
    }
  };
  auto apply = [&](int i, int j, const v16f& acc, const v16f& sp, int g) {
#pragma unroll
    for (int r = 0; r < 16; ++r) apply_element(i, j, acc, sp, g, r);
  };
  auto finish_tile = [&](int i, int j, const v16f& acc, h4 sai, h4 sbj, int g) {
    apply(i, j, acc, scale_product(sai, sbj), g);
  };

  // This wave's packed operand bytes of one stage: for tile row i (A) / column j (B), the
  // lane's row, chunks 2kh and 2kh+1 (stage bytes 32kh .. 32kh+31).  On an INT4 stage these
  // are four units of 16 codes: chunk 2kh is the lane's K=32 slice of the first K=64 fp6
  // operand, chunk 2kh+1 of the second; on an INT8 stage, its K slices of two K=32 int8
  // operands.
  auto read_a = [&](const uint8_t* la, int i) {
    return cat(lds_chunk(la, a_row, i, 2 * kh), lds_chunk(la, a_row, i, 2 * kh + 1));
  };
  auto read_b = [&](const uint8_t* lb, int j) {
    return cat(lds_chunk(lb, b_row, j, 2 * kh), lds_chunk(lb, b_row, j, 2 * kh + 1));
  };
  auto read_packed = [&](const uint8_t* la, const uint8_t* lb, v8i (&pa)[T::kTM], v8i (&pb)[T::kTN]) {
#pragma unroll
    for (int i = 0; i < T::kTM; ++i) pa[i] = read_a(la, i);
#pragma unroll
    for (int j = 0; j < T::kTN; ++j) pb[j] = read_b(lb, j);
  };

  // Stage ring.  Stage t (t = ga, ga+1, ...) lives in LDS buffer (t - ga) % NBUF.  While group s
  // is multiplied, its packed operands and scales are in registers; stage s+1 has landed and
  // each wave reads it into the registers that group s's decode has just freed; the copies of
  // stages s+2 .. s+NBUF are in flight (stage s+NBUF issued at the start of group s, into the
  // buffer stage s came from).  The one barrier per group comes after this wave's copy of stage
  // s+2 has landed and its reads of stage s+1 have completed: after it stage s+2 is visible to
  // all and the buffer of stage s+1 may be refilled.  Scales travel with their stage: the scale
  // of stage t is loaded into sreg[(t - ga) % NBUF] just before stage t's copy is issued, and
  // written to LDS at the start of group t-2 (its buffer's previous stage was read during group
  // t-NBUF-1; loads complete in order, so waiting for that scale waits only for the copies of
  // stages up to t-1, which the ring needs by then anyway).
  constexpr int kPerStage = 2 * T::kDma + (kAcc ? 0 : T::kSPT);   // vector-memory operations per stage
  constexpr int kInFlight = (NBUF - 2) * kPerStage;         // at most this many once stage s+2 landed
  static_assert(kInFlight <= 63, "vmcnt range");
  uint16_t sreg[NBUF][T::kSPT];
  auto scale_load = [&](int q, int stage) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < T::kSPT; ++u) sreg[q][u] = load_scale(ad, stage, G, M, N, u);
  };
  auto scale_store = [&](int q) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < T::kSPT; ++u) LS(q)[vtid + u * T::kThreads] = scale_operand(sreg[q][u]);
  };
#pragma unroll
  for (int q = 0; q < NBUF; ++q) {
    if (!kAcc) scale_load(q, ga + q);
    __builtin_amdgcn_sched_barrier(0);
    dma_stage(ad, LA(q), LB(q), min(ga + q, G));
    __builtin_amdgcn_sched_barrier(0);
  }
  if (!kAcc) {
    scale_store(0);
    scale_store(1);
  }
  __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(kInFlight));   // stages ga and ga+1 have landed
  ring_barrier();
  v8i pa[T::kTM], pb[T::kTN];
  h4 sa[T::kTM], sb[T::kTN];
  if (!kAcc) read_scales(LS(0), sa, sb);
  read_packed(LA(0), LB(0), pa, pb);
  __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(63));             // buffer 0 read by this wave
  ring_barrier();                                              // ... and by all: it may be refilled

  // INT4 group s in ring position P (stage s in buffer P).  A wave issues in order and stalls
  // on an instruction whose operand an MFMA still computes, so each group is laid out as six
  // slots per tile row i, each one MFMA followed by vector work that does not depend on the
  // MFMAs in flight:
  //   1  scale product (i, 0)      decode A row i, first half (i = 0: and B column 0, first half)
  //   2  tile (i, 0), K 0..63      decode A row i, second half (i = 0: B column 0, second half);
  //                                read the next stage's B column 0 (i = 0)
  //   3  tile (i, 0), K 64..127    apply tile (i-1, 1) (i > 0); read the next stage's A row i
  //   4  scale product (i, 1)      decode B column 1 and read the next stage's (i = 0)
  //   5  tile (i, 1), K 0..63      apply tile (i, 0), first half
  //   6  tile (i, 1), K 64..127    apply tile (i, 0), second half; after the last row, read
  //                                the next stage's scales
  // An apply thus follows at least two MFMAs that do not feed it.  The group's last tile is
  // applied after the barrier, by which time its MFMAs have finished.  Each slot is a
  // scheduling region whose MFMA is pinned ahead of its vector work.  (Against the previous
  // two-region layout, whose scheduler put each apply right behind the MFMA feeding it, this
  // raises the cycles in which MFMA and vector work overlap by a third; the time of a whole
  // Llama-7B layer changes by about 1%, since the chip runs these shapes at its power limit.)
  static_assert(T::kTN == 2, "tile rows are processed as pairs of 32x32 tiles");
  // Fair turns (kFair: a grid of one round with two workgroups on some compute units).  A SIMD
  // issues the older of two ready waves first, so of two workgroups sharing a compute unit the
  // one dispatched first runs ahead and the other finishes alone.  Workgroups b and
  // b + fair_cus (the first and second on a compute unit) instead take the higher priority in
  // turns, by a bit of the real-time clock read at the start of each group and applied after
  // its barrier.
  const uint32_t fair_parity = kFair ? (blockIdx.x / (unsigned)fair_cus) & 1u : 0u;
  auto int4_group = [&](auto ring, int s) __attribute__((always_inline)) {
    constexpr int p = decltype(ring)::kCur, pn = decltype(ring)::kNext, p2 = decltype(ring)::kAfterNext;
    const uint32_t tnow = kFair ? (uint32_t)__builtin_amdgcn_s_memrealtime() : 0u;
    // scale of stage s+2 into its buffer (read during group s+1)
    if (!kAcc) scale_store(p2);
    // refill buffer p (stage s was read during group s-1, before the last barrier)
    if (!kAcc) scale_load(p, s + NBUF);
    __builtin_amdgcn_sched_barrier(0);
    dma_stage(ad, LA(p), LB(p), min(s + NBUF, G));            // past the row end: unused
    __builtin_amdgcn_sched_barrier(0);
    h4 san[T::kTM], sbn[T::kTN];
    v8i b0[2], b1[2];                                          // fp6 operands of the B columns
    v16f acc1, sp1;
#pragma unroll
    for (int i = 0; i < T::kTM; ++i) {
      v8i a0, a1;
      v16f acc0, sp0;
      sp0 = scale_product(sa[i], sb[0]);
      a0 = fp6_operand(pa[i], 0);
      if (i == 0) b0[0] = fp6_operand(pb[0], 0);
      ATOM_SLOT(16, 0);
      acc0 = mma_fp6(a0, b0[0], v16f{});
      a1 = fp6_operand(pa[i], 1);
      if (i == 0) {
        b1[0] = fp6_operand(pb[0], 1);
        pb[0] = read_b(LB(pn), 0);
      }
      ATOM_SLOT(16, 2);
      acc0 = mma_fp6(a1, b1[0], acc0);
      if (i > 0) apply(i - 1, 1, acc1, sp1, s);
      pa[i] = read_a(LA(pn), i);
      ATOM_SLOT(16, 2);
      sp1 = scale_product(sa[i], sb[1]);
      if (i == 0) {
        b0[1] = fp6_operand(pb[1], 0);
        b1[1] = fp6_operand(pb[1], 1);
        pb[1] = read_b(LB(pn), 1);
      }
      ATOM_SLOT(16, 2);
      acc1 = mma_fp6(a0, b0[1], v16f{});
#pragma unroll
      for (int r = 0; r < 8; ++r) apply_element(i, 0, acc0, sp0, s, r);
      ATOM_SLOT(8, 0);
      acc1 = mma_fp6(a1, b1[1], acc1);
#pragma unroll
      for (int r = 8; r < 16; ++r) apply_element(i, 0, acc0, sp0, s, r);
      if (i == T::kTM - 1 && !kAcc) read_scales(LS(pn), san, sbn);   // this group's are all used
      ATOM_SLOT(8, 4);
    }
    __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(kInFlight));   // own copy of stage s+2 landed, reads done
    ring_barrier();
    // the second workgroup on the compute unit takes 2 on its turn and 1 off it, the first 1 and
    // 0: where their clock reads straddle a turn, the second wins the tie the older would win
    // (event-timed 2048 x 11008 x 4096, four alternating pairs: 83.4-83.9 -> 82.9-83.3 us)
    if constexpr (kFair) set_priority_0_to_2((((tnow >> kFairBit) ^ fair_parity) & 1u) + fair_parity);
    apply(T::kTM - 1, 1, acc1, sp1, s);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < T::kTM; ++i) sa[i] = san[i];
#pragma unroll
    for (int j = 0; j < T::kTN; ++j) sb[j] = sbn[j];
  };
  {
    int s = ga;
    for (; s + NBUF <= gb; s += NBUF) ring_turn<0, NBUF>(int4_group, s);
    ring_tail<0, NBUF>(int4_group, s, gb);
    if constexpr (SUB > 1 && T::kWaves > 1)   // parts get floor or ceil of (G-1)/SUB groups
      if (gb - ga < (G - 1 + SUB - 1) / SUB) wg_barrier();
  }

  // INT8 outlier group: stage G-1 (its packed operands are in pa / pb, the group's scales in
  // sa / sb) and stage G (landed in buffer (G - ga) % 3), each two K=32 int8 MFMAs per tile.
  if (last_split) {
    v16i acc[T::kTM][T::kTN];
    auto lo = [](v8i v) { return v4i{v[0], v[1], v[2], v[3]}; };
    auto hi = [](v8i v) { return v4i{v[4], v[5], v[6], v[7]}; };
#pragma unroll
    for (int i = 0; i < T::kTM; ++i)
#pragma unroll
      for (int j = 0; j < T::kTN; ++j) {
        acc[i][j] = mma_i8(lo(pa[i]), lo(pb[j]), v16i{});
        acc[i][j] = mma_i8(hi(pa[i]), hi(pb[j]), acc[i][j]);
      }
    const int pg = (G - ga) % NBUF;                 // stage G's buffer
#pragma unroll
    for (int q = 0; q < NBUF; ++q)
      if (pg == q) read_packed(LA(q), LB(q), pa, pb);
#pragma unroll
    for (int i = 0; i < T::kTM; ++i)
#pragma unroll
      for (int j = 0; j < T::kTN; ++j) {
        acc[i][j] = mma_i8(lo(pa[i]), lo(pb[j]), acc[i][j]);
        acc[i][j] = mma_i8(hi(pa[i]), hi(pb[j]), acc[i][j]);
        v16f accf;
#pragma unroll
        for (int r = 0; r < 16; ++r) accf[r] = (float)acc[i][j][r];   // |acc| <= 128*127*127 < 2^24: exact
        finish_tile(i, j, accf, sa[i], sb[j], G - 1);
      }
  }
  __builtin_amdgcn_s_waitcnt(0);                    // no copy into LDS outlives the workgroup

  // K parts: part v's partial of MFMA tile t goes to slot t of region v (stage buffer A v, or
  // B v - NBUF), 16 floats per lane in the accumulator layout; the wave of part t then adds
  // the SUB partials of tile t in part order, so the sum does not depend on timing.
  if constexpr (SUB > 1) {
    auto region = [&](int v) -> float* {   // v must fold to a constant: only buffers < NBUF exist
      return reinterpret_cast<float*>(v < NBUF ? LA0(v) : LB0(v - NBUF));
    };
    constexpr int kRegions = SUB * T::kWaves;     // one per wave of the workgroup
    const int me = sub * T::kWaves + wave;
    float* mine = nullptr;
#pragma unroll
    for (int v = 0; v < kRegions; ++v)
      if (v == me) mine = region(v);
    __syncthreads();                                  // every part is done with the stage buffers
#pragma unroll
    for (int i = 0; i < T::kTM; ++i)
#pragma unroll
      for (int j = 0; j < T::kTN; ++j) {
        float* d = mine + ((i * T::kTN + j) * 64 + lane) * 16;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<float4*>(d + 4 * q) =
              float4{yacc[i][j][4 * q], yacc[i][j][4 * q + 1], yacc[i][j][4 * q + 2], yacc[i][j][4 * q + 3]};
      }
    __syncthreads();
    v16f sum;
    if (sub < T::kTM * T::kTN) {
#pragma unroll
    for (int v = 0; v < SUB; ++v) {
      // the same wave position in part v (a compile-time region for each wave position)
      const float* src = nullptr;
#pragma unroll
      for (int w = 0; w < T::kWaves; ++w)
        if (w == wave) src = region(v * T::kWaves + w);
      src += (sub * 64 + lane) * 16;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 x = *reinterpret_cast<const float4*>(src + 4 * q);
        if (v == 0) {
          sum[4 * q] = x.x; sum[4 * q + 1] = x.y; sum[4 * q + 2] = x.z; sum[4 * q + 3] = x.w;
        } else {
          sum[4 * q] += x.x; sum[4 * q + 1] += x.y; sum[4 * q + 2] += x.z; sum[4 * q + 3] += x.w;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < T::kTM; ++i)
#pragma unroll
      for (int j = 0; j < T::kTN; ++j)
        if (i * T::kTN + j == sub) yacc[i][j] = sum;
    }
  }
  // the MFMA tiles this wave stores (all of them, or with K parts the one it added up)
  auto owns = [&](int i, int j) { return SUB == 1 || i * T::kTN + j == sub; };

  // Store.  Each lane writes four runs of four consecutive outputs per tile.  A split piece
  // writes its whole fp32 tile (16-byte stores; rows and columns past Y land in the piece's
  // own scratch tile and are never read).  A whole tile writes Y with 8-byte fp16 stores when
  // it lies inside Y and every row start is 8-byte aligned (N % 4 == 0), element by element
  // otherwise.
  if (!kAcc) {
    if (is_piece) {
      float* tile = part + ((size_t)split * rem + (lin - full)) * (BM * BN);
#pragma unroll
      for (int i = 0; i < T::kTM; ++i) {
        const int r = wm * T::kWTM + i * 32 + acc_row(lane);
#pragma unroll
        for (int j = 0; j < T::kTN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int c = wn * T::kWTN + j * 32 + acc_col(lane, q);
            *reinterpret_cast<float4*>(tile + r * BN + c) =
                float4{yacc[i][j][4 * q], yacc[i][j][4 * q + 1], yacc[i][j][4 * q + 2], yacc[i][j][4 * q + 3]};
          }
      }
    } else if (m0 + BM <= M && n0 + BN <= N && (N & 3) == 0) {   // uniform
#pragma unroll
      for (int i = 0; i < T::kTM; ++i) {
        const size_t m = (size_t)(m0 + wm * T::kWTM + i * 32 + acc_row(lane));
#pragma unroll
        for (int j = 0; j < T::kTN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (!owns(i, j)) continue;
            const int n = n0 + wn * T::kWTN + j * 32 + acc_col(lane, q);
            ushort4 o;
            o.x = __half_as_ushort(__float2half_rn(0.5f * yacc[i][j][4 * q]));
            o.y = __half_as_ushort(__float2half_rn(0.5f * yacc[i][j][4 * q + 1]));
            o.z = __half_as_ushort(__float2half_rn(0.5f * yacc[i][j][4 * q + 2]));
            o.w = __half_as_ushort(__float2half_rn(0.5f * yacc[i][j][4 * q + 3]));
            *reinterpret_cast<ushort4*>(Y + m * N + n) = o;
          }
      }
    } else {
#pragma unroll
      for (int i = 0; i < T::kTM; ++i)
#pragma unroll
        for (int j = 0; j < T::kTN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int m = m0 + wm * T::kWTM + i * 32 + acc_row(lane);
            const int n = n0 + wn * T::kWTN + j * 32 + acc_col(lane, r >> 2) + (r & 3);
            if (owns(i, j) && m < M && n < N) Y[(size_t)m * N + n] = __half_as_ushort(__float2half_rn(0.5f * yacc[i][j][r]));
          }
    }
  }
}

// The tiled GEMM: one workgroup per output tile or split-K piece.
template <int BM, int BN, int WAVES_M, int WAVES_N, int NBUF, bool kAcc, bool kFair = false>
__global__ __launch_bounds__(WAVES_M* WAVES_N * 64) __attribute__((amdgpu_waves_per_eu(kAcc ? 1 : 2))) void gemm_w4a4_kernel(
    const uint8_t* __restrict__ Xq, const uint16_t* __restrict__ sx, const uint8_t* __restrict__ Wq,
    const uint16_t* __restrict__ sw, int M, int N, int K, uint16_t* __restrict__ Y, int32_t* __restrict__ acc_out,
    int full, int rem, int splits, float* __restrict__ part, int fair_cus, int late_from) {
  // Workgroups of later rounds (id >= late_from) issue at priority 1: a late tile shares its
  // compute unit with a partner already part way through, and should not wait behind it (the
  // older wave wins otherwise), so the two finish closer together.  1024 x 4096 x 11008 (688
  // tiles for 512 slots, event-timed): 60.6-61.3 -> 59.7-60.0 us.
  if (!kFair) set_priority_from_bit0((uint32_t)__builtin_amdgcn_readfirstlane((int)blockIdx.x >= late_from ? 1 : 0));
  // Work assignment.  Workgroups go to the 8 XCDs round-robin by id.  Each XCD gets an equal
  // share of the split pieces followed by an equal share of the whole tiles, each share a
  // contiguous run in tile order (so an XCD's L2 sees a compact block of X and W), and the
  // pieces are dispatched first so that the whole tiles fill in behind them.
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const int npieces = rem * splits;
  const int nblocks = full + npieces;
  const int xcd = blockIdx.x % kXcds, local = blockIdx.x / kXcds;
  const int qb = nblocks / kXcds, rb = nblocks % kXcds;   // workgroups on XCD x: qb + (x < rb)
  const int qp = npieces / kXcds, rp = npieces % kXcds;   // pieces on XCD x: qp + (x < rp)
  const int px = qp + (xcd < rp ? 1 : 0);
  const int pbase = xcd * qp + min(xcd, rp);
  int lin, split = 0, nsplit = 1;
  if (local < px) {
    const int piece = pbase + local;
    lin = full + piece % rem;
    split = piece / rem;
    nsplit = splits;
  } else {
    lin = (xcd * qb + min(xcd, rb)) - pbase + (local - px);
  }
  gemm_tile<BM, BN, WAVES_M, WAVES_N, NBUF, kAcc, 1, kFair>(Xq, sx, Wq, sw, M, N, K, Y, acc_out, lin, split, nsplit,
                                                            full, rem, part, fair_cus);
}

// One 64 x 64 output tile per workgroup of SUB K parts of WM x WN waves (see gemm_tile), for
// grids that have too few tiles to give every SIMD a wave otherwise.
template <int BM, int WM, int WN, int SUB, int NBUF>
__global__ __launch_bounds__(SUB * WM * WN * 64) __attribute__((amdgpu_waves_per_eu(2))) void gemm_w4a4_kpart_kernel(
    const uint8_t* __restrict__ Xq, const uint16_t* __restrict__ sx, const uint8_t* __restrict__ Wq,
    const uint16_t* __restrict__ sw, int M, int N, int K, uint16_t* __restrict__ Y, int tiles) {
  // whole tiles only: XCD x takes a contiguous run of the tile order (as gemm_w4a4_kernel does)
  const int xcd = blockIdx.x % kXcds, local = blockIdx.x / kXcds;
  const int qb = tiles / kXcds, rb = tiles % kXcds;
  const int lin = xcd * qb + min(xcd, rb) + local;
  gemm_tile<BM, BM, WM, WN, NBUF, false, SUB>(Xq, sx, Wq, sw, M, N, K, Y, nullptr, lin, 0, 1, tiles, 0, nullptr);
}

// 128 x 128 workgroup tile, 2 x 2 waves of 64 x 64 (2 x 2 MFMA tiles of 32 x 32 each).
constexpr int kBM = 128, kBN = 128, kWavesM = 2, kWavesN = 2, kRing = 3;
// Split-K.  Grids of fewer than kSplitMinTiles tiles split every tile, aiming at about one
// workgroup per compute unit; a piece keeps at least kSplitMinGroups INT4 groups.  Larger
// grids are not split, not even a last partial round of tiles: with every compute unit busy
// the chip runs at its power limit, so spreading a tail lowers the clock about as much as it
// adds parallelism, and the partial sums and the second kernel are pure cost (measured:
// 1024 x 4096 x 11008 with its last 176 of 688 tiles split in two spans the same time, and
// 600 x 2048 x 15300 with 88 of 600 split three ways is slower).
constexpr int kSplitMinTiles = 128, kSplitTargetBlocks = 256, kSplitMinGroups = 4, kSplitMax = 8;
// 64 x 64 output tiles, two waves of 32 x 64 (one 32 x 32 MFMA tile row, two columns): for grids
// with fewer than kSplitMinTiles tiles of 128 x 128 but at least k64MinTiles of 64 x 64 that
// are too short for K parts (below), whole small tiles replace split-K (no partial sums, no
// second kernel, no scratch).  Measured on 256 x 4096 x 4096 (kernel trace): 16.0 us against
// 19.9 us for four split-K pieces of 128 x 128 plus 4.4 us for their finalize kernel.  A deeper
// ring helps neither these tiles (event-timed: 3 or 4 buffers 18.3 us, 6 buffers 21.5 us, 8
// buffers 22.2 us) nor the K parts (3 buffers 14.4 us, 4 buffers 14.6 us, four parts of four
// buffers 14.7 us), so they keep three.  The group accumulators of both run on these tiles.
constexpr int k64 = 64, k64WavesM = 2, k64WavesN = 1, k64Ring = 3, k64MinTiles = 192;
// K parts: 64 x 64 tiles, two parts of two waves of 32 x 64 each taking half of the groups
// (gemm_w4a4_kpart_kernel).  Grids of fewer than kSplitMinTiles tiles of 128 x 128 take them
// when they have at least kPartTiles tiles of 64 x 64, or at least kPartMinTiles and no more
// than kPartMaxGroups groups; otherwise split-K (more workgroups on a long K).  Measured
// (kernel trace, split-K time including its finalize): 256x4096x4096 15.7 (whole 64 x 64
// tiles) -> 12.7 us; 128x4096x4096 20.4 -> 12.0; 64x4096x4096 16.8 -> 11.6; 33x4096x8448
// 21.6 -> 12.4; 64x4096x11008 21.9 -> 12.1; 17x32768x10753 64.4 -> 58.5; but 64x11008x4096
// (64 tiles, 86 groups) 20.0 with split-K against 22.8.
constexpr int kParts = 2, kPartMinGroups = 2 * kParts, kPartTiles = 128, kPartMinTiles = 64, kPartMaxGroups = 48;

// Y of the split tiles = fp16(0.5 * sum over pieces of the partial tiles), pieces added in
// order.  blockIdx.y = split tile (tile full + blockIdx.y in tile order); four consecutive
// outputs of one tile row per thread.  The piece count S is a template argument so that all S
// loads are in flight before the first add: with a run-time count the loop waits for each load
// in turn (64 x 4096 x 4096, seven pieces: the GEMM call takes 14.5 us instead of 19.6 us).
template <int S>
__global__ __launch_bounds__(256) void gemm_splitk_finish_kernel(const float* __restrict__ part, int full, int rem,
                                                                 int M, int N, uint16_t* __restrict__ Y) {
  const int t = blockIdx.y;
  const int e = (blockIdx.x * 256 + threadIdx.x) * 4;       // element of the tile, < kBM * kBN
  const int tiles_m = (M + kBM - 1) / kBM, tiles_n = (N + kBN - 1) / kBN;
  const int2 tc = tile_coords(full + t, tiles_m, tiles_n);
  const int m = tc.x * kBM + e / kBN, n = tc.y * kBN + e % kBN;
  const float* src = part + (size_t)t * (kBM * kBN) + e;
  float4 v[S];
#pragma unroll
  for (int k = 0; k < S; ++k) v[k] = *reinterpret_cast<const float4*>(src + (size_t)k * rem * (kBM * kBN));
  float4 acc = v[0];
#pragma unroll
  for (int k = 1; k < S; ++k) {
    acc.x += v[k].x;
    acc.y += v[k].y;
    acc.z += v[k].z;
    acc.w += v[k].w;
  }
  if (m >= M) return;
  const uint16_t o[4] = {__half_as_ushort(__float2half_rn(0.5f * acc.x)), __half_as_ushort(__float2half_rn(0.5f * acc.y)),
                         __half_as_ushort(__float2half_rn(0.5f * acc.z)), __half_as_ushort(__float2half_rn(0.5f * acc.w))};
  uint16_t* dst = Y + (size_t)m * N + n;
  if (n + 4 <= N && (N & 3) == 0) {
    *reinterpret_cast<ushort4*>(dst) = ushort4{o[0], o[1], o[2], o[3]};
  } else {
    for (int i = 0; i < 4; ++i)
      if (n + i < N) dst[i] = o[i];
  }
}


// ---------------------------------------------------------------------------------------------
// Activation quantize and GEMM in one persistent launch.
//
// One workgroup per resident slot.  Each first quantizes its own few token rows (exactly as
// atom_quantize_act does, into Xq / sx), makes those stores visible at device scope and adds
// their count to the ready count of their 64-row block (release).  Then it runs its share of
// the 128 x 128 output tiles (the tiled GEMM's own XCD-aware order: each XCD takes a contiguous
// run of tiles, its workgroups interleaved over the run), and before each tile waits until the
// tile's row blocks are complete (acquire).  No workgroup waits before it has quantized its
// rows, so with every workgroup resident (the grid is the resident count for an otherwise idle
// GPU) every wait ends.  The wait is bounded all the same: one that gives up sets the
// workspace's timeout flag and the workgroup goes on (the outputs are then not valid).  Leaving,
// each workgroup counts itself on its XCD's exit counter; the last of an XCD counts the XCD on
// the global one, and the last XCD resets every count, so the workspace is zero again for the
// next call (and for a graph replay) without a memset.  Work items come from no shared queue:
// device-scope atomics on one address serialize across the XCDs (a queue item per tile and row
// group made the launch 2.5x slower than the two separate kernels).
//
// Workspace (int32 words, zero before the first call and after every call):
//   [0] XCDs done, [1 .. 8] workgroups done per XCD, [9] timeout flag (sticky: set by a wait
//   that gave up, never cleared by the kernel), [10] wait limit (0: default; > 0: that many
//   polls; < 0: every wait gives up at once, a forced failure that exercises the flag),
//   [16 + b] rows of 64-row block b quantized.
constexpr int kLinXcdsDone = 0, kLinXcdDone = 1, kLinTimeout = 9, kLinWaitLimit = 10, kLinBlocks = 16;
constexpr int kLinBlockRows = 64;
constexpr int kLinDefaultPolls = 1 << 20;

__device__ __forceinline__ int lin_load_acquire(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
}

template <int CHUNKS, int PASSES>
__global__ __launch_bounds__(kBM * 2) __attribute__((amdgpu_waves_per_eu(2))) void linear_fused_kernel(
    const uint16_t* __restrict__ X, const int32_t* __restrict__ perm, const uint8_t* __restrict__ Wq,
    const uint16_t* __restrict__ sw, int M, int N, int K, uint8_t* __restrict__ Xq, uint16_t* __restrict__ sx,
    uint16_t* __restrict__ Y, int* __restrict__ ws, int rows_per_wg) {
  static_assert(kBM + kBN == rowq::kThreads, "the GEMM tile's threads are the row quantizer's");
  __shared__ __attribute__((aligned(16))) uint32_t qlds[rowq::staged_stride(CHUNKS * 8 * rowq::kThreads) * 8];
  const int nwg = gridDim.x, b = blockIdx.x;

  // ---- this workgroup's token rows [r0, r1) (rows_per_wg is a power of two: inside one 64-row
  // block, or whole blocks)
  const int r0 = (int)min((long long)b * rows_per_wg, (long long)M), r1 = min(r0 + rows_per_wg, M);
  if (r0 < r1) {
    rowq::RowQuant<CHUNKS, PASSES, kRowW4A4> rq(X, perm, M, K, Xq, sx, qlds);
    rq.load_perm();
    rq.prefetch(r0);
    rq.finish_offsets();
    for (int r = r0; r < r1; ++r) {
      __syncthreads();                               // everyone finished reading the previous row
      rq.stage();
      __syncthreads();
      if (r + 1 < r1) rq.prefetch(r + 1);
      rq.quantize(r, 0, 1);
    }
    // every wave's code and scale stores complete and visible at device scope, then the rows
    // are counted
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    if (threadIdx.x == 0)
      for (int blk = r0 / kLinBlockRows; blk * kLinBlockRows < r1; ++blk)
        __hip_atomic_fetch_add(ws + kLinBlocks + blk, min(r1, (blk + 1) * kLinBlockRows) - max(r0, blk * kLinBlockRows),
                               __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  }

  // ---- this workgroup's tiles: XCD x (workgroups b = x, x + 8, ...) takes a contiguous run of
  // the tile order, its workgroups interleaved over it
  const int tiles_m = (M + kBM - 1) / kBM, tiles_n = (N + kBN - 1) / kBN, tiles = tiles_m * tiles_n;
  const int xcd = b % kXcds, local = b / kXcds;
  const int nx = (nwg - xcd + kXcds - 1) / kXcds;                  // workgroups on this XCD
  const int qt = tiles / kXcds, rt = tiles % kXcds;
  const int t0 = xcd * qt + min(xcd, rt), t1 = t0 + qt + (xcd < rt ? 1 : 0);
  const int limit_word = ws[kLinWaitLimit];
  const int limit = limit_word > 0 ? limit_word : kLinDefaultPolls;
  for (int lin = t0 + local; lin < t1; lin += nx) {
    const int2 tc = tile_coords(lin, tiles_m, tiles_n);
    if (threadIdx.x == 0) {
      const int m0 = tc.x * kBM, m1 = min(m0 + kBM, M);
      if (limit_word < 0) __hip_atomic_store(ws + kLinTimeout, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      for (int blk = m0 / kLinBlockRows; limit_word >= 0 && blk * kLinBlockRows < m1; ++blk) {
        const int want = min(kLinBlockRows, M - blk * kLinBlockRows);
        int polls = 0;
        while (lin_load_acquire(ws + kLinBlocks + blk) < want) {
          if (++polls > limit) {
            __hip_atomic_store(ws + kLinTimeout, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
          }
          __builtin_amdgcn_s_sleep(2);
        }
      }
    }
    __syncthreads();                                 // the tile's rows are visible to every wave (and
                                                     // the previous tile's LDS is free)
    gemm_tile<kBM, kBN, kWavesM, kWavesN, kRing, false>(Xq, sx, Wq, sw, M, N, K, Y, nullptr, lin, 0, 1, tiles, 0,
                                                        nullptr);
  }

  // ---- leave: the last workgroup of the last XCD resets every count for the next call
  if (threadIdx.x == 0) {
    const int xcds = min(nwg, kXcds);
    const int done = __hip_atomic_fetch_add(ws + kLinXcdDone + xcd, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if (done == nx - 1 &&
        __hip_atomic_fetch_add(ws + kLinXcdsDone, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) == xcds - 1) {
      const int nblocks = (M + kLinBlockRows - 1) / kLinBlockRows;
      for (int blk = 0; blk < nblocks; ++blk)
        __hip_atomic_store(ws + kLinBlocks + blk, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      for (int x = 0; x < kXcds; ++x) __hip_atomic_store(ws + kLinXcdDone + x, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(ws + kLinXcdsDone, 0, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

template <int CHUNKS, int PASSES>
hipError_t launch_linear_fused_inst(const uint16_t* X, const int32_t* perm, const uint8_t* Wq, const uint16_t* sw,
                                    int M, int N, int K, uint8_t* Xq, uint16_t* sx, uint16_t* Y, int* ws,
                                    hipStream_t stream) {
  // persistent: as many workgroups as are resident at once (queried once per process and
  // instantiation on the device current at the first call)
  static const int resident = [] {
    int dev = 0, cus = 256, per_cu = 2;
    if (hipGetDevice(&dev) == hipSuccess) {
      int n = 0;
      if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0) cus = n;
    }
    int b = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, linear_fused_kernel<CHUNKS, PASSES>, kBM * 2, 0) ==
            hipSuccess && b > 0)
      per_cu = b;
    return cus * per_cu;
  }();
  // rows per workgroup: the least power of two that gives every row a workgroup; the grid is the
  // resident count, fewer when there are fewer rows and tiles
  const int tiles = ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
  int rpw = 1;
  while ((long long)rpw * resident < M) rpw *= 2;
  const int grid = min(resident, max((M + rpw - 1) / rpw, tiles));
  hipLaunchKernelGGL((linear_fused_kernel<CHUNKS, PASSES>), dim3(grid), dim3(kBM * 2), 0, stream, X, perm, Wq, sw, M,
                     N, K, Xq, sx, Y, ws, rpw);
  return hipGetLastError();
}

// Split-K scratch for callers that cannot allocate (atom_gemm_noalloc): the largest split plan
// of any valid shape needs 315 partial tiles of 64 KiB (63 tiles in 5 pieces, e.g. M = 17,
// N = 8000, K = 32768; a split grid has at most 64 tiles when M <= 64 and 32 otherwise, since
// grids of 128 tiles of 64 x 64 or more take K parts), so 384 tiles cover every shape.  Each GPU the library runs on holds its own copy until the
// process ends.  In host code this name is not a device address: the address comes from
// hipGetSymbolAddress, per device.
constexpr size_t kStaticScratchBytes = (size_t)384 * kBM * kBN * sizeof(float);   // 24 MiB
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

}  // namespace

GemmPlan gemm_plan(int M, int N, int K) {
  if (M <= kSmallMaxM) return GemmPlan{0, 0, 1, 1, 0};
  const int tiles = ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
  const int tiles64 = ((M + k64 - 1) / k64) * ((N + k64 - 1) / k64);
  const int G = K / ATOM_GROUP;
  if (tiles < kSplitMinTiles && G - 1 >= kPartMinGroups &&
      (tiles64 >= kPartTiles || (tiles64 >= kPartMinTiles && G <= kPartMaxGroups)))
    return GemmPlan{tiles64, 0, 1, 0, 0, 1};
  if (tiles < kSplitMinTiles && tiles64 >= k64MinTiles) return GemmPlan{tiles64, 0, 1, 0, 1};
  return gemm_plan_tiled(M, N, K);
}

GemmPlan gemm_plan_tiled(int M, int N, int K) {
  const int tiles = ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
  const int G = K / ATOM_GROUP;
  if (tiles >= kSplitMinTiles) return GemmPlan{tiles, 0, 1, 0, 0};
  const int s = min(min((kSplitTargetBlocks + tiles - 1) / tiles, (G - 1) / kSplitMinGroups), kSplitMax);
  return s < 2 ? GemmPlan{tiles, 0, 1, 0, 0} : GemmPlan{0, tiles, s, 0, 0};
}

int64_t gemm_workspace_bytes(const GemmPlan& plan) {
  if (plan.small || plan.tile64 || plan.kpart) return 0;
  return plan.rem > 0 ? (int64_t)plan.rem * plan.splits * kBM * kBN * (int64_t)sizeof(float) : 0;
}

// Compute units of the device current at the first call (queried once per process; the
// initialisation of a function-local static is thread-safe).  256 if the query fails.
int compute_units() {
  static const int cus = [] {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        n > 0)
      return n;
    return 256;
  }();
  return cus;
}

hipError_t launch_gemm(const uint8_t* Xq, const uint16_t* sx, const uint8_t* Wq, const uint16_t* sw, int M, int N,
                       int K, uint16_t* Y, float* part, const GemmPlan& plan, hipStream_t stream) {
  if (plan.small) return launch_gemm_small(Xq, sx, Wq, sw, M, N, K, Y, stream);
  if (plan.kpart) {
    if (plan.rem != 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm_w4a4_kpart_kernel<k64, k64WavesM, k64WavesN, kParts, k64Ring>), dim3(plan.full),
                       dim3(kParts * k64WavesM * k64WavesN * 64), 0, stream,
                       Xq, sx, Wq, sw, M, N, K, Y, plan.full);
    return hipGetLastError();
  }
  if (plan.tile64) {
    if (plan.rem != 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm_w4a4_kernel<k64, k64, k64WavesM, k64WavesN, k64Ring, false>), dim3(plan.full),
                       dim3(k64WavesM * k64WavesN * 64), 0, stream, Xq, sx, Wq, sw, M, N, K, Y, (int32_t*)nullptr,
                       plan.full, 0, 1, (float*)nullptr, 0, plan.full);
    return hipGetLastError();
  }
  if (plan.rem > 0 && (plan.splits < 2 || plan.splits > kSplitMax)) return hipErrorInvalidValue;
  const int blocks = plan.full + plan.rem * plan.splits;
  // Fair turns (a kernel of their own) for a grid of one round: at most two workgroups on every
  // compute unit, some with two.  With more rounds an early finish lets a later tile start
  // sooner, which is worth more.  Event-timed, 2048 x 11008 x 4096 (512 tiles on 256 compute
  // units): 87.1 -> 85.2 us; 1024 x 4096 x 11008 (688 tiles) ran 60.3 -> 61.7 us with them.
  const int cus = compute_units();
  if (blocks > cus && blocks <= 2 * cus)
    hipLaunchKernelGGL((gemm_w4a4_kernel<kBM, kBN, kWavesM, kWavesN, kRing, false, true>), dim3(blocks),
                       dim3(kWavesM * kWavesN * 64), 0, stream, Xq, sx, Wq, sw, M, N, K, Y, (int32_t*)nullptr,
                       plan.full, plan.rem, plan.splits, part, cus, blocks);
  else
    hipLaunchKernelGGL((gemm_w4a4_kernel<kBM, kBN, kWavesM, kWavesN, kRing, false>), dim3(blocks),
                       dim3(kWavesM * kWavesN * 64), 0, stream, Xq, sx, Wq, sw, M, N, K, Y, (int32_t*)nullptr,
                       plan.full, plan.rem, plan.splits, part, 0, blocks > 2 * cus ? 2 * cus : blocks);
  if (plan.rem > 0) return launch_splitk_finish(part, plan, M, N, Y, stream);
  return hipGetLastError();
}

hipError_t launch_splitk_finish(const float* part, const GemmPlan& plan, int M, int N, uint16_t* Y,
                                hipStream_t stream) {
  using Finish = void (*)(const float*, int, int, int, int, uint16_t*);
  static constexpr Finish kFinish[kSplitMax + 1] = {
      nullptr, nullptr, gemm_splitk_finish_kernel<2>, gemm_splitk_finish_kernel<3>, gemm_splitk_finish_kernel<4>,
      gemm_splitk_finish_kernel<5>, gemm_splitk_finish_kernel<6>, gemm_splitk_finish_kernel<7>,
      gemm_splitk_finish_kernel<8>};
  if (plan.rem <= 0 || plan.splits < 2 || plan.splits > kSplitMax) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kFinish[plan.splits], dim3(kBM * kBN / 4 / 256, plan.rem), dim3(256), 0, stream, part,
                     plan.full, plan.rem, M, N, Y);
  return hipGetLastError();
}


int64_t linear_fused_workspace_bytes(int M) {
  const int64_t words = kLinBlocks + (M + kLinBlockRows - 1) / kLinBlockRows;
  return (words * 4 + 255) / 256 * 256;
}

bool linear_fused_supported(int M, int N, int K) {
  const GemmPlan plan = gemm_plan(M, N, K);
  return !plan.small && !plan.tile64 && !plan.kpart && plan.rem == 0 && K <= 12288;
}

hipError_t launch_linear_fused(const uint16_t* X, const int32_t* perm, const uint8_t* Wq, const uint16_t* sw, int M,
                               int N, int K, uint8_t* Xq, uint16_t* sx, uint16_t* Y, int* ws, hipStream_t stream) {
  if (!linear_fused_supported(M, N, K)) return hipErrorInvalidValue;
  if (K <= 4096) return launch_linear_fused_inst<2, 1>(X, perm, Wq, sw, M, N, K, Xq, sx, Y, ws, stream);
  if (K <= 8192) return launch_linear_fused_inst<4, 2>(X, perm, Wq, sw, M, N, K, Xq, sx, Y, ws, stream);
  return launch_linear_fused_inst<6, 3>(X, perm, Wq, sw, M, N, K, Xq, sx, Y, ws, stream);
}

int64_t static_scratch_bytes() { return (int64_t)kStaticScratchBytes; }

hipError_t static_scratch_address(void** out) {
  // the device address of `scratch` on the current device, looked up once per device
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

hipError_t launch_gemm_group_acc(const uint8_t* Xq, const uint8_t* Wq, int M, int N, int K, int32_t* acc,
                                 hipStream_t stream) {
  const GemmPlan plan = gemm_plan(M, N, K);
  if (plan.small) return launch_gemm_small_group_acc(Xq, Wq, M, N, K, acc, stream);
  if (plan.tile64 || plan.kpart) {   // the same 64 x 64 tiles, one workgroup of two waves each
    hipLaunchKernelGGL((gemm_w4a4_kernel<k64, k64, k64WavesM, k64WavesN, k64Ring, true>), dim3(plan.full),
                       dim3(k64WavesM * k64WavesN * 64), 0, stream, Xq, (const uint16_t*)nullptr, Wq,
                       (const uint16_t*)nullptr, M, N, K, (uint16_t*)nullptr, acc, plan.full, 0, 1, (float*)nullptr,
                       0, plan.full);
    return hipGetLastError();
  }
  const dim3 grid(((N + kBN - 1) / kBN) * ((M + kBM - 1) / kBM));
  hipLaunchKernelGGL((gemm_w4a4_kernel<kBM, kBN, kWavesM, kWavesN, kRing, true>), grid, dim3(kWavesM * kWavesN * 64), 0,
                     stream, Xq, (const uint16_t*)nullptr, Wq, (const uint16_t*)nullptr, M, N, K,
                     (uint16_t*)nullptr, acc, (int)grid.x, 0, 1, (float*)nullptr, 0, (int)grid.x);
  return hipGetLastError();
}

}  // namespace atom
