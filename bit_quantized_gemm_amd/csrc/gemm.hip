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

#include "atom_internal.h"

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

__device__ __forceinline__ v16i mma_i8(v4i a, v4i b, v16i c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(b, a, c, 0, 0, 0);
}

// Output row (within a 32x32 tile) and first of four consecutive columns held by element
// group q (elements 4q .. 4q+3) of a lane's accumulator.
__device__ __forceinline__ int acc_row(int lane) { return lane & 31; }
__device__ __forceinline__ int acc_col(int lane, int q) { return q * 8 + (lane >> 5) * 4; }

// Chunk position swizzle of LDS row r (rows are 64 bytes)
__device__ __forceinline__ int chunk_swz(int r) { return (r >> 2) & 3; }

// s_waitcnt immediate (vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8): wait until at
// most n vector-memory operations of this wave are outstanding and all its LDS operations
// have completed.  n = 63 leaves vector memory alone.
constexpr int wait_vm_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4); }

// Workgroup barrier that does not wait for this wave's outstanding vector-memory operations
// (__syncthreads would drain every copy in flight).  The empty asm statements keep the
// compiler from moving memory operations across it; callers wait for what must be complete.
__device__ __forceinline__ void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Compile-time ring position of a stage buffer.
template <int P>
struct Ring {
  static constexpr int kCur = P, kNext = (P + 1) % 3;
};


template <int BM, int BN, int WAVES_M, int WAVES_N>
struct Tile {
  static constexpr int kThreads = WAVES_M * WAVES_N * 64;
  static constexpr int kWTM = BM / WAVES_M;            // wave tile rows
  static constexpr int kWTN = BN / WAVES_N;            // wave tile columns
  static constexpr int kTM = kWTM / 32;                // MFMA tiles per wave (rows)
  static constexpr int kTN = kWTN / 32;                // MFMA tiles per wave (columns)
  static constexpr int kWaves = WAVES_M * WAVES_N;
  static constexpr int kDma = BM / kWaves / 16;        // LDS-DMA instructions per wave per stage and tile
  static_assert(kWTM % 32 == 0 && kWTN % 32 == 0, "wave tile must be a multiple of 32");
  static_assert(BM + BN == kThreads, "one scale per thread per stage");
  static_assert(BM == BN && kDma * kWaves * 16 == BM, "each wave copies whole 16-row slabs of A and B");
};

// Per-thread addressing of the stage copy, fixed for the whole K loop.  Wave w copies tile
// rows [w * BM / W, (w + 1) * BM / W) of A and the same rows of B (W waves), 16 rows per
// LDS-DMA instruction: lane i of instruction h lands at LDS row r = w * BM / W + 16h + i / 4,
// position i % 4, so it loads chunk (i % 4) ^ chunk_swz(r) of that row.  Rows past M / N
// repeat the last valid row.  Thread t < BM carries the activation scale of tile row t,
// thread BM + u the weight scale of tile column u.
template <int NDMA>
struct StageAddr {
  __amdgpu_buffer_rsrc_t a_rsrc, b_rsrc;  // the workgroup's rows of Xq / Wq
  int a_voff[NDMA], b_voff[NDMA];          // byte offset of this lane's chunk in stage 0
  int lds_row0;                            // first LDS row of this wave's copy (wave-uniform)
  const uint16_t* s_src;                   // this thread's scale in group 0
  bool s_is_x;                             // activation (stride M) or weight (stride N) scale
};

// One LDS-DMA instruction: lane i loads 16 bytes at voff + soff of the buffer and writes them
// to lds + 16 i (lds is wave-uniform).  Not a template: the LDS address-space cast exists
// only for the device.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rsrc, uint8_t* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}

// Copy stage s of this wave's rows into LDS (asynchronous; tracked by vmcnt).
template <int NDMA>
__device__ __forceinline__ void dma_stage(const StageAddr<NDMA>& ad, uint8_t* la, uint8_t* lb, int s) {
  const int soff = s * kStageBytes;
#pragma unroll
  for (int h = 0; h < NDMA; ++h) {
    lds_dma16(ad.a_rsrc, la + (ad.lds_row0 + 16 * h) * kLdsRow, ad.a_voff[h], soff);
    lds_dma16(ad.b_rsrc, lb + (ad.lds_row0 + 16 * h) * kLdsRow, ad.b_voff[h], soff);
  }
}

// This thread's scale of stage s (group min(s, G-1): the INT8 group fills two stages).
template <int NDMA>
__device__ __forceinline__ uint16_t load_scale(const StageAddr<NDMA>& ad, int s, int G, int M, int N) {
  const int g = min(s, G - 1);
  const size_t ox = (size_t)g * M, ow = (size_t)g * N;   // uniform
  return ad.s_src[ad.s_is_x ? ox : ow];
}

// kAcc = false: Y output.  kAcc = true: write the per-group integer accumulators instead.
// Split-K (Y output only): the first `full` tiles run whole; the INT4 groups of each of the
// last `rem` tiles are divided among `splits` pieces (the last piece also takes the INT8
// group), each writing its fp32 tile sum, still carrying the factor 2 of the scale
// products, tile-major to part[(piece split * rem + tile - full) * BM * BN].
template <int BM, int BN, int WAVES_M, int WAVES_N, bool kAcc>
__global__ __launch_bounds__(WAVES_M* WAVES_N * 64) __attribute__((amdgpu_waves_per_eu(kAcc ? 1 : 2))) void gemm_w4a4_kernel(
    const uint8_t* __restrict__ Xq, const uint16_t* __restrict__ sx, const uint8_t* __restrict__ Wq,
    const uint16_t* __restrict__ sw, int M, int N, int K, uint16_t* __restrict__ Y, int32_t* __restrict__ acc_out,
    int full, int rem, int splits, float* __restrict__ part) {
  using T = Tile<BM, BN, WAVES_M, WAVES_N>;
  // Three stage buffers, each its own object: the compiler then knows that a copy into one
  // does not write what is read from another, and waits only where a buffer is really shared.
  __shared__ __attribute__((aligned(16))) uint8_t la0[BM * kLdsRow], la1[BM * kLdsRow], la2[BM * kLdsRow];
  __shared__ __attribute__((aligned(16))) uint8_t lb0[BN * kLdsRow], lb1[BN * kLdsRow], lb2[BN * kLdsRow];
  __shared__ __attribute__((aligned(16))) h4 ls0[BM + BN], ls1[BM + BN], ls2[BM + BN];   // sx rows, then sw
  auto LA = [&](int p) -> uint8_t* { return p == 0 ? la0 : p == 1 ? la1 : la2; };
  auto LB = [&](int p) -> uint8_t* { return p == 0 ? lb0 : p == 1 ? lb1 : lb2; };
  auto LS = [&](int p) -> h4* { return p == 0 ? ls0 : p == 1 ? ls1 : ls2; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WAVES_N;
  const int wn = wave % WAVES_N;
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
  const bool is_piece = nsplit > 1;
  const int2 tc = tile_coords(lin, tiles_m, tiles_n);
  const int m0 = tc.x * BM, n0 = tc.y * BN;
  const int G = K / ATOM_GROUP;
  // this workgroup's INT4 groups [ga, gb); the last piece also takes the INT8 group
  const int ga = split * (G - 1) / nsplit, gb = (split + 1) * (G - 1) / nsplit;
  const bool last_split = split == nsplit - 1;
  const int S = G + 1;                                  // stages per row
  const size_t rbytes = (size_t)S * kStageBytes;        // = (K-128)/2 + 128
  const int l32 = lane & 31;                            // row (A) / column (B) inside a 32x32 tile
  const int kh = lane >> 5;                             // which K half of an operand this lane supplies

  // ---- per-lane stage-copy addresses
  StageAddr<T::kDma> ad;
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
    ad.s_is_x = tid < BM;
    ad.s_src = kAcc ? nullptr : ad.s_is_x ? sx + min(m0 + tid, M - 1) : sw + min(n0 + tid - BM, N - 1);
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
  auto apply = [&](int i, int j, const v16f& acc, const v16f& sp, int g) {
    if (kAcc) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * T::kWTM + i * 32 + acc_row(lane);
        const int n = n0 + wn * T::kWTN + j * 32 + acc_col(lane, r >> 2) + (r & 3);
        if (m < M && n < N) acc_out[((size_t)g * M + m) * N + n] = (int32_t)acc[r];   // exact integers
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) yacc[i][j][r] = __builtin_fmaf(acc[r], sp[r], yacc[i][j][r]);
    }
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

  // Stage ring.  Stage t (t = ga, ga+1, ...) lives in LDS buffer (t - ga) % 3.  While group s
  // is multiplied, its packed operands and scales are in registers; stage s+1 has landed and
  // each wave reads it into the registers that group s's decode has just freed; the copies
  // of stage s+2 (issued at the start of group s-1) and stage s+3 (issued at the start of
  // group s, into the buffer stage s came from) are in flight.  The one barrier per group
  // comes after this wave's copy of stage s+2 has landed and its reads of stage s+1 have
  // completed: after it stage s+2 is visible to all and the buffer of stage s+1 may be
  // refilled.  Scales take the same ring: each thread's scale of stage t is loaded into
  // `sreg` during group t-4 and written to LDS at the start of group t-3.
  constexpr int kPerStage = 2 * T::kDma + (kAcc ? 0 : 1);   // vector-memory operations per stage
  uint16_t sreg = 0;
  {
    uint16_t s0 = 0, s1 = 0, s2 = 0;
    if (!kAcc) {
      s0 = load_scale(ad, ga, G, M, N);
      s1 = load_scale(ad, ga + 1, G, M, N);
      s2 = load_scale(ad, ga + 2, G, M, N);
    }
    __builtin_amdgcn_sched_barrier(0);
    dma_stage(ad, la0, lb0, ga);
    dma_stage(ad, la1, lb1, min(ga + 1, G));
    dma_stage(ad, la2, lb2, min(ga + 2, G));
    __builtin_amdgcn_sched_barrier(0);
    if (!kAcc) {
      sreg = load_scale(ad, ga + 3, G, M, N);
      ls0[tid] = scale_operand(s0);
      ls1[tid] = scale_operand(s1);
      ls2[tid] = scale_operand(s2);
    }
    __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(kPerStage));   // stages ga and ga+1 have landed
    wg_barrier();
  }
  v8i pa[T::kTM], pb[T::kTN];
  h4 sa[T::kTM], sb[T::kTN];
  if (!kAcc) read_scales(ls0, sa, sb);
  read_packed(la0, lb0, pa, pb);
  __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(63));             // buffer 0 read by this wave
  wg_barrier();                                                // ... and by all: it may be refilled

  // INT4 group s in ring position P (stage s in buffer P).  A wave issues in order, so nothing
  // may wait on the MFMA issued just before it.  Per tile row i: region a decodes A row i
  // (and every B column at i = 0), reads the matching operands of stage s+1, issues the scale
  // product and the two K=64 fp6 MFMAs of tile (i, 0), then applies tile (i-1, 1); region b
  // issues the scale product and MFMAs of tile (i, 1), then applies tile (i, 0).  Each apply
  // thus comes after three MFMAs that do not feed it, so a tile's sums (the exact group sum
  // in fp32) and its scale product are complete when they are used, and no more than two
  // tiles' sums and scale products are live at a time.  The scheduling fences keep this order.
  static_assert(T::kTN == 2, "tile rows are processed as pairs of 32x32 tiles");
  auto int4_group = [&](auto ring, int s) {
    constexpr int p = decltype(ring)::kCur, pn = decltype(ring)::kNext;
    // refill buffer p (stage s was read during group s-1, before the last barrier)
    if (!kAcc) {
      LS(p)[tid] = scale_operand(sreg);
      sreg = load_scale(ad, s + 4, G, M, N);
    }
    __builtin_amdgcn_sched_barrier(0);
    dma_stage(ad, LA(p), LB(p), min(s + 3, G));               // past the row end: unused
    __builtin_amdgcn_sched_barrier(0);
    v16f acc0, sp0, acc1, sp1;                                 // tiles (i, 0) and (i, 1)
    v8i b0[2], b1[2];                                          // fp6 operands of the B columns
    h4 san[T::kTM], sbn[T::kTN];
#pragma unroll
    for (int i = 0; i < T::kTM; ++i) {
      const v8i a0 = fp6_operand(pa[i], 0), a1 = fp6_operand(pa[i], 1);
      if (i == 0) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          b0[j] = fp6_operand(pb[j], 0);
          b1[j] = fp6_operand(pb[j], 1);
          pb[j] = read_b(LB(pn), j);
        }
        if (!kAcc) read_scales(LS(pn), san, sbn);
      }
      pa[i] = read_a(LA(pn), i);
      sp0 = scale_product(sa[i], sb[0]);
      acc0 = mma_fp6(a0, b0[0], v16f{});
      acc0 = mma_fp6(a1, b1[0], acc0);
      if (i > 0) apply(i - 1, 1, acc1, sp1, s);
      __builtin_amdgcn_sched_barrier(0);
      sp1 = scale_product(sa[i], sb[1]);
      acc1 = mma_fp6(a0, b0[1], v16f{});
      acc1 = mma_fp6(a1, b1[1], acc1);
      apply(i, 0, acc0, sp0, s);
      __builtin_amdgcn_sched_barrier(0);
    }
    apply(T::kTM - 1, 1, acc1, sp1, s);
    __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(kPerStage));   // own copy of stage s+2 landed, reads done
    wg_barrier();
#pragma unroll
    for (int i = 0; i < T::kTM; ++i) sa[i] = san[i];
#pragma unroll
    for (int j = 0; j < T::kTN; ++j) sb[j] = sbn[j];
  };
  {
    int s = ga;
    for (; s + 3 <= gb; s += 3) {
      int4_group(Ring<0>{}, s);
      int4_group(Ring<1>{}, s + 1);
      int4_group(Ring<2>{}, s + 2);
    }
    if (s < gb) int4_group(Ring<0>{}, s++);
    if (s < gb) int4_group(Ring<1>{}, s++);
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
    const int pg = (G - ga) % 3;
    if (pg == 0) read_packed(la0, lb0, pa, pb);
    else if (pg == 1) read_packed(la1, lb1, pa, pb);
    else read_packed(la2, lb2, pa, pb);
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
            if (m < M && n < N) Y[(size_t)m * N + n] = __half_as_ushort(__float2half_rn(0.5f * yacc[i][j][r]));
          }
    }
  }
}

// 128 x 128 workgroup tile, 2 x 2 waves of 64 x 64 (2 x 2 MFMA tiles of 32 x 32 each).
constexpr int kBM = 128, kBN = 128, kWavesM = 2, kWavesN = 2;
// Split-K.  Grids of fewer than kSplitMinTiles tiles split every tile, aiming at about one
// workgroup per compute unit; a piece keeps at least kSplitMinGroups INT4 groups.  Larger
// grids are not split, not even a last partial round of tiles: with every compute unit busy
// the chip runs at its power limit, so spreading a tail lowers the clock about as much as it
// adds parallelism, and the partial sums and the second kernel are pure cost (measured:
// 1024 x 4096 x 11008 with its last 176 of 688 tiles split in two spans the same time, and
// 600 x 2048 x 15300 with 88 of 600 split three ways is slower).
constexpr int kSplitMinTiles = 128, kSplitTargetBlocks = 256, kSplitMinGroups = 4, kSplitMax = 8;

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

}  // namespace

GemmPlan gemm_plan(int M, int N, int K) {
  if (M <= kSmallMaxM) return GemmPlan{0, 0, 1, 1};
  return gemm_plan_tiled(M, N, K);
}

GemmPlan gemm_plan_tiled(int M, int N, int K) {
  const int tiles = ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
  const int G = K / ATOM_GROUP;
  if (tiles >= kSplitMinTiles) return GemmPlan{tiles, 0, 1, 0};
  const int s = min(min((kSplitTargetBlocks + tiles - 1) / tiles, (G - 1) / kSplitMinGroups), kSplitMax);
  return s < 2 ? GemmPlan{tiles, 0, 1, 0} : GemmPlan{0, tiles, s, 0};
}

int64_t gemm_workspace_bytes(const GemmPlan& plan) {
  if (plan.small) return 0;
  return plan.rem > 0 ? (int64_t)plan.rem * plan.splits * kBM * kBN * (int64_t)sizeof(float) : 0;
}

hipError_t launch_gemm(const uint8_t* Xq, const uint16_t* sx, const uint8_t* Wq, const uint16_t* sw, int M, int N,
                       int K, uint16_t* Y, float* part, const GemmPlan& plan, hipStream_t stream) {
  if (plan.small) return launch_gemm_small(Xq, sx, Wq, sw, M, N, K, Y, stream);
  if (plan.rem > 0 && (plan.splits < 2 || plan.splits > kSplitMax)) return hipErrorInvalidValue;
  const int blocks = plan.full + plan.rem * plan.splits;
  hipLaunchKernelGGL((gemm_w4a4_kernel<kBM, kBN, kWavesM, kWavesN, false>), dim3(blocks),
                     dim3(kWavesM * kWavesN * 64), 0, stream, Xq, sx, Wq, sw, M, N, K, Y, (int32_t*)nullptr,
                     plan.full, plan.rem, plan.splits, part);
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

hipError_t launch_gemm_group_acc(const uint8_t* Xq, const uint8_t* Wq, int M, int N, int K, int32_t* acc,
                                 hipStream_t stream) {
  const dim3 grid(((N + kBN - 1) / kBN) * ((M + kBM - 1) / kBM));
  hipLaunchKernelGGL((gemm_w4a4_kernel<kBM, kBN, kWavesM, kWavesN, true>), grid, dim3(kWavesM * kWavesN * 64), 0,
                     stream, Xq, (const uint16_t*)nullptr, Wq, (const uint16_t*)nullptr, M, N, K,
                     (uint16_t*)nullptr, acc, (int)grid.x, 0, 1, (float*)nullptr);
  return hipGetLastError();
}

}  // namespace atom
