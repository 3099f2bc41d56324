// W4A8 GEMM for gfx950: INT8 activation codes in every 128-channel group against the W4
// weights (INT4 bulk, INT8 outlier group), a variant beside the W4A4 path.
//
// Y[m,n] = sum over groups g of acc_g[m,n] * sx[g,m] * sw[g,n], acc_g the exact integer dot
// product of the codes of group g, as for W4A4 (quantization record of "Atom (mixed-precision
// block-outlier low-bit quantization for serving)", Fields "Bits", "Weight group size",
// "notes": per-group scales, the 128-channel INT8 group).  INT8 activation codes are not exact
// fp6 or fp8 values, so every group runs on v_mfma_i32_32x32x32_i8.
//
// Operands.  Activation rows are K two's-complement bytes; a lane's 16 bytes of a K = 32 slice
// feed the MFMA as they are.  Weight rows keep the INT4 groups as offset-binary nibbles (byte j
// of each 8-code block holds c_j + 8 and c_{j+4} + 8): for 16 consecutive codes (two words
// w0, w1) the int8 operand is {w0 & 0x0F0F0F0F, (w0 >> 4) & 0x0F0F0F0F, w1 & .., (w1 >> 4) & ..},
// the biased codes c + 8 in order.  The MFMA then sums a * (c + 8); one more MFMA per K slice
// with the constant -8 as weight operand puts -8 * sum(a) into the accumulator first, so the
// result is the exact sum of a * c.  The INT8 outlier group's weights are two's-complement
// bytes and need no correction.  Every partial sum is an integer below 2^31.
//
// K slices.  In a K = 32 slice t of a group, lane l supplies row (activations: token; weights:
// output column) l & 31 and the 16 codes 32 t + 16 (l >> 5) .. + 15; both operands use the same
// assignment, so every code of the group meets its partner once.  The weights are the first
// operand, so a 32x32 accumulator holds its output tile transposed: lane l owns output row
// l & 31, element r is column (r >> 2) * 8 + (l >> 5) * 4 + (r & 3).
//
// Scales and epilogue.  As in the W4A4 kernel: one v_mfma_f32_32x32x8_f16 with each lane's
// fp16 scale in K slot 0 of its half gives 2 * sx * sw exactly in the accumulator layout; the
// int32 group sum (|acc| < 2^21, so its conversion to fp32 is exact) is added with one fp32 fma
// per element and group; the factor 2 goes at the store (or stays in a split piece's partial
// tile, which the split-K finalize removes).
//
// Work layout.  One workgroup of 4 waves per 128 x 128 output tile (2 x 2 waves of 64 x 64,
// each 2 x 2 MFMA tiles), tiles in the banded order of the W4A4 kernel; with caller scratch, a
// grid of few tiles splits each tile's groups among pieces whose fp32 partial tiles the W4A4
// split-K finalize adds.  Per group the activation stage (128 rows x 128 bytes) and the weight
// stage (128 rows x 64 or 128 bytes) are staged in LDS, rows padded to 144 bytes (the 16 lanes
// of a 16-byte read hit 16 distinct bank groups), double-buffered: the next group's loads are
// in flight in registers while the current group is multiplied.  Pieces of many groups (long K)
// take gemm_w4a8_ring_kernel instead: the same computation with the stages copied straight
// from global memory into a ring of three LDS buffers (LDS-DMA: no registers, no LDS store
// instructions), two stages ahead of the group being multiplied, one barrier per group; its
// stage rows are unpadded, with 16-byte chunks at swizzled positions (the INT8 group's weights
// fill two 64-byte stages, its activations one).
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "atom_internal.h"
#include "lds_ring.h"

namespace atom {
namespace {

typedef int32_t v4i __attribute__((ext_vector_type(4)));
typedef int32_t v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));

constexpr int kTile = 128;                 // output tile rows and columns
constexpr int kThreads = 256;              // 4 waves
constexpr int kLdsRow = 144;               // staged row: 128 bytes + 16 padding

// The ring kernel (long K)
constexpr int kRowA = 128;                 // staged activation row: one group of int8 codes
constexpr int kRowW = 64;                  // staged weight row: one INT4 group, half the INT8 group
constexpr int kRing = 3;                   // stage buffers
// Pieces of at least this many INT4 groups take the ring kernel.  Kernel trace, Llama-7B
// shapes, register-staged -> ring: 2048x11008x4096 (85 groups) 173.6 -> 158.7 us; but
// 1024x4096x11008 (31 groups) 103.5 -> 113.3 us and 256x4096x4096 (4 pieces of ~8) 17.0 ->
// 20.0 us: the ring costs more per tile (two stages copied before the first group, wider
// bursts) and less per group.
constexpr int kRingMinGroups = 64;
constexpr int kDmaA = kTile / 4 * kRowA / 16 / 64;   // LDS-DMA instructions per wave and stage: 4
constexpr int kDmaW = kTile / 4 * kRowW / 16 / 64;   // 2

// Position of 16-byte chunk c of staged row r.  Activation rows (8 chunks): the 16 lanes of a
// 16-byte read take 16 consecutive rows at one chunk; row parity picks the half of the banks
// and (r >> 1) & 7 one of 8 positions, so the 16 reads hit distinct banks.  Weight rows (4
// chunks): as in the W4A4 kernel, (r >> 2) & 3.
__device__ __forceinline__ int pos_a(int r, int c) { return c ^ ((r >> 1) & 7); }
__device__ __forceinline__ int pos_w(int r, int c) { return c ^ ((r >> 2) & 3); }
constexpr uint32_t kNibbles = 0x0F0F0F0Fu;
constexpr int32_t kMinus8 = (int32_t)0xF8F8F8F8u;   // four int8 -8

__device__ __forceinline__ v16i mma_i8(v4i w, v4i x, v16i c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(w, x, c, 0, 0, 0);
}

// Compile-time selector of the weight group kind (INT4 nibbles or the INT8 outlier group).
template <bool B>
struct WeightKind {
  static constexpr bool value = B;
};
using Int4W = WeightKind<false>;
using Int8W = WeightKind<true>;

// 16 biased INT4 codes (two words of nibbles) -> int8 operand of the codes + 8
__device__ __forceinline__ v4i unpack_nibbles(uint2 w) {
  return v4i{(int)(w.x & kNibbles), (int)((w.x >> 4) & kNibbles), (int)(w.y & kNibbles),
             (int)((w.y >> 4) & kNibbles)};
}

template <bool kAcc>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void gemm_w4a8_kernel(
    const uint8_t* __restrict__ Xq, const uint16_t* __restrict__ sx, const uint8_t* __restrict__ Wq,
    const uint16_t* __restrict__ sw, int M, int N, int K, uint16_t* __restrict__ Y, int32_t* __restrict__ acc_out,
    int rem, int splits, float* __restrict__ part, int late_from) {
  // Workgroups of later rounds (id >= late_from) issue at priority 1, so that a late tile does
  // not trail the partner it joins part way through (a SIMD otherwise issues the older wave
  // first).  Event-timed 1024 x 4096 x 11008 (688 tiles for 512 slots): 109.4-109.6 ->
  // 106.1-106.7 us.  One asm statement with its own skip, outside the main loop.
  {
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)blockIdx.x >= late_from ? 1 : 0);
    asm volatile(
        "s_bitcmp1_b32 %0, 0\n\t"
        "s_cbranch_scc0 1f\n\t"
        "s_setprio 1\n\t"
        "s_branch 2f\n"
        "1:\n\t"
        "s_setprio 0\n"
        "2:"
        :
        : "s"(hi)
        : "scc");
  }
  __shared__ __attribute__((aligned(16))) uint8_t la[2][kTile * kLdsRow];
  __shared__ __attribute__((aligned(16))) uint8_t lb[2][kTile * kLdsRow];
  __shared__ __attribute__((aligned(16))) h4 ls[2][2 * kTile];        // sx of the tile rows, then sw

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, kh = lane >> 5;
  const int tiles_m = (M + kTile - 1) / kTile, tiles_n = (N + kTile - 1) / kTile;
  // Split plan (rem > 0): workgroup p is piece p / rem of tile p % rem; each piece takes a
  // contiguous range of INT4 groups, the last piece also the INT8 group.
  const bool split_mode = rem > 0;   // uniform
  const int lin = split_mode ? (int)blockIdx.x % rem : (int)blockIdx.x;
  const int split = split_mode ? (int)blockIdx.x / rem : 0, nsplit = split_mode ? splits : 1;
  const int2 tc = tile_coords(lin, tiles_m, tiles_n);
  const int m0 = tc.x * kTile, n0 = tc.y * kTile;
  const int G = K / ATOM_GROUP;
  const int ga = split * (G - 1) / nsplit, gb = (split + 1) * (G - 1) / nsplit;   // INT4 groups [ga, gb)
  const bool last_split = split == nsplit - 1;
  const int klo = K - ATOM_OUTLIERS;
  const size_t rbw = (size_t)klo / 2 + ATOM_OUTLIERS;      // weight row bytes

  // Stage copy: thread tid moves chunks q = tid + 256 i (16 bytes each); activation chunk q is
  // row q / 8, bytes 16 (q % 8) of the group; weight chunk q of an INT4 group is row q / 4,
  // bytes 16 (q % 4) (two chunks per thread), of the INT8 group row q / 8, bytes 16 (q % 8)
  // (four).  Rows past M / N repeat the last valid row (their results are never stored).
  struct Stage {
    uint4 a0, a1, a2, a3, w0, w1, w2, w3;
    uint16_t s;
  };
  auto xload = [&](int g, int i) {
    const int q = tid + kThreads * i;
    return *reinterpret_cast<const uint4*>(Xq + (size_t)min(m0 + (q >> 3), M - 1) * K + (size_t)g * ATOM_GROUP +
                                           16 * (q & 7));
  };
  auto wload4 = [&](int g, int i) {   // INT4 group, chunks 0..511
    const int q = tid + kThreads * i;
    return *reinterpret_cast<const uint4*>(Wq + (size_t)min(n0 + (q >> 2), N - 1) * rbw + (size_t)g * 64 + 16 * (q & 3));
  };
  auto wload8 = [&](int i) {          // INT8 group, chunks 0..1023
    const int q = tid + kThreads * i;
    return *reinterpret_cast<const uint4*>(Wq + (size_t)min(n0 + (q >> 3), N - 1) * rbw + klo / 2 + 16 * (q & 7));
  };
  auto load_stage = [&](auto int8w_tag, int g) {
    constexpr bool kInt8W = decltype(int8w_tag)::value;
    Stage st;
    st.a0 = xload(g, 0);
    st.a1 = xload(g, 1);
    st.a2 = xload(g, 2);
    st.a3 = xload(g, 3);
    if (kInt8W) {
      st.w0 = wload8(0);
      st.w1 = wload8(1);
      st.w2 = wload8(2);
      st.w3 = wload8(3);
    } else {
      st.w0 = wload4(g, 0);
      st.w1 = wload4(g, 1);
      st.w2 = st.w3 = uint4{0, 0, 0, 0};
    }
    st.s = 0;
    if (!kAcc)
      st.s = tid < kTile ? sx[(size_t)g * M + min(m0 + tid, M - 1)] : sw[(size_t)g * N + min(n0 + tid - kTile, N - 1)];
    return st;
  };
  auto lds_a = [&](int buf, int i) -> uint4* {
    const int q = tid + kThreads * i;
    return reinterpret_cast<uint4*>(&la[buf][(q >> 3) * kLdsRow + 16 * (q & 7)]);
  };
  auto lds_w4 = [&](int buf, int i) -> uint4* {
    const int q = tid + kThreads * i;
    return reinterpret_cast<uint4*>(&lb[buf][(q >> 2) * kLdsRow + 16 * (q & 3)]);
  };
  auto lds_w8 = [&](int buf, int i) -> uint4* {
    const int q = tid + kThreads * i;
    return reinterpret_cast<uint4*>(&lb[buf][(q >> 3) * kLdsRow + 16 * (q & 7)]);
  };
  auto store_stage = [&](auto int8w_tag, const Stage& st, int buf) {
    constexpr bool kInt8W = decltype(int8w_tag)::value;
    *lds_a(buf, 0) = st.a0;
    *lds_a(buf, 1) = st.a1;
    *lds_a(buf, 2) = st.a2;
    *lds_a(buf, 3) = st.a3;
    if (kInt8W) {
      *lds_w8(buf, 0) = st.w0;
      *lds_w8(buf, 1) = st.w1;
      *lds_w8(buf, 2) = st.w2;
      *lds_w8(buf, 3) = st.w3;
    } else {
      *lds_w4(buf, 0) = st.w0;
      *lds_w4(buf, 1) = st.w1;
    }
    if (!kAcc) ls[buf][tid] = h4{__builtin_bit_cast(_Float16, st.s), (_Float16)0, (_Float16)0, (_Float16)0};
  };

  v16f yacc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) yacc[i][j][r] = 0.0f;

  // Group g from LDS buffer buf into the Y accumulators (or, kAcc, to acc_out).
  auto compute = [&](auto int8w_tag, int g, int buf) {
    constexpr bool kInt8W = decltype(int8w_tag)::value;
    h4 sa[2], sb[2];
    if (!kAcc) {
#pragma unroll
      for (int i = 0; i < 2; ++i) sa[i] = ls[buf][wm * 64 + i * 32 + l32];
#pragma unroll
      for (int j = 0; j < 2; ++j) sb[j] = ls[buf][kTile + wn * 64 + j * 32 + l32];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      __builtin_amdgcn_sched_barrier(0);   // one tile row's operands live at a time
      const uint8_t* arow = &la[buf][(wm * 64 + i * 32 + l32) * kLdsRow + 16 * kh];
      v4i a[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) a[t] = *reinterpret_cast<const v4i*>(arow + 32 * t);
      v16i corr = {};
      if (!kInt8W) {
#pragma unroll
        for (int t = 0; t < 4; ++t) corr = mma_i8(v4i{kMinus8, kMinus8, kMinus8, kMinus8}, a[t], corr);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint8_t* brow = &lb[buf][(wn * 64 + j * 32 + l32) * kLdsRow];
        v16i acc = corr;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          v4i b;
          if (kInt8W)
            b = *reinterpret_cast<const v4i*>(brow + 32 * t + 16 * kh);
          else
            b = unpack_nibbles(*reinterpret_cast<const uint2*>(brow + 16 * t + 8 * kh));
          acc = mma_i8(b, a[t], acc);
        }
        if (kAcc) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int m = m0 + wm * 64 + i * 32 + l32;
            const int n = n0 + wn * 64 + j * 32 + (r >> 2) * 8 + kh * 4 + (r & 3);
            if (m < M && n < N) acc_out[((size_t)g * M + m) * N + n] = acc[r];
          }
        } else {
          const v16f sp = __builtin_amdgcn_mfma_f32_32x32x8f16(sb[j], sa[i], v16f{}, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 16; ++r) yacc[i][j][r] = __builtin_fmaf((float)acc[r], sp[r], yacc[i][j][r]);
        }
      }
    }
  };

  // INT4 groups ga .. gb-1, the next group's loads in flight during each; then (last piece)
  // the INT8 group.  Buffer (g - ga) % 2 holds group g.
  store_stage(Int4W{}, load_stage(Int4W{}, ga), 0);
  __syncthreads();
  for (int g = ga; g < gb - 1; ++g) {
    const Stage next = load_stage(Int4W{}, g + 1);
    compute(Int4W{}, g, (g - ga) & 1);
    store_stage(Int4W{}, next, (g - ga + 1) & 1);
    __syncthreads();
  }
  if (last_split) {
    const Stage next = load_stage(Int8W{}, G - 1);
    compute(Int4W{}, gb - 1, (gb - 1 - ga) & 1);
    store_stage(Int8W{}, next, (gb - ga) & 1);
    __syncthreads();
    compute(Int8W{}, G - 1, (gb - ga) & 1);
  } else {
    compute(Int4W{}, gb - 1, (gb - 1 - ga) & 1);
  }

  if (kAcc) return;
  if (split_mode) {   // the piece's fp32 tile (factor 2 kept), row-major, to its scratch slot
    float* tile = part + ((size_t)split * rem + lin) * (kTile * kTile);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = wm * 64 + i * 32 + l32;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = wn * 64 + j * 32 + q * 8 + kh * 4;
          *reinterpret_cast<float4*>(tile + r * kTile + c) =
              float4{yacc[i][j][4 * q], yacc[i][j][4 * q + 1], yacc[i][j][4 * q + 2], yacc[i][j][4 * q + 3]};
        }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int m = m0 + wm * 64 + i * 32 + l32;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + wn * 64 + j * 32 + q * 8 + kh * 4;
        const uint16_t o[4] = {__half_as_ushort(__float2half_rn(0.5f * yacc[i][j][4 * q])),
                               __half_as_ushort(__float2half_rn(0.5f * yacc[i][j][4 * q + 1])),
                               __half_as_ushort(__float2half_rn(0.5f * yacc[i][j][4 * q + 2])),
                               __half_as_ushort(__float2half_rn(0.5f * yacc[i][j][4 * q + 3]))};
        if (m >= M) continue;
        uint16_t* dst = Y + (size_t)m * N + n;
        if (n + 4 <= N && (N & 3) == 0) {
          *reinterpret_cast<ushort4*>(dst) = ushort4{o[0], o[1], o[2], o[3]};
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < N) dst[e] = o[e];
        }
      }
  }
}

// Long K: the same tile and group computation with the stage copies on an LDS-DMA ring.
template <bool kAcc>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void gemm_w4a8_ring_kernel(
    const uint8_t* __restrict__ Xq, const uint16_t* __restrict__ sx, const uint8_t* __restrict__ Wq,
    const uint16_t* __restrict__ sw, int M, int N, int K, uint16_t* __restrict__ Y, int32_t* __restrict__ acc_out,
    int rem, int splits, float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) uint8_t la0[kTile * kRowA], la1[kTile * kRowA], la2[kTile * kRowA];
  __shared__ __attribute__((aligned(16))) uint8_t lw0[kTile * kRowW], lw1[kTile * kRowW], lw2[kTile * kRowW];
  __shared__ __attribute__((aligned(16))) h4 ls0[2 * kTile], ls1[2 * kTile], ls2[2 * kTile];   // sx, then sw
  auto LA = [&](int p) -> uint8_t* { return p == 0 ? la0 : p == 1 ? la1 : la2; };
  auto LW = [&](int p) -> uint8_t* { return p == 0 ? lw0 : p == 1 ? lw1 : lw2; };
  auto LS = [&](int p) -> h4* { return p == 0 ? ls0 : p == 1 ? ls1 : ls2; };

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, kh = lane >> 5;
  const int tiles_m = (M + kTile - 1) / kTile, tiles_n = (N + kTile - 1) / kTile;
  // Split plan (rem > 0): workgroup p is piece p / rem of tile p % rem; each piece takes a
  // contiguous range of INT4 groups, the last piece also the INT8 group.
  const bool split_mode = rem > 0;   // uniform
  const int lin = split_mode ? (int)blockIdx.x % rem : (int)blockIdx.x;
  const int split = split_mode ? (int)blockIdx.x / rem : 0, nsplit = split_mode ? splits : 1;
  const int2 tc = tile_coords(lin, tiles_m, tiles_n);
  const int m0 = tc.x * kTile, n0 = tc.y * kTile;
  const int G = K / ATOM_GROUP;
  const int ga = split * (G - 1) / nsplit, gb = (split + 1) * (G - 1) / nsplit;   // INT4 groups [ga, gb)
  const bool last_split = split == nsplit - 1;
  const int klo = K - ATOM_OUTLIERS;
  const int rbw = klo / 2 + ATOM_OUTLIERS;      // weight row bytes

  // Stage copies.  Stage t (t = ga, ga+1, ...) is group t for t < G-1; the INT8 group G-1 is
  // stages G-1 and G: its activations (128 bytes) in stage G-1 (stage G repeats them), its
  // weights' first and second 64 bytes in stages G-1 and G.  The weight bytes of stage t thus
  // start at 64 t for every t, the activation bytes at 128 min(t, G-1).  Wave w copies rows
  // 32 w .. 32 w + 31 of both; lane i of instruction h lands at LDS row 32 w + 8 h + i / 8,
  // position i % 8 (activations), or row 32 w + 16 h + i / 4, position i % 4 (weights), and
  // loads the chunk stored there.  Rows past M / N repeat the last valid row.
  __amdgpu_buffer_rsrc_t a_rsrc, w_rsrc;
  int a_voff[kDmaA], w_voff[kDmaW];
  const int row0 = __builtin_amdgcn_readfirstlane(wave) * (kTile / 4);
  {
    const int rows_a = min(kTile, M - m0), rows_w = min(kTile, N - n0);
    a_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)(Xq + (size_t)m0 * K), (short)0, rows_a * K, 0x00020000);
    w_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)(Wq + (size_t)n0 * rbw), (short)0, rows_w * rbw, 0x00020000);
#pragma unroll
    for (int h = 0; h < kDmaA; ++h) {
      const int r = row0 + 8 * h + lane / 8;
      a_voff[h] = min(r, rows_a - 1) * K + pos_a(r, lane & 7) * 16;
    }
#pragma unroll
    for (int h = 0; h < kDmaW; ++h) {
      const int r = row0 + 16 * h + lane / 4;
      w_voff[h] = min(r, rows_w - 1) * rbw + pos_w(r, lane & 3) * 16;
    }
  }
  auto dma_stage = [&](int p, int t) __attribute__((always_inline)) {
    const int sa_off = min(t, G - 1) * kRowA, sw_off = min(t, G) * kRowW;
#pragma unroll
    for (int h = 0; h < kDmaA; ++h) lds_dma16(a_rsrc, LA(p) + (row0 + 8 * h) * kRowA, a_voff[h], sa_off);
#pragma unroll
    for (int h = 0; h < kDmaW; ++h) lds_dma16(w_rsrc, LW(p) + (row0 + 16 * h) * kRowW, w_voff[h], sw_off);
  };
  // Thread tid < 128 carries the activation scale of tile row tid, thread 128 + u the weight
  // scale of tile column u; stage t's scale (group min(t, G-1)) is loaded with its copy and
  // written to LDS, as the finished operand (scale, 0, 0, 0), during group t-1.
  const uint16_t* s_src = kAcc ? nullptr : tid < kTile ? sx + min(m0 + tid, M - 1) : sw + min(n0 + tid - kTile, N - 1);
  const bool s_is_x = tid < kTile;
  auto load_scale = [&](int t) -> uint16_t {
    const int g = min(t, G - 1);
    return s_src[s_is_x ? (size_t)g * M : (size_t)g * N];
  };
  auto scale_operand = [](uint16_t v) {
    return h4{__builtin_bit_cast(_Float16, v), (_Float16)0, (_Float16)0, (_Float16)0};
  };
  constexpr int kPerStage = kDmaA + kDmaW + (kAcc ? 0 : 1);   // vector-memory operations per stage

  v16f yacc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) yacc[i][j][r] = 0.0f;

  // Group g from stage buffers (activations and first weight half pa / pw, second weight half
  // pw2 for the INT8 group) into the Y accumulators (or, kAcc, to acc_out).
  auto compute = [&](auto int8w_tag, int g, const uint8_t* sa_buf, const uint8_t* sw_buf, const uint8_t* sw2_buf,
                     const h4* ls) __attribute__((always_inline)) {
    constexpr bool kInt8W = decltype(int8w_tag)::value;
    h4 sa[2], sb[2];
    if (!kAcc) {
#pragma unroll
      for (int i = 0; i < 2; ++i) sa[i] = ls[wm * 64 + i * 32 + l32];
#pragma unroll
      for (int j = 0; j < 2; ++j) sb[j] = ls[kTile + wn * 64 + j * 32 + l32];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      __builtin_amdgcn_sched_barrier(0);   // one tile row's operands live at a time
      const int ra = wm * 64 + i * 32 + l32;
      const uint8_t* arow = sa_buf + ra * kRowA;
      v4i a[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) a[t] = *reinterpret_cast<const v4i*>(arow + pos_a(ra, 2 * t + kh) * 16);
      v16i corr = {};
      if (!kInt8W) {
#pragma unroll
        for (int t = 0; t < 4; ++t) corr = mma_i8(v4i{kMinus8, kMinus8, kMinus8, kMinus8}, a[t], corr);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int rw = wn * 64 + j * 32 + l32;
        v16i acc = corr;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          v4i b;
          if (kInt8W) {   // 16 bytes at 32 t + 16 kh of the 128-byte row: half t / 2
            const uint8_t* wrow = (t < 2 ? sw_buf : sw2_buf) + rw * kRowW;
            b = *reinterpret_cast<const v4i*>(wrow + pos_w(rw, 2 * (t & 1) + kh) * 16);
          } else {        // 8 bytes at 16 t + 8 kh of the 64-byte row
            const uint8_t* wrow = sw_buf + rw * kRowW;
            b = unpack_nibbles(*reinterpret_cast<const uint2*>(wrow + pos_w(rw, t) * 16 + 8 * kh));
          }
          acc = mma_i8(b, a[t], acc);
        }
        if (kAcc) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int m = m0 + wm * 64 + i * 32 + l32;
            const int n = n0 + wn * 64 + j * 32 + (r >> 2) * 8 + kh * 4 + (r & 3);
            if (m < M && n < N) acc_out[((size_t)g * M + m) * N + n] = acc[r];
          }
        } else {
          const v16f sp = __builtin_amdgcn_mfma_f32_32x32x8f16(sb[j], sa[i], v16f{}, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 16; ++r) yacc[i][j][r] = __builtin_fmaf((float)acc[r], sp[r], yacc[i][j][r]);
        }
      }
    }
  };

  // Ring.  Stage t lives in buffer (t - ga) % 3.  During group s: stage s's copy has landed and
  // is multiplied; stage s+1's copy is in flight (issued during group s-1) and its scale is
  // written to LDS; stage s+2's copy is issued into the buffer stage s-1 came from (read during
  // group s-1, before the last barrier).  The one barrier per group comes after this wave's
  // copy of stage s+1 has landed and its reads of stage s are done.
  uint16_t sreg[kRing];
  if (!kAcc) sreg[0] = load_scale(ga);
  dma_stage(0, ga);
  if (!kAcc) sreg[1] = load_scale(ga + 1);
  dma_stage(1, ga + 1);
  if (!kAcc) ls0[tid] = scale_operand(sreg[0]);
  __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(kPerStage));   // stage ga has landed
  wg_barrier();
  auto int4_group = [&](auto ring, int s) __attribute__((always_inline)) {
    constexpr int p = decltype(ring)::kCur, p1 = decltype(ring)::kNext, p2 = decltype(ring)::kAfterNext;
    if (!kAcc) LS(p1)[tid] = scale_operand(sreg[p1]);
    if (!kAcc) sreg[p2] = load_scale(s + 2);
    __builtin_amdgcn_sched_barrier(0);
    dma_stage(p2, s + 2);                               // past the row end: unused
    __builtin_amdgcn_sched_barrier(0);
    compute(Int4W{}, s, LA(p), LW(p), LW(p), LS(p));
    __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(kPerStage));   // own copy of stage s+1 landed, reads done
    wg_barrier();
  };
  {
    int s = ga;
    for (; s + kRing <= gb; s += kRing) ring_turn<0, kRing>(int4_group, s);
    ring_tail<0, kRing>(int4_group, s, gb);
  }
  if (last_split) {   // the INT8 group: stages G-1 (landed) and G (its copy issued during G-2)
    __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));
    wg_barrier();
    const int p = (G - 1 - ga) % kRing;
#pragma unroll
    for (int pp = 0; pp < kRing; ++pp)
      if (pp == p) compute(Int8W{}, G - 1, LA(pp), LW(pp), LW((pp + 1) % kRing), LS(pp));
  }
  __builtin_amdgcn_s_waitcnt(0);                    // no copy into LDS outlives the workgroup

  if (kAcc) return;
  if (split_mode) {   // the piece's fp32 tile (factor 2 kept), row-major, to its scratch slot
    float* tile = part + ((size_t)split * rem + lin) * (kTile * kTile);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = wm * 64 + i * 32 + l32;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = wn * 64 + j * 32 + q * 8 + kh * 4;
          *reinterpret_cast<float4*>(tile + r * kTile + c) =
              float4{yacc[i][j][4 * q], yacc[i][j][4 * q + 1], yacc[i][j][4 * q + 2], yacc[i][j][4 * q + 3]};
        }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int m = m0 + wm * 64 + i * 32 + l32;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + wn * 64 + j * 32 + q * 8 + kh * 4;
        const uint16_t o[4] = {__half_as_ushort(__float2half_rn(0.5f * yacc[i][j][4 * q])),
                               __half_as_ushort(__float2half_rn(0.5f * yacc[i][j][4 * q + 1])),
                               __half_as_ushort(__float2half_rn(0.5f * yacc[i][j][4 * q + 2])),
                               __half_as_ushort(__float2half_rn(0.5f * yacc[i][j][4 * q + 3]))};
        if (m >= M) continue;
        uint16_t* dst = Y + (size_t)m * N + n;
        if (n + 4 <= N && (N & 3) == 0) {
          *reinterpret_cast<ushort4*>(dst) = ushort4{o[0], o[1], o[2], o[3]};
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < N) dst[e] = o[e];
        }
      }
  }
}

}  // namespace

hipError_t launch_gemm_w4a8(const uint8_t* Xq, const uint16_t* sx, const uint8_t* Wq, const uint16_t* sw, int M,
                            int N, int K, uint16_t* Y, int32_t* acc, float* part, const GemmPlan& plan,
                            hipStream_t stream) {
  const int tiles = ((M + kTile - 1) / kTile) * ((N + kTile - 1) / kTile);
  const bool split = !acc && plan.rem > 0 && part;
  const dim3 grid(split ? plan.rem * plan.splits : tiles);
  // the ring for pieces of many groups, the register-staged kernel otherwise (measured below)
  const int groups = (K / ATOM_GROUP - 1) / (split ? plan.splits : 1);
  const bool ring = groups >= kRingMinGroups;
  if (acc) {
    if (ring)
      hipLaunchKernelGGL(gemm_w4a8_ring_kernel<true>, grid, dim3(kThreads), 0, stream, Xq, sx, Wq, sw, M, N, K, Y, acc,
                         0, 1, (float*)nullptr);
    else
      hipLaunchKernelGGL(gemm_w4a8_kernel<true>, grid, dim3(kThreads), 0, stream, Xq, sx, Wq, sw, M, N, K, Y, acc, 0,
                         1, (float*)nullptr, (int)grid.x);
  } else {
    if (ring)
      hipLaunchKernelGGL(gemm_w4a8_ring_kernel<false>, grid, dim3(kThreads), 0, stream, Xq, sx, Wq, sw, M, N, K, Y,
                         (int32_t*)nullptr, split ? plan.rem : 0, split ? plan.splits : 1, part);
    else
      hipLaunchKernelGGL(gemm_w4a8_kernel<false>, grid, dim3(kThreads), 0, stream, Xq, sx, Wq, sw, M, N, K, Y,
                         (int32_t*)nullptr, split ? plan.rem : 0, split ? plan.splits : 1, part,
                         (int)grid.x > 2 * compute_units() ? 2 * compute_units() : (int)grid.x);
  }
  if (split) return launch_splitk_finish(part, plan, M, N, Y, stream);
  return hipGetLastError();
}

}  // namespace atom
