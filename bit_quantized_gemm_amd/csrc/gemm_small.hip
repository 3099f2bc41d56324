// W4A4 GEMM for few token rows (M <= 16, the decode regime) on gfx950.
//
// Same product as gemm.hip (per 128-channel group g: an exact integer dot product of the
// codes, scaled by sx[g,m] * sw[g,n] in fp32 and summed over groups; quantization record of
// "Atom: Low-bit Quantization for Efficient and Accurate LLM Serving", Fields "Bits",
// "Weight group size", "notes"), organised for a different bound.  With at most 16 rows of
// activations every weight byte is used at most 16 times, so the time to beat is that of
// reading the packed weights once from HBM; 128 x 128 tiles would waste 7/8 of every MFMA and
// leave the copies latency-bound.
//
// Work layout.  A workgroup owns 16 output columns.  K is cut into ranges of at most MAXG
// INT4 groups (the last range also takes the INT8 outlier group): 4, or 6 when ranges of 4
// would need more than 16 waves, or 8 (at most 4 waves) when there are more column blocks than
// two workgroups of 8 waves per compute unit can hold at once; the workgroup has one wave per
// range, at most 16, and a wave takes every 16th range when there are more.  A wave issues every load of a range at once straight into registers (no LDS
// staging, no barrier), then runs one 16 x 16 x 128 fp6 MFMA per group.  At the end the waves'
// fp32 sums meet in LDS and wave 0 adds them in wave order and writes Y: one kernel, no
// scratch, deterministic.
//
// Operands.  Lane l supplies row (A: weight column n0 + l % 16; B: token row l % 16) and the
// K slice l / 16 of each operand: the 32 codes in bytes 16 (l / 16) .. 16 (l / 16) + 15 of the
// group's 64-byte stage, two packed units, which four bit operations per unit turn into six
// words of fp6 e2m3 fields (the subnormal q / 8; the layout is described in atom_internal.h).
// Both operands use the same assignment, so every code of the group meets its partner once.
// With the weights as the first operand the 16 x 16 accumulator holds the output transposed:
// lane l owns token row l % 16 and the four consecutive output columns 4 (l / 16) .. + 3.
//
// Scales.  v_mfma_f32_16x16x16_f16 with each lane's fp16 scale in element 0 of its four
// K values gives 4 * sw * sx exactly (four equal exact products) in the accumulator layout;
// the factor 4 is removed at the end (a power of two: no rounding).
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "atom_internal.h"

namespace atom {
namespace {

typedef int32_t v8i __attribute__((ext_vector_type(8)));
typedef int32_t v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));

constexpr int kCols = 16;                    // output columns per workgroup
constexpr int kScaleE8M0 = 127 + 3;          // 2^3: the e2m3 subnormal q / 8 counts as q

// Two packed units (16 bytes) -> the fp6 operand of their 32 codes (six words; the last two
// are not read by the fp6 MFMA).
__device__ __forceinline__ v8i fp6_operand(uint4 v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  v8i r;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const uint32_t w0 = w[2 * u], w1 = w[2 * u + 1];
    r[3 * u] = (int)(w0 & ~kFp6Exp0);
    r[3 * u + 1] = (int)(w1 & ~kFp6Exp1);
    r[3 * u + 2] = (int)((w0 & kFp6Exp0) | (w1 & kFp6Exp1));
  }
  r[6] = 0;
  r[7] = 0;
  return r;
}

__device__ __forceinline__ h4 scale_operand(uint16_t v) {
  return h4{__builtin_bit_cast(_Float16, v), (_Float16)0, (_Float16)0, (_Float16)0};
}

constexpr int kMaxWaves = 16;                // waves (K ranges in flight) per workgroup
constexpr int kDeepMinBlocks = 512;          // column blocks beyond which ranges of 8 are taken

// The kAcc stores sit under a per-lane branch (token rows past M store nothing).  Left alone,
// the compiler sinks the operand decode and the MFMA that feed a store into that branch; the
// decode then runs with those lanes switched off, and the matrix core, which reads every lane,
// multiplies stale operand registers for their rows.  An empty asm statement that takes the
// result as an in/out operand pins the MFMA (and everything it reads) before the branch.
__device__ __forceinline__ void keep_in_all_lanes(v4f& v) { asm volatile("" : "+v"(v)); }

// blockIdx.x: column block (columns n0 = 16 blockIdx.x ..); wave w handles K ranges w, w + waves, ...
// kAcc = true: write each group's exact integer sums to acc_out [G, M, N] instead of Y (the
// same loads, decode and MFMAs; no scales are read).
template <int MAXG, bool kAcc>
__global__ __launch_bounds__(MAXG == 8 ? 256 : kMaxWaves * 64) void gemm_w4a4_small_kernel(const uint8_t* __restrict__ Xq,
                                                                         const uint16_t* __restrict__ sx,
                                                                         const uint8_t* __restrict__ Wq,
                                                                         const uint16_t* __restrict__ sw, int M,
                                                                         int N, int K, int ranges,
                                                                         uint16_t* __restrict__ Y,
                                                                         int32_t* __restrict__ acc_out) {
  __shared__ v4f red[kMaxWaves][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, waves = blockDim.x >> 6;
  const int r = lane & 15, slice = lane >> 4;
  const int G = K / ATOM_GROUP;
  const size_t rb = (size_t)(K - ATOM_OUTLIERS) / 2 + ATOM_OUTLIERS;
  const int n0 = blockIdx.x * kCols;
  // rows past N / M repeat the last valid one; their results are never stored
  const int n = min(n0 + r, N - 1), m = min(r, M - 1);
  const uint8_t* wrow = Wq + (size_t)n * rb + 16 * slice;
  const uint8_t* xrow = Xq + (size_t)m * rb + 16 * slice;
  const int c0 = n0 + 4 * slice;                     // this lane's first output column
  // kAcc: this lane's sums of group g are token row r, columns c0 .. c0 + 3
  auto store_acc = [&](int g, v4f a) {
    if (r >= M) return;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (c0 + j < N) acc_out[((size_t)g * M + r) * N + c0 + j] = (int32_t)a[j];   // exact integers
  };

  v4f yacc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int range = wave; range < ranges; range += waves) {
    const int ga = range * (G - 1) / ranges, gb = (range + 1) * (G - 1) / ranges;   // 1 .. MAXG
    const int ng = gb - ga;                                                         // uniform
    const bool last = range == ranges - 1;                                          // uniform
    // Every load of the range is issued, unconditionally, before any of it is used (a load
    // under a branch would first wait for all earlier ones).  Groups past the range's end
    // repeat its last group, and outside the last range the INT8 group's loads repeat group
    // ga's bytes and scales: in bounds, cached, never used.
    uint4 wl[MAXG], xl[MAXG];
    uint16_t wsc[MAXG], xsc[MAXG];
#pragma unroll
    for (int i = 0; i < MAXG; ++i) {
      const int g = min(ga + i, gb - 1);
      wl[i] = *reinterpret_cast<const uint4*>(wrow + (size_t)g * 64);
      xl[i] = *reinterpret_cast<const uint4*>(xrow + (size_t)g * 64);
      if (!kAcc) {
        wsc[i] = sw[(size_t)g * N + n];
        xsc[i] = sx[(size_t)g * M + m];
      }
    }
    // INT8 outlier group: the 16-byte K slice of each 64-byte half
    const size_t o8 = last ? rb - ATOM_OUTLIERS : (size_t)ga * 64;
    const size_t c8 = last ? 64 : 0;
    const int g8 = last ? G - 1 : ga;
    v4i w8[2], x8[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      w8[c] = *reinterpret_cast<const v4i*>(Wq + (size_t)n * rb + o8 + 16 * slice + c8 * c);
      x8[c] = *reinterpret_cast<const v4i*>(Xq + (size_t)m * rb + o8 + 16 * slice + c8 * c);
    }
    const uint16_t wsc8 = kAcc ? (uint16_t)0 : sw[(size_t)g8 * N + n];
    const uint16_t xsc8 = kAcc ? (uint16_t)0 : sx[(size_t)g8 * M + m];
    __builtin_amdgcn_sched_barrier(0);   // keep every load ahead of the first use
    // Branch-free as well (a load used only under a branch gets sunk into it): a repeated
    // group gets a zero scale product and adds exactly +0.
#pragma unroll
    for (int i = 0; i < MAXG; ++i) {
      const v8i a = fp6_operand(wl[i]);
      const v8i b = fp6_operand(xl[i]);
      // cbsz = blgp = 2: both operands fp6 e2m3
      const v4f acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, v4f{}, 2, 2, 0, kScaleE8M0, 0, kScaleE8M0);
      if (kAcc) {
        v4f a4 = acc;
        keep_in_all_lanes(a4);
        if (i < ng) store_acc(ga + i, a4);
        continue;
      }
      const uint16_t ws = i < ng ? wsc[i] : (uint16_t)0;
      const v4f sp = __builtin_amdgcn_mfma_f32_16x16x16f16(scale_operand(ws), scale_operand(xsc[i]), v4f{}, 0, 0, 0);
#pragma unroll
      for (int j = 0; j < 4; ++j) yacc[j] = __builtin_fmaf(acc[j], sp[j], yacc[j]);
    }
    {   // INT8 group, counted by the last range only (zero scale product elsewhere)
      v4i acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(w8[0], x8[0], v4i{}, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(w8[1], x8[1], acc, 0, 0, 0);
      if (kAcc) {
        v4f a4 = v4f{(float)acc[0], (float)acc[1], (float)acc[2], (float)acc[3]};
        keep_in_all_lanes(a4);
        if (last) store_acc(G - 1, a4);
        continue;
      }
      const uint16_t ws = last ? wsc8 : (uint16_t)0;
      const v4f sp = __builtin_amdgcn_mfma_f32_16x16x16f16(scale_operand(ws), scale_operand(xsc8), v4f{}, 0, 0, 0);
#pragma unroll
      for (int j = 0; j < 4; ++j) yacc[j] = __builtin_fmaf((float)acc[j], sp[j], yacc[j]);   // |acc| < 2^24: exact
    }
  }

  if (kAcc) return;
  red[wave][lane] = yacc;
  __syncthreads();
  if (wave != 0) return;
  v4f y = red[0][lane];
  for (int w = 1; w < waves; ++w) {
    const v4f v = red[w][lane];
#pragma unroll
    for (int j = 0; j < 4; ++j) y[j] += v[j];
  }
  // lane: token row r, columns n0 + 4 slice .. + 3; the factor 4 of the scale products goes
  if (r >= M) return;
  uint16_t* dst = Y + (size_t)r * N + c0;
  const uint16_t o[4] = {__half_as_ushort(__float2half_rn(0.25f * y[0])), __half_as_ushort(__float2half_rn(0.25f * y[1])),
                         __half_as_ushort(__float2half_rn(0.25f * y[2])), __half_as_ushort(__float2half_rn(0.25f * y[3]))};
  if (c0 + 4 <= N && (N & 3) == 0) {
    *reinterpret_cast<ushort4*>(dst) = ushort4{o[0], o[1], o[2], o[3]};
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (c0 + j < N) dst[j] = o[j];
  }
}

}  // namespace

namespace {
// Range plan: ranges of 4 groups while they fit one wave each; beyond 16 ranges, ranges of 6
// (fewer waves that take a second range).  Measured on 16-token batches (event-timed): 16 x
// 11008 x 4096 (85 INT4 groups) 11.3 -> 10.7 us with ranges of 6; with 31 INT4 groups ranges of
// 6 are slower (16 x 4096 x 11008: 11.1 -> 11.4 us), and ranges of 2 are slower everywhere.
// More than 512 column blocks with at most 32 INT4 groups: ranges of 8 in workgroups of at most
// 4 waves (160 VGPRs, three workgroups per compute unit), so that every block is resident at
// once instead of 1.34 rounds of 8-wave workgroups (kernel trace, 16 x 4096 x 11008: 8.96 ->
// 8.17 us; its 688 blocks).
template <bool kAcc>
hipError_t launch_small(const uint8_t* Xq, const uint16_t* sx, const uint8_t* Wq, const uint16_t* sw, int M, int N,
                        int K, uint16_t* Y, int32_t* acc, hipStream_t stream) {
  const int G = K / ATOM_GROUP;
  const bool wide = (G - 1 + 3) / 4 > kMaxWaves;
  const bool deep = !wide && G - 1 <= 4 * 8 && (N + kCols - 1) / kCols > kDeepMinBlocks;
  const int maxg = wide ? 6 : deep ? 8 : 4;
  const int ranges = (G - 1 + maxg - 1) / maxg;
  const int waves = ranges < kMaxWaves ? ranges : kMaxWaves;
  const dim3 grid((N + kCols - 1) / kCols), block(64 * waves);
  if (deep)
    hipLaunchKernelGGL((gemm_w4a4_small_kernel<8, kAcc>), grid, block, 0, stream, Xq, sx, Wq, sw, M, N, K, ranges, Y,
                       acc);
  else if (wide)
    hipLaunchKernelGGL((gemm_w4a4_small_kernel<6, kAcc>), grid, block, 0, stream, Xq, sx, Wq, sw, M, N, K, ranges, Y,
                       acc);
  else
    hipLaunchKernelGGL((gemm_w4a4_small_kernel<4, kAcc>), grid, block, 0, stream, Xq, sx, Wq, sw, M, N, K, ranges, Y,
                       acc);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_gemm_small(const uint8_t* Xq, const uint16_t* sx, const uint8_t* Wq, const uint16_t* sw, int M,
                             int N, int K, uint16_t* Y, hipStream_t stream) {
  return launch_small<false>(Xq, sx, Wq, sw, M, N, K, Y, nullptr, stream);
}

hipError_t launch_gemm_small_group_acc(const uint8_t* Xq, const uint8_t* Wq, int M, int N, int K, int32_t* acc,
                                       hipStream_t stream) {
  return launch_small<true>(Xq, nullptr, Wq, nullptr, M, N, K, nullptr, acc, stream);
}

}  // namespace atom
