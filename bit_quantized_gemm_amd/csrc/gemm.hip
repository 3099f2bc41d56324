// W4A4 grouped GEMM for gfx950 on int8 MFMA.
//
// Y[m,n] = sum over 128-channel groups g of acc_g[m,n] * sx[g,m] * sw[g,n], with
// acc_g = exact integer dot product of the codes of group g.  The method runs this product
// on integer operators (index page of "Atom: Low-bit Quantization for Efficient and Accurate
// LLM Serving", Abstract; quantization record, "notes": an integer-operator path).  gfx950
// has no 4-bit MFMA, so the INT4 groups are widened to int8 in registers and fed to
// v_mfma_i32_16x16x64_i8; the INT8 outlier group (record, "notes": a 128-channel
// high-precision group) feeds the same instruction without widening.
//
// Nibble widening.  For a packed word w holding codes c0..c7 (c_{2j} in the low nibble of
// byte j), w & 0xF0F0F0F0 holds 16*c_{2j+1} and (w << 4) & 0xF0F0F0F0 holds 16*c_{2j} as
// int8 bytes.  Both operands are widened the same way, so an MFMA over the "low" words and
// one over the "high" words together cover every channel of the group once, and the
// accumulator holds 256 * acc_g exactly (|256*acc_g| <= 128*112*112 < 2^21).  The factor
// 1/256 is folded into the fp32 activation scale (a power of two: exact).
//
// Tiling: a 256-thread workgroup computes a 128x128 tile of Y; its four waves each own a
// 64x64 sub-tile held as 4x4 MFMA tiles of 16x16.  Per group, the packed A and B tiles
// (64 bytes per row, 128 for the INT8 group) are staged in LDS with 16-byte loads; each lane
// reads one 16-byte word per MFMA tile row, widens it, and issues two MFMAs per tile.
// After each group the int32 accumulators are scaled into fp32 and cleared.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "atom_internal.h"

namespace atom {
namespace {

typedef int32_t v4i __attribute__((ext_vector_type(4)));

constexpr int kBM = 128;
constexpr int kBN = 128;
constexpr int kThreads = 256;
constexpr int kRowStride = 128 + 16;     // LDS bytes per staged row (INT8 group needs 128)

__device__ __forceinline__ v4i widen_lo(uint4 p) {
  v4i r;
  r[0] = (int32_t)((p.x << 4) & 0xF0F0F0F0u);
  r[1] = (int32_t)((p.y << 4) & 0xF0F0F0F0u);
  r[2] = (int32_t)((p.z << 4) & 0xF0F0F0F0u);
  r[3] = (int32_t)((p.w << 4) & 0xF0F0F0F0u);
  return r;
}

__device__ __forceinline__ v4i widen_hi(uint4 p) {
  v4i r;
  r[0] = (int32_t)(p.x & 0xF0F0F0F0u);
  r[1] = (int32_t)(p.y & 0xF0F0F0F0u);
  r[2] = (int32_t)(p.z & 0xF0F0F0F0u);
  r[3] = (int32_t)(p.w & 0xF0F0F0F0u);
  return r;
}

__device__ __forceinline__ v4i as_v4i(uint4 p) {
  v4i r;
  r[0] = (int32_t)p.x;
  r[1] = (int32_t)p.y;
  r[2] = (int32_t)p.z;
  r[3] = (int32_t)p.w;
  return r;
}

// kAcc = false: Y output.  kAcc = true: write the per-group integer accumulators instead.
template <bool kAcc>
__global__ __launch_bounds__(kThreads) void gemm_w4a4_kernel(const uint8_t* __restrict__ Xq,
                                                             const uint16_t* __restrict__ sx,
                                                             const uint8_t* __restrict__ Wq,
                                                             const uint16_t* __restrict__ sw, int M, int N, int K,
                                                             uint16_t* __restrict__ Y, int32_t* __restrict__ acc_out) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_a[kBM * kRowStride];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b[kBN * kRowStride];
  __shared__ __attribute__((aligned(16))) float lds_sx[kBM];
  __shared__ __attribute__((aligned(16))) float lds_sw[kBN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1;          // wave row in the 2x2 wave grid
  const int wn = wave & 1;
  const int m0 = blockIdx.y * kBM;
  const int n0 = blockIdx.x * kBN;
  const int G = K / ATOM_GROUP;
  const size_t rb = (size_t)((K - ATOM_OUTLIERS) / 2 + ATOM_OUTLIERS);

  const int l16 = lane & 15;          // row (A) / column (B) inside a 16-wide MFMA tile
  const int kq = lane >> 4;           // which 16-byte quarter of the 64-byte K chunk

  float yacc[4][4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) yacc[i][j][r] = 0.0f;

  for (int g = 0; g < G; ++g) {
    const bool tail = g == G - 1;
    const int chunks = tail ? 8 : 4;               // 16-byte chunks per row for this group
    const size_t goff = (size_t)g * 64;            // byte offset of the group in a packed row

    // ---- stage the A and B tiles of this group (rows past M/N repeat the last row)
    for (int i = tid; i < kBM * chunks; i += kThreads) {
      const int r = i / chunks, ch = i % chunks;
      const int gm = min(m0 + r, M - 1);
      *reinterpret_cast<uint4*>(lds_a + r * kRowStride + ch * 16) =
          *reinterpret_cast<const uint4*>(Xq + (size_t)gm * rb + goff + ch * 16);
    }
    for (int i = tid; i < kBN * chunks; i += kThreads) {
      const int r = i / chunks, ch = i % chunks;
      const int gn = min(n0 + r, N - 1);
      *reinterpret_cast<uint4*>(lds_b + r * kRowStride + ch * 16) =
          *reinterpret_cast<const uint4*>(Wq + (size_t)gn * rb + goff + ch * 16);
    }
    if (!kAcc) {
      const float f = tail ? 1.0f : (1.0f / 256.0f);
      if (tid < kBM) {
        const int gm = min(m0 + tid, M - 1);
        lds_sx[tid] = __half2float(__ushort_as_half(sx[(size_t)g * M + gm])) * f;
      } else {
        const int t = tid - kBM;
        const int gn = min(n0 + t, N - 1);
        lds_sw[t] = __half2float(__ushort_as_half(sw[(size_t)g * N + gn]));
      }
    }
    __syncthreads();

    // ---- integer products of this group
    v4i acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = v4i{0, 0, 0, 0};

#pragma unroll
    for (int half = 0; half < 2; ++half) {
      v4i af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ra = wm * 64 + i * 16 + l16;
        const int rbw = wn * 64 + i * 16 + l16;
        if (!tail) {
          const uint4 pa = *reinterpret_cast<const uint4*>(lds_a + ra * kRowStride + kq * 16);
          const uint4 pb = *reinterpret_cast<const uint4*>(lds_b + rbw * kRowStride + kq * 16);
          af[i] = half ? widen_hi(pa) : widen_lo(pa);
          bf[i] = half ? widen_hi(pb) : widen_lo(pb);
        } else {
          af[i] = as_v4i(*reinterpret_cast<const uint4*>(lds_a + ra * kRowStride + half * 64 + kq * 16));
          bf[i] = as_v4i(*reinterpret_cast<const uint4*>(lds_b + rbw * kRowStride + half * 64 + kq * 16));
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
    }

    // ---- epilogue of this group
    if (kAcc) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int m = m0 + wm * 64 + i * 16 + kq * 4 + r;
            const int n = n0 + wn * 64 + j * 16 + l16;
            if (m < M && n < N) {
              const int32_t v = tail ? acc[i][j][r] : (acc[i][j][r] >> 8);   // exact: a multiple of 256
              acc_out[((size_t)g * M + m) * N + n] = v;
            }
          }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 s4 = *reinterpret_cast<const float4*>(&lds_sx[wm * 64 + i * 16 + kq * 4]);
        const float sxr[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float swc = lds_sw[wn * 64 + j * 16 + l16];
#pragma unroll
          for (int r = 0; r < 4; ++r)
            yacc[i][j][r] = __builtin_fmaf((float)acc[i][j][r], sxr[r] * swc, yacc[i][j][r]);
        }
      }
    }
    __syncthreads();
  }

  if (!kAcc) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = m0 + wm * 64 + i * 16 + kq * 4 + r;
          const int n = n0 + wn * 64 + j * 16 + l16;
          if (m < M && n < N) Y[(size_t)m * N + n] = __half_as_ushort(__float2half_rn(yacc[i][j][r]));
        }
  }
}

}  // namespace

hipError_t launch_gemm(const uint8_t* Xq, const uint16_t* sx, const uint8_t* Wq, const uint16_t* sw, int M, int N,
                       int K, uint16_t* Y, hipStream_t stream) {
  const dim3 grid((N + kBN - 1) / kBN, (M + kBM - 1) / kBM);
  hipLaunchKernelGGL(gemm_w4a4_kernel<false>, grid, dim3(kThreads), 0, stream, Xq, sx, Wq, sw, M, N, K, Y,
                     (int32_t*)nullptr);
  return hipGetLastError();
}

hipError_t launch_gemm_group_acc(const uint8_t* Xq, const uint8_t* Wq, int M, int N, int K, int32_t* acc,
                                 hipStream_t stream) {
  const dim3 grid((N + kBN - 1) / kBN, (M + kBM - 1) / kBM);
  hipLaunchKernelGGL(gemm_w4a4_kernel<true>, grid, dim3(kThreads), 0, stream, Xq, (const uint16_t*)nullptr, Wq,
                     (const uint16_t*)nullptr, M, N, K, (uint16_t*)nullptr, acc);
  return hipGetLastError();
}

}  // namespace atom
