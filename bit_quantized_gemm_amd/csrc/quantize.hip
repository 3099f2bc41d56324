// Row quantize for gfx950: reorder through perm, per-128 group absmax, fp16 scale,
// INT4 codes packed two per byte, INT8 codes for the 128-channel outlier tail.
//
// One kernel serves both the runtime activation quantize (rows = tokens) and the offline
// weight pack (rows = output channels): the quantization record "Atom (mixed-precision
// block-outlier low-bit quantization for serving)" gives one rule for both operands
// (Field "Bits": w4a4; "Weight group size": 128; "notes": each contiguous 128-element group is
// quantized independently, plus one 128-channel high-precision group).
//
// Work layout: one 256-thread workgroup per row.  The fp16 row is staged in LDS with
// 16-byte loads, then every thread gathers 8 consecutive reordered elements through perm
// (a group of 128 is 16 neighbouring lanes), reduces the group absmax across those 16 lanes,
// and writes its 8 codes as one 32-bit word (INT4) or 8 bytes (INT8 tail): each group's
// 16 lanes store a contiguous 64- or 128-byte run.
//
// Exact codes without a per-element IEEE division: with r = 1/s correctly rounded,
// t = x*r, e = fma(-t, s, x), u = fma(e, r, t), the integer nearest u (ties to even) equals
// the integer nearest the correctly rounded fp32 quotient x/s for every fp16 x and every
// fp16 scale s this rule can produce (checked over all 2.0e9 such pairs on the CPU).
// Adding 1.5*2^23 rounds the clamped value to that integer with ties to even and leaves its
// two's-complement low byte in the low bits of the sum.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "atom_internal.h"

#pragma clang fp contract(off)

namespace atom {
namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = 8;

__device__ __forceinline__ float half_bits_to_float(uint16_t h) { return __half2float(__ushort_as_half(h)); }

// Code of x for scale s (> 0) with reciprocal r, as the low byte of the returned word.
__device__ __forceinline__ uint32_t code_bits(float x, float s, float r, float qmax) {
  const float t = x * r;
  const float e = __builtin_fmaf(-t, s, x);
  const float u = __builtin_fmaf(e, r, t);
  const float v = __builtin_fminf(__builtin_fmaxf(u, -qmax), qmax);
  return __float_as_uint(v + 12582912.0f);
}

__global__ __launch_bounds__(kThreads) void row_quantize_kernel(const uint16_t* __restrict__ X,
                                                                const int32_t* __restrict__ perm, int rows, int K,
                                                                uint8_t* __restrict__ Q, uint16_t* __restrict__ S) {
  extern __shared__ uint4 lds_row4[];
  const uint16_t* lds_row = reinterpret_cast<const uint16_t*>(lds_row4);
  const int row = blockIdx.x;
  const int G = K / ATOM_GROUP;
  const int klo = K - ATOM_OUTLIERS;
  const size_t rb = (size_t)(klo / 2 + ATOM_OUTLIERS);

  const uint4* src = reinterpret_cast<const uint4*>(X + (size_t)row * K);
  for (int i = threadIdx.x; i < K / 8; i += kThreads) lds_row4[i] = src[i];
  __syncthreads();

  uint8_t* qrow = Q + (size_t)row * rb;
  const unsigned kmax = (unsigned)(K - 1);
  for (int c = threadIdx.x * kPerThread; c < K; c += kThreads * kPerThread) {
    const int g = c / ATOM_GROUP;
    const bool tail = g == G - 1;
    const int4 p0 = *reinterpret_cast<const int4*>(perm + c);
    const int4 p1 = *reinterpret_cast<const int4*>(perm + c + 4);
    const int pi[kPerThread] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
    float x[kPerThread];
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const unsigned idx = __builtin_elementwise_min((unsigned)pi[i], kmax);   // bad perm: clamp, no fault
      x[i] = half_bits_to_float(lds_row[idx]);
      a = __builtin_fmaxf(a, __builtin_fabsf(x[i]));
    }
    // group absmax over the 16 lanes that share this group
    a = __builtin_fmaxf(a, __shfl_xor(a, 1));
    a = __builtin_fmaxf(a, __shfl_xor(a, 2));
    a = __builtin_fmaxf(a, __shfl_xor(a, 4));
    a = __builtin_fmaxf(a, __shfl_xor(a, 8));

    const float qmax = tail ? 127.0f : 7.0f;
    const __half s16 = __float2half_rn(a / qmax);      // correctly rounded fp32 divide, then RNE to fp16
    const float s = __half2float(s16);
    uint32_t b[kPerThread];
    if (s > 0.0f) {
      const float r = 1.0f / s;
#pragma unroll
      for (int i = 0; i < kPerThread; ++i) b[i] = code_bits(x[i], s, r, qmax);
    } else {
#pragma unroll
      for (int i = 0; i < kPerThread; ++i) b[i] = 0;
    }
    if (!tail) {
      uint32_t w = 0;
#pragma unroll
      for (int i = 0; i < kPerThread; ++i) w |= (b[i] & 0xfu) << (4 * i);
      *reinterpret_cast<uint32_t*>(qrow + c / 2) = w;
    } else {
      uint2 w;
      w.x = (b[0] & 0xff) | ((b[1] & 0xff) << 8) | ((b[2] & 0xff) << 16) | ((b[3] & 0xff) << 24);
      w.y = (b[4] & 0xff) | ((b[5] & 0xff) << 8) | ((b[6] & 0xff) << 16) | ((b[7] & 0xff) << 24);
      *reinterpret_cast<uint2*>(qrow + klo / 2 + (c - klo)) = w;
    }
    if ((threadIdx.x & 15) == 0) S[(size_t)g * rows + row] = __half_as_ushort(s16);
  }
}

}  // namespace

hipError_t launch_row_quantize(const uint16_t* X, const int32_t* perm, int rows, int K, uint8_t* Q, uint16_t* S,
                               hipStream_t stream) {
  const size_t lds = (size_t)K * sizeof(uint16_t);
  hipLaunchKernelGGL(row_quantize_kernel, dim3(rows), dim3(kThreads), lds, stream, X, perm, rows, K, Q, S);
  return hipGetLastError();
}

}  // namespace atom
