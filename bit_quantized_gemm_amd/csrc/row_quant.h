// Device-side row quantizer for gfx950, shared by the row quantize kernel (quantize.hip) and the
// fused quantize + GEMM kernel (linear.hip): reorder through perm, per-128 group absmax, fp16
// scale, INT4 codes packed four bits each, INT8 codes for the 128-channel outlier tail (the
// quantization record "Atom (mixed-precision block-outlier low-bit quantization for serving)",
// Fields "Bits", "Weight group size", "notes").  The arithmetic and the packed layouts are
// described at the top of quantize.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "atom_internal.h"

namespace atom {
namespace rowq {


typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kPerThread = 16;                       // reordered elements per thread per pass
constexpr int kLanesPerGroup = ATOM_GROUP / kPerThread;   // 8

// Column stride (32-bit words) of the staged row: the smallest value >= K/16 that is 8 mod 64.
__host__ __device__ constexpr int staged_stride(int K) { return K / 16 + ((8 - K / 16) & 63); }

// max over the 8 lanes of a group (lanes 8k..8k+7) via DPP: xor 1, xor 2 (quad perms), then
// the half-row mirror (lane i <-> 7-i), which pairs the two quads of the group.  The values
// are absolute values (sign bit clear), whose order as unsigned integers is their order as
// floats, so the maximum is taken on the bits.
__device__ __forceinline__ float group_max8(float a) {
  unsigned u = __builtin_bit_cast(unsigned, a);
  u = max(u, (unsigned)__builtin_amdgcn_mov_dpp((int)u, 0xB1, 0xF, 0xF, false));
  u = max(u, (unsigned)__builtin_amdgcn_mov_dpp((int)u, 0x4E, 0xF, 0xF, false));
  u = max(u, (unsigned)__builtin_amdgcn_mov_dpp((int)u, 0x141, 0xF, 0xF, false));
  return __builtin_bit_cast(float, u);
}

// Quotient of x for scale s (> 0) with reciprocal r; its nearest integer (ties to even),
// clamped to [-qmax, qmax], is the code.
__device__ __forceinline__ float code_quotient(_Float16 xh, float s, float r) {
  const float x = (float)xh;
  // t = x * r, written as an fma with +0 so that it cannot become a plain multiply of a
  // converted x: the two differ only in the sign of a zero product, which then rounds to the
  // same code 0
  const float t = __builtin_fmaf(x, r, 0.0f);
  const float e = __builtin_fmaf(-t, s, x);
  return __builtin_fmaf(e, r, t);
}

// The smallest normal fp16 value.  A normal scale is a / qmax rounded to fp16, within a
// relative 2^-11 of it, so every quotient of the group lies below qmax + 1/2 and rounds into
// [-qmax, qmax] by itself; only a subnormal scale (tiny groups) can need the clamp.
constexpr float kMinNormalHalf = 6.103515625e-05f;

// Adding 1.5 * 2^23 rounds to an integer (ties to even) and leaves it in the low bits.
constexpr float kRound = 12582912.0f;

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x6 __attribute__((ext_vector_type(6)));

// fp16 pair (rint(a) + 1536, rint(b) + 1536), each rounded once from the exact fp32 sum
// (v_fma_mix computes a * 1 + 1536 unrounded and rounds to fp16, whose spacing is 1 on
// [1024, 2048)): ties go to the even integer, as 1536 is even.  Subtracting 1536 afterwards
// gives the integers exactly, with +0 for a zero code.
__device__ __forceinline__ h2 round_pair_biased(float a, float b, float bias) {
  uint32_t d;
  asm("v_fma_mixlo_f16 %0, %1, 1.0, %2\n\tv_fma_mixhi_f16 %0, %3, 1.0, %2" : "=&v"(d) : "v"(a), "s"(bias), "v"(b));
  return __builtin_bit_cast(h2, d);
}
constexpr float kBias16 = 1536.0f;

// low bytes of a,b,c,d -> one word [a, b, c, d]
__device__ __forceinline__ uint32_t pack4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const uint32_t ab = __builtin_amdgcn_perm(b, a, 0x0C0C0400u);   // [a.b0, b.b0, 0, 0]
  const uint32_t cd = __builtin_amdgcn_perm(d, c, 0x04000C0Cu);   // [0, 0, c.b0, d.b0]
  return ab | cd;
}


constexpr int kPassElems = kThreads * kPerThread;    // 4096 reordered elements per pass

// One workgroup of kThreads threads quantizing whole rows.  CHUNKS: 16-byte row chunks each
// thread prefetches (K <= CHUNKS * 2048).  PASSES: passes of 4096 reordered elements per row
// whose gather offsets stay in registers (K <= PASSES * 4096); 0 = read perm from memory on
// every row.  Use: construct, load_perm(), prefetch(first row), finish_offsets(), then per row:
// barrier, stage(), barrier, [prefetch(next row)], quantize(row, ...).  perm's loads go out
// first and the first row's right behind them, so the offsets are computed while the row is
// still in flight.
template <int CHUNKS, int PASSES, int FMT>
struct RowQuant {
  const uint16_t* __restrict__ X;
  const int32_t* __restrict__ perm;
  int rows, K;
  uint8_t* __restrict__ Q;
  uint16_t* __restrict__ S;
  uint32_t* lds_words;                               // the staged row: staged_stride(K) * 8 words
  const int QP, G, klo, nchunks;
  const size_t rb;
  const unsigned kmax;
  int offs[PASSES > 0 ? PASSES : 1][kPerThread];
  u32x4 pre[CHUNKS];

  __device__ __forceinline__ RowQuant(const uint16_t* X_, const int32_t* perm_, int rows_, int K_, uint8_t* Q_,
                                      uint16_t* S_, uint32_t* lds)
      : X(X_), perm(perm_), rows(rows_), K(K_), Q(Q_), S(S_), lds_words(lds), QP(staged_stride(K_)),
        G(K_ / ATOM_GROUP), klo(K_ - ATOM_OUTLIERS),
        nchunks(K_ / 8),                              // 16-byte chunks per row
        rb(FMT == kRowA8 ? (size_t)K_ : (size_t)((K_ - ATOM_OUTLIERS) / 2 + ATOM_OUTLIERS)),
        kmax((unsigned)(K_ - 1)) {}

  // The gather offsets of this thread's passes are kept in registers (PASSES > 0):
  // load_perm() reads its perm entries into them, finish_offsets() turns those into offsets.
  __device__ __forceinline__ void load_perm() {
    if (PASSES > 0) {
#pragma unroll
      for (int ps = 0; ps < (PASSES > 0 ? PASSES : 1); ++ps) {
        const int c = threadIdx.x * kPerThread + ps * kPassElems;
        if (c < K) read_perm(c, offs[ps]);
      }
    }
  }
  __device__ __forceinline__ void finish_offsets() {
    if (PASSES > 0) {
#pragma unroll
      for (int ps = 0; ps < (PASSES > 0 ? PASSES : 1); ++ps) {
        const int c = threadIdx.x * kPerThread + ps * kPassElems;
        if (c < K) perm_to_offsets(offs[ps]);
      }
    }
  }

  // perm entries c .. c+15
  __device__ __forceinline__ void read_perm(int c, int (&off)[kPerThread]) const {
#pragma unroll
    for (int v = 0; v < kPerThread / 4; ++v) {
      const int4 p = *reinterpret_cast<const int4*>(perm + c + 4 * v);
      off[4 * v] = p.x;
      off[4 * v + 1] = p.y;
      off[4 * v + 2] = p.z;
      off[4 * v + 3] = p.w;
    }
  }

  // The 16 perm entries in off -> LDS byte offsets of those elements in the staged row
  // (clamped: a bad perm gives garbage, never an out-of-range read).
  __device__ __forceinline__ void perm_to_offsets(int (&off)[kPerThread]) const {
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) {
      const unsigned e = __builtin_elementwise_min((unsigned)off[u], kmax);
      off[u] = (int)((((e & 15) >> 1) * QP + (e >> 4)) * 4 + (e & 1) * 2);
    }
  }

  // LDS byte offsets of this thread's 16 reordered elements at position c.
  __device__ __forceinline__ void gather_offsets(int c, int (&off)[kPerThread]) const {
    read_perm(c, off);
    perm_to_offsets(off);
  }

  // Loads of this thread's chunks of `row` into registers (in flight until stage()).  Every
  // load is issued (a chunk past the row end reloads the last one, which stage() skips), so the
  // compiler's wait counts for loads issued before these need not allow for missing ones.
  __device__ __forceinline__ void prefetch(int row) {
    const u32x4* src = reinterpret_cast<const u32x4*>(X + (size_t)row * K);
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i) pre[i] = src[min((int)threadIdx.x + i * kThreads, nchunks - 1)];
  }

  // The prefetched row into LDS, stored by columns (see quantize.hip).  The caller brackets
  // this with workgroup barriers.
  __device__ __forceinline__ void stage() {
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i) {
      const int c = threadIdx.x + i * kThreads;
      if (c < nchunks) {
        // chunk c = elements 8c .. 8c+7 = words 4 (c % 2) .. 4 (c % 2) + 3 of column c / 2
        uint32_t* w = lds_words + (c & 1) * 4 * QP + (c >> 1);
        w[0] = pre[i].x;
        w[QP] = pre[i].y;
        w[2 * QP] = pre[i].z;
        w[3 * QP] = pre[i].w;
      }
    }
  }

    // Quantize the 16 reordered elements at position c (gather offsets off) of the LDS row.
    __device__ __forceinline__ void quantize16(int c, const int (&off)[kPerThread], uint8_t* qrow, int row) {
      const int g = c / ATOM_GROUP;
      const bool tail = FMT == kRowA8 || g == G - 1;     // INT8 codes
      // The elements stay fp16: the absmax is taken in fp16 (exact), and each fp32 step that
      // reads x takes it as a mixed-precision fma operand, so no element is converted.
      _Float16 x[kPerThread];
      _Float16 ah = (_Float16)0.0f;
  #pragma unroll
      for (int i = 0; i < kPerThread; ++i) {
        x[i] = __builtin_bit_cast(_Float16, *reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(lds_words) + off[i]));
        ah = __builtin_fmaxf16(ah, __builtin_fabsf16(x[i]));
      }
      const float a = group_max8((float)ah);

      const float qmax = tail ? 127.0f : 7.0f;
      // s = fp16_rne(fl32(a / qmax)) without a divide: q1 (the quotient through the rounded
      // reciprocal, corrected once) can differ from the fp32 quotient, but never in its fp16
      // rounding, for any fp16 a and either qmax (checked over all fp16 values on the CPU)
      const float qinv = tail ? 1.0f / 127.0f : 1.0f / 7.0f;
      const float q0 = a * qinv;
      const float q1 = __builtin_fmaf(__builtin_fmaf(-q0, qmax, a), qinv, q0);
      const __half s16 = __float2half_rn(q1);
      const float s = __half2float(s16);
      // r = fl32(1 / s): the hardware reciprocal (within one ulp) refined by one Newton step is
      // the correctly rounded reciprocal for every fp16 s > 0 (checked on the CPU for all three
      // starting values within one ulp).  s == 0 (an all-zero group, or a scale that underflows
      // fp16): r = 0 makes every code 0, since then t = 0, e = x, u = 0 for the group's (zero)
      // elements; no branch needed
      const float r0 = __builtin_amdgcn_rcpf(s);
      const float r = s > 0.0f ? __builtin_fmaf(__builtin_fmaf(-s, r0, 1.0f), r0, r0) : 0.0f;
      float v[kPerThread];
  #pragma unroll
      for (int i = 0; i < kPerThread; ++i) v[i] = code_quotient(x[i], s, r);
      // the clamp, only where a group of the wave has a subnormal scale (a uniform branch)
      if (__builtin_amdgcn_ballot_w64(s > 0.0f && s < kMinNormalHalf) != 0) {
  #pragma unroll
        for (int i = 0; i < kPerThread; ++i) v[i] = __builtin_amdgcn_fmed3f(v[i], -qmax, qmax);
      }
      if (!tail && FMT == kRowW4A8) {
        // offset-binary nibbles: adding 1.5 * 2^23 + 8 leaves code + 8 (1 .. 15) in the low
        // byte; block k (codes 8k .. 8k+7) is the word whose byte j holds codes 8k+j and 8k+j+4
        uint32_t bb[kPerThread];
  #pragma unroll
        for (int i = 0; i < kPerThread; ++i) bb[i] = __float_as_uint(v[i] + (kRound + 8.0f));
        uint2 w;
        w.x = pack4(bb[0], bb[1], bb[2], bb[3]) | (pack4(bb[4], bb[5], bb[6], bb[7]) << 4);
        w.y = pack4(bb[8], bb[9], bb[10], bb[11]) | (pack4(bb[12], bb[13], bb[14], bb[15]) << 4);
        *reinterpret_cast<uint2*>(qrow + c / 2) = w;
      } else if (!tail) {
        // INT4 unit: the integer codes as fp16, then one conversion to fp6 e2m3 with scale 8
        // (code / 8, exact on the subnormal grid) that packs field i at bits 6i of T0:T1:T2; T2
        // is then folded into the exponent bits of T0 and T1
        h16 n;
  #pragma unroll
        for (int i = 0; i < kPerThread; i += 2) {
          const h2 p = round_pair_biased(v[i], v[i + 1], kBias16) - h2{(_Float16)kBias16, (_Float16)kBias16};
          n[i] = p.x;
          n[i + 1] = p.y;
        }
        const u32x6 t = __builtin_amdgcn_cvt_scalef32_pk32_fp6_f16(
            __builtin_shufflevector(n, n, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, -1, -1, -1, -1, -1, -1,
                                    -1, -1, -1, -1, -1, -1, -1, -1, -1, -1),
            8.0f);
        uint2 w;
        w.x = t[0] | (t[2] & kFp6Exp0);
        w.y = t[1] | (t[2] & kFp6Exp1);
        *reinterpret_cast<uint2*>(qrow + c / 2) = w;
      } else {
        uint32_t b[kPerThread];                            // two's-complement code in the low byte
  #pragma unroll
        for (int i = 0; i < kPerThread; ++i) b[i] = __float_as_uint(v[i] + kRound);
        u32x4 w;
        w.x = pack4(b[0], b[1], b[2], b[3]);
        w.y = pack4(b[4], b[5], b[6], b[7]);
        w.z = pack4(b[8], b[9], b[10], b[11]);
        w.w = pack4(b[12], b[13], b[14], b[15]);
        *reinterpret_cast<u32x4*>(qrow + (FMT == kRowA8 ? c : klo / 2 + (c - klo))) = w;
      }
      if ((threadIdx.x & (kLanesPerGroup - 1)) == 0) S[(size_t)g * rows + row] = __half_as_ushort(s16);
    }

  // Quantize the staged row `row`: every pass (split == 1), or pass `part` only.
  __device__ __forceinline__ void quantize(int row, int part, int split) {
    uint8_t* qrow = Q + (size_t)row * rb;
    if (PASSES > 0) {
#pragma unroll
      for (int ps = 0; ps < (PASSES > 0 ? PASSES : 1); ++ps) {
        const int c = threadIdx.x * kPerThread + ps * kPassElems;
        if (c < K && (split == 1 || ps == part)) quantize16(c, offs[ps], qrow, row);
      }
    } else {
      for (int c = threadIdx.x * kPerThread; c < K; c += kPassElems) {
        int off[kPerThread];
        gather_offsets(c, off);
        quantize16(c, off, qrow, row);
      }
    }
  }
};

}  // namespace rowq
}  // namespace atom
