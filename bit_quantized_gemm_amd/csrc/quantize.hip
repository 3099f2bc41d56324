// Row quantize for gfx950: reorder through perm, per-128 group absmax, fp16 scale,
// INT4 codes packed four bits each, INT8 codes for the 128-channel outlier tail.
//
// One kernel serves both the runtime activation quantize (rows = tokens) and the offline
// weight pack (rows = output channels): the quantization record "Atom (mixed-precision
// block-outlier low-bit quantization for serving)" gives one rule for both operands
// (Field "Bits": w4a4; "Weight group size": 128; "notes": each contiguous 128-element group is
// quantized independently, plus one 128-channel high-precision group).
//
// Work layout.  Persistent workgroups of 256 threads walk the rows (for jobs of 2048 rows or
// more, each XCD owns whole 64-row blocks, whose fp16 scales share cache lines).  A row is
// staged in LDS (fp16, 16-byte loads); the next row's loads are issued into registers before
// the current row is processed, so HBM reads overlap the arithmetic.  The staged row is stored by
// columns: original element e = 16q + r sits in 32-bit word (r / 2) * QP + q, half r % 2,
// where QP >= K/16 is padded to 8 mod 64.  A thread reads 16 consecutive reordered elements,
// which for neighbouring lanes lie 16 elements apart in the row, so the lanes of one read hit
// consecutive words (distinct banks) instead of words 32 bytes apart, and the four 32-bit
// writes of a 16-byte chunk from 64 lanes cover all 64 banks.  The gather offsets through perm are
// computed once per workgroup and kept in registers (no memory traffic in the row loop, so
// nothing else waits behind the prefetch).  Each thread gathers 16 consecutive
// reordered elements through perm; a group of 128 is 8 neighbouring lanes, whose absmax is
// combined with DPP row operations.  Each thread writes its 16 codes as 8 bytes (INT4) or
// 16 bytes (INT8 tail), so a group's 8 lanes store one contiguous 64- or 128-byte run.
//
// Exact codes without a per-element IEEE division (a Markstein-style quotient correction):
// with r = 1/s correctly rounded, t = x*r, e = fma(-t, s, x) (the remainder, rounded once)
// and u = fma(e, r, t), the integer nearest clamp(u) (ties to even) equals the clamped integer
// nearest the correctly rounded fp32 quotient x/s for every fp16 scale s this rule can produce
// and every fp16 x up to the largest absmax giving that scale (tests/quotient_exhaustive.c
// walks all 1.8e9 such pairs for both qmax with IEEE fused multiply-adds on the CPU).  The
// scale itself and r come from a reciprocal and one correction step each, not from an IEEE
// divide (exact for every fp16 input, see quantize16).  INT8 codes: adding 1.5*2^23 rounds
// the clamped value to that integer with ties to even and leaves its two's-complement low
// byte in the low bits of the sum.  INT4 codes: a mixed-precision fma rounds u + 1536 once
// to fp16 (spacing 1 there), which after subtracting 1536 is the integer code as an fp16
// value, +0 for a zero code.
//
// Packed INT4 layout (chosen so that a GEMM turns 16 codes into fp6 e2m3 MFMA operands with
// four bit operations): a unit of 16 consecutive codes c0..c15 is 8 bytes.  Code c_i is the
// fp6 e2m3 field f_i = |c_i| | (c_i < 0) << 5 (the subnormal c_i / 8) at bits 6i .. 6i+5 of a
// 96-bit string T0:T1:T2; the exponent bits (3 and 4 of every field) are zero, and T2's bits
// lie exactly at the exponent positions of T0 (kFp6Exp0) and T1 (kFp6Exp1), so the unit is
// stored as the words T0 | (T2 & kFp6Exp0), T1 | (T2 & kFp6Exp1).  T0:T1:T2 is what
// v_cvt_scalef32_pk32_fp6_f16 returns for the 16 fp16 codes with scale 8 (it rounds
// value / scale to e2m3 to nearest even and packs value i at bits 6i; the codes are exact
// there, and a zero code is +0, so no field reads as the negative zero 0x20).
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "atom_internal.h"

#pragma clang fp contract(off)

namespace atom {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kPerThread = 16;                       // reordered elements per thread per pass
constexpr int kLanesPerGroup = ATOM_GROUP / kPerThread;   // 8
constexpr int kXcdCount = 8;                         // accelerator complex dies, each with its own L2
constexpr int kRowBlock = 64;                        // rows whose fp16 scales fill one 128-byte line
constexpr int kBlockedMinRows = 2048;                // jobs of at least this many rows use XCD row blocks

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

// Clamped quotient of x for scale s (> 0) with reciprocal r; its nearest integer (ties to
// even) is the code.
__device__ __forceinline__ float code_value(_Float16 xh, float s, float r, float qmax) {
  const float x = (float)xh;
  // t = x * r, written as an fma with +0 so that it cannot become a plain multiply of a
  // converted x: the two differ only in the sign of a zero product, which then rounds to the
  // same code 0
  const float t = __builtin_fmaf(x, r, 0.0f);
  const float e = __builtin_fmaf(-t, s, x);
  const float u = __builtin_fmaf(e, r, t);
  return __builtin_amdgcn_fmed3f(u, -qmax, qmax);
}

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

// CHUNKS: 16-byte row chunks each thread prefetches (K <= CHUNKS * 2048).
// PASSES: passes of 4096 reordered elements per row whose gather offsets stay in registers
// for the whole kernel (K <= PASSES * 4096); 0 = read perm from memory on every row.
// Work items: split == 1: item = one row, all passes; split == PASSES: item = one pass of one
// row (item / split = row, item % split = pass), used when there are fewer rows than resident
// workgroups, so that a short batch still spreads over the chip (each item stages the whole
// row, which an arbitrary reorder needs; the repeated row reads hit in L2).
template <int CHUNKS, int PASSES, int FMT>
__global__ __launch_bounds__(kThreads) void row_quantize_kernel(const uint16_t* __restrict__ X,
                                                                const int32_t* __restrict__ perm, int rows, int K,
                                                                int split, uint8_t* __restrict__ Q,
                                                                uint16_t* __restrict__ S) {
  extern __shared__ uint32_t lds_words[];
  const uint8_t* lds_bytes = reinterpret_cast<const uint8_t*>(lds_words);
  const int QP = staged_stride(K);
  const int G = K / ATOM_GROUP;
  const int klo = K - ATOM_OUTLIERS;
  const size_t rb = FMT == kRowA8 ? (size_t)K : (size_t)(klo / 2 + ATOM_OUTLIERS);
  const int nchunks = K / 8;                         // 16-byte chunks per row
  const unsigned kmax = (unsigned)(K - 1);
  constexpr int kPassElems = kThreads * kPerThread;  // 4096

  // LDS byte offsets of this thread's 16 reordered elements (clamped: a bad perm gives
  // garbage, never an out-of-range read)
  auto gather_offsets = [&](int c, int (&off)[kPerThread]) {
#pragma unroll
    for (int v = 0; v < kPerThread / 4; ++v) {
      const int4 p = *reinterpret_cast<const int4*>(perm + c + 4 * v);
      const unsigned e[4] = {__builtin_elementwise_min((unsigned)p.x, kmax), __builtin_elementwise_min((unsigned)p.y, kmax),
                             __builtin_elementwise_min((unsigned)p.z, kmax), __builtin_elementwise_min((unsigned)p.w, kmax)};
#pragma unroll
      for (int u = 0; u < 4; ++u) off[4 * v + u] = (int)((((e[u] & 15) >> 1) * QP + (e[u] >> 4)) * 4 + (e[u] & 1) * 2);
    }
  };
  int offs[PASSES > 0 ? PASSES : 1][kPerThread];
  if (PASSES > 0) {
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
      const int c = threadIdx.x * kPerThread + ps * kPassElems;
      if (c < K) gather_offsets(c, offs[ps]);
    }
  }

  u32x4 pre[CHUNKS];
  auto prefetch = [&](int row) {
    const u32x4* src = reinterpret_cast<const u32x4*>(X + (size_t)row * K);
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i) {
      const int c = threadIdx.x + i * kThreads;
      if (c < nchunks) pre[i] = src[c];
    }
  };

  // Quantize the 16 reordered elements at position c (gather offsets off) of the LDS row.
  auto quantize16 = [&](int c, const int (&off)[kPerThread], uint8_t* qrow, int row) {
    const int g = c / ATOM_GROUP;
    const bool tail = FMT == kRowA8 || g == G - 1;     // INT8 codes
    // The elements stay fp16: the absmax is taken in fp16 (exact), and each fp32 step that
    // reads x takes it as a mixed-precision fma operand, so no element is converted.
    _Float16 x[kPerThread];
    _Float16 ah = (_Float16)0.0f;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      x[i] = __builtin_bit_cast(_Float16, *reinterpret_cast<const uint16_t*>(lds_bytes + off[i]));
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
    for (int i = 0; i < kPerThread; ++i) v[i] = code_value(x[i], s, r, qmax);
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
  };

  // Work items of this workgroup, k = 0, 1, ...  Large jobs (one item per row) give each XCD
  // whole 64-row blocks (block b to XCD b % 8, workgroups reach the XCDs round-robin), so the
  // 2-byte scale stores of a block's rows, which share cache lines of the group-major scale
  // array, meet in one L2; the XCD's workgroups interleave over its rows.
  const bool blocked = split == 1 && rows >= kBlockedMinRows && gridDim.x >= kXcdCount;   // uniform
  const int xcd = blockIdx.x % kXcdCount, wx = blockIdx.x / kXcdCount;
  const int nx = ((int)gridDim.x - xcd + kXcdCount - 1) / kXcdCount;      // workgroups on this XCD
  const int nblk = (rows + kRowBlock - 1) / kRowBlock;
  const int myblk = (nblk - xcd + kXcdCount - 1) / kXcdCount;               // blocks xcd, xcd + 8, ...
  const int rx = myblk * kRowBlock - ((nblk - 1) % kXcdCount == xcd ? nblk * kRowBlock - rows : 0);
  const int items = rows * split;
  auto valid = [&](int k) {
    return blocked ? wx + k * nx < rx : (int)blockIdx.x + k * (int)gridDim.x < items;
  };
  auto row_of = [&](int k) {
    if (blocked) {
      const int t = wx + k * nx;
      return kRowBlock * (xcd + kXcdCount * (t / kRowBlock)) + t % kRowBlock;
    }
    return ((int)blockIdx.x + k * (int)gridDim.x) / split;
  };
  if (valid(0)) prefetch(row_of(0));
  for (int k = 0; valid(k); ++k) {
    const int row = row_of(k);
    const int part = blocked ? 0 : ((int)blockIdx.x + k * (int)gridDim.x) - row * split;
    __syncthreads();                                 // everyone finished reading the previous row
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
    __syncthreads();
    if (valid(k + 1)) prefetch(row_of(k + 1));       // next item's loads fly meanwhile

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
}

// Resident workgroups of one instantiation: per compute unit (for its largest row's LDS) and
// the compute-unit count, queried on the current device.
struct Residency {
  int per_cu, cus;
};

template <int CHUNKS, int PASSES, int FMT>
Residency query_residency() {
  Residency r{2, 256};                               // fallbacks if a query fails
  int dev = 0, n = 0, b = 0;
  if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
      n > 0)
    r.cus = n;
  const size_t lds_max = (size_t)staged_stride(CHUNKS * 8 * kThreads) * 8 * sizeof(uint32_t);   // largest row of this range
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, row_quantize_kernel<CHUNKS, PASSES, FMT>, kThreads, lds_max) ==
          hipSuccess && b > 0)
    r.per_cu = b;
  return r;
}

template <int CHUNKS, int PASSES, int FMT>
hipError_t launch_rq(const uint16_t* X, const int32_t* perm, int rows, int K, uint8_t* Q, uint16_t* S,
                     hipStream_t stream) {
  const size_t lds = (size_t)staged_stride(K) * 8 * sizeof(uint32_t);
  // queried once per process and instantiation (the initialisation of a function-local static
  // is thread-safe), on the device current at the first call
  static const Residency res = query_residency<CHUNKS, PASSES, FMT>();
  const int per_cu = res.per_cu, cus = res.cus;
  const int lim = per_cu * cus;
  // passes of a row as separate items when the rows alone leave resident slots empty
  const int passes = (K + kThreads * kPerThread - 1) / (kThreads * kPerThread);
  const int split = (PASSES > 1 && rows < lim) ? passes : 1;
  const long long items = (long long)rows * split;
  const int grid = items < lim ? (int)items : lim;   // persistent: one wave of workgroups
  hipLaunchKernelGGL((row_quantize_kernel<CHUNKS, PASSES, FMT>), dim3(grid), dim3(kThreads), lds, stream, X, perm, rows,
                     K, split, Q, S);
  return hipGetLastError();
}


template <int FMT>
hipError_t launch_rq_fmt(const uint16_t* X, const int32_t* perm, int rows, int K, uint8_t* Q, uint16_t* S,
                         hipStream_t stream) {
  if (K <= 4096) return launch_rq<2, 1, FMT>(X, perm, rows, K, Q, S, stream);
  if (K <= 8192) return launch_rq<4, 2, FMT>(X, perm, rows, K, Q, S, stream);
  if (K <= 12288) return launch_rq<6, 3, FMT>(X, perm, rows, K, Q, S, stream);
  if (K <= 16384) return launch_rq<8, 4, FMT>(X, perm, rows, K, Q, S, stream);
  return launch_rq<ATOM_MAX_K / 8 / kThreads, 0, FMT>(X, perm, rows, K, Q, S, stream);
}

}  // namespace

hipError_t launch_row_quantize(const uint16_t* X, const int32_t* perm, int rows, int K, uint8_t* Q, uint16_t* S,
                               RowFormat fmt, hipStream_t stream) {
  switch (fmt) {
    case kRowW4A4: return launch_rq_fmt<kRowW4A4>(X, perm, rows, K, Q, S, stream);
    case kRowA8: return launch_rq_fmt<kRowA8>(X, perm, rows, K, Q, S, stream);
    case kRowW4A8: return launch_rq_fmt<kRowW4A8>(X, perm, rows, K, Q, S, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace atom
