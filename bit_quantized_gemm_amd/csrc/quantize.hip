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
// walks all 1.8e9 such pairs for both qmax with IEEE fused multiply-adds on the CPU).  For a
// normal scale the clamp never changes that integer (the same walk checks it), so the kernel
// clamps only in a wave that holds a group with a subnormal scale.  The scale itself and r
// come from a reciprocal and one correction step each, not from an IEEE divide (exact for
// every fp16 input, see quantize16).  INT8 codes: adding 1.5*2^23 rounds the (clamped) value
// to that integer with ties to even and leaves its two's-complement low byte in the low bits
// of the sum.  INT4 codes: a mixed-precision fma rounds u + 1536 once
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
#include "row_quant.h"

#pragma clang fp contract(off)

namespace atom {
namespace {

using rowq::kLanesPerGroup;
using rowq::kPassElems;
using rowq::kPerThread;
using rowq::kThreads;
using rowq::RowQuant;
using rowq::staged_stride;

constexpr int kXcdCount = 8;                         // accelerator complex dies, each with its own L2
constexpr int kRowBlock = 64;                        // rows whose fp16 scales fill one 128-byte line
constexpr int kBlockedMinRows = 2048;                // jobs of at least this many rows use XCD row blocks

// CHUNKS / PASSES as for RowQuant.
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
  RowQuant<CHUNKS, PASSES, FMT> rq(X, perm, rows, K, Q, S, lds_words);
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
  rq.load_perm();
  rq.prefetch(valid(0) ? row_of(0) : 0);            // unconditional (see RowQuant::prefetch)
  rq.finish_offsets();
  for (int k = 0; valid(k); ++k) {
    const int row = row_of(k);
    const int part = blocked ? 0 : ((int)blockIdx.x + k * (int)gridDim.x) - row * split;
    __syncthreads();                                 // everyone finished reading the previous row
    rq.stage();
    __syncthreads();
    if (valid(k + 1)) rq.prefetch(row_of(k + 1));    // next item's loads fly meanwhile
    rq.quantize(row, part, split);
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
  // longer rows read perm on every row; rows up to 32768 keep two workgroups per compute unit
  if (K <= 32768) return launch_rq<16, 0, FMT>(X, perm, rows, K, Q, S, stream);
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
