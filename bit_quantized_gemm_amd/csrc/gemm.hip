// W4A4 grouped GEMM for gfx950 on the matrix cores.
//
// Y[m,n] = sum over 128-channel groups g of acc_g[m,n] * sx[g,m] * sw[g,n], with
// acc_g = exact integer dot product of the codes of group g.  The method runs this product
// on integer operators (index page of "Atom: Low-bit Quantization for Efficient and Accurate
// LLM Serving", Abstract; quantization record, "notes": an integer-operator path, not FP4).
//
// INT4 groups.  gfx950 has no 4-bit integer MFMA.  An INT4 code q in [-7, 7] is exactly the
// fp8 e4m3 subnormal with bits (q < 0) << 7 | |q| (value q * 2^-9), and the packed
// sign-magnitude layout turns a 32-bit word of eight codes into four such bytes with one AND
// (even codes: w & 0x87878787) or one rotate and one AND (odd codes: rotr(w, 4) & 0x87878787).
// v_mfma_scale_f32_32x32x64_f8f6f4 with unit-exponent scales 2^9 * 2^9 then returns the
// group's integer dot product exactly in fp32: every product and partial sum is an integer
// of magnitude below 2^24.  The INT4 groups thus run at the dense fp8 rate (equal to the int8
// rate) and their accumulators are already fp32.
//
// INT8 outlier group (record, "notes": a 128-channel high-precision group): int8 codes feed
// v_mfma_i32_32x32x32_i8 directly; its int32 accumulators are converted once.
//
// Scales.  The rank-one product sx[g,:] (x) sw[g,:] of a 32x32 output tile comes from one
// v_mfma_f32_32x32x8_f16 whose only nonzero K column/row holds the fp16 scales: fp16 x fp16
// is exact in fp32, and the product lands in the accumulator layout.  The epilogue per output
// element and group is then a single fp32 FMA.
//
// Pipeline.  A packed row is a sequence of 64-byte stages: stage s < G-1 is INT4 group s,
// stages G-1 and G are the two 64-byte halves of the INT8 outlier group.  Each thread loads
// its 16-byte chunks of a stage of the A (activation) and B (weight) tiles with buffer loads
// (the stage offset is a scalar), decodes them once into fp8 bytes (INT8 stages are copied
// as they are), and writes them to LDS (double-buffered); every wave then reads ready MFMA
// operands.  The loads of stage s+2 are in flight while stage s+1 is written to LDS and stage
// s is multiplied; one barrier per stage.
//
// LDS layout.  A staged row is 128 bytes = eight 16-byte chunks: chunk q (0..3) holds the
// even-code bytes of packed chunk q, chunk 4 + q its odd-code bytes (INT8 stages use chunks
// 0..3 raw).  Chunk c of row r is stored at position c ^ h((r >> 1) & 7), h a rotation of
// three bits, so that the 16 lanes of a ds_read_b128 group (16 consecutive rows, one chunk)
// and those of a ds_write_b128 group (4 rows x 4 chunks) each cover all 16 bank groups.
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
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));   // native vector: stays in VGPRs
typedef _Float16 h4 __attribute__((ext_vector_type(4)));

constexpr int kStageBytes = 64;          // bytes of one stage of a packed row
constexpr int kLdsRow = 128;             // bytes of one staged (decoded) row in LDS
constexpr int kXcds = 8;                 // accelerator complex dies (each with its own L2)
constexpr int kScaleE8M0 = 127 + 9;      // 2^9: the e4m3 subnormal q * 2^-9 counts as q

__device__ __forceinline__ uint32_t rotr4(uint32_t w) { return __builtin_amdgcn_alignbit(w, w, 4); }

__device__ __forceinline__ u32x4 fp8_even(u32x4 w) { return w & 0x87878787u; }

__device__ __forceinline__ u32x4 fp8_odd(u32x4 w) {
  return u32x4{rotr4(w.x), rotr4(w.y), rotr4(w.z), rotr4(w.w)} & 0x87878787u;
}

__device__ __forceinline__ v16f mma_fp8(v8i a, v8i b, v16f c) {
  // cbsz = blgp = 0: both operands fp8 e4m3; opsel 0 and E8M0 scale 2^9 on both sides
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, kScaleE8M0, 0, kScaleE8M0);
}

__device__ __forceinline__ v16i mma_i8(v4i a, v4i b, v16i c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

// h: rotation of three bits, b2 b1 b0 -> b0 b2 b1
__device__ __forceinline__ int chunk_swz(int row) {
  const int k = (row >> 1) & 7;
  return ((k & 1) << 2) | (k >> 1);
}

__device__ __forceinline__ int lds_pos(int row, int chunk) { return row * kLdsRow + ((chunk ^ chunk_swz(row)) << 4); }

template <int BM, int BN, int WAVES_M, int WAVES_N>
struct Tile {
  static constexpr int kThreads = WAVES_M * WAVES_N * 64;
  static constexpr int kWTM = BM / WAVES_M;            // wave tile rows
  static constexpr int kWTN = BN / WAVES_N;            // wave tile columns
  static constexpr int kTM = kWTM / 32;                // MFMA tiles per wave (rows)
  static constexpr int kTN = kWTN / 32;                // MFMA tiles per wave (columns)
  static constexpr int kAPer = BM * 4 / kThreads;      // 16-byte A chunks per thread per stage
  static constexpr int kBPer = BN * 4 / kThreads;
  static_assert(kWTM % 32 == 0 && kWTN % 32 == 0, "wave tile must be a multiple of 32");
  static_assert(kAPer * kThreads == BM * 4 && kBPer * kThreads == BN * 4, "chunks must divide evenly");
  static_assert(BM + BN <= kThreads, "one scale per thread per stage");
};

// Registers holding one stage in flight between global memory and LDS.
template <int APER, int BPER>
struct StageRegs {
  u32x4 a[APER];
  u32x4 b[BPER];
  uint16_t s;
};

// Per-thread addressing of the global -> LDS copy, fixed for the whole K loop.
template <int APER, int BPER>
struct StageAddr {
  __amdgpu_buffer_rsrc_t a_rsrc, b_rsrc;  // the workgroup's rows of Xq / Wq
  int a_voff[APER], b_voff[BPER];          // byte offset of this thread's chunk in stage 0
  int a_lds[APER], b_lds[BPER];            // LDS offset of chunk q (even codes, or the INT8 chunk)
  int a_lds_odd[APER], b_lds_odd[BPER];    // LDS offset of chunk 4 + q (odd codes)
  const uint16_t* s_src;                   // this thread's scale column (or null)
  size_t s_stride;
};

template <int APER, int BPER>
__device__ __forceinline__ void load_stage(StageRegs<APER, BPER>& st, const StageAddr<APER, BPER>& ad, int s, int G) {
  const int soff = s * kStageBytes;
#pragma unroll
  for (int p = 0; p < APER; ++p)
    st.a[p] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ad.a_rsrc, ad.a_voff[p], soff, 0));
#pragma unroll
  for (int p = 0; p < BPER; ++p)
    st.b[p] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ad.b_rsrc, ad.b_voff[p], soff, 0));
  if (ad.s_src) st.s = ad.s_src[(size_t)min(s, G - 1) * ad.s_stride];
}

template <int BM, int BN, bool kAcc>
__device__ __forceinline__ void store_scale(uint16_t s, uint16_t* lsx, uint16_t* lsw, int tid) {
  if (!kAcc) {
    if (tid < BM) lsx[tid] = s;
    else if (tid < BM + BN) lsw[tid - BM] = s;
  }
}

// INT4 stage: decode every chunk into its even- and odd-code fp8 chunks.
template <int BM, int BN, bool kAcc, int APER, int BPER>
__device__ __forceinline__ void store_stage_int4(const StageRegs<APER, BPER>& st, const StageAddr<APER, BPER>& ad,
                                                 uint8_t* la, uint8_t* lb, uint16_t* lsx, uint16_t* lsw, int tid) {
#pragma unroll
  for (int p = 0; p < APER; ++p) {
    *reinterpret_cast<u32x4*>(la + ad.a_lds[p]) = fp8_even(st.a[p]);
    *reinterpret_cast<u32x4*>(la + ad.a_lds_odd[p]) = fp8_odd(st.a[p]);
  }
#pragma unroll
  for (int p = 0; p < BPER; ++p) {
    *reinterpret_cast<u32x4*>(lb + ad.b_lds[p]) = fp8_even(st.b[p]);
    *reinterpret_cast<u32x4*>(lb + ad.b_lds_odd[p]) = fp8_odd(st.b[p]);
  }
  store_scale<BM, BN, kAcc>(st.s, lsx, lsw, tid);
}

// INT8 stage: chunks are already int8 codes.
template <int BM, int BN, bool kAcc, int APER, int BPER>
__device__ __forceinline__ void store_stage_int8(const StageRegs<APER, BPER>& st, const StageAddr<APER, BPER>& ad,
                                                 uint8_t* la, uint8_t* lb, uint16_t* lsx, uint16_t* lsw, int tid) {
#pragma unroll
  for (int p = 0; p < APER; ++p) *reinterpret_cast<u32x4*>(la + ad.a_lds[p]) = st.a[p];
#pragma unroll
  for (int p = 0; p < BPER; ++p) *reinterpret_cast<u32x4*>(lb + ad.b_lds[p]) = st.b[p];
  store_scale<BM, BN, kAcc>(st.s, lsx, lsw, tid);
}

// kAcc = false: Y output.  kAcc = true: write the per-group integer accumulators instead.
template <int BM, int BN, int WAVES_M, int WAVES_N, bool kAcc>
__global__ __launch_bounds__(WAVES_M* WAVES_N * 64) __attribute__((amdgpu_waves_per_eu(2))) void gemm_w4a4_kernel(
    const uint8_t* __restrict__ Xq, const uint16_t* __restrict__ sx, const uint8_t* __restrict__ Wq,
    const uint16_t* __restrict__ sw, int M, int N, int K, uint16_t* __restrict__ Y, int32_t* __restrict__ acc_out) {
  using T = Tile<BM, BN, WAVES_M, WAVES_N>;
  __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][BM * kLdsRow];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b[2][BN * kLdsRow];
  __shared__ __attribute__((aligned(16))) uint16_t lds_sx[2][BM];
  __shared__ __attribute__((aligned(16))) uint16_t lds_sw[2][BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WAVES_N;
  const int wn = wave % WAVES_N;
  // Tile order: workgroups go to the 8 XCDs round-robin by id; renumber them so that each
  // XCD gets a contiguous run of tiles, M fastest, so an XCD's L2 holds one slice of W.
  const int tiles_m = (M + BM - 1) / BM;
  const int ntiles = tiles_m * ((N + BN - 1) / BN);
  const int xcd = blockIdx.x % kXcds, local = blockIdx.x / kXcds;
  const int q = ntiles / kXcds, rem = ntiles % kXcds;
  const int lin = xcd < rem ? xcd * (q + 1) + local : rem * (q + 1) + (xcd - rem) * q + local;
  const int m0 = (lin % tiles_m) * BM;
  const int n0 = (lin / tiles_m) * BN;
  const int G = K / ATOM_GROUP;
  const int S = G + 1;                                  // stages per row
  const size_t rbytes = (size_t)S * kStageBytes;        // = (K-128)/2 + 128
  const int l32 = lane & 31;                            // row (A) / column (B) inside a 32x32 tile
  const int kh = lane >> 5;                             // which K half of an operand this lane supplies

  // ---- per-thread staging addresses (rows past M / N repeat the last valid row)
  StageAddr<T::kAPer, T::kBPer> ad;
  {
    const int rows_a = min(BM, M - m0), rows_b = min(BN, N - n0);
    ad.a_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)(Xq + (size_t)m0 * rbytes), (short)0,
                                                  (int)(rows_a * rbytes), 0x00020000);
    ad.b_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)(Wq + (size_t)n0 * rbytes), (short)0,
                                                  (int)(rows_b * rbytes), 0x00020000);
#pragma unroll
    for (int p = 0; p < T::kAPer; ++p) {
      const int c = tid + p * T::kThreads, r = c / 4, qc = c % 4;
      ad.a_voff[p] = min(r, rows_a - 1) * (int)rbytes + qc * 16;
      ad.a_lds[p] = lds_pos(r, qc);
      ad.a_lds_odd[p] = lds_pos(r, 4 + qc);
    }
#pragma unroll
    for (int p = 0; p < T::kBPer; ++p) {
      const int c = tid + p * T::kThreads, r = c / 4, qc = c % 4;
      ad.b_voff[p] = min(r, rows_b - 1) * (int)rbytes + qc * 16;
      ad.b_lds[p] = lds_pos(r, qc);
      ad.b_lds_odd[p] = lds_pos(r, 4 + qc);
    }
    ad.s_src = nullptr;
    ad.s_stride = 0;
    if (!kAcc) {
      if (tid < BM) {
        ad.s_src = sx + min(m0 + tid, M - 1);
        ad.s_stride = (size_t)M;
      } else if (tid < BM + BN) {
        ad.s_src = sw + min(n0 + tid - BM, N - 1);
        ad.s_stride = (size_t)N;
      }
    }
  }

  StageRegs<T::kAPer, T::kBPer> st;
  v16f yacc[T::kTM][T::kTN];
#pragma unroll
  for (int i = 0; i < T::kTM; ++i)
#pragma unroll
    for (int j = 0; j < T::kTN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) yacc[i][j][r] = 0.0f;
  v16f accf[T::kTM][T::kTN];                            // group sums: exact integers in fp32

  // 16-byte LDS chunk c of the row supplying this lane in tile i (A) / j (B).  The swizzle
  // term depends only on l32 (tile rows start at multiples of 32).
  const int lane_swz = chunk_swz(l32);
  auto lds_a_chunk = [&](int buf, int i, int c) {
    return *reinterpret_cast<const v4i*>(lds_a[buf] + (wm * T::kWTM + i * 32 + l32) * kLdsRow + ((c ^ lane_swz) << 4));
  };
  auto lds_b_chunk = [&](int buf, int j, int c) {
    return *reinterpret_cast<const v4i*>(lds_b[buf] + (wn * T::kWTN + j * 32 + l32) * kLdsRow + ((c ^ lane_swz) << 4));
  };
  // 32-byte fp8 operand of half h (0: even codes, 1: odd codes): chunks 4h + 2kh and 4h + 2kh + 1
  auto fp8_a = [&](int buf, int i, int h) {
    const v4i lo = lds_a_chunk(buf, i, 4 * h + 2 * kh), hi = lds_a_chunk(buf, i, 4 * h + 2 * kh + 1);
    return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };
  auto fp8_b = [&](int buf, int j, int h) {
    const v4i lo = lds_b_chunk(buf, j, 4 * h + 2 * kh), hi = lds_b_chunk(buf, j, 4 * h + 2 * kh + 1);
    return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };

  // One INT4 group: two K=64 fp8 MFMAs per tile (even codes, then odd codes).
  auto mma_int4 = [&](int buf) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      v8i bf[T::kTN];
#pragma unroll
      for (int j = 0; j < T::kTN; ++j) bf[j] = fp8_b(buf, j, h);
#pragma unroll
      for (int i = 0; i < T::kTM; ++i) {
        const v8i af = fp8_a(buf, i, h);
#pragma unroll
        for (int j = 0; j < T::kTN; ++j) accf[i][j] = mma_fp8(af, bf[j], h == 0 ? v16f{} : accf[i][j]);
      }
    }
  };

  // One 64-channel half of the INT8 outlier group: two K=32 int8 MFMAs per tile.
  auto mma_int8_half = [&](int buf, bool first, v16i (&acc)[T::kTM][T::kTN]) {
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      v4i bf[T::kTN];
#pragma unroll
      for (int j = 0; j < T::kTN; ++j) bf[j] = lds_b_chunk(buf, j, 2 * kh + w);
#pragma unroll
      for (int i = 0; i < T::kTM; ++i) {
        const v4i af = lds_a_chunk(buf, i, 2 * kh + w);
#pragma unroll
        for (int j = 0; j < T::kTN; ++j) acc[i][j] = mma_i8(af, bf[j], (first && w == 0) ? v16i{} : acc[i][j]);
      }
    }
  };

  // Scale the group sums of group g (scales in LDS buffer buf) into yacc, or (kAcc) write them.
  auto epilogue = [&](int buf, int g) {
    if (kAcc) {
#pragma unroll
      for (int i = 0; i < T::kTM; ++i)
#pragma unroll
        for (int j = 0; j < T::kTN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int m = m0 + wm * T::kWTM + i * 32 + (r >> 2) * 8 + kh * 4 + (r & 3);
            const int n = n0 + wn * T::kWTN + j * 32 + l32;
            if (m < M && n < N) acc_out[((size_t)g * M + m) * N + n] = (int32_t)accf[i][j][r];
          }
    } else {
      // rank-one scale operands: K column 0 of A holds sx, K row 0 of B holds sw (lanes < 32)
      h4 sa[T::kTM], sb[T::kTN];
#pragma unroll
      for (int i = 0; i < T::kTM; ++i) {
        const uint16_t h = kh == 0 ? lds_sx[buf][wm * T::kWTM + i * 32 + l32] : (uint16_t)0;
        sa[i] = h4{__builtin_bit_cast(_Float16, h), (_Float16)0, (_Float16)0, (_Float16)0};
      }
#pragma unroll
      for (int j = 0; j < T::kTN; ++j) {
        const uint16_t h = kh == 0 ? lds_sw[buf][wn * T::kWTN + j * 32 + l32] : (uint16_t)0;
        sb[j] = h4{__builtin_bit_cast(_Float16, h), (_Float16)0, (_Float16)0, (_Float16)0};
      }
#pragma unroll
      for (int i = 0; i < T::kTM; ++i)
#pragma unroll
        for (int j = 0; j < T::kTN; ++j) {
          const v16f sp = __builtin_amdgcn_mfma_f32_32x32x8f16(sa[i], sb[j], v16f{}, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 16; ++r) yacc[i][j][r] = __builtin_fmaf(accf[i][j][r], sp[r], yacc[i][j][r]);
        }
    }
  };

  load_stage(st, ad, 0, G);
  store_stage_int4<BM, BN, kAcc>(st, ad, lds_a[0], lds_b[0], lds_sx[0], lds_sw[0], tid);   // G >= 2: stage 0 is INT4
  load_stage(st, ad, 1, G);
  __syncthreads();

  // INT4 groups: stages 0 .. G-2
  for (int s = 0; s < G - 1; ++s) {
    const int buf = s & 1;
    mma_int4(buf);
    // stage s+1 into the other buffer (released by the last barrier), then start stage s+2
    if (s + 1 < G - 1)
      store_stage_int4<BM, BN, kAcc>(st, ad, lds_a[buf ^ 1], lds_b[buf ^ 1], lds_sx[buf ^ 1], lds_sw[buf ^ 1], tid);
    else
      store_stage_int8<BM, BN, kAcc>(st, ad, lds_a[buf ^ 1], lds_b[buf ^ 1], lds_sx[buf ^ 1], lds_sw[buf ^ 1], tid);
    load_stage(st, ad, s + 2, G);                    // s+2 <= G: always a valid stage
    epilogue(buf, s);
    __syncthreads();
  }
  // INT8 outlier group: stages G-1 and G
  {
    v16i acc[T::kTM][T::kTN];
    const int buf = (G - 1) & 1;
    mma_int8_half(buf, true, acc);
    store_stage_int8<BM, BN, kAcc>(st, ad, lds_a[buf ^ 1], lds_b[buf ^ 1], lds_sx[buf ^ 1], lds_sw[buf ^ 1], tid);
    __syncthreads();
    mma_int8_half(buf ^ 1, false, acc);
#pragma unroll
    for (int i = 0; i < T::kTM; ++i)
#pragma unroll
      for (int j = 0; j < T::kTN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) accf[i][j][r] = (float)acc[i][j][r];   // |acc| <= 128*127*127 < 2^24
    epilogue(buf ^ 1, G - 1);
  }

  if (!kAcc) {
#pragma unroll
    for (int i = 0; i < T::kTM; ++i)
#pragma unroll
      for (int j = 0; j < T::kTN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = m0 + wm * T::kWTM + i * 32 + (r >> 2) * 8 + kh * 4 + (r & 3);
          const int n = n0 + wn * T::kWTN + j * 32 + l32;
          if (m < M && n < N) Y[(size_t)m * N + n] = __half_as_ushort(__float2half_rn(yacc[i][j][r]));
        }
  }
}

// 128 x 128 workgroup tile, 2 x 2 waves of 64 x 64 (2 x 2 MFMA tiles of 32 x 32 each).
constexpr int kBM = 128, kBN = 128, kWavesM = 2, kWavesN = 2;

}  // namespace

hipError_t launch_gemm(const uint8_t* Xq, const uint16_t* sx, const uint8_t* Wq, const uint16_t* sw, int M, int N,
                       int K, uint16_t* Y, hipStream_t stream) {
  const dim3 grid(((N + kBN - 1) / kBN) * ((M + kBM - 1) / kBM));
  hipLaunchKernelGGL((gemm_w4a4_kernel<kBM, kBN, kWavesM, kWavesN, false>), grid, dim3(kWavesM * kWavesN * 64), 0,
                     stream, Xq, sx, Wq, sw, M, N, K, Y, (int32_t*)nullptr);
  return hipGetLastError();
}

hipError_t launch_gemm_group_acc(const uint8_t* Xq, const uint8_t* Wq, int M, int N, int K, int32_t* acc,
                                 hipStream_t stream) {
  const dim3 grid(((N + kBN - 1) / kBN) * ((M + kBM - 1) / kBM));
  hipLaunchKernelGGL((gemm_w4a4_kernel<kBM, kBN, kWavesM, kWavesN, true>), grid, dim3(kWavesM * kWavesN * 64), 0,
                     stream, Xq, (const uint16_t*)nullptr, Wq, (const uint16_t*)nullptr, M, N, K,
                     (uint16_t*)nullptr, acc);
  return hipGetLastError();
}

}  // namespace atom
