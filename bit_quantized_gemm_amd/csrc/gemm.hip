// W4A4 grouped GEMM for gfx950 on int8 MFMA.
//
// Y[m,n] = sum over 128-channel groups g of acc_g[m,n] * sx[g,m] * sw[g,n], with
// acc_g = exact integer dot product of the codes of group g.  The method runs this product
// on integer operators (index page of "Atom: Low-bit Quantization for Efficient and Accurate
// LLM Serving", Abstract; quantization record, "notes": an integer-operator path).  gfx950
// has no 4-bit MFMA, so the INT4 groups are widened to int8 in registers and fed to
// v_mfma_i32_32x32x32_i8; the INT8 outlier group (record, "notes": a 128-channel
// high-precision group) feeds the same instruction without widening.
//
// Nibble widening.  For a packed word w holding codes c0..c7 (c_{2j} in the low nibble of
// byte j), w & 0xF0F0F0F0 holds 16*c_{2j+1} and (w << 4) & 0xF0F0F0F0 holds 16*c_{2j} as
// int8 bytes.  Both operands are widened the same way, so the MFMAs over the "low" words and
// those over the "high" words together cover every channel of the group once, and the
// accumulator holds 256 * acc_g exactly (|256*acc_g| <= 128*112*112 < 2^21, so its fp32
// conversion is exact too).
//
// Scales.  The rank-one product sx[g,:] (x) sw[g,:] of a 32x32 output tile comes from one
// v_mfma_f32_32x32x8_f16 whose only nonzero K column/row holds the fp16 scales: fp16 x fp16
// is exact in fp32, and the product lands in the accumulator layout.  The epilogue per output
// element and group is then one int->fp32 conversion and one fp32 FMA.  The outlier group's
// scale product is multiplied by 256 so that the whole sum carries the same factor 256, which
// the final store removes (a power of two: exact).
//
// Pipeline.  A packed row is a sequence of 64-byte stages: stage s < G-1 is INT4 group s,
// stages G-1 and G are the two 64-byte halves of the INT8 outlier group.  Each thread loads
// its 16-byte chunks of a stage of the A (activation) and B (weight) tiles with buffer loads
// (the stage offset is a scalar), widens them once, and writes the int8 operands to LDS
// (double-buffered); every wave then reads ready-to-use MFMA operands.  The loads of stage
// s+2 are in flight while stage s+1 is written to LDS and stage s is multiplied; one barrier
// per stage.
//
// LDS layout.  A staged row is 128 bytes = eight 16-byte chunks: chunk h*4 + q holds the
// widened low (h = 0) or high (h = 1) nibbles of packed chunk q (the INT8 stages use chunks
// 0..3 raw).  Chunk c of row r is stored at chunk position c ^ ((r >> 1) & 7), so the 16
// lanes of a ds_read_b128 group (16 consecutive rows, same chunk) hit 16 different bank
// groups.
//
// Waves.  A workgroup of WAVES_M x WAVES_N waves computes a BM x BN tile of Y; each wave
// owns a (BM/WAVES_M) x (BN/WAVES_N) sub-tile held as 32x32 MFMA tiles.  Lane l of a wave
// supplies row (A) / column (B) l & 31 of a tile and K half l >> 5 of each chunk pair.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "atom_internal.h"

namespace atom {
namespace {

typedef int32_t v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef int32_t v4i __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));   // native vector: stays in VGPRs
typedef _Float16 h4 __attribute__((ext_vector_type(4)));

constexpr int kStageBytes = 64;          // bytes of one stage of a packed row
constexpr int kXcds = 8;                 // accelerator complex dies (each with its own L2)

__device__ __forceinline__ v4i widen_lo(u32x4 p) {
  return v4i{(int32_t)((p.x << 4) & 0xF0F0F0F0u), (int32_t)((p.y << 4) & 0xF0F0F0F0u),
             (int32_t)((p.z << 4) & 0xF0F0F0F0u), (int32_t)((p.w << 4) & 0xF0F0F0F0u)};
}

__device__ __forceinline__ v4i widen_hi(u32x4 p) {
  return v4i{(int32_t)(p.x & 0xF0F0F0F0u), (int32_t)(p.y & 0xF0F0F0F0u), (int32_t)(p.z & 0xF0F0F0F0u),
             (int32_t)(p.w & 0xF0F0F0F0u)};
}

__device__ __forceinline__ v4i as_v4i(u32x4 p) { return v4i{(int32_t)p.x, (int32_t)p.y, (int32_t)p.z, (int32_t)p.w}; }

__device__ __forceinline__ v16i mma_i8(v4i a, v4i b, v16i c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v16i mma_i8_first(v4i a, v4i b) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, v16i{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0}, 0, 0, 0);
}

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

constexpr int kLdsRow = 128;             // bytes of one staged (widened) row in LDS

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
  int a_lds[APER], b_lds[BPER];            // LDS byte offset of the widened-low chunk
  int a_lds_hi[APER], b_lds_hi[BPER];      // LDS byte offset of the widened-high chunk
  const uint16_t* s_src;                   // this thread's scale column (or null)
  size_t s_stride;
};

__device__ __forceinline__ int swizzled(int row, int chunk) { return row * kLdsRow + ((chunk ^ ((row >> 1) & 7)) << 4); }

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

// INT4 stage: widen every chunk into its low- and high-nibble int8 chunks.
template <int BM, int BN, bool kAcc, int APER, int BPER>
__device__ __forceinline__ void store_stage_int4(const StageRegs<APER, BPER>& st, const StageAddr<APER, BPER>& ad,
                                                 uint8_t* la, uint8_t* lb, uint16_t* lsx, uint16_t* lsw, int tid) {
#pragma unroll
  for (int p = 0; p < APER; ++p) {
    *reinterpret_cast<v4i*>(la + ad.a_lds[p]) = widen_lo(st.a[p]);
    *reinterpret_cast<v4i*>(la + ad.a_lds_hi[p]) = widen_hi(st.a[p]);
  }
#pragma unroll
  for (int p = 0; p < BPER; ++p) {
    *reinterpret_cast<v4i*>(lb + ad.b_lds[p]) = widen_lo(st.b[p]);
    *reinterpret_cast<v4i*>(lb + ad.b_lds_hi[p]) = widen_hi(st.b[p]);
  }
  if (!kAcc) {
    if (tid < BM) lsx[tid] = st.s;
    else if (tid < BM + BN) lsw[tid - BM] = st.s;
  }
}

// INT8 stage: chunks are already int8 codes.
template <int BM, int BN, bool kAcc, int APER, int BPER>
__device__ __forceinline__ void store_stage_int8(const StageRegs<APER, BPER>& st, const StageAddr<APER, BPER>& ad,
                                                 uint8_t* la, uint8_t* lb, uint16_t* lsx, uint16_t* lsw, int tid) {
#pragma unroll
  for (int p = 0; p < APER; ++p) *reinterpret_cast<u32x4*>(la + ad.a_lds[p]) = st.a[p];
#pragma unroll
  for (int p = 0; p < BPER; ++p) *reinterpret_cast<u32x4*>(lb + ad.b_lds[p]) = st.b[p];
  if (!kAcc) {
    if (tid < BM) lsx[tid] = st.s;
    else if (tid < BM + BN) lsw[tid - BM] = st.s;
  }
}

// kAcc = false: Y output.  kAcc = true: write the per-group integer accumulators instead.
template <int BM, int BN, int WAVES_M, int WAVES_N, bool kAcc>
__global__ __launch_bounds__(WAVES_M* WAVES_N * 64) __attribute__((amdgpu_waves_per_eu(4))) void gemm_w4a4_kernel(
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
  const int kh = lane >> 5;                             // which 32-byte half of the stage this lane reads

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
      const int c = tid + p * T::kThreads, r = c / 4, q = c % 4;
      ad.a_voff[p] = min(r, rows_a - 1) * (int)rbytes + q * 16;
      ad.a_lds[p] = swizzled(r, q);
      ad.a_lds_hi[p] = swizzled(r, 4 + q);
    }
#pragma unroll
    for (int p = 0; p < T::kBPer; ++p) {
      const int c = tid + p * T::kThreads, r = c / 4, q = c % 4;
      ad.b_voff[p] = min(r, rows_b - 1) * (int)rbytes + q * 16;
      ad.b_lds[p] = swizzled(r, q);
      ad.b_lds_hi[p] = swizzled(r, 4 + q);
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
  v16i acc[T::kTM][T::kTN];

  // This lane's 16-byte operand word of tile i (A) / j (B): chunk h*4 + kh*2 + w of its row.
  // The swizzle term depends only on l32 (tile rows start at multiples of 32).
  const int lane_swz = (l32 >> 1) & 7;
  auto lds_a_word = [&](int buf, int i, int h, int w) {
    return *reinterpret_cast<const v4i*>(lds_a[buf] + (wm * T::kWTM + i * 32 + l32) * kLdsRow +
                                         (((h * 4 + kh * 2 + w) ^ lane_swz) << 4));
  };
  auto lds_b_word = [&](int buf, int j, int h, int w) {
    return *reinterpret_cast<const v4i*>(lds_b[buf] + (wn * T::kWTN + j * 32 + l32) * kLdsRow +
                                         (((h * 4 + kh * 2 + w) ^ lane_swz) << 4));
  };

  // One INT4 group: four K=32 MFMAs per tile (widened low / high nibbles of two chunk words).
  auto mma_int4 = [&](int buf) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        v4i af[T::kTM], bf[T::kTN];
#pragma unroll
        for (int i = 0; i < T::kTM; ++i) af[i] = lds_a_word(buf, i, h, w);
#pragma unroll
        for (int j = 0; j < T::kTN; ++j) bf[j] = lds_b_word(buf, j, h, w);
#pragma unroll
        for (int i = 0; i < T::kTM; ++i)
#pragma unroll
          for (int j = 0; j < T::kTN; ++j)
            acc[i][j] = (h == 0 && w == 0) ? mma_i8_first(af[i], bf[j]) : mma_i8(af[i], bf[j], acc[i][j]);
      }
  };

  // One 64-channel half of the INT8 outlier group: two K=32 MFMAs per tile.
  auto mma_int8 = [&](int buf, bool first) {
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      v4i af[T::kTM], bf[T::kTN];
#pragma unroll
      for (int i = 0; i < T::kTM; ++i) af[i] = lds_a_word(buf, i, 0, w);
#pragma unroll
      for (int j = 0; j < T::kTN; ++j) bf[j] = lds_b_word(buf, j, 0, w);
#pragma unroll
      for (int i = 0; i < T::kTM; ++i)
#pragma unroll
        for (int j = 0; j < T::kTN; ++j)
          acc[i][j] = (first && w == 0) ? mma_i8_first(af[i], bf[j]) : mma_i8(af[i], bf[j], acc[i][j]);
    }
  };

  // Tile row i of an INT4 group (tiles (i, 0..kTN-1)): four K=32 MFMAs per tile.
  auto mma_int4_row = [&](int buf, int i) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const v4i af = lds_a_word(buf, i, h, w);
#pragma unroll
        for (int j = 0; j < T::kTN; ++j) {
          const v4i bf = lds_b_word(buf, j, h, w);
          acc[i][j] = (h == 0 && w == 0) ? mma_i8_first(af, bf) : mma_i8(af, bf, acc[i][j]);
        }
      }
  };

  // fp16 scale operands of one group for this lane: K column 0 of A holds sx (lanes < 32),
  // K row 0 of B holds sw.
  auto read_scales = [&](int buf, h4 (&sa)[T::kTM], h4 (&sb)[T::kTN]) {
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
  };

  // Epilogue of tile row i: yacc += float(acc) * (sx (x) sw); `outlier` scales the product by
  // 256 so that every group's contribution carries the factor 256 of the widened groups.
  auto epi_row = [&](int i, h4 sai, const h4 (&sb)[T::kTN], bool outlier) {
#pragma unroll
    for (int j = 0; j < T::kTN; ++j) {
      v16f sp = __builtin_amdgcn_mfma_f32_32x32x8f16(sai, sb[j], v16f{}, 0, 0, 0);
      if (outlier) sp *= 256.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) yacc[i][j][r] = __builtin_fmaf((float)acc[i][j][r], sp[r], yacc[i][j][r]);
    }
  };

  // Scale the finished integer accumulators of group g into the fp32 output accumulators,
  // or (kAcc) write them out.  `widened`: the accumulators carry the factor 256.
  auto epilogue = [&](int buf, int g, bool widened) {
    if (kAcc) {
#pragma unroll
      for (int i = 0; i < T::kTM; ++i)
#pragma unroll
        for (int j = 0; j < T::kTN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int m = m0 + wm * T::kWTM + i * 32 + (r >> 2) * 8 + kh * 4 + (r & 3);
            const int n = n0 + wn * T::kWTN + j * 32 + l32;
            if (m < M && n < N) acc_out[((size_t)g * M + m) * N + n] = widened ? (acc[i][j][r] >> 8) : acc[i][j][r];
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
          v16f sp = __builtin_amdgcn_mfma_f32_32x32x8f16(sa[i], sb[j], v16f{}, 0, 0, 0);
          if (!widened) sp *= 256.0f;
#pragma unroll
          for (int r = 0; r < 16; ++r) yacc[i][j][r] = __builtin_fmaf((float)acc[i][j][r], sp[r], yacc[i][j][r]);
        }
    }
  };

  load_stage(st, ad, 0, G);
  store_stage_int4<BM, BN, kAcc>(st, ad, lds_a[0], lds_b[0], lds_sx[0], lds_sw[0], tid);   // G >= 2: stage 0 is INT4
  load_stage(st, ad, 1, G);
  __syncthreads();

  {
    for (int s = 0; s < G - 1; ++s) {
      const int buf = s & 1;
      mma_int4(buf);
      if (s + 1 < G - 1)
        store_stage_int4<BM, BN, kAcc>(st, ad, lds_a[buf ^ 1], lds_b[buf ^ 1], lds_sx[buf ^ 1], lds_sw[buf ^ 1], tid);
      else
        store_stage_int8<BM, BN, kAcc>(st, ad, lds_a[buf ^ 1], lds_b[buf ^ 1], lds_sx[buf ^ 1], lds_sw[buf ^ 1], tid);
      load_stage(st, ad, s + 2, G);                  // s+2 <= G: always a valid stage
      epilogue(buf, s, true);
      __syncthreads();
    }
    const int buf = (G - 1) & 1;
    mma_int8(buf, true);
    store_stage_int8<BM, BN, kAcc>(st, ad, lds_a[buf ^ 1], lds_b[buf ^ 1], lds_sx[buf ^ 1], lds_sw[buf ^ 1], tid);
    __syncthreads();
    mma_int8(buf ^ 1, false);
    epilogue(buf ^ 1, G - 1, false);
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
          if (m < M && n < N)
            Y[(size_t)m * N + n] = __half_as_ushort(__float2half_rn(yacc[i][j][r] * (1.0f / 256.0f)));
        }
  }
}

// 128 x 128 workgroup tile, 2 x 2 waves of 64 x 64 (2 x 2 MFMA tiles of 32 x 32 each).
constexpr int kBM = 128, kBN = 128, kWavesM = 2, kWavesN = 4;

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
