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
// 1/256 is folded into the fp32 weight scale (a power of two: exact).
//
// Pipeline.  A packed row is a sequence of 64-byte stages: stage s < G-1 is INT4 group s,
// stages G-1 and G are the two 64-byte halves of the INT8 outlier group.  Each stage of the
// A (activation) and B (weight) tiles plus the group's scales goes global -> registers ->
// LDS (double-buffered).  The loads of stage s+2 are in flight while stage s+1 is written
// to LDS and stage s is multiplied; one barrier per stage.
//
// Waves.  A workgroup of WAVES_M x WAVES_N waves computes a BM x BN tile of Y; each wave
// owns a (BM/WAVES_M) x (BN/WAVES_N) sub-tile held as 16x16 MFMA tiles.  Each lane reads one
// 16-byte word per tile row or column per stage from LDS and widens it in registers.
// After every group the int32 accumulators are scaled into the fp32 output accumulators.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "atom_internal.h"

namespace atom {
namespace {

typedef int32_t v4i __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));   // native vector: stays in VGPRs

constexpr int kStageBytes = 64;          // bytes of one stage of a packed row

__device__ __forceinline__ v4i widen_lo(u32x4 p) {
  return v4i{(int32_t)((p.x << 4) & 0xF0F0F0F0u), (int32_t)((p.y << 4) & 0xF0F0F0F0u),
             (int32_t)((p.z << 4) & 0xF0F0F0F0u), (int32_t)((p.w << 4) & 0xF0F0F0F0u)};
}

__device__ __forceinline__ v4i widen_hi(u32x4 p) {
  return v4i{(int32_t)(p.x & 0xF0F0F0F0u), (int32_t)(p.y & 0xF0F0F0F0u), (int32_t)(p.z & 0xF0F0F0F0u),
             (int32_t)(p.w & 0xF0F0F0F0u)};
}

__device__ __forceinline__ v4i as_v4i(u32x4 p) { return v4i{(int32_t)p.x, (int32_t)p.y, (int32_t)p.z, (int32_t)p.w}; }

__device__ __forceinline__ float h2f(uint16_t h) { return __half2float(__ushort_as_half(h)); }

template <int BM, int BN, int WAVES_M, int WAVES_N>
struct Tile {
  static constexpr int kThreads = WAVES_M * WAVES_N * 64;
  static constexpr int kWTM = BM / WAVES_M;            // wave tile rows
  static constexpr int kWTN = BN / WAVES_N;            // wave tile columns
  static constexpr int kTM = kWTM / 16;                // MFMA tiles per wave (rows)
  static constexpr int kTN = kWTN / 16;                // MFMA tiles per wave (columns)
  static constexpr int kAPer = BM * 4 / kThreads;      // 16-byte A chunks per thread per stage
  static constexpr int kBPer = BN * 4 / kThreads;
  static_assert(kWTM % 16 == 0 && kWTN % 16 == 0, "wave tile must be a multiple of 16");
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

template <int APER, int BPER>
__device__ __forceinline__ void load_stage(StageRegs<APER, BPER>& st, const uint8_t* const (&a_src)[APER],
                                           const uint8_t* const (&b_src)[BPER], const uint16_t* s_src,
                                           size_t s_stride, int s, int G) {
  const size_t off = (size_t)s * kStageBytes;
#pragma unroll
  for (int p = 0; p < APER; ++p) st.a[p] = *reinterpret_cast<const u32x4*>(a_src[p] + off);
#pragma unroll
  for (int p = 0; p < BPER; ++p) st.b[p] = *reinterpret_cast<const u32x4*>(b_src[p] + off);
  if (s_src) st.s = s_src[(size_t)min(s, G - 1) * s_stride];
}

template <int BM, int BN, int NT, bool kAcc, int APER, int BPER>
__device__ __forceinline__ void store_stage(const StageRegs<APER, BPER>& st, uint8_t* la, uint8_t* lb, uint16_t* lsx,
                                            uint16_t* lsw, int tid) {
#pragma unroll
  for (int p = 0; p < APER; ++p) *reinterpret_cast<u32x4*>(la + (tid + p * NT) * 16) = st.a[p];
#pragma unroll
  for (int p = 0; p < BPER; ++p) *reinterpret_cast<u32x4*>(lb + (tid + p * NT) * 16) = st.b[p];
  if (!kAcc) {
    if (tid < BM) lsx[tid] = st.s;
    else if (tid < BM + BN) lsw[tid - BM] = st.s;
  }
}

// kAcc = false: Y output.  kAcc = true: write the per-group integer accumulators instead.
template <int BM, int BN, int WAVES_M, int WAVES_N, bool kAcc>
__global__ __launch_bounds__(WAVES_M* WAVES_N * 64) __attribute__((amdgpu_waves_per_eu(2))) void gemm_w4a4_kernel(
    const uint8_t* __restrict__ Xq, const uint16_t* __restrict__ sx, const uint8_t* __restrict__ Wq,
    const uint16_t* __restrict__ sw, int M, int N, int K, uint16_t* __restrict__ Y, int32_t* __restrict__ acc_out) {
  using T = Tile<BM, BN, WAVES_M, WAVES_N>;
  __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][BM * kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b[2][BN * kStageBytes];
  __shared__ __attribute__((aligned(16))) uint16_t lds_sx[2][BM];
  __shared__ __attribute__((aligned(16))) uint16_t lds_sw[2][BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WAVES_N;
  const int wn = wave % WAVES_N;
  const int m0 = blockIdx.y * BM;
  const int n0 = blockIdx.x * BN;
  const int G = K / ATOM_GROUP;
  const int S = G + 1;                                  // stages per row
  const size_t rbytes = (size_t)S * kStageBytes;        // = (K-128)/2 + 128
  const int l16 = lane & 15;                            // row (A) / column (B) inside a 16x16 tile
  const int kq = lane >> 4;                             // 16-byte quarter of the 64-byte stage

  // ---- per-thread global source pointers (rows past M / N repeat the last valid row)
  const uint8_t* a_src[T::kAPer];
  const uint8_t* b_src[T::kBPer];
#pragma unroll
  for (int p = 0; p < T::kAPer; ++p) {
    const int c = tid + p * T::kThreads;
    a_src[p] = Xq + (size_t)min(m0 + c / 4, M - 1) * rbytes + (c % 4) * 16;
  }
#pragma unroll
  for (int p = 0; p < T::kBPer; ++p) {
    const int c = tid + p * T::kThreads;
    b_src[p] = Wq + (size_t)min(n0 + c / 4, N - 1) * rbytes + (c % 4) * 16;
  }
  const uint16_t* s_src = nullptr;                      // this thread's scale column
  size_t s_stride = 0;
  if (!kAcc) {
    if (tid < BM) {
      s_src = sx + min(m0 + tid, M - 1);
      s_stride = (size_t)M;
    } else if (tid < BM + BN) {
      s_src = sw + min(n0 + tid - BM, N - 1);
      s_stride = (size_t)N;
    }
  }

  StageRegs<T::kAPer, T::kBPer> st;
  float yacc[T::kTM][T::kTN][4];
#pragma unroll
  for (int i = 0; i < T::kTM; ++i)
#pragma unroll
    for (int j = 0; j < T::kTN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) yacc[i][j][r] = 0.0f;
  v4i acc[T::kTM][T::kTN];

  // LDS reads of this lane: row l16 of each 16-row tile, 16-byte quarter kq of the stage
  auto lds_a_word = [&](int buf, int i) {
    return *reinterpret_cast<const u32x4*>(lds_a[buf] + (wm * T::kWTM + i * 16 + l16) * kStageBytes + kq * 16);
  };
  auto lds_b_word = [&](int buf, int j) {
    return *reinterpret_cast<const u32x4*>(lds_b[buf] + (wn * T::kWTN + j * 16 + l16) * kStageBytes + kq * 16);
  };

  // One INT4 group: low-nibble MFMAs start the accumulators, high-nibble MFMAs finish them.
  auto mma_int4 = [&](int buf) {
    u32x4 pa[T::kTM], pb[T::kTN];
#pragma unroll
    for (int i = 0; i < T::kTM; ++i) pa[i] = lds_a_word(buf, i);
#pragma unroll
    for (int j = 0; j < T::kTN; ++j) pb[j] = lds_b_word(buf, j);
#pragma unroll
    for (int i = 0; i < T::kTM; ++i) {
      const v4i a_lo = widen_lo(pa[i]);
#pragma unroll
      for (int j = 0; j < T::kTN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a_lo, widen_lo(pb[j]), v4i{0, 0, 0, 0}, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < T::kTM; ++i) {
      const v4i a_hi = widen_hi(pa[i]);
#pragma unroll
      for (int j = 0; j < T::kTN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a_hi, widen_hi(pb[j]), acc[i][j], 0, 0, 0);
    }
  };

  // One 64-channel half of the INT8 outlier group (no widening).
  auto mma_int8 = [&](int buf, bool first) {
    v4i bf[T::kTN];
#pragma unroll
    for (int j = 0; j < T::kTN; ++j) bf[j] = as_v4i(lds_b_word(buf, j));
#pragma unroll
    for (int i = 0; i < T::kTM; ++i) {
      const v4i af = as_v4i(lds_a_word(buf, i));
#pragma unroll
      for (int j = 0; j < T::kTN; ++j)
        acc[i][j] = first ? __builtin_amdgcn_mfma_i32_16x16x64_i8(af, bf[j], v4i{0, 0, 0, 0}, 0, 0, 0)
                          : __builtin_amdgcn_mfma_i32_16x16x64_i8(af, bf[j], acc[i][j], 0, 0, 0);
    }
  };

  // Scale the finished integer accumulators of group g into the fp32 output accumulators,
  // or (kAcc) write them out.  wscale undoes the x256 of the nibble widening.
  auto epilogue = [&](int buf, int g, float wscale, bool widened) {
    if (kAcc) {
#pragma unroll
      for (int i = 0; i < T::kTM; ++i)
#pragma unroll
        for (int j = 0; j < T::kTN; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int m = m0 + wm * T::kWTM + i * 16 + kq * 4 + r;
            const int n = n0 + wn * T::kWTN + j * 16 + l16;
            if (m < M && n < N) acc_out[((size_t)g * M + m) * N + n] = widened ? (acc[i][j][r] >> 8) : acc[i][j][r];
          }
    } else {
      float swv[T::kTN];
#pragma unroll
      for (int j = 0; j < T::kTN; ++j) swv[j] = h2f(lds_sw[buf][wn * T::kWTN + j * 16 + l16]) * wscale;
#pragma unroll
      for (int i = 0; i < T::kTM; ++i) {
        const uint2 s4 = *reinterpret_cast<const uint2*>(&lds_sx[buf][wm * T::kWTM + i * 16 + kq * 4]);
        const float sxv[4] = {h2f((uint16_t)(s4.x & 0xffff)), h2f((uint16_t)(s4.x >> 16)),
                              h2f((uint16_t)(s4.y & 0xffff)), h2f((uint16_t)(s4.y >> 16))};
#pragma unroll
        for (int j = 0; j < T::kTN; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            yacc[i][j][r] = __builtin_fmaf((float)acc[i][j][r], sxv[r] * swv[j], yacc[i][j][r]);
      }
    }
  };

  load_stage(st, a_src, b_src, s_src, s_stride, 0, G);
  store_stage<BM, BN, T::kThreads, kAcc>(st, lds_a[0], lds_b[0], lds_sx[0], lds_sw[0], tid);
  load_stage(st, a_src, b_src, s_src, s_stride, 1, G);
  __syncthreads();

  // INT4 groups: stages 0 .. G-2
  for (int s = 0; s < G - 1; ++s) {
    const int buf = s & 1;
    mma_int4(buf);
    // stage s+1 into the other buffer (released by the last barrier), then start stage s+2
    store_stage<BM, BN, T::kThreads, kAcc>(st, lds_a[buf ^ 1], lds_b[buf ^ 1], lds_sx[buf ^ 1], lds_sw[buf ^ 1], tid);
    load_stage(st, a_src, b_src, s_src, s_stride, s + 2, G);   // s+2 <= G: always a valid stage
    epilogue(buf, s, 1.0f / 256.0f, true);
    __syncthreads();
  }
  // INT8 outlier group: stages G-1 and G
  {
    const int buf = (G - 1) & 1;
    mma_int8(buf, true);
    store_stage<BM, BN, T::kThreads, kAcc>(st, lds_a[buf ^ 1], lds_b[buf ^ 1], lds_sx[buf ^ 1], lds_sw[buf ^ 1],
                                           tid);   // stage G
    __syncthreads();
    mma_int8(buf ^ 1, false);
    epilogue(buf ^ 1, G - 1, 1.0f, false);
  }

  if (!kAcc) {
#pragma unroll
    for (int i = 0; i < T::kTM; ++i)
#pragma unroll
      for (int j = 0; j < T::kTN; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = m0 + wm * T::kWTM + i * 16 + kq * 4 + r;
          const int n = n0 + wn * T::kWTN + j * 16 + l16;
          if (m < M && n < N) Y[(size_t)m * N + n] = __half_as_ushort(__float2half_rn(yacc[i][j][r]));
        }
  }
}

// 128 x 128 workgroup tile, 2 x 2 waves of 64 x 64.
constexpr int kBM = 128, kBN = 128, kWavesM = 2, kWavesN = 2;

}  // namespace

hipError_t launch_gemm(const uint8_t* Xq, const uint16_t* sx, const uint8_t* Wq, const uint16_t* sw, int M, int N,
                       int K, uint16_t* Y, hipStream_t stream) {
  const dim3 grid((N + kBN - 1) / kBN, (M + kBM - 1) / kBM);
  hipLaunchKernelGGL((gemm_w4a4_kernel<kBM, kBN, kWavesM, kWavesN, false>), grid, dim3(kWavesM * kWavesN * 64), 0,
                     stream, Xq, sx, Wq, sw, M, N, K, Y, (int32_t*)nullptr);
  return hipGetLastError();
}

hipError_t launch_gemm_group_acc(const uint8_t* Xq, const uint8_t* Wq, int M, int N, int K, int32_t* acc,
                                 hipStream_t stream) {
  const dim3 grid((N + kBN - 1) / kBN, (M + kBM - 1) / kBM);
  hipLaunchKernelGGL((gemm_w4a4_kernel<kBM, kBN, kWavesM, kWavesN, true>), grid, dim3(kWavesM * kWavesN * 64), 0,
                     stream, Xq, (const uint16_t*)nullptr, Wq, (const uint16_t*)nullptr, M, N, K,
                     (uint16_t*)nullptr, acc);
  return hipGetLastError();
}

}  // namespace atom
