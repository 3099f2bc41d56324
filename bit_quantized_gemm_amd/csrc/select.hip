// Outlier channel statistic and selection (offline calibration step) for gfx950.
//
// Atom keeps a small set of input channels at higher precision as one 128-channel group
// (quantization record "Atom (mixed-precision block-outlier low-bit quantization for
// serving)", Fields "Activation scheme" and "notes").  The pages leave the selection rule
// open; the layer ranks channels by their sum of squares over calibration tokens.
//
// Exactness: an fp16 value x is an integer multiple of 2^-24, so x^2 * 2^48 is an integer
// below 2^80.  Each channel accumulates those integers in an unsigned 128-bit register
// (no rounding, order-free) and converts the exact total once to fp64 with round-to-nearest-
// even.  The statistic is therefore bit-identical to the correctly rounded exact sum.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "atom_internal.h"

namespace atom {
namespace {

typedef unsigned __int128 u128;

// |x| * 2^24 for an fp16 bit pattern, as an integer (exact; inf/NaN are not meaningful).
__device__ __forceinline__ uint64_t fp16_abs_units(uint16_t h) {
  const uint32_t e = (h >> 10) & 0x1f;
  const uint32_t m = h & 0x3ff;
  if (e == 0) return m;                                  // subnormal: m * 2^-24
  return (uint64_t)(m | 0x400) << (e - 1);               // (1024+m) * 2^(e-25)
}

// Round the exact value S * 2^-48 to the nearest fp64 (ties to even).
__device__ double u128_scaled_to_double(u128 S) {
  const uint64_t hi = (uint64_t)(S >> 64);
  const uint64_t lo = (uint64_t)S;
  if (hi == 0 && lo < (1ull << 53)) return ldexp((double)lo, -48);   // exact
  const int top = hi ? 127 - __clzll(hi) : 63 - __clzll(lo);          // index of the leading bit
  const int shift = top - 52;                                         // drop this many bits
  u128 mant = S >> shift;
  const u128 rem = S - (mant << shift);
  const u128 half = (u128)1 << (shift - 1);
  if (rem > half || (rem == half && (mant & 1))) mant += 1;
  int e = shift;
  if (mant >> 53) { mant >>= 1; e += 1; }                             // carried into a new bit
  return ldexp((double)(uint64_t)mant, e - 48);
}

constexpr int kStatThreads = 1024;   // 16 waves; each lane owns one channel of a 64-wide slab
constexpr int kStatWaves = kStatThreads / 64;

__global__ __launch_bounds__(kStatThreads) void channel_stat_kernel(const uint16_t* __restrict__ X, int M, int K,
                                                                    double* __restrict__ stat) {
  __shared__ uint64_t part_lo[kStatWaves][64];
  __shared__ uint64_t part_hi[kStatWaves][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int c = blockIdx.x * 64 + lane;          // K is a multiple of 128, so c < K always
  u128 acc = 0;
  for (int m = wave; m < M; m += kStatWaves) {
    const uint64_t v = fp16_abs_units(X[(size_t)m * K + c]);
    acc += (u128)v * v;
  }
  part_lo[wave][lane] = (uint64_t)acc;
  part_hi[wave][lane] = (uint64_t)(acc >> 64);
  __syncthreads();
  if (wave == 0) {
    u128 tot = 0;
    for (int w = 0; w < kStatWaves; ++w) tot += ((u128)part_hi[w][lane] << 64) | part_lo[w][lane];
    stat[c] = u128_scaled_to_double(tot);
  }
}

// Rank of channel c = #{c' : stat[c'] > stat[c]} + #{c' < c : stat[c'] == stat[c]}.
// The 128 channels of rank < 128 are the outliers.  The flag is written into perm, which
// build_perm_kernel then overwrites with the permutation.
constexpr int kRankThreads = 256;
constexpr int kRankChunk = 2048;

__global__ __launch_bounds__(kRankThreads) void outlier_flag_kernel(const double* __restrict__ stat, int K,
                                                                    int32_t* __restrict__ flags) {
  __shared__ double chunk[kRankChunk];
  const int c = blockIdx.x * kRankThreads + threadIdx.x;
  const double mine = c < K ? stat[c] : 0.0;
  int rank = 0;
  for (int base = 0; base < K; base += kRankChunk) {
    const int n = min(kRankChunk, K - base);
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += kRankThreads) chunk[i] = stat[base + i];
    __syncthreads();
    for (int i = 0; i < n; ++i) {
      const double o = chunk[i];
      rank += (o > mine) | ((o == mine) & (base + i < c));
    }
  }
  if (c < K) flags[c] = rank < ATOM_OUTLIERS ? 1 : 0;
}

// Stable partition: non-outlier channels ascending, then outlier channels ascending.
// Positions are always inside [0, K), whatever the flags hold.
constexpr int kPermThreads = 1024;

__global__ __launch_bounds__(kPermThreads) void build_perm_kernel(int32_t* __restrict__ perm, int K) {
  __shared__ uint8_t flag[ATOM_MAX_K];
  __shared__ int cnt_out[kPermThreads];
  __shared__ int total_out;
  const int t = threadIdx.x;
  const int per = (K + kPermThreads - 1) / kPermThreads;
  const int lo = min(K, t * per), hi = min(K, lo + per);
  int mine = 0;
  for (int j = lo; j < hi; ++j) {
    const uint8_t f = perm[j] != 0;
    flag[j] = f;
    mine += f;
  }
  cnt_out[t] = mine;
  __syncthreads();
  // inclusive scan over the per-thread outlier counts (Hillis-Steele)
  for (int off = 1; off < kPermThreads; off <<= 1) {
    const int v = t >= off ? cnt_out[t - off] : 0;
    __syncthreads();
    cnt_out[t] += v;
    __syncthreads();
  }
  if (t == kPermThreads - 1) total_out = cnt_out[t];
  __syncthreads();
  int out_before = cnt_out[t] - mine;
  int non_before = lo - out_before;
  const int tail0 = K - total_out;
  for (int j = lo; j < hi; ++j) {
    if (flag[j]) perm[tail0 + out_before++] = j;
    else perm[non_before++] = j;
  }
}

}  // namespace

hipError_t launch_channel_stat(const uint16_t* X, int M, int K, double* stat, hipStream_t stream) {
  hipLaunchKernelGGL(channel_stat_kernel, dim3(K / 64), dim3(kStatThreads), 0, stream, X, M, K, stat);
  return hipGetLastError();
}

hipError_t launch_select_outliers(const double* stat, int K, int32_t* perm, hipStream_t stream) {
  hipLaunchKernelGGL(outlier_flag_kernel, dim3((K + kRankThreads - 1) / kRankThreads), dim3(kRankThreads), 0,
                     stream, stat, K, perm);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(build_perm_kernel, dim3(1), dim3(kPermThreads), 0, stream, perm, K);
  return hipGetLastError();
}

}  // namespace atom
