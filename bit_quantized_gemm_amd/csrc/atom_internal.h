// Internal launcher declarations shared by the host API and the kernel sources.
// Every launcher enqueues on `stream` and returns hipGetLastError() after its launches;
// arguments are validated by the caller (atom_api.cpp) before any launcher runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "atom.h"

namespace atom {

// Packed INT4 unit (16 codes, 8 bytes; written by the row quantize, read by the GEMMs): the
// codes' fp6 e2m3 fields (c / 8 as a subnormal: |c| in bits 0-2, sign in bit 5) at bits 6i of
// a 96-bit string T0:T1:T2, stored as T0 | (T2 & kFp6Exp0), T1 | (T2 & kFp6Exp1).  The masks
// are the exponent bits (3 and 4 of each field) of T0 and T1, always zero for INT4 codes;
// T2's nonzero bits are exactly their union, so T2 = (w0 & kFp6Exp0) | (w1 & kFp6Exp1).
constexpr uint32_t kFp6Exp0 = 0x18618618u, kFp6Exp1 = 0x86186186u;

hipError_t launch_channel_stat(const uint16_t* X, int M, int K, double* stat, hipStream_t stream);
hipError_t launch_select_outliers(const double* stat, int K, int32_t* perm, hipStream_t stream);
// Packed row formats the row quantize writes.
//   kRowW4A4: INT4 groups in the fp6-fold units above, INT8 outlier group last; (K-128)/2 + 128 bytes.
//   kRowA8:   every group INT8 (qmax 127), one two's-complement byte per code; K bytes.
//   kRowW4A8: INT4 groups as offset-binary nibbles (byte j of each 8-code block holds c_j + 8
//             and c_{j+4} + 8 in its low and high nibble), INT8 outlier group last; (K-128)/2 + 128 bytes.
enum RowFormat { kRowW4A4 = 0, kRowA8 = 1, kRowW4A8 = 2 };
hipError_t launch_row_quantize(const uint16_t* X, const int32_t* perm, int rows, int K, uint8_t* Q,
                               uint16_t* S, RowFormat fmt, hipStream_t stream);
// Split-K plan of a GEMM: the first `full` output tiles (in the kernel's tile order) run whole;
// each of the last `rem` tiles is divided into `splits` pieces along K, whose fp32 partial
// tiles go to caller scratch and are added by a second kernel.  rem == 0: no split.  The
// kernel takes any mix; gemm_plan returns either no split or every tile split.
// small != 0 instead selects the few-rows kernel (gemm_small.hip), which needs no scratch.
// tile64 != 0 instead runs whole 64 x 64 output tiles (two waves of 32 x 64 each), for grids
// that have too few 128 x 128 tiles to fill the GPU but enough 64 x 64 ones: no split, no scratch.
// kpart != 0 instead runs whole 64 x 64 output tiles with four waves each, every wave a
// quarter of the K range, added in LDS at the end: no scratch, no second kernel.
struct GemmPlan {
  int full, rem, splits;
  int small;
  int tile64;
  int kpart;
};
// Few-rows kernel: at most kSmallMaxM token rows.
constexpr int kSmallMaxM = 16;
// Compute units of the device current at the first call (queried once per process; 256 if
// the query fails).
int compute_units();

GemmPlan gemm_plan(int M, int N, int K);
// The same plan for the 128 x 128 tiled kernels only (no few-rows branch).
GemmPlan gemm_plan_tiled(int M, int N, int K);
// Adds the fp32 partial tiles of a split plan (tile-major, piece p of split tile t at
// part[(p * rem + t) * 128 * 128], row-major inside the tile, carrying the factor 2 of the scale
// products) in piece order and writes Y.
hipError_t launch_splitk_finish(const float* part, const GemmPlan& plan, int M, int N, uint16_t* Y,
                                hipStream_t stream);

// Output tile order of the tiled GEMM kernels: tiles are numbered in bands of kBandM tile rows,
// M fastest inside a band, so a run of 64 consecutive tiles is an 8 x 8 block.  Returns the
// tile's row and column index.
constexpr int kBandM = 8;
__host__ __device__ inline int2 tile_coords(int lin, int tiles_m, int tiles_n) {
  const int band = lin / (kBandM * tiles_n), first_m = band * kBandM;
  const int band_m = min(tiles_m - first_m, kBandM);     // tile rows in this band
  const int in_band = lin - band * kBandM * tiles_n;
  return int2{first_m + in_band % band_m, in_band / band_m};
}
// Scratch bytes the plan needs (0 when it writes Y directly).
int64_t gemm_workspace_bytes(const GemmPlan& plan);
// `part` holds gemm_workspace_bytes(plan) bytes of scratch when that is > 0, else unused.
hipError_t launch_gemm(const uint8_t* Xq, const uint16_t* sx, const uint8_t* Wq, const uint16_t* sw, int M, int N,
                       int K, uint16_t* Y, float* part, const GemmPlan& plan, hipStream_t stream);
// The library's static split-K scratch (atom_gemm_noalloc): its size, and its device address on
// the current device (looked up once per device; no allocation).
int64_t static_scratch_bytes();
hipError_t static_scratch_address(void** out);
// Few-rows kernel (M <= kSmallMaxM), Y written directly.
hipError_t launch_gemm_small(const uint8_t* Xq, const uint16_t* sx, const uint8_t* Wq, const uint16_t* sw, int M,
                             int N, int K, uint16_t* Y, hipStream_t stream);
// Per-group integer sums [G, M, N] from the kernel atom_gemm runs for this shape (the few-rows
// kernel for M <= kSmallMaxM, the tiled kernel otherwise).
hipError_t launch_gemm_group_acc(const uint8_t* Xq, const uint8_t* Wq, int M, int N, int K, int32_t* acc,
                                 hipStream_t stream);
// Activation quantize + GEMM in one persistent launch (gemm.hip), for shapes whose GEMM runs whole
// 128 x 128 tiles and K <= 12288 (linear_fused_supported).  ws: linear_fused_workspace_bytes(M)
// bytes, zero before the first call and left zero by every call.
bool linear_fused_supported(int M, int N, int K);
int64_t linear_fused_workspace_bytes(int M);
hipError_t launch_linear_fused(const uint16_t* X, const int32_t* perm, const uint8_t* Wq, const uint16_t* sw, int M,
                               int N, int K, uint8_t* Xq, uint16_t* sx, uint16_t* Y, int* ws, hipStream_t stream);
hipError_t launch_gemm_small_group_acc(const uint8_t* Xq, const uint8_t* Wq, int M, int N, int K, int32_t* acc,
                                       hipStream_t stream);
// W4A8 GEMM (gemm_w4a8.hip): Xq in kRowA8 rows, Wq in kRowW4A8 rows.  acc != nullptr: write
// the per-group int32 accumulators [G, M, N] instead of Y.
// plan: gemm_plan_tiled(M, N, K), or an unsplit plan; `part` holds gemm_workspace_bytes(plan)
// bytes when the plan splits.
hipError_t launch_gemm_w4a8(const uint8_t* Xq, const uint16_t* sx, const uint8_t* Wq, const uint16_t* sw, int M,
                            int N, int K, uint16_t* Y, int32_t* acc, float* part, const GemmPlan& plan,
                            hipStream_t stream);

}  // namespace atom
