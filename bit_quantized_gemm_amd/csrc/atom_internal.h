// Internal launcher declarations shared by the host API and the kernel sources.
// Every launcher enqueues on `stream` and returns hipGetLastError() after its launches;
// arguments are validated by the caller (atom_api.cpp) before any launcher runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "atom.h"

namespace atom {

hipError_t launch_channel_stat(const uint16_t* X, int M, int K, double* stat, hipStream_t stream);
hipError_t launch_select_outliers(const double* stat, int K, int32_t* perm, hipStream_t stream);
hipError_t launch_row_quantize(const uint16_t* X, const int32_t* perm, int rows, int K, uint8_t* Q,
                               uint16_t* S, hipStream_t stream);
// Number of workgroups a tile's K range is divided among (1: no split-K).
int gemm_splits(int M, int N, int K);
// splits > 1: `part` holds splits * M * N floats of scratch; splits == 1: `part` unused.
hipError_t launch_gemm(const uint8_t* Xq, const uint16_t* sx, const uint8_t* Wq, const uint16_t* sw, int M, int N,
                       int K, uint16_t* Y, float* part, int splits, hipStream_t stream);
hipError_t launch_gemm_group_acc(const uint8_t* Xq, const uint8_t* Wq, int M, int N, int K, int32_t* acc,
                                 hipStream_t stream);

}  // namespace atom
