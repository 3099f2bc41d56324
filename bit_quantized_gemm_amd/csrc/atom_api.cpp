// Host side of the C ABI declared in include/atom.h: argument validation (all of it before
// any HIP call), then the kernel launches on the caller's stream.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "atom_internal.h"

namespace {

struct Range {
  uintptr_t lo, hi;   // [lo, hi)
};

Range range_of(const void* p, uint64_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{a, a + (uintptr_t)bytes};
}

bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_k(int32_t K) { return K >= 2 * ATOM_GROUP && K <= ATOM_MAX_K && K % ATOM_GROUP == 0; }

bool valid_rows(int32_t r) { return r >= 1 && r <= ATOM_MAX_ROWS; }

// GEMM shapes: both row counts valid and the 128 x 128 output tiles (a 1-D grid, with split-K
// pieces on top) well inside the 32-bit grid range.
bool valid_gemm(int32_t M, int32_t N, int32_t K) {
  if (!valid_k(K) || !valid_rows(M) || !valid_rows(N)) return false;
  const uint64_t tiles = (uint64_t)((M + 127) / 128) * (uint64_t)((N + 127) / 128);
  return tiles <= ATOM_MAX_TILES;
}

int hip_status(hipError_t e) { return e == hipSuccess ? ATOM_OK : ATOM_E_HIP; }

// Every output must be disjoint from every input and from the other outputs.
int check_overlap(const Range* in, int n_in, const Range* out, int n_out) {
  for (int o = 0; o < n_out; ++o) {
    for (int i = 0; i < n_in; ++i)
      if (overlaps(out[o], in[i])) return ATOM_E_OVERLAP;
    for (int p = o + 1; p < n_out; ++p)
      if (overlaps(out[o], out[p])) return ATOM_E_OVERLAP;
  }
  return ATOM_OK;
}

// rb = bytes of one packed output row (W4A4 and W4A8 weights: (K-128)/2 + 128; A8: K)
int check_row_quantize(const void* X, const int32_t* perm, int32_t rows, int32_t K, void* Q, void* S, bool a8) {
  if (!X || !perm || !Q || !S) return ATOM_E_NULL;
  if (!valid_k(K) || !valid_rows(rows)) return ATOM_E_SHAPE;
  if (!aligned16(X) || !aligned16(perm) || !aligned16(Q) || !aligned16(S)) return ATOM_E_ALIGN;
  const uint64_t G = (uint64_t)K / ATOM_GROUP;
  const uint64_t rb = a8 ? (uint64_t)K : (uint64_t)atom_row_bytes(K);
  const Range in[2] = {range_of(X, (uint64_t)rows * K * 2), range_of(perm, (uint64_t)K * 4)};
  const Range out[2] = {range_of(Q, (uint64_t)rows * rb), range_of(S, G * rows * 2)};
  return check_overlap(in, 2, out, 2);
}

}  // namespace

extern "C" {

int64_t atom_row_bytes(int32_t K) {
  if (!valid_k(K)) return -(int64_t)ATOM_E_SHAPE;
  return (int64_t)(K - ATOM_OUTLIERS) / 2 + ATOM_OUTLIERS;
}

int32_t atom_num_groups(int32_t K) {
  if (!valid_k(K)) return -ATOM_E_SHAPE;
  return K / ATOM_GROUP;
}

const char* atom_strerror(int status) {
  switch (status) {
    case ATOM_OK: return "ok";
    case ATOM_E_NULL: return "a required pointer is NULL";
    case ATOM_E_SHAPE: return "invalid shape: K must be a multiple of 128 in [256, 65536] and rows in [1, 2^24]";
    case ATOM_E_ALIGN: return "a pointer is not 16-byte aligned";
    case ATOM_E_OVERLAP: return "an output buffer overlaps an input or another output";
    case ATOM_E_HIP: return "the HIP runtime reported an error when enqueuing a kernel";
    case ATOM_E_SCRATCH: return "the shape needs more split-K scratch than the library's static buffer holds";
    default: return "unknown status";
  }
}

int atom_channel_stat(const void* X, int32_t M, int32_t K, double* stat, void* stream) {
  if (!X || !stat) return ATOM_E_NULL;
  if (!valid_k(K) || !valid_rows(M)) return ATOM_E_SHAPE;
  if (!aligned16(X) || !aligned16(stat)) return ATOM_E_ALIGN;
  const Range in[1] = {range_of(X, (uint64_t)M * K * 2)};
  const Range out[1] = {range_of(stat, (uint64_t)K * 8)};
  if (int s = check_overlap(in, 1, out, 1)) return s;
  return hip_status(atom::launch_channel_stat(static_cast<const uint16_t*>(X), M, K, stat,
                                              static_cast<hipStream_t>(stream)));
}

int atom_select_outliers(const double* stat, int32_t K, int32_t* perm, void* stream) {
  if (!stat || !perm) return ATOM_E_NULL;
  if (!valid_k(K)) return ATOM_E_SHAPE;
  if (!aligned16(stat) || !aligned16(perm)) return ATOM_E_ALIGN;
  const Range in[1] = {range_of(stat, (uint64_t)K * 8)};
  const Range out[1] = {range_of(perm, (uint64_t)K * 4)};
  if (int s = check_overlap(in, 1, out, 1)) return s;
  return hip_status(atom::launch_select_outliers(stat, K, perm, static_cast<hipStream_t>(stream)));
}

int atom_pack_weights(const void* W, const int32_t* perm, int32_t N, int32_t K, void* Wq, void* sw, void* stream) {
  if (int s = check_row_quantize(W, perm, N, K, Wq, sw, false)) return s;
  return hip_status(atom::launch_row_quantize(static_cast<const uint16_t*>(W), perm, N, K,
                                              static_cast<uint8_t*>(Wq), static_cast<uint16_t*>(sw), atom::kRowW4A4,
                                              static_cast<hipStream_t>(stream)));
}

int atom_quantize_act(const void* X, const int32_t* perm, int32_t M, int32_t K, void* Xq, void* sx, void* stream) {
  if (int s = check_row_quantize(X, perm, M, K, Xq, sx, false)) return s;
  return hip_status(atom::launch_row_quantize(static_cast<const uint16_t*>(X), perm, M, K,
                                              static_cast<uint8_t*>(Xq), static_cast<uint16_t*>(sx), atom::kRowW4A4,
                                              static_cast<hipStream_t>(stream)));
}

int64_t atom_gemm_workspace_bytes(int32_t M, int32_t N, int32_t K) {
  if (!valid_gemm(M, N, K)) return -(int64_t)ATOM_E_SHAPE;
  return atom::gemm_workspace_bytes(atom::gemm_plan(M, N, K));
}

int atom_gemm_ws(const void* Xq, const void* sx, const void* Wq, const void* sw, int32_t M, int32_t N, int32_t K,
                 void* Y, void* workspace, int64_t workspace_bytes, void* stream) {
  if (!Xq || !sx || !Wq || !sw || !Y) return ATOM_E_NULL;
  if (!valid_gemm(M, N, K)) return ATOM_E_SHAPE;
  if (!aligned16(Xq) || !aligned16(sx) || !aligned16(Wq) || !aligned16(sw) || !aligned16(Y)) return ATOM_E_ALIGN;
  atom::GemmPlan plan = atom::gemm_plan(M, N, K);
  int64_t need = atom::gemm_workspace_bytes(plan);
  if (need > 0 && (!workspace || workspace_bytes < need)) {   // too little scratch: the 128 x 128 kernel, unsplit
    plan = atom::GemmPlan{((M + 127) / 128) * ((N + 127) / 128), 0, 1, 0};
    need = 0;
  }
  const bool split = need > 0;
  if (split && !aligned16(workspace)) return ATOM_E_ALIGN;
  const uint64_t G = (uint64_t)K / ATOM_GROUP;
  const uint64_t rb = (uint64_t)atom_row_bytes(K);
  const Range in[4] = {range_of(Xq, (uint64_t)M * rb), range_of(sx, G * M * 2), range_of(Wq, (uint64_t)N * rb),
                       range_of(sw, G * N * 2)};
  const Range out[2] = {range_of(Y, (uint64_t)M * N * 2), range_of(workspace, split ? (uint64_t)need : 0)};
  if (int s = check_overlap(in, 4, out, split ? 2 : 1)) return s;
  return hip_status(atom::launch_gemm(static_cast<const uint8_t*>(Xq), static_cast<const uint16_t*>(sx),
                                      static_cast<const uint8_t*>(Wq), static_cast<const uint16_t*>(sw), M, N, K,
                                      static_cast<uint16_t*>(Y), static_cast<float*>(workspace), plan,
                                      static_cast<hipStream_t>(stream)));
}

int atom_gemm(const void* Xq, const void* sx, const void* Wq, const void* sw, int32_t M, int32_t N, int32_t K, void* Y,
              void* stream) {
  return atom_gemm_ws(Xq, sx, Wq, sw, M, N, K, Y, nullptr, 0, stream);
}

int atom_gemm_noalloc(const void* Xq, const void* sx, const void* Wq, const void* sw, int32_t M, int32_t N, int32_t K,
                      void* Y, void* stream) {
  if (!Xq || !sx || !Wq || !sw || !Y) return ATOM_E_NULL;
  if (!valid_gemm(M, N, K)) return ATOM_E_SHAPE;
  if (!aligned16(Xq) || !aligned16(sx) || !aligned16(Wq) || !aligned16(sw) || !aligned16(Y)) return ATOM_E_ALIGN;
  const atom::GemmPlan plan = atom::gemm_plan(M, N, K);
  const int64_t need = atom::gemm_workspace_bytes(plan);
  if (need > atom::static_scratch_bytes()) return ATOM_E_SCRATCH;
  const uint64_t G = (uint64_t)K / ATOM_GROUP;
  const uint64_t rb = (uint64_t)atom_row_bytes(K);
  const Range in[4] = {range_of(Xq, (uint64_t)M * rb), range_of(sx, G * M * 2), range_of(Wq, (uint64_t)N * rb),
                       range_of(sw, G * N * 2)};
  const Range out[1] = {range_of(Y, (uint64_t)M * N * 2)};
  if (int st = check_overlap(in, 4, out, 1)) return st;
  void* part = nullptr;
  if (need > 0 && atom::static_scratch_address(&part) != hipSuccess) return ATOM_E_HIP;
  return hip_status(atom::launch_gemm(static_cast<const uint8_t*>(Xq), static_cast<const uint16_t*>(sx),
                                      static_cast<const uint8_t*>(Wq), static_cast<const uint16_t*>(sw), M, N, K,
                                      static_cast<uint16_t*>(Y), static_cast<float*>(part), plan,
                                      static_cast<hipStream_t>(stream)));
}

int atom_gemm_group_acc(const void* Xq, const void* Wq, int32_t M, int32_t N, int32_t K, int32_t* acc,
                        void* stream) {
  if (!Xq || !Wq || !acc) return ATOM_E_NULL;
  if (!valid_gemm(M, N, K)) return ATOM_E_SHAPE;
  if (!aligned16(Xq) || !aligned16(Wq) || !aligned16(acc)) return ATOM_E_ALIGN;
  const uint64_t G = (uint64_t)K / ATOM_GROUP;
  const uint64_t rb = (uint64_t)atom_row_bytes(K);
  const Range in[2] = {range_of(Xq, (uint64_t)M * rb), range_of(Wq, (uint64_t)N * rb)};
  const Range out[1] = {range_of(acc, G * M * N * 4)};
  if (int s = check_overlap(in, 2, out, 1)) return s;
  return hip_status(atom::launch_gemm_group_acc(static_cast<const uint8_t*>(Xq), static_cast<const uint8_t*>(Wq), M,
                                                N, K, acc, static_cast<hipStream_t>(stream)));
}

// ---- fused runtime forward (activation quantize + GEMM)

int64_t atom_linear_workspace_bytes(int32_t M, int32_t N, int32_t K) {
  if (!valid_gemm(M, N, K)) return -(int64_t)ATOM_E_SHAPE;
  return atom::linear_fused_workspace_bytes(M) + atom::gemm_workspace_bytes(atom::gemm_plan(M, N, K));
}

int atom_linear(const void* X, const int32_t* perm, const void* Wq, const void* sw, int32_t M, int32_t N, int32_t K,
                void* Xq, void* sx, void* Y, void* workspace, int64_t workspace_bytes, void* stream) {
  if (!X || !perm || !Wq || !sw || !Xq || !sx || !Y || !workspace) return ATOM_E_NULL;
  if (!valid_gemm(M, N, K)) return ATOM_E_SHAPE;
  const int64_t need = atom_linear_workspace_bytes(M, N, K);
  if (workspace_bytes < need) return ATOM_E_SHAPE;
  if (!aligned16(X) || !aligned16(perm) || !aligned16(Wq) || !aligned16(sw) || !aligned16(Xq) || !aligned16(sx) ||
      !aligned16(Y) || !aligned16(workspace))
    return ATOM_E_ALIGN;
  const uint64_t G = (uint64_t)K / ATOM_GROUP;
  const uint64_t rb = (uint64_t)atom_row_bytes(K);
  const Range in[4] = {range_of(X, (uint64_t)M * K * 2), range_of(perm, (uint64_t)K * 4),
                       range_of(Wq, (uint64_t)N * rb), range_of(sw, G * N * 2)};
  const Range out[4] = {range_of(Xq, (uint64_t)M * rb), range_of(sx, G * M * 2), range_of(Y, (uint64_t)M * N * 2),
                        range_of(workspace, (uint64_t)need)};
  if (int st = check_overlap(in, 4, out, 4)) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (atom::linear_fused_supported(M, N, K))
    return hip_status(atom::launch_linear_fused(static_cast<const uint16_t*>(X), perm, static_cast<const uint8_t*>(Wq),
                                                static_cast<const uint16_t*>(sw), M, N, K, static_cast<uint8_t*>(Xq),
                                                static_cast<uint16_t*>(sx), static_cast<uint16_t*>(Y),
                                                static_cast<int*>(workspace), s));
  // two launches: the quantize, then the GEMM with the split-K part of the workspace
  hipError_t e = atom::launch_row_quantize(static_cast<const uint16_t*>(X), perm, M, K, static_cast<uint8_t*>(Xq),
                                           static_cast<uint16_t*>(sx), atom::kRowW4A4, s);
  if (e != hipSuccess) return ATOM_E_HIP;
  const atom::GemmPlan plan = atom::gemm_plan(M, N, K);
  float* part = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + atom::linear_fused_workspace_bytes(M));
  return hip_status(atom::launch_gemm(static_cast<const uint8_t*>(Xq), static_cast<const uint16_t*>(sx),
                                      static_cast<const uint8_t*>(Wq), static_cast<const uint16_t*>(sw), M, N, K,
                                      static_cast<uint16_t*>(Y), atom::gemm_workspace_bytes(plan) > 0 ? part : nullptr,
                                      plan, s));
}

// ---- W4A8 variant

int atom_quantize_act_a8(const void* X, const int32_t* perm, int32_t M, int32_t K, void* Xq, void* sx,
                         void* stream) {
  if (int s = check_row_quantize(X, perm, M, K, Xq, sx, true)) return s;
  return hip_status(atom::launch_row_quantize(static_cast<const uint16_t*>(X), perm, M, K,
                                              static_cast<uint8_t*>(Xq), static_cast<uint16_t*>(sx), atom::kRowA8,
                                              static_cast<hipStream_t>(stream)));
}

int atom_pack_weights_w4a8(const void* W, const int32_t* perm, int32_t N, int32_t K, void* Wq, void* sw,
                           void* stream) {
  if (int s = check_row_quantize(W, perm, N, K, Wq, sw, false)) return s;
  return hip_status(atom::launch_row_quantize(static_cast<const uint16_t*>(W), perm, N, K,
                                              static_cast<uint8_t*>(Wq), static_cast<uint16_t*>(sw), atom::kRowW4A8,
                                              static_cast<hipStream_t>(stream)));
}

static int w4a8_common(const void* Xq, const void* sx, const void* Wq, const void* sw, int32_t M, int32_t N,
                       int32_t K, void* Y, int32_t* acc, void* workspace, int64_t workspace_bytes, void* stream) {
  const bool want_acc = acc != nullptr;
  if (!Xq || !Wq || (want_acc ? false : (!sx || !sw || !Y))) return ATOM_E_NULL;
  if (!valid_gemm(M, N, K)) return ATOM_E_SHAPE;
  if (!aligned16(Xq) || !aligned16(Wq)) return ATOM_E_ALIGN;
  if (!want_acc && (!aligned16(sx) || !aligned16(sw) || !aligned16(Y))) return ATOM_E_ALIGN;
  if (want_acc && !aligned16(acc)) return ATOM_E_ALIGN;
  const uint64_t G = (uint64_t)K / ATOM_GROUP;
  const uint64_t rbw = (uint64_t)atom_row_bytes(K);
  if (want_acc) {
    const Range in[2] = {range_of(Xq, (uint64_t)M * K), range_of(Wq, (uint64_t)N * rbw)};
    const Range out[1] = {range_of(acc, G * M * N * 4)};
    if (int s = check_overlap(in, 2, out, 1)) return s;
    return hip_status(atom::launch_gemm_w4a8(static_cast<const uint8_t*>(Xq), nullptr,
                                             static_cast<const uint8_t*>(Wq), nullptr, M, N, K, nullptr, acc,
                                             nullptr, atom::GemmPlan{0, 0, 1, 0}, static_cast<hipStream_t>(stream)));
  }
  atom::GemmPlan plan = atom::gemm_plan_tiled(M, N, K);
  int64_t need = atom::gemm_workspace_bytes(plan);
  if (need > 0 && (!workspace || workspace_bytes < need)) {   // too little scratch: unsplit
    plan = atom::GemmPlan{((M + 127) / 128) * ((N + 127) / 128), 0, 1, 0};
    need = 0;
  }
  const bool split = need > 0;
  if (split && !aligned16(workspace)) return ATOM_E_ALIGN;
  const Range in[4] = {range_of(Xq, (uint64_t)M * K), range_of(sx, G * M * 2), range_of(Wq, (uint64_t)N * rbw),
                       range_of(sw, G * N * 2)};
  const Range out[2] = {range_of(Y, (uint64_t)M * N * 2), range_of(workspace, split ? (uint64_t)need : 0)};
  if (int s = check_overlap(in, 4, out, split ? 2 : 1)) return s;
  return hip_status(atom::launch_gemm_w4a8(static_cast<const uint8_t*>(Xq), static_cast<const uint16_t*>(sx),
                                           static_cast<const uint8_t*>(Wq), static_cast<const uint16_t*>(sw), M, N,
                                           K, static_cast<uint16_t*>(Y), nullptr,
                                           split ? static_cast<float*>(workspace) : nullptr, plan,
                                           static_cast<hipStream_t>(stream)));
}

int atom_gemm_w4a8(const void* Xq, const void* sx, const void* Wq, const void* sw, int32_t M, int32_t N, int32_t K,
                   void* Y, void* stream) {
  return w4a8_common(Xq, sx, Wq, sw, M, N, K, Y, nullptr, nullptr, 0, stream);
}

int64_t atom_gemm_w4a8_workspace_bytes(int32_t M, int32_t N, int32_t K) {
  if (!valid_gemm(M, N, K)) return -(int64_t)ATOM_E_SHAPE;
  return atom::gemm_workspace_bytes(atom::gemm_plan_tiled(M, N, K));
}

int atom_gemm_w4a8_ws(const void* Xq, const void* sx, const void* Wq, const void* sw, int32_t M, int32_t N,
                      int32_t K, void* Y, void* workspace, int64_t workspace_bytes, void* stream) {
  return w4a8_common(Xq, sx, Wq, sw, M, N, K, Y, nullptr, workspace, workspace_bytes, stream);
}

int atom_gemm_w4a8_group_acc(const void* Xq, const void* Wq, int32_t M, int32_t N, int32_t K, int32_t* acc,
                             void* stream) {
  if (!acc) return ATOM_E_NULL;
  return w4a8_common(Xq, nullptr, Wq, nullptr, M, N, K, nullptr, acc, nullptr, 0, stream);
}

}  // extern "C"
