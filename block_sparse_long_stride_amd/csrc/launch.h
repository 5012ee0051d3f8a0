// Host-side launchers of the libxattn kernels.  Arguments are validated by
// the C-ABI layer (xattn_api.cpp) before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace xattn {

struct Shape {
  int hq, hkv, L, d, causal;
  bool bf16;
};

// Compute units per XCD of the current device (cached per device).
int cus_per_xcd();

// ---- block scores ---------------------------------------------------------
// Workspace of the bf16 scoring path: per (head, 32-row group of reshaped rows)
//   P: [NB][32] fp32 partial block sums (each against its own snapshot max)
//   M: [nct][32] fp32 snapshot max (log2 units) per 64-column range
//   Z: [nct][32] fp32 snapshot sum of exp2 against that max
// Sampling pattern of the scoring product: key sub-row paired with query
// sub-row a inside each SxS tile.  custom == 0 is the antidiagonal, S-1-a;
// otherwise v[0 .. S) is a permutation of 0 .. S-1 (S <= kMaxPhase).
constexpr int kMaxPhase = 64;
struct PhaseMap {
  int32_t custom;
  int32_t v[kMaxPhase];
};
size_t score_workspace_bytes(const Shape& s, int S, int B);
// Fixed scratch of the allocation-free scoring entry point (a static device
// array in score_bf16.hip): its size, and this device's address of it
// (looked up once per device with hipGetSymbolAddress).
constexpr size_t kScoreScratchBytes = (size_t)64 << 20;
hipError_t score_scratch_ptr(void** out);
hipError_t launch_score_bf16(const Shape& s, const void* Q, const void* K, int S, int B,
                             const PhaseMap& phase, float* scores, void* ws, hipStream_t st);
hipError_t launch_score_fp32(const Shape& s, const void* Q, const void* K, int S, int B,
                             const PhaseMap& phase, float* scores, hipStream_t st);

// ---- selection --------------------------------------------------------------
constexpr int kMaxHeads = 128;
constexpr int kMaxSelectBlocks = 4096;
struct TauArray {
  float v[kMaxHeads];
};
hipError_t launch_select(int hq, int NB, int causal, const float* scores, const TauArray& tau,
                         uint64_t* mask, int32_t* idx, int32_t* counts, hipStream_t st);
// Scoring GEMM, then finishing and threshold selection fused in one kernel
// (no score matrix in memory); antidiagonal pattern, bf16 inputs.  ws as for
// launch_score_bf16.
hipError_t launch_score_select_bf16(const Shape& s, const void* Q, const void* K, int S, int B,
                                    const TauArray& tau, uint64_t* mask, int32_t* idx,
                                    int32_t* counts, void* ws, hipStream_t st);
// Fixed-count cut rules on the same ranking: Top-K (k blocks) and Top-Ratio
// (the nearest integer to ratio * valid blocks), both clamped to [1, valid].
hipError_t launch_select_topk(int hq, int NB, int causal, const float* scores, int k_blocks,
                              uint64_t* mask, int32_t* idx, int32_t* counts, hipStream_t st);
hipError_t launch_select_topratio(int hq, int NB, int causal, const float* scores, float ratio,
                                  uint64_t* mask, int32_t* idx, int32_t* counts, hipStream_t st);

// ---- threshold calibration -----------------------------------------------------
// err[h] = sum (O_sparse - O_dense)^2 / sum O_dense^2 over head h's per_head
// elements (bf16 or fp32), accumulated in float64 in a fixed order.
hipError_t launch_head_error(int hq, size_t per_head, bool bf16, const void* O_sparse,
                             const void* O_dense, double* err, hipStream_t st);
// Host DP: distributes exactly `steps` reduction steps over H heads with
// err[h*(R+1) + k] the error of head h after k steps; writes levels[H] and
// returns minus the summed error of the chosen levels.
double tau_dp(int H, int R, const double* err, int steps, int* levels);

// ---- attention ---------------------------------------------------------------
// idx == nullptr selects dense mode (every key block, causal-limited).
// LDS bytes one bf16 attention work-group needs (d in {64, 128}, B in {64, 128}).
size_t flash_bf16_lds_bytes(int d, int B, int NB, bool sparse);
constexpr size_t kLdsBytesPerCu = 160 * 1024;   // gfx950

hipError_t launch_flash_bf16(const Shape& s, const void* Q, const void* K, const void* V,
                             int B, const int32_t* idx, const int32_t* counts, void* O,
                             hipStream_t st);
// LDS bytes one fp32 attention work-group needs (key/value tiles, and the
// block bitmap in sparse mode).
size_t flash_fp32_lds_bytes(int d, int NB, bool sparse);
hipError_t launch_flash_fp32(const Shape& s, const void* Q, const void* K, const void* V,
                             int B, const int32_t* idx, const int32_t* counts, void* O,
                             hipStream_t st);

}  // namespace xattn
