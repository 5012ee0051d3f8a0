// Threshold block selection: find_blocks(A, tau) ("XAttention: Block Sparse
// Attention with Antidiagonal Scoring", papercache.org summary, section 2.2;
// chapterpal.com Knowl 2).  One wavefront per (head, query block), four rows
// per workgroup.
//
// The smallest set of key blocks whose score sum reaches tau is a prefix of
// the blocks ranked by score (descending; equal scores keep the lower block
// first), and the first prefix whose float64 sum is >= tau ends it.  The
// wave finds where that prefix ends without sorting the row (a bitwise
// search over the score keys, select_row.h) and emits the bitmask, the
// ascending block ids (padded with -1) and the count.
//
// The same kernel serves the two fixed-count cut rules of the ablation on
// block selection strategies (chapterpal.com Knowl 9, "Selection Strategy";
// papercache.org summary, ablation "block selection strategy"): Top-K keeps
// the k highest-ranked blocks, Top-Ratio the nearest integer to ratio times
// the number of valid blocks (halves up); both keep at least one and at most
// every valid block.
#include "common.h"
#include "launch.h"
#include "select_row.h"

namespace xattn {
namespace {

struct SelectParams {
  const float* scores;
  uint64_t* mask;
  int32_t* idx;
  int32_t* counts;
  int NB, causal, nwords, rows;
  int rule;        // CutRule
  int topk;        // kTopK: blocks kept
  float ratio;     // kTopRatio: share of the valid blocks kept
  TauArray tau;    // kThreshold: per-head tau
};

template <int EPL>
__global__ __launch_bounds__(kSelectThreads) void select_kernel(SelectParams p) {
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int row = blockIdx.x * kSelectRowsPerBlock + wave;
  if (row >= p.rows) return;
  const int h = row / p.NB;
  const int qb = row % p.NB;
  const int n = p.causal ? qb + 1 : p.NB;
  const float* srow = p.scores + (size_t)row * p.NB;
  const CutSpec cut{p.rule, p.topk, p.ratio, p.rule == kThreshold ? p.tau.v[h] : 1.0f};
  rank_and_cut<EPL>([&](int i) { return srow[i]; }, n, p.NB, p.nwords, cut,
                    p.mask + (size_t)row * p.nwords, p.idx + (size_t)row * p.NB, p.counts + row);
}

template <int EPL>
hipError_t launch_epl(SelectParams sp, int rows, hipStream_t st) {
  sp.rows = rows;
  const int blocks = (rows + kSelectRowsPerBlock - 1) / kSelectRowsPerBlock;
  hipLaunchKernelGGL((select_kernel<EPL>), dim3(blocks), dim3(kSelectThreads), 0, st, sp);
  return hipGetLastError();
}

SelectParams make_params(int NB, int causal, const float* scores, uint64_t* mask, int32_t* idx,
                         int32_t* counts) {
  SelectParams sp{};
  sp.scores = scores;
  sp.mask = mask;
  sp.idx = idx;
  sp.counts = counts;
  sp.NB = NB;
  sp.causal = causal;
  sp.nwords = (NB + 63) / 64;
  return sp;
}

hipError_t launch_rows(const SelectParams& sp, int rows, hipStream_t st) {
  // registers per lane: NB <= 64 * EPL (NB <= kMaxSelectBlocks = 4096)
  if (rows == 0) return hipSuccess;
  if (sp.NB <= 256) return launch_epl<4>(sp, rows, st);
  if (sp.NB <= 1024) return launch_epl<16>(sp, rows, st);
  return launch_epl<64>(sp, rows, st);
}

}  // namespace

hipError_t launch_select(int hq, int NB, int causal, const float* scores, const TauArray& tau,
                         uint64_t* mask, int32_t* idx, int32_t* counts, hipStream_t st) {
  SelectParams sp = make_params(NB, causal, scores, mask, idx, counts);
  sp.rule = kThreshold;
  sp.tau = tau;
  return launch_rows(sp, hq * NB, st);
}

hipError_t launch_select_topk(int hq, int NB, int causal, const float* scores, int k_blocks,
                              uint64_t* mask, int32_t* idx, int32_t* counts, hipStream_t st) {
  SelectParams sp = make_params(NB, causal, scores, mask, idx, counts);
  sp.rule = kTopK;
  sp.topk = k_blocks;
  return launch_rows(sp, hq * NB, st);
}

hipError_t launch_select_topratio(int hq, int NB, int causal, const float* scores, float ratio,
                                  uint64_t* mask, int32_t* idx, int32_t* counts, hipStream_t st) {
  SelectParams sp = make_params(NB, causal, scores, mask, idx, counts);
  sp.rule = kTopRatio;
  sp.ratio = ratio;
  return launch_rows(sp, hq * NB, st);
}

}  // namespace xattn
