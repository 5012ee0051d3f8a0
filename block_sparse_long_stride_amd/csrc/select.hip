// Threshold block selection: find_blocks(A, tau) ("XAttention: Block Sparse
// Attention with Antidiagonal Scoring", papercache.org summary, section 2.2;
// chapterpal.com Knowl 2).  One workgroup per (head, query block).
//
// The smallest set of key blocks whose score sum reaches tau is a prefix of
// the blocks ranked by score.  The kernel ranks the valid blocks with an LDS
// bitonic sort of 64-bit keys (order-preserving score bits, then the inverted
// block id, so equal scores keep the lower block first), forms the prefix sums
// of the ranked scores in float64, cuts at the first prefix >= tau, and emits
// the bitmask, the ascending block ids (padded with -1) and the count.
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
  int NB, causal, nwords;
  int rule;        // CutRule
  int topk;        // kTopK: blocks kept
  float ratio;     // kTopRatio: share of the valid blocks kept
  TauArray tau;    // kThreshold: per-head tau
};

template <int CAP>
__global__ __launch_bounds__(kSelectThreads) void select_kernel(SelectParams p) {
  __shared__ SelectScratch<CAP> sh;
  const int row = blockIdx.x;
  const int h = row / p.NB;
  const int qb = row % p.NB;
  const int n = p.causal ? qb + 1 : p.NB;
  const float* srow = p.scores + (size_t)row * p.NB;
  const CutSpec cut{p.rule, p.topk, p.ratio, p.rule == kThreshold ? p.tau.v[h] : 1.0f};
  rank_and_cut<CAP>(sh, [&](int i) { return srow[i]; }, n, p.NB, p.nwords, cut,
                    p.mask + (size_t)row * p.nwords, p.idx + (size_t)row * p.NB, p.counts + row);
}

template <int CAP>
hipError_t launch_cap(const SelectParams& sp, int rows, hipStream_t st) {
  hipLaunchKernelGGL((select_kernel<CAP>), dim3(rows), dim3(kSelectThreads), 0, st, sp);
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
  if (sp.NB <= 256) return launch_cap<256>(sp, rows, st);
  if (sp.NB <= 1024) return launch_cap<1024>(sp, rows, st);
  return launch_cap<4096>(sp, rows, st);
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
