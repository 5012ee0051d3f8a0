// Ranking and cut of one row of block scores, shared by the selection kernel
// (scores read from global memory) and the fused scoring + selection kernel
// (scores produced in LDS).  See select.hip for the rules.
#pragma once

#include "common.h"

namespace xattn {

constexpr int kSelectThreads = 256;

enum CutRule : int { kThreshold = 0, kTopK = 1, kTopRatio = 2 };

struct CutSpec {
  int rule;     // CutRule
  int topk;     // kTopK: blocks kept
  float ratio;  // kTopRatio: share of the valid blocks kept
  float tau;    // kThreshold: this head's tau
};

template <int CAP>
struct SelectScratch {
  uint64_t keys[CAP];
  double part[kSelectThreads];
  uint32_t bits[CAP / 32];
  int off[CAP / 32];
  int cut;
};

// monotone map of float bits to unsigned (total order for finite values)
__device__ __forceinline__ uint32_t order_bits(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unorder_bits(uint32_t u) {
  return __builtin_bit_cast(float, (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

// Called by all kSelectThreads threads of a workgroup.  score_at(i) gives the
// score of key block i < n (the valid blocks); outputs one row of mask
// (nwords uint64), idx (NB int32, ascending then -1) and the count.
template <int CAP, class ScoreAt>
__device__ void rank_and_cut(SelectScratch<CAP>& sh, const ScoreAt& score_at, int n, int NB,
                             int nwords, const CutSpec& cut, uint64_t* mask_row, int32_t* idx_row,
                             int32_t* count_out) {
  const int tid = threadIdx.x;
  constexpr int kThreads = kSelectThreads;
  uint64_t* keys = sh.keys;
  double* part = sh.part;
  uint32_t* bits = sh.bits;
  int n2 = 1;
  while (n2 < n) n2 <<= 1;
  for (int i = tid; i < n2; i += kThreads)
    keys[i] = (i < n) ? (((uint64_t)order_bits(score_at(i)) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)i))
                      : 0ull;
  for (int i = tid; i < CAP / 32; i += kThreads) bits[i] = 0u;
  if (tid == 0) sh.cut = n;
  __syncthreads();

  // bitonic sort, descending
  for (int k = 2; k <= n2; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < n2 / 2; i += kThreads) {
        const int lo = ((i & ~(j - 1)) << 1) | (i & (j - 1));
        const int hi = lo | j;
        const uint64_t a = keys[lo], b = keys[hi];
        const bool desc = (lo & k) == 0;
        if (desc ? (a < b) : (a > b)) {
          keys[lo] = b;
          keys[hi] = a;
        }
      }
      __syncthreads();
    }
  }

  if (cut.rule != kThreshold) {   // fixed count: no prefix sums needed
    int k = cut.rule == kTopK ? cut.topk : (int)floor((double)cut.ratio * (double)n + 0.5);
    k = k < 1 ? 1 : (k > n ? n : k);
    if (tid == 0) sh.cut = k;
  }
  // prefix sums in float64 over the ranked scores: a contiguous chunk per thread
  const float tau = cut.rule == kThreshold ? cut.tau : 1.0f;
  const int per = (n + kThreads - 1) / kThreads;
  const int b0 = tid * per, b1 = min(n, b0 + per);
  double local = 0.0;
  for (int i = b0; i < b1; ++i) local += (double)unorder_bits((uint32_t)(keys[i] >> 32));
  part[tid] = local;
  __syncthreads();
  // inclusive scan of the per-thread sums (Hillis-Steele)
  for (int o = 1; o < kThreads; o <<= 1) {
    const double v = (tid >= o) ? part[tid - o] : 0.0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  if (tau < 1.0f) {
    double run = (tid > 0) ? part[tid - 1] : 0.0;
    for (int i = b0; i < b1; ++i) {
      run += (double)unorder_bits((uint32_t)(keys[i] >> 32));
      if (run >= (double)tau) {
        atomicMin(&sh.cut, i + 1);
        break;
      }
    }
  }
  __syncthreads();
  const int kstar = sh.cut;

  for (int i = tid; i < kstar; i += kThreads) {
    const uint32_t kb = 0xFFFFFFFFu - (uint32_t)(keys[i] & 0xFFFFFFFFull);
    atomicOr(&bits[kb >> 5], 1u << (kb & 31));
  }
  __syncthreads();

  const int nw32 = (NB + 31) / 32;
  for (int w = tid; w < nwords; w += kThreads) {
    const uint64_t lo = bits[2 * w];
    const uint64_t hi = (2 * w + 1 < nw32) ? bits[2 * w + 1] : 0u;
    mask_row[w] = lo | (hi << 32);
  }
  if (tid == 0) {
    int acc = 0;
    for (int w = 0; w < nw32; ++w) {
      sh.off[w] = acc;
      acc += __builtin_popcount(bits[w]);
    }
  }
  __syncthreads();
  for (int w = tid; w < nw32; w += kThreads) {
    uint32_t b = bits[w];
    int o = sh.off[w];
    while (b) {
      const int bit = __builtin_ctz(b);
      idx_row[o++] = 32 * w + bit;
      b &= b - 1;
    }
  }
  for (int i = kstar + tid; i < NB; i += kThreads) idx_row[i] = -1;
  if (tid == 0) *count_out = kstar;
}

}  // namespace xattn
