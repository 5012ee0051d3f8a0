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

namespace xattn {
namespace {

constexpr int kThreads = 256;

enum CutRule : int { kThreshold = 0, kTopK = 1, kTopRatio = 2 };

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

// monotone map of float bits to unsigned (total order for finite values)
__device__ __forceinline__ uint32_t order_bits(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unorder_bits(uint32_t u) {
  return __builtin_bit_cast(float, (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

template <int CAP>
__global__ __launch_bounds__(kThreads) void select_kernel(SelectParams p) {
  __shared__ uint64_t keys[CAP];
  __shared__ double part[kThreads];
  __shared__ uint32_t bits[CAP / 32];
  __shared__ int s_cut;
  __shared__ int s_off[CAP / 32];

  const int row = blockIdx.x;
  const int h = row / p.NB;
  const int qb = row % p.NB;
  const int tid = threadIdx.x;
  const int n = p.causal ? qb + 1 : p.NB;
  int n2 = 1;
  while (n2 < n) n2 <<= 1;
  const float* srow = p.scores + (size_t)row * p.NB;

  for (int i = tid; i < n2; i += kThreads)
    keys[i] = (i < n) ? (((uint64_t)order_bits(srow[i]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)i))
                      : 0ull;
  for (int i = tid; i < CAP / 32; i += kThreads) bits[i] = 0u;
  if (tid == 0) s_cut = n;
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

  if (p.rule != kThreshold) {   // fixed count: no prefix sums needed
    int k = p.rule == kTopK ? p.topk : (int)floor((double)p.ratio * (double)n + 0.5);
    k = k < 1 ? 1 : (k > n ? n : k);
    if (tid == 0) s_cut = k;
  }
  // prefix sums in float64 over the ranked scores: a contiguous chunk per thread
  const float tau = p.rule == kThreshold ? p.tau.v[h] : 1.0f;
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
        atomicMin(&s_cut, i + 1);
        break;
      }
    }
  }
  __syncthreads();
  const int kstar = s_cut;

  for (int i = tid; i < kstar; i += kThreads) {
    const uint32_t kb = 0xFFFFFFFFu - (uint32_t)(keys[i] & 0xFFFFFFFFull);
    atomicOr(&bits[kb >> 5], 1u << (kb & 31));
  }
  __syncthreads();

  const int nw32 = (p.NB + 31) / 32;
  for (int w = tid; w < p.nwords; w += kThreads) {
    const uint64_t lo = bits[2 * w];
    const uint64_t hi = (2 * w + 1 < nw32) ? bits[2 * w + 1] : 0u;
    p.mask[(size_t)row * p.nwords + w] = lo | (hi << 32);
  }
  if (tid == 0) {
    int acc = 0;
    for (int w = 0; w < nw32; ++w) {
      s_off[w] = acc;
      acc += __builtin_popcount(bits[w]);
    }
  }
  __syncthreads();
  int32_t* irow = p.idx + (size_t)row * p.NB;
  for (int w = tid; w < nw32; w += kThreads) {
    uint32_t b = bits[w];
    int o = s_off[w];
    while (b) {
      const int bit = __builtin_ctz(b);
      irow[o++] = 32 * w + bit;
      b &= b - 1;
    }
  }
  for (int i = kstar + tid; i < p.NB; i += kThreads) irow[i] = -1;
  if (tid == 0) p.counts[row] = kstar;
}

template <int CAP>
hipError_t launch_cap(const SelectParams& sp, int rows, hipStream_t st) {
  hipLaunchKernelGGL((select_kernel<CAP>), dim3(rows), dim3(kThreads), 0, st, sp);
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
