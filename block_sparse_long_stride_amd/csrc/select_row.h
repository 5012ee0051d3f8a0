// Ranking and cut of one row of block scores by one wavefront, shared by the
// selection kernel (scores read from global memory) and the fused scoring +
// selection kernel (scores produced in LDS).  See select.hip for the rules.
//
// The kept set is a prefix of the valid blocks ranked by score (descending,
// the lower block first on equal scores), so it is fixed by a threshold value
// v and a tie count m: every block scoring above v, plus the m lowest blocks
// scoring exactly v.  The row is never sorted.  The wave holds element
// i = j * 64 + lane of the row in register j and finds v bit by bit over
// the order-preserving 32-bit score keys (31 or 32 passes):
//   - Top-K / Top-Ratio: v is the k-th largest score; each pass counts the
//     keys at or above a candidate with ballots.
//   - threshold tau: only non-negative scores raise a running sum, so the cut
//     lies among them; v is the largest score whose "at or above" sum (in
//     float64) still reaches tau, and m the ties at v taken one by one until
//     the sum reaches tau.  If the non-negative scores sum to less than tau
//     every valid block is kept.
// Each float64 sum is accumulated per lane in register order, then reduced by
// a fixed DPP butterfly, so every lane and every call sees the same bits.
#pragma once

#include "common.h"

namespace xattn {

constexpr int kSelectThreads = 256;
constexpr int kSelectRowsPerBlock = kSelectThreads / 64;   // one row per wave

enum CutRule : int { kThreshold = 0, kTopK = 1, kTopRatio = 2 };

struct CutSpec {
  int rule;     // CutRule
  int topk;     // kTopK: blocks kept
  float ratio;  // kTopRatio: share of the valid blocks kept
  float tau;    // kThreshold: this head's tau
};

// -0.0 ranks as +0.0 (equal scores)
__device__ __forceinline__ float canonical_zero(float f) {
  return __builtin_bit_cast(uint32_t, f) == 0x80000000u ? 0.0f : f;
}

// monotone map of float bits to unsigned (total order for finite values);
// non-negative floats map to keys >= 0x80000000
__device__ __forceinline__ uint32_t order_bits(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unorder_bits(uint32_t u) {
  return __builtin_bit_cast(float, (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

// The value of x in the lane that the DPP control CTRL pairs with this one
// (every lane written).
template <int CTRL>
__device__ __forceinline__ double dpp_pair(double x) {
  const u32x2_t v = __builtin_bit_cast(u32x2_t, x);
  u32x2_t w;
  w[0] = (uint32_t)__builtin_amdgcn_mov_dpp((int)v[0], CTRL, 0xF, 0xF, false);
  w[1] = (uint32_t)__builtin_amdgcn_mov_dpp((int)v[1], CTRL, 0xF, 0xF, false);
  return __builtin_bit_cast(double, w);
}
// row_bcast (CTRL 0x142: lane 15 of each row into the next row; 0x143: lane 31
// into rows 2 and 3) into the rows of ROWS; 0 in the other rows.
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_bcast(double x) {
  const u32x2_t v = __builtin_bit_cast(u32x2_t, x);
  u32x2_t w;
  w[0] = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v[0], CTRL, ROWS, 0xF, false);
  w[1] = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v[1], CTRL, ROWS, 0xF, false);
  return __builtin_bit_cast(double, w);
}
__device__ __forceinline__ double lane63(double x) {
  const u32x2_t v = __builtin_bit_cast(u32x2_t, x);
  u32x2_t w;
  w[0] = (uint32_t)__builtin_amdgcn_readlane((int)v[0], 63);
  w[1] = (uint32_t)__builtin_amdgcn_readlane((int)v[1], 63);
  return __builtin_bit_cast(double, w);
}

// Sum over the 64 lanes in a fixed order (the same bits on every call): pairs
// l^1, then l^2 within quads, the two quads of each 8 lanes, the two halves of
// each row of 16 (each add's operands are the same in both lanes of a pair,
// and addition commutes), then (r3 + r2) + (r1 + r0) over the row sums.
__device__ __forceinline__ double wave_sum(double x) {
  x += dpp_pair<0xB1>(x);    // quad_perm [1,0,3,2]
  x += dpp_pair<0x4E>(x);    // quad_perm [2,3,0,1]
  x += dpp_pair<0x141>(x);   // row_half_mirror
  x += dpp_pair<0x140>(x);   // row_mirror
  x += dpp_bcast<0x142, 0xA>(x);   // rows 1, 3: r1 + r0, r3 + r2
  x += dpp_bcast<0x143, 0x8>(x);   // row 3: (r3 + r2) + (r1 + r0)
  return lane63(x);
}

// Minimum over the 64 lanes (exact, so the order does not matter).
__device__ __forceinline__ double wave_min(double x) {
  x = __builtin_fmin(x, dpp_pair<0xB1>(x));
  x = __builtin_fmin(x, dpp_pair<0x4E>(x));
  x = __builtin_fmin(x, dpp_pair<0x141>(x));
  x = __builtin_fmin(x, dpp_pair<0x140>(x));
  const u32x2_t v = __builtin_bit_cast(u32x2_t, x);
  double r[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    u32x2_t w;
    w[0] = (uint32_t)__builtin_amdgcn_readlane((int)v[0], 16 * q);
    w[1] = (uint32_t)__builtin_amdgcn_readlane((int)v[1], 16 * q);
    r[q] = __builtin_bit_cast(double, w);
  }
  return __builtin_fmin(__builtin_fmin(r[0], r[1]), __builtin_fmin(r[2], r[3]));
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
  x = min(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false));
  x = min(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false));
  x = min(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x141, 0xF, 0xF, false));
  x = min(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x140, 0xF, 0xF, false));
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)x, 0);
  const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)x, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)x, 32);
  const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)x, 48);
  return min(min(a, b), min(c, d));
}

__device__ __forceinline__ int wave_count(bool b) { return __popcll(__ballot(b)); }

// Writes one row: mask words (nwords), ascending block ids then -1 (NB), count.
// above(j) / tie(j): element j * 64 + lane is above the threshold / equal to
// it; the m lowest tied elements are kept after every element above.  Only
// registers j < JL can hold a valid block.
template <int JL, class Above, class Tie>
__device__ __forceinline__ void emit_row(const Above& above, const Tie& tie, int m, int NB,
                                         int nwords, uint64_t* mask_row, int32_t* idx_row,
                                         int32_t* count_out) {
  const int lane = threadIdx.x & 63;
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  uint64_t word = 0ull;   // mask word `lane`
  int base = 0, ties_seen = 0;
#pragma unroll
  for (int j = 0; j < JL; ++j) {
    const bool eq = tie(j);
    const uint64_t eqm = __ballot(eq);
    const bool sel = above(j) || (eq && ties_seen + __popcll(eqm & below) < m);
    ties_seen += __popcll(eqm);
    const uint64_t selm = __ballot(sel);
    if (sel) idx_row[base + __popcll(selm & below)] = j * 64 + lane;
    base += __popcll(selm);
    if (lane == j) word = selm;
  }
  if (lane < nwords) mask_row[lane] = word;
  for (int i = base + lane; i < NB; i += 64) idx_row[i] = -1;
  if (lane == 0) *count_out = base;
}

// rank_and_cut for a row whose valid blocks all sit in registers j < JL.
template <int JL, class ScoreAt>
__device__ __forceinline__ void rank_and_cut_live(const ScoreAt& score_at, int n, int NB,
                                                  int nwords, const CutSpec& cut,
                                                  uint64_t* mask_row, int32_t* idx_row,
                                                  int32_t* count_out) {
  const int lane = threadIdx.x & 63;
  auto valid = [&](int j) { return j * 64 + lane < n; };

  if (cut.rule == kThreshold && cut.tau < 1.0f) {
    const double tau = (double)cut.tau;
    double d[JL];   // scores; -1 past n (below every candidate, which is >= +0)
#pragma unroll
    for (int j = 0; j < JL; ++j)
      d[j] = valid(j) ? (double)canonical_zero(score_at(j * 64 + lane)) : -1.0;
    // sum and count of the scores >= cv, for a candidate cv >= +0 (a select,
    // not a multiply by 0/1: an infinite score times 0 would be NaN)
    auto sum_ge = [&](double cv, int& cnt) -> double {
      double s = 0.0;
      int c = 0;
#pragma unroll
      for (int j = 0; j < JL; ++j) {
        const bool ge = d[j] >= cv;
        s += ge ? d[j] : 0.0;
        c += wave_count(ge);
      }
      cnt = c;
      return wave_sum(s);
    };
    bool keep_all = true;
    double v = 0.0;
    int m = 0;
    int c_lo;   // scores >= the lower end of the search interval
    if (sum_ge(0.0, c_lo) >= tau) {
      keep_all = false;
      // Search interval [t, t_hi] of keys, t_hi + 1 the last candidate that
      // failed (none yet: no bound); c_hi = scores at or above that bound.
      // Once one score is left in the interval it is the answer.
      uint32_t t = 0x80000000u;   // key of +0.0
      int c_hi = 0;
#pragma unroll 1
      for (int b = 30; b >= 0 && c_lo - c_hi > 1; --b) {
        const uint32_t c = t | (1u << b);
        int cnt;
        if (sum_ge((double)unorder_bits(c), cnt) >= tau) {
          t = c;
          c_lo = cnt;
        } else {
          c_hi = cnt;
        }
      }
      // v = the smallest score >= t: the one left in the interval, or t
      // itself after every bit
      const double lo = (double)unorder_bits(t);
      double mn = __builtin_inf();
#pragma unroll
      for (int j = 0; j < JL; ++j) mn = __builtin_fmin(mn, d[j] >= lo ? d[j] : __builtin_inf());
      v = wave_min(mn);
      // the blocks above v, then the blocks at v in ascending order until the
      // running sum reaches tau
      double run = 0.0;
      int ties = 0;
      {
        double sg = 0.0;
#pragma unroll
        for (int j = 0; j < JL; ++j) {
          sg += d[j] > v ? d[j] : 0.0;
          ties += wave_count(d[j] == v);
        }
        run = wave_sum(sg);
      }
      while (m < ties) {
        run += v;
        ++m;
        if (run >= tau) break;
      }
    }
    emit_row<JL>([&](int j) { return valid(j) && (keep_all || d[j] > v); },
                 [&](int j) { return !keep_all && d[j] == v; }, m, NB, nwords, mask_row, idx_row,
                 count_out);
  } else {
    // a fixed number k of blocks (tau >= 1 keeps every valid block)
    int k = n;
    if (cut.rule == kTopK) k = cut.topk;
    else if (cut.rule == kTopRatio) k = (int)floor((double)cut.ratio * (double)n + 0.5);
    k = k < 1 ? 1 : (k > n ? n : k);
    uint32_t key[JL];   // 0 past n (below every candidate, which is >= 1)
#pragma unroll
    for (int j = 0; j < JL; ++j)
      key[j] = valid(j) ? order_bits(canonical_zero(score_at(j * 64 + lane))) : 0u;
    auto count_ge = [&](uint32_t c) -> int {
      int s = 0;
#pragma unroll
      for (int j = 0; j < JL; ++j) s += wave_count(key[j] >= c);
      return s;
    };
    // t = the k-th largest key: the largest t with at least k keys >= t.
    // Search interval [t, t_hi] as in the threshold rule; counts of valid
    // keys >= t (c_lo) and >= t_hi + 1 (c_hi).
    uint32_t t = 0;
    int c_lo = n, c_hi = 0;
#pragma unroll 1
    for (int b = 31; b >= 0 && c_lo - c_hi > 1; --b) {
      const uint32_t c = t | (1u << b);
      const int cnt = count_ge(c);
      if (cnt >= k) {
        t = c;
        c_lo = cnt;
      } else {
        c_hi = cnt;
      }
    }
    // the smallest valid key >= t
    uint32_t mn = 0xFFFFFFFFu;
#pragma unroll
    for (int j = 0; j < JL; ++j) mn = min(mn, (valid(j) && key[j] >= t) ? key[j] : 0xFFFFFFFFu);
    t = wave_min_u32(mn);
    int above = 0;
#pragma unroll
    for (int j = 0; j < JL; ++j) above += wave_count(key[j] > t);
    const int m = k - above;
    emit_row<JL>([&](int j) { return key[j] > t; }, [&](int j) { return key[j] == t && valid(j); },
                 m, NB, nwords, mask_row, idx_row, count_out);
  }
}

// The smallest register count JL (a multiple of G) that holds the row's n
// valid blocks.
template <int EPL, int G, int JL, class ScoreAt>
__device__ __forceinline__ void cut_dispatch(int jn, const ScoreAt& score_at, int n, int NB,
                                             int nwords, const CutSpec& cut, uint64_t* mask_row,
                                             int32_t* idx_row, int32_t* count_out) {
  if constexpr (JL >= EPL) {
    rank_and_cut_live<EPL>(score_at, n, NB, nwords, cut, mask_row, idx_row, count_out);
  } else {
    if (jn <= JL)
      rank_and_cut_live<JL>(score_at, n, NB, nwords, cut, mask_row, idx_row, count_out);
    else
      cut_dispatch<EPL, G, JL + G>(jn, score_at, n, NB, nwords, cut, mask_row, idx_row, count_out);
  }
}

// Called by one whole wavefront.  1 <= n <= NB <= 64 * EPL, EPL <= 64;
// score_at(i) gives the score of key block i < n (the valid blocks); outputs
// one row of mask (nwords uint64), idx (NB int32, ascending then -1) and the
// count.  The work scales with the registers that hold valid blocks.
template <int EPL, class ScoreAt>
__device__ __forceinline__ void rank_and_cut(const ScoreAt& score_at, int n, int NB, int nwords,
                                             const CutSpec& cut, uint64_t* mask_row,
                                             int32_t* idx_row, int32_t* count_out) {
  static_assert(EPL >= 1 && EPL <= 64, "one mask word per lane");
  constexpr int G = EPL >= 8 ? EPL / 8 : 1;
  const int jn = (n + 63) >> 6;
  cut_dispatch<EPL, G, G>(jn, score_at, n, NB, nwords, cut, mask_row, idx_row, count_out);
}

}  // namespace xattn
