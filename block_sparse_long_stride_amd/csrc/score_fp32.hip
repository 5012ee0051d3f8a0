// Block scores of XAttention (papercache.org summary, section 2.2,
// Algorithm 1) for fp32 inputs: a plain SIMT kernel for small fp32 problems,
// kept in fp32 end to end.  One workgroup per (head, query block).
//
// For each of the B/S reshaped rows R of the query block, pass 1 finds the
// softmax max and denominator over the valid columns (c <= R when causal) of
// z = sum_a <Q[R*S+a], K[c*S+S-1-a]> * log2(e)/sqrt(d*S); pass 2 recomputes
// z per key block and sums exp2(z - m)/Z over the (B/S)x(B/S) tile, divided by
// B/S.
#include "common.h"
#include "launch.h"

namespace xattn {
namespace {

constexpr int kThreads = 256;

struct Fp32ScoreParams {
  const float* Q;
  const float* K;
  float* scores;
  int L, d, S, bs, NB, Lr, group, causal;
  float scale_log2;
  PhaseMap phase;   // key sub-row per query sub-row (default: antidiagonal)
};

__device__ float reshaped_dot(const float* Qh, const float* Kg, int R, int c, int S, int d,
                             const PhaseMap& ph) {
  float acc = 0.f;
  for (int a = 0; a < S; ++a) {
    const float* q = Qh + (size_t)(R * S + a) * d;
    const float* k = Kg + (size_t)(c * S + (ph.custom ? ph.v[a] : S - 1 - a)) * d;
    for (int e = 0; e < d; ++e) acc = fmaf(q[e], k[e], acc);
  }
  return acc;
}

__global__ __launch_bounds__(kThreads) void score_fp32_kernel(Fp32ScoreParams p) {
  __shared__ float s_m[kThreads];
  __shared__ float s_z[kThreads];
  __shared__ float row_m[256];
  __shared__ float row_invz[256];
  const int qb = blockIdx.x % p.NB;
  const int h = blockIdx.x / p.NB;
  const int g = h / p.group;
  const float* Qh = p.Q + (size_t)h * p.L * p.d;
  const float* Kg = p.K + (size_t)g * p.L * p.d;
  const int tid = threadIdx.x;
  const int ncols = p.causal ? (qb + 1) * p.bs : p.Lr;

  // pass 1: per-row max and denominator (online, then a tree over threads)
  for (int r = 0; r < p.bs; ++r) {
    const int R = qb * p.bs + r;
    const int lim = p.causal ? R + 1 : p.Lr;
    float m = -INFINITY, z = 0.f;
    for (int c = tid; c < lim; c += kThreads) {
      const float x = reshaped_dot(Qh, Kg, R, c, p.S, p.d, p.phase) * p.scale_log2;
      if (x > m) {
        z = z * fast_exp2(m - x) + 1.f;
        m = x;
      } else {
        z += fast_exp2(x - m);
      }
    }
    s_m[tid] = m;
    s_z[tid] = z;
    __syncthreads();
    for (int o = kThreads / 2; o > 0; o >>= 1) {
      if (tid < o) {
        const float m1 = s_m[tid], m2 = s_m[tid + o];
        const float mm = fmaxf(m1, m2);
        float zz = 0.f;
        if (m1 != -INFINITY) zz += s_z[tid] * fast_exp2(m1 - mm);
        if (m2 != -INFINITY) zz += s_z[tid + o] * fast_exp2(m2 - mm);
        s_m[tid] = mm;
        s_z[tid] = zz;
      }
      __syncthreads();
    }
    if (tid == 0) {
      row_m[r] = s_m[0];
      row_invz[r] = 1.f / s_z[0];
    }
    __syncthreads();
  }

  // pass 2: tile sums, one key block per thread
  float* out = p.scores + ((size_t)h * p.NB + qb) * p.NB;
  for (int kb = tid; kb < p.NB; kb += kThreads) {
    float acc = 0.f;
    if (!p.causal || kb <= qb) {
      for (int r = 0; r < p.bs; ++r) {
        const int R = qb * p.bs + r;
        for (int c = kb * p.bs; c < (kb + 1) * p.bs && c < ncols; ++c) {
          if (p.causal && c > R) continue;
          const float x = reshaped_dot(Qh, Kg, R, c, p.S, p.d, p.phase) * p.scale_log2;
          acc += fast_exp2(x - row_m[r]) * row_invz[r];
        }
      }
      acc /= (float)p.bs;
    }
    out[kb] = acc;
  }
}

}  // namespace

hipError_t launch_score_fp32(const Shape& s, const void* Q, const void* K, int S, int B,
                             const PhaseMap& phase, float* scores, hipStream_t st) {
  Fp32ScoreParams p;
  p.Q = (const float*)Q;
  p.K = (const float*)K;
  p.scores = scores;
  p.L = s.L;
  p.d = s.d;
  p.S = S;
  p.bs = B / S;
  p.NB = s.L / B;
  p.Lr = s.L / S;
  p.group = s.hq / s.hkv;
  p.causal = s.causal;
  p.scale_log2 = (float)(1.4426950408889634 / __builtin_sqrt((double)s.d * S));
  p.phase = phase;
  hipLaunchKernelGGL(score_fp32_kernel, dim3(s.hq * p.NB), dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace xattn
