// Block scores of XAttention (papercache.org summary, section 2.2,
// Algorithm 1) for fp32 inputs, kept in fp32 end to end.  When B/S divides 32
// the reshaped products run on the matrix cores (score_fp32_mfma_kernel);
// otherwise a SIMT kernel, one workgroup per (head, query block):
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

// Matrix-core version for B/S dividing 32: one workgroup of four waves per 32
// reshaped rows of one head, its waves taking the 32-column tiles in turn.  A
// tile T[c][R] = sum_f K_r[c][f] Q_r[R][f] (f over the S*d features of the
// reshaped rows; K_r takes key sub-row S-1-a, or the pattern's, for feature
// chunk a) is built from 32x32x2 fp32 MFMAs, step t pairing features 2t and
// 2t+1 (a feature past S*d reads 0), with the operands read from memory; each
// lane then holds row R0 + l32 and the columns 8(v/4) + 4 hi + v%4 of
// register v.  Pass 1 reduces every row's max and denominator over its lanes,
// the two lane halves and the four waves; pass 2 recomputes the tiles.  As
// B/S divides 32, every (query block, key block) square of (B/S)^2 entries
// lies inside one tile, so its sum takes lane shuffles only.
constexpr int kMfmaWaves = 4;

__global__ __launch_bounds__(kMfmaWaves * 64) void score_fp32_mfma_kernel(Fp32ScoreParams p) {
  __shared__ float s_m[kMfmaWaves][32];
  __shared__ float s_z[kMfmaWaves][32];
  const int ngroups = (p.Lr + 31) / 32;
  const int rg = blockIdx.x % ngroups;
  const int h = blockIdx.x / ngroups;
  const int g = h / p.group;
  const float* Qh = p.Q + (size_t)h * p.L * p.d;
  const float* Kg = p.K + (size_t)g * p.L * p.d;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int R0 = rg * 32;
  const int R = R0 + l32;                      // this lane's reshaped row
  const int F = p.S * p.d;
  const int nsteps = (F + 1) / 2;
  const int ctop = p.causal ? min(p.Lr, R0 + 32) : p.Lr;   // columns some row of the group sees
  const int ntiles = (ctop + 31) / 32;

  auto qfeat = [&](int f) -> float {
    if (f >= F || R >= p.Lr) return 0.f;
    const int a = f / p.d, e = f - a * p.d;
    return Qh[(size_t)(R * p.S + a) * p.d + e];
  };
  auto kfeat = [&](int c, int f) -> float {
    if (f >= F || c >= p.Lr) return 0.f;
    const int a = f / p.d, e = f - a * p.d;
    const int ka = p.phase.custom ? p.phase.v[a] : p.S - 1 - a;
    return Kg[(size_t)(c * p.S + ka) * p.d + e];
  };
  auto tile = [&](int c0) -> f32x16_t {
    f32x16_t acc = f32x16_t{};
    for (int t = 0; t < nsteps; ++t)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(kfeat(c0 + l32, 2 * t + hi), qfeat(2 * t + hi), acc, 0, 0, 0);
    return acc;
  };
  auto col_of = [&](int c0, int v) -> int { return c0 + 8 * (v >> 2) + 4 * hi + (v & 3); };
  auto visible = [&](int c) -> bool { return R < p.Lr && c < p.Lr && (!p.causal || c <= R); };

  // pass 1: row max and denominator
  float m = -INFINITY, z = 0.f;
  for (int tt = wave; tt < ntiles; tt += kMfmaWaves) {
    const f32x16_t acc = tile(tt * 32);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      if (!visible(col_of(tt * 32, v))) continue;
      const float x = acc[v] * p.scale_log2;
      if (x > m) {
        z = z * fast_exp2(m - x) + 1.f;
        m = x;
      } else {
        z += fast_exp2(x - m);
      }
    }
  }
  auto merge = [](float& m1, float& z1, float m2, float z2) {
    const float mm = fmaxf(m1, m2);
    float zz = 0.f;
    if (m1 != -INFINITY) zz += z1 * fast_exp2(m1 - mm);
    if (m2 != -INFINITY) zz += z2 * fast_exp2(m2 - mm);
    m1 = mm;
    z1 = zz;
  };
  merge(m, z, __shfl_xor(m, 32), __shfl_xor(z, 32));
  if (hi == 0) {
    s_m[wave][l32] = m;
    s_z[wave][l32] = z;
  }
  __syncthreads();
  float M = -INFINITY, Z = 0.f;
  for (int w = 0; w < kMfmaWaves; ++w) merge(M, Z, s_m[w][l32], s_z[w][l32]);
  const float invZ = Z > 0.f ? 1.f / Z : 0.f;

  // pass 2: block sums of the tiles
  const int bs = p.bs;
  float* out = p.scores + (size_t)h * p.NB * p.NB;
  for (int tt = wave; tt < ntiles; tt += kMfmaWaves) {
    const int c0 = tt * 32;
    const f32x16_t acc = tile(c0);
    float pv[16];
#pragma unroll
    for (int v = 0; v < 16; ++v)
      pv[v] = visible(col_of(c0, v)) ? fast_exp2(acc[v] * p.scale_log2 - M) * invZ : 0.f;
    for (int kbl = 0; kbl < 32 / bs; ++kbl) {
      float sum = 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if ((8 * (v >> 2) + 4 * hi + (v & 3)) / bs == kbl) sum += pv[v];
      for (int off = 1; off < bs; off <<= 1) sum += __shfl_xor(sum, off);   // rows of the query block
      sum += __shfl_xor(sum, 32);                                           // the other lane half
      const int qb = R / bs, kb = c0 / bs + kbl;
      if (hi == 0 && l32 % bs == 0 && R < p.Lr && kb < p.NB) out[(size_t)qb * p.NB + kb] = sum / (float)bs;
    }
  }
  // key blocks past the causal limit of the group's query blocks are 0
  if (p.causal) {
    const int qb0 = R0 / bs, qb1 = min(R0 + 32, p.Lr) / bs, kb0 = ctop / bs;
    for (int i = tid; i < (qb1 - qb0) * (p.NB - kb0); i += blockDim.x)
      out[(size_t)(qb0 + i / (p.NB - kb0)) * p.NB + kb0 + i % (p.NB - kb0)] = 0.f;
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
  if (32 % p.bs == 0) {
    hipLaunchKernelGGL(score_fp32_mfma_kernel, dim3(s.hq * ((p.Lr + 31) / 32)), dim3(kMfmaWaves * 64), 0,
                       st, p);
  } else {
    hipLaunchKernelGGL(score_fp32_kernel, dim3(s.hq * p.NB), dim3(kThreads), 0, st, p);
  }
  return hipGetLastError();
}

}  // namespace xattn
