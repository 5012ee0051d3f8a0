// Block-sparse and dense attention for fp32 inputs (papercache.org summary,
// section 1 step 3).  One workgroup per (query head, query block), key/value
// tiles of 32 rows staged in LDS, online softmax in fp32.  Query blocks of a
// multiple of 32 rows run on the matrix cores (32x32x2 fp32 MFMAs, one wave
// per 32 query rows); other block sizes use a SIMT kernel, one thread per
// query row.
#include "common.h"
#include "launch.h"

namespace xattn {
namespace {

constexpr int kKT = 32;

struct Fp32FlashParams {
  const float* Q;
  const float* K;
  const float* V;
  float* O;
  const int32_t* idx;
  const int32_t* counts;
  int L, B, NB, group, causal;
  float scale_log2;
};

template <int D>
__global__ __launch_bounds__(256) void flash_fp32_kernel(Fp32FlashParams p) {
  __shared__ float sK[kKT][D];
  __shared__ float sV[kKT][D];
  const int qb = blockIdx.x % p.NB;
  const int h = blockIdx.x / p.NB;
  const int g = h / p.group;
  const int tid = threadIdx.x;
  const int qrow = qb * p.B + tid;
  const bool live = tid < p.B;
  const float* Kg = p.K + (size_t)g * p.L * D;
  const float* Vg = p.V + (size_t)g * p.L * D;

  float q[D], o[D];
#pragma unroll
  for (int e = 0; e < D; ++e) {
    q[e] = live ? p.Q[((size_t)h * p.L + qrow) * D + e] : 0.f;
    o[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f;

  // One key block: stream its keys through LDS and update the online softmax.
  auto visit = [&](int kb) {
    for (int t0 = 0; t0 < p.B; t0 += kKT) {
      const int nk = min(kKT, p.B - t0);
      const int key0 = kb * p.B + t0;
      __syncthreads();
      for (int i = tid; i < nk * D; i += blockDim.x) {
        sK[i / D][i % D] = Kg[(size_t)(key0 + i / D) * D + i % D];
        sV[i / D][i % D] = Vg[(size_t)(key0 + i / D) * D + i % D];
      }
      __syncthreads();
      if (!live) continue;
      for (int k = 0; k < nk; ++k) {
        if (p.causal && key0 + k > qrow) break;
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < D; ++e) dot = fmaf(q[e], sK[k][e], dot);
        const float z = dot * p.scale_log2;
        const float mnew = fmaxf(m, z);
        const float alpha = fast_exp2(m - mnew);
        const float pz = fast_exp2(z - mnew);
        l = l * alpha + pz;
#pragma unroll
        for (int e = 0; e < D; ++e) o[e] = fmaf(pz, sV[k][e], o[e] * alpha);
        m = mnew;
      }
    }
  };
  if (p.idx) {
    // The list as a set: a bitmap in LDS (invalid entries dropped, repeats
    // kept once), walked in ascending block order by the whole workgroup.
    extern __shared__ uint32_t s_bits[];
    const int nw32 = (p.NB + 31) / 32;
    for (int w = tid; w < nw32; w += blockDim.x) s_bits[w] = 0u;
    __syncthreads();
    int cnt = p.counts[(size_t)h * p.NB + qb];
    cnt = cnt < 0 ? 0 : (cnt > p.NB ? p.NB : cnt);
    const int32_t* list = p.idx + ((size_t)h * p.NB + qb) * p.NB;
    for (int j = tid; j < cnt; j += blockDim.x) {
      const int kb = list[j];
      if (kb < 0 || kb >= p.NB || (p.causal && kb > qb)) continue;
      atomicOr(&s_bits[kb >> 5], 1u << (kb & 31));
    }
    __syncthreads();
    for (int w = 0; w < nw32; ++w) {
      uint32_t bits = s_bits[w];
      while (bits) {
        visit(32 * w + __builtin_ctz(bits));
        bits &= bits - 1;
      }
    }
  } else {
    const int nkb = p.causal ? qb + 1 : p.NB;
    for (int kb = 0; kb < nkb; ++kb) visit(kb);
  }
  if (!live) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int e = 0; e < D; ++e) p.O[((size_t)h * p.L + qrow) * D + e] = o[e] * inv;
}

// Row stride (floats) of the matrix-core kernel's LDS tiles: one float of
// padding makes the column reads of S (32 key rows, one feature each) fall in
// distinct banks.
template <int D>
constexpr int kPadRow = D + 1;

// Matrix-core version.  Per 32-key tile a wave computes S^T = K Q^T: the two
// reduction indices of MFMA step t are the features t and t + D/2, so lane
// (l32, hi) feeds K[key0 + l32][t + hi D/2] and Q[row l32][t + hi D/2] and
// reads contiguous features.  Each lane then holds its query row's scores for
// the keys 8 (v / 4) + 4 hi + v % 4 of register v; the online softmax (exp2
// domain, exact rescale) keeps P in those registers, and step v of
// O^T += V^T P^T pairs exactly the two keys the lane halves hold in register
// v, so P is used where it lies: A = V[that key][d0 + l32], B = p[v].
template <int D>
__global__ __launch_bounds__(512) void flash_fp32_mfma_kernel(Fp32FlashParams p) {
  constexpr int kRow = kPadRow<D>;
  __shared__ float sK[kKT * kRow];
  __shared__ float sV[kKT * kRow];
  const int qb = blockIdx.x % p.NB;
  const int h = blockIdx.x / p.NB;
  const int g = h / p.group;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int qwave0 = qb * p.B + wave * 32;
  const int qrow = qwave0 + l32;
  const float* Kg = p.K + (size_t)g * p.L * D;
  const float* Vg = p.V + (size_t)g * p.L * D;

  float q[D / 2];
#pragma unroll
  for (int t = 0; t < D / 2; ++t) q[t] = p.Q[((size_t)h * p.L + qrow) * D + t + hi * (D / 2)];
  f32x16_t o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) o[i] = f32x16_t{};
  float m = -INFINITY, l = 0.f;   // running max (log2 units) and this lane's share of the sum

  auto visit = [&](int kb) {
    for (int t0 = 0; t0 < p.B; t0 += kKT) {
      const int key0 = kb * p.B + t0;
      __syncthreads();
      for (int i = tid; i < kKT * D; i += blockDim.x) {
        sK[(i / D) * kRow + i % D] = Kg[(size_t)(key0 + i / D) * D + i % D];
        sV[(i / D) * kRow + i % D] = Vg[(size_t)(key0 + i / D) * D + i % D];
      }
      __syncthreads();
      if (p.causal && key0 > qwave0 + 31) continue;   // the whole tile is above this wave's rows
      f32x16_t sacc = f32x16_t{};
#pragma unroll
      for (int t = 0; t < D / 2; ++t)
        sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(sK[l32 * kRow + t + hi * (D / 2)], q[t], sacc, 0, 0, 0);
      float z[16];
      float mloc = -INFINITY;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = key0 + 8 * (v >> 2) + 4 * hi + (v & 3);
        z[v] = (p.causal && key > qrow) ? -INFINITY : sacc[v] * p.scale_log2;
        mloc = fmaxf(mloc, z[v]);
      }
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32));   // the row's other 16 keys
      const float mnew = fmaxf(m, mloc);
      const float mref = mnew == -INFINITY ? 0.f : mnew;   // no visible key yet: p = 0
      const float alpha = fast_exp2(m - mref);              // m == -inf gives 0
      float pv[16], rs = 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        pv[v] = fast_exp2(z[v] - mref);
        rs += pv[v];
      }
      l = l * alpha + rs;
      m = mnew;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        o[dt] *= alpha;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = 8 * (v >> 2) + 4 * hi + (v & 3);
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(sV[key * kRow + dt * 32 + l32], pv[v], o[dt], 0, 0, 0);
        }
      }
    }
  };
  if (p.idx) {
    // the list as a set, as in the SIMT kernel below
    extern __shared__ uint32_t s_bits[];
    const int nw32 = (p.NB + 31) / 32;
    for (int w = tid; w < nw32; w += blockDim.x) s_bits[w] = 0u;
    __syncthreads();
    int cnt = p.counts[(size_t)h * p.NB + qb];
    cnt = cnt < 0 ? 0 : (cnt > p.NB ? p.NB : cnt);
    const int32_t* list = p.idx + ((size_t)h * p.NB + qb) * p.NB;
    for (int j = tid; j < cnt; j += blockDim.x) {
      const int kb = list[j];
      if (kb < 0 || kb >= p.NB || (p.causal && kb > qb)) continue;
      atomicOr(&s_bits[kb >> 5], 1u << (kb & 31));
    }
    __syncthreads();
    for (int w = 0; w < nw32; ++w) {
      uint32_t bits = s_bits[w];
      while (bits) {
        visit(32 * w + __builtin_ctz(bits));
        bits &= bits - 1;
      }
    }
  } else {
    const int nkb = p.causal ? qb + 1 : p.NB;
    for (int kb = 0; kb < nkb; ++kb) visit(kb);
  }
  // lane holds O[qrow][32 dt + 8 (v / 4) + 4 hi + v % 4]
  const float ltot = l + __shfl_xor(l, 32);
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  float* op = p.O + ((size_t)h * p.L + qrow) * D;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) op[dt * 32 + 8 * (v >> 2) + 4 * hi + (v & 3)] = o[dt][v] * inv;
}

template <int D>
hipError_t launch(const Fp32FlashParams& fp, int hq, hipStream_t st) {
  const size_t bitmap_bytes = fp.idx ? (size_t)((fp.NB + 31) / 32) * sizeof(uint32_t) : 0;
  if (fp.B % 32 == 0) {
    hipLaunchKernelGGL((flash_fp32_mfma_kernel<D>), dim3(hq * fp.NB), dim3(fp.B * 2), bitmap_bytes, st,
                       fp);
  } else {
    const int threads = (fp.B + 63) / 64 * 64;
    hipLaunchKernelGGL((flash_fp32_kernel<D>), dim3(hq * fp.NB), dim3(threads), bitmap_bytes, st, fp);
  }
  return hipGetLastError();
}

}  // namespace

size_t flash_fp32_lds_bytes(int d, int NB, bool sparse) {
  // the matrix-core kernel's padded tiles (the larger of the two kernels' needs)
  return (size_t)2 * kKT * (d + 1) * sizeof(float) +
         (sparse ? (size_t)((NB + 31) / 32) * sizeof(uint32_t) : 0);
}

hipError_t launch_flash_fp32(const Shape& s, const void* Q, const void* K, const void* V,
                             int B, const int32_t* idx, const int32_t* counts, void* O,
                             hipStream_t st) {
  Fp32FlashParams fp;
  fp.Q = (const float*)Q;
  fp.K = (const float*)K;
  fp.V = (const float*)V;
  fp.O = (float*)O;
  fp.idx = idx;
  fp.counts = counts;
  fp.L = s.L;
  fp.B = B;
  fp.NB = s.L / B;
  fp.group = s.hq / s.hkv;
  fp.causal = s.causal;
  fp.scale_log2 = (float)(1.4426950408889634 / __builtin_sqrt((double)s.d));
  switch (s.d) {
    case 32: return launch<32>(fp, s.hq, st);
    case 64: return launch<64>(fp, s.hq, st);
    case 128: return launch<128>(fp, s.hq, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace xattn
