// Block-sparse and dense attention for fp32 inputs: a SIMT kernel for small
// fp32 problems (papercache.org summary, section 1 step 3).  One workgroup per
// (query head, query block), one thread per query row, key/value tiles of 32
// rows staged in LDS, online softmax in fp32.
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

template <int D>
hipError_t launch(const Fp32FlashParams& fp, int hq, hipStream_t st) {
  const int threads = (fp.B + 63) / 64 * 64;
  const size_t bitmap_bytes = fp.idx ? (size_t)((fp.NB + 31) / 32) * sizeof(uint32_t) : 0;
  hipLaunchKernelGGL((flash_fp32_kernel<D>), dim3(hq * fp.NB), dim3(threads), bitmap_bytes, st, fp);
  return hipGetLastError();
}

}  // namespace

size_t flash_fp32_lds_bytes(int d, int NB, bool sparse) {
  return (size_t)2 * kKT * d * sizeof(float) + (sparse ? (size_t)((NB + 31) / 32) * sizeof(uint32_t) : 0);
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
