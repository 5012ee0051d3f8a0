// Per-head threshold calibration ("XAttention: Block Sparse Attention with
// Antidiagonal Scoring", papercache.org summary, section 2.3 "minimum
// threshold prediction"; chapterpal.com Knowl 3).
//
// head_error_kernel: the performance proxy of one head, the relative squared
// error sum (O_sparse - O_dense)^2 / sum O_dense^2 over its [L][d] output.
// One workgroup per head streams both outputs (16-byte loads), accumulates in
// float64 per thread and reduces in a fixed tree order, so the result does
// not depend on scheduling.
//
// tau_dp (host): distributes exactly `steps` threshold-reduction steps over
// the heads, each head taking k = 0 .. R steps; D[h][m] is the best value of
// minus the summed error of heads 0 .. h-1 with m steps in total (R = 1 is
// the printed recurrence D[h][m] = max(D[h-1][m], P(h, m))).  Ties keep the
// smaller k for the later head.
#include <vector>

#include "common.h"
#include "launch.h"

namespace xattn {
namespace {

constexpr int kErrThreads = 1024;

struct HeadErrParams {
  const void* A;   // sparse output
  const void* B;   // dense output
  double* err;     // [hq]
  size_t n;        // elements per head (L * d)
};

// Adds one 16-byte chunk of each output (8 bf16 or 4 fp32 values).
template <bool BF16>
__device__ __forceinline__ void accumulate(u32x4_t va, u32x4_t vb, double& num, double& den) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (BF16) {
      const double a0 = bf16_bits_to_f32(va[i] & 0xFFFFu), a1 = bf16_bits_to_f32(va[i] >> 16);
      const double b0 = bf16_bits_to_f32(vb[i] & 0xFFFFu), b1 = bf16_bits_to_f32(vb[i] >> 16);
      num += (a0 - b0) * (a0 - b0) + (a1 - b1) * (a1 - b1);
      den += b0 * b0 + b1 * b1;
    } else {
      // reinterpret the whole vectors, then index (a bit_cast of one subscripted
      // element of an ext_vector_type value reads element 0 on this compiler)
      const double av = __builtin_bit_cast(f32x4_t, va)[i], bv = __builtin_bit_cast(f32x4_t, vb)[i];
      num += (av - bv) * (av - bv);
      den += bv * bv;
    }
  }
}

template <bool BF16>
__global__ __launch_bounds__(kErrThreads) void head_error_kernel(HeadErrParams p) {
  __shared__ double s_num[kErrThreads];
  __shared__ double s_den[kErrThreads];
  const int h = blockIdx.x, tid = threadIdx.x;
  constexpr size_t kEsz = BF16 ? 2 : 4;
  const size_t chunks = p.n * kEsz / 16;   // 16-byte chunks per head (n * size is a multiple of 16)
  const u32x4_t* a = (const u32x4_t*)((const char*)p.A + (size_t)h * p.n * kEsz);
  const u32x4_t* b = (const u32x4_t*)((const char*)p.B + (size_t)h * p.n * kEsz);
  double num = 0.0, den = 0.0;
  for (size_t i = tid; i < chunks; i += kErrThreads) {
    const u32x4_t va = a[i], vb = b[i];
    accumulate<BF16>(va, vb, num, den);
  }
  s_num[tid] = num;
  s_den[tid] = den;
  __syncthreads();
  for (int o = kErrThreads / 2; o > 0; o >>= 1) {
    if (tid < o) {
      s_num[tid] += s_num[tid + o];
      s_den[tid] += s_den[tid + o];
    }
    __syncthreads();
  }
  if (tid == 0) p.err[h] = s_den[0] > 0.0 ? s_num[0] / s_den[0] : 0.0;
}

}  // namespace

hipError_t launch_head_error(int hq, size_t per_head, bool bf16, const void* O_sparse,
                             const void* O_dense, double* err, hipStream_t st) {
  HeadErrParams p;
  p.A = O_sparse;
  p.B = O_dense;
  p.err = err;
  p.n = per_head;
  if (bf16) hipLaunchKernelGGL((head_error_kernel<true>), dim3(hq), dim3(kErrThreads), 0, st, p);
  else hipLaunchKernelGGL((head_error_kernel<false>), dim3(hq), dim3(kErrThreads), 0, st, p);
  return hipGetLastError();
}

double tau_dp(int H, int R, const double* err, int steps, int* levels) {
  const double NEG = -__builtin_inf();
  const size_t W = (size_t)steps + 1;
  std::vector<double> D((size_t)(H + 1) * W, NEG);
  std::vector<int> take((size_t)(H + 1) * W, 0);
  D[0] = 0.0;
  for (int h = 1; h <= H; ++h)
    for (int m = 0; m <= steps; ++m)
      for (int k = 0; k <= (R < m ? R : m); ++k) {
        const double prev = D[(size_t)(h - 1) * W + (m - k)];
        if (prev == NEG) continue;
        const double cand = prev - err[(size_t)(h - 1) * (R + 1) + k];
        double& cur = D[(size_t)h * W + m];
        if (cand > cur) {
          cur = cand;
          take[(size_t)h * W + m] = k;
        }
      }
  int m = steps;
  for (int h = H; h >= 1; --h) {
    levels[h - 1] = take[(size_t)h * W + m];
    m -= levels[h - 1];
  }
  return D[(size_t)H * W + steps];
}

}  // namespace xattn
