// Block-sparse and dense attention for bf16 on gfx950 ("XAttention: Block
// Sparse Attention with Antidiagonal Scoring", papercache.org summary,
// section 1 step 3: attention computed on the selected blocks only).
//
// One workgroup per (query head, query block of B rows); each of its B/32
// waves owns 32 query rows.  Key/value blocks -- the selected ones in sparse
// mode, all causal-visible ones in dense mode -- stream through LDS in tiles
// of 64 keys: K row-major, V transposed with a key permutation that matches
// the MFMA operand layout.  Per tile a wave computes S^T = K Q^T with
// 32x32x16 bf16 MFMAs (so each lane owns one query row), applies the causal
// mask and an online softmax in the exp2 domain, and accumulates
// O^T += V^T P^T with P rounded to bf16.  Query head h reads key/value head
// h / (hq / hkv).
#include "common.h"
#include "launch.h"

namespace xattn {
namespace {

constexpr int kKT = 64;           // keys per LDS tile
constexpr int kKPad = 8;
constexpr int kVPad = 8;
constexpr int kVtRow = kKT + kVPad;

struct FlashParams {
  const uint16_t* Q;
  const uint16_t* K;
  const uint16_t* V;
  uint16_t* O;
  const int32_t* idx;      // nullptr: dense
  const int32_t* counts;
  int L, hq, group, NB, causal;
  int nwork, grid;
  float scale_log2;        // log2(e) / sqrt(d)
};

// Position of key k (0..63) of a tile inside a transposed V row: within each
// group of 16 keys, bits 2 and 3 are swapped, so that the 8 keys lane-half
// `hi` feeds to the MFMA k-slots of one 16-key step are contiguous.
__device__ __forceinline__ int vt_pos(int k) {
  return (k & ~15) | (k & 3) | ((k & 4) << 1) | ((k & 8) >> 1);
}

template <int D, int BQ>
__global__ __launch_bounds__(BQ * 2) void flash_bf16_kernel(FlashParams p) {
  constexpr int kThreads = BQ * 2;
  constexpr int kKRow = D + kKPad;
  constexpr int kTilesPerBlock = BQ / kKT;
  constexpr int kChunks = kKT * D / 8;                 // 16-byte chunks per K (or V) tile
  constexpr int kPerThread = kChunks / kThreads;
  __shared__ __attribute__((aligned(16))) uint16_t sK[kKT * kKRow];
  __shared__ __attribute__((aligned(16))) uint16_t sVt[D * kVtRow];

  const int w = xcd_swizzle(blockIdx.x, p.grid);
  if (w >= p.nwork) return;
  const int qb = p.NB - 1 - w / p.hq;     // longest causal rows first
  const int h = w % p.hq;
  const int g = h / p.group;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int qrow = qb * BQ + wave * 32 + l32;   // this lane's query token
  const int qwave0 = qb * BQ + wave * 32;

  const uint16_t* Kg = p.K + (size_t)g * p.L * D;
  const uint16_t* Vg = p.V + (size_t)g * p.L * D;

  // query fragments (B operand of S^T = K Q^T): lane holds Q[qrow][16t + 8hi .. +8]
  bf16x8_t qf[D / 16];
  {
    const uint16_t* qp = p.Q + ((size_t)h * p.L + qrow) * D + hi * 8;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) qf[t] = as_bf16x8(*(const u32x4_t*)(qp + 16 * t));
  }

  int nkb;
  const int32_t* list = nullptr;
  if (p.idx) {
    nkb = p.counts[(size_t)h * p.NB + qb];
    nkb = nkb < 0 ? 0 : (nkb > p.NB ? p.NB : nkb);
    list = p.idx + ((size_t)h * p.NB + qb) * p.NB;
  } else {
    nkb = p.causal ? qb + 1 : p.NB;
  }
  const int ntiles = nkb * kTilesPerBlock;
  auto tile_key0 = [&](int n) -> int {   // first key of tile n, or -1 to skip it
    const int j = n / kTilesPerBlock;
    const int kb = list ? list[j] : j;
    if (kb < 0 || kb >= p.NB || (p.causal && kb > qb)) return -1;
    return kb * BQ + (n % kTilesPerBlock) * kKT;
  };

  f32x16_t o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) o[i] = f32x16_t{};
  float m = -INFINITY;   // running max (log2 units) of this lane's query row
  float lsum = 0.f;      // this lane's share of the running denominator

  u32x4_t rk[kPerThread], rv[kPerThread];
  auto prefetch = [&](int key0) {
#pragma unroll
    for (int c = 0; c < kPerThread; ++c) {
      const int ch = tid + c * kThreads;
      const int key = ch / (D / 8), col = (ch % (D / 8)) * 8;
      const size_t off = (size_t)(key0 + key) * D + col;
      rk[c] = *(const u32x4_t*)(Kg + off);
      rv[c] = *(const u32x4_t*)(Vg + off);
    }
  };

  int key0_next = ntiles > 0 ? tile_key0(0) : -1;
  if (key0_next >= 0) prefetch(key0_next);
  for (int n = 0; n < ntiles; ++n) {
    const int key0 = key0_next;
    __syncthreads();
    if (key0 >= 0) {
#pragma unroll
      for (int c = 0; c < kPerThread; ++c) {
        const int ch = tid + c * kThreads;
        const int key = ch / (D / 8), col = (ch % (D / 8)) * 8;
        *(u32x4_t*)&sK[key * kKRow + col] = rk[c];
        const int pos = vt_pos(key);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t two = rv[c][e];
          sVt[(col + 2 * e) * kVtRow + pos] = (uint16_t)(two & 0xFFFFu);
          sVt[(col + 2 * e + 1) * kVtRow + pos] = (uint16_t)(two >> 16);
        }
      }
    }
    __syncthreads();
    if (n + 1 < ntiles) {
      key0_next = tile_key0(n + 1);
      if (key0_next >= 0) prefetch(key0_next);
    }
    if (key0 < 0) continue;
    if (p.causal && key0 > qwave0 + 31) continue;   // whole tile right of this wave's rows

    // S^T (64 keys x 32 queries) as two 32x32 tiles
    f32x16_t s[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      s[i] = f32x16_t{};
#pragma unroll
      for (int t = 0; t < D / 16; ++t) {
        const bf16x8_t kf = as_bf16x8(*(const u32x4_t*)&sK[(i * 32 + l32) * kKRow + 16 * t + 8 * hi]);
        s[i] = mfma_32x32x16(kf, qf[t], s[i]);
      }
    }
    // scale, mask, running max
    const bool diag = p.causal && (key0 + kKT - 1 > qwave0);
    float mloc = -INFINITY;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float z = s[i][v] * p.scale_log2;
        if (diag) {
          const int key = key0 + 32 * i + 8 * (v >> 2) + 4 * hi + (v & 3);
          if (key > qrow) z = -INFINITY;
        }
        s[i][v] = z;
        mloc = fmaxf(mloc, z);
      }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    // No branch on per-row values: MFMAs below must run with the whole wave.
    // A row with nothing visible yet keeps m = -inf and gets p = 0, alpha = 0.
    const float mnew = fmaxf(m, mloc);
    const float mref = (mnew == -INFINITY) ? 0.f : mnew;
    const float alpha = fast_exp2(m - mref);  // m == -inf gives 0
    m = mnew;
    float rs = 0.f;
    bf16x8_t pf[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = u >> 1, v0 = (u & 1) * 8;
      uint32_t pk[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float z0 = s[i][v0 + 2 * e], z1 = s[i][v0 + 2 * e + 1];
        const float p0 = fast_exp2(z0 - mref), p1 = fast_exp2(z1 - mref);
        rs += p0 + p1;
        pk[e] = pack_bf16x2(p0, p1);
      }
      pf[u] = as_bf16x8(u32x4_t{pk[0], pk[1], pk[2], pk[3]});
    }
    lsum = lsum * alpha + rs;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      o[dt] *= alpha;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bf16x8_t vf = as_bf16x8(*(const u32x4_t*)&sVt[(dt * 32 + l32) * kVtRow + 16 * u + 8 * hi]);
        o[dt] = mfma_32x32x16(vf, pf[u], o[dt]);
      }
    }
  }

  // normalise and store: lane holds O[qrow][32 dt + 8 g + 4 hi + r]
  const float ltot = lsum + __shfl_xor(lsum, 32);
  const float inv = ltot > 0.f ? 1.0f / ltot : 0.f;
  uint16_t* op = p.O + ((size_t)h * p.L + qrow) * D;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) {
      const int col = dt * 32 + 8 * gg + 4 * hi;
      u32x2_t v;
      v[0] = pack_bf16x2(o[dt][4 * gg] * inv, o[dt][4 * gg + 1] * inv);
      v[1] = pack_bf16x2(o[dt][4 * gg + 2] * inv, o[dt][4 * gg + 3] * inv);
      *(u32x2_t*)(op + col) = v;
    }
}

template <int D, int BQ>
hipError_t launch(const FlashParams& fp, hipStream_t st) {
  hipLaunchKernelGGL((flash_bf16_kernel<D, BQ>), dim3(fp.grid), dim3(BQ * 2), 0, st, fp);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_flash_bf16(const Shape& s, const void* Q, const void* K, const void* V,
                             int B, const int32_t* idx, const int32_t* counts, void* O,
                             hipStream_t st) {
  FlashParams fp;
  fp.Q = (const uint16_t*)Q;
  fp.K = (const uint16_t*)K;
  fp.V = (const uint16_t*)V;
  fp.O = (uint16_t*)O;
  fp.idx = idx;
  fp.counts = counts;
  fp.L = s.L;
  fp.hq = s.hq;
  fp.group = s.hq / s.hkv;
  fp.NB = s.L / B;
  fp.causal = s.causal;
  fp.nwork = fp.NB * s.hq;
  fp.grid = (fp.nwork + kNumXcd - 1) / kNumXcd * kNumXcd;
  fp.scale_log2 = (float)(1.4426950408889634 / __builtin_sqrt((double)s.d));
  if (s.d == 128) return B == 128 ? launch<128, 128>(fp, st) : launch<128, 64>(fp, st);
  return B == 128 ? launch<64, 128>(fp, st) : launch<64, 64>(fp, st);
}

}  // namespace xattn
