// Block scores of XAttention ("XAttention: Block Sparse Attention with
// Antidiagonal Scoring", papercache.org summary, section 2.2, Algorithm 1)
// for bf16 inputs on gfx950.
//
// Algorithm 1 multiplies a stride-S reshape of the queries (phases S-1 .. 0
// appended along features) by a reshape of the keys (phases 0 .. S-1).  The
// product entry (R, c) is sum_a <Q[R*S+a], K[c*S+S-1-a]>: the antidiagonal sum
// of the SxS tile (R, c) of Q K^T.  Here it is one GEMM with M = N = L/S and
// K-dimension S*d: the query operand is Q's own memory read as an (L/S) x (S*d)
// matrix, and the key operand reads sub-row S-1-a of key group c for feature
// chunk a -- the reshape is folded into the global load addresses and never
// materialised.  Other sampling patterns of the pattern-geometry ablation
// (chapterpal.com Knowl 9: diagonal, random) only change which key sub-row a
// chunk reads (a permutation of 0 .. S-1), so they run the same kernel.
//
// Kernel 1 (score_gemm): MFMA 32x32x16 bf16 GEMM over lower-triangular (causal)
// or all 256x256 tiles of the reshaped matrix, computed transposed (rows =
// key columns c, columns = query rows R) so that each lane owns one reshaped
// row R.  Its epilogue masks c > R, scales by log2(e)/sqrt(d*S) and, per
// 64-column range of each row, writes the range max m, the range sum of
// exp2(z - m) and the per-key-block sums of exp2(z - m).  The (L/S)^2 matrix
// never reaches HBM.
// Kernel 2 (score_fixup): per 32 reshaped rows, combines the range snapshots
// into the row's softmax max and denominator, rescales the partial block sums,
// adds the B/S rows of each query block and divides by B/S.
// Kernel 2' (score_select_fused, xattn_score_select): kernel 2 with the
// threshold selection of its query blocks' rows in the same workgroup.
#include <algorithm>
#include <atomic>

#include "common.h"
#include "launch.h"
#include "select_row.h"

namespace xattn {
namespace {

constexpr int kWavesC = 4;       // waves along c
constexpr int kWavesR = 2;       // waves along R
constexpr int kWaves = kWavesC * kWavesR;   // two waves per SIMD
constexpr int kWaveC = 64;       // key columns c per wave
constexpr int kWaveR = 128;      // query rows R per wave
constexpr int kTileC = kWaveC * kWavesC;    // reshaped columns c per workgroup tile
constexpr int kTileR = kWaveR * kWavesR;    // reshaped rows R per workgroup tile
constexpr int kRangeCols = 64;   // columns per softmax snapshot
constexpr int kKC = 64;          // reduction chunk (elements of S*d): 128-byte LDS rows
constexpr int kRowBytes = kKC * 2;
constexpr int kStageBytes = (kTileC + kTileR) * kRowBytes;   // 64 KB
constexpr int kRowsPerCopy = 1024 / kRowBytes;               // rows per 1 KB copy
constexpr int kDmaPerWave = kStageBytes / 1024 / kWaves;     // 1 KB copies per wave per chunk
constexpr int kDmaK = kTileC * kRowBytes / 1024 / kWaves;    // of which key-row copies

struct GemmParams {
  const uint16_t* Q;
  const uint16_t* K;
  float* P;   // [hq][nR32][NB][32]
  float* M;   // [hq][nR32][nct][32]
  float* Z;   // [hq][nR32][nct][32]
  int L, S, group, NB, Lr, nR32, nct;
  int causal, ntr, ntc, tiles_per_head, nwork;
  int per_xcd, wg_per_xcd;   // work items per XCD (at most), workgroups per XCD
  int deal;                  // consecutive work items per dealt chunk
  float scale_log2;
  PhaseMap phase;   // key sub-row per query sub-row (default: antidiagonal)
};

// LDS rows hold one 64-element (128-byte) chunk of a reshaped row; their
// eight 16-byte pieces are XOR-swizzled by (row / 2) mod 8, so that 16
// consecutive rows read at the same piece fall in 16 distinct 16-byte bank
// groups (64 four-byte banks): conflict-free 16-byte fragment reads.
__device__ __forceinline__ int piece_slot(int row, int piece) { return piece ^ ((row >> 1) & 7); }

// Epilogue of a wave's 64-column range (accumulator blocks I0, I0+1) with no
// masked column: per row R (one per lane and 32-row block j) the range max
// (the scale is positive, so the max of the scaled values is the scaled
// max), the range sum of exp2(z - m) and the per-key-block sums.  Each block
// sum is finished by one exchange between the two half-waves: a lane keeps
// the four-column sums of the block it stores and hands the other
// half-wave's block to its partner, so every lane stores and no store is
// predicated beyond the row bound.
template <int BS, int I0>
__device__ __forceinline__ void epilogue_interior(const GemmParams& p, f32x16_t (&acc)[2][4], int h,
                                                  int R_lane0, int cw, int hi) {
  const int kb0 = cw / BS, ct = cw / kRangeCols;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int R = R_lane0 + j * 32;
    float mr = acc[I0][j][0];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) mr = fmaxf(mr, acc[I0 + i][j][v]);
    float m = mr * p.scale_log2;
    m = fmaxf(m, __shfl_xor(m, 32));
    float s[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float acc4 = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) acc4 += fast_exp2(acc[I0 + i][j][4 * q + r] * p.scale_log2 - m);
        s[i][q] = acc4;
      }
    float zsum = 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) zsum += s[i][q];
    zsum += __shfl_xor(zsum, 32);
    if (R >= p.Lr) continue;
    const size_t rowbase = (size_t)h * p.nR32 + (R >> 5);
    if (hi == 0) {
      p.M[(rowbase * p.nct + ct) * 32 + (R & 31)] = m;
      p.Z[(rowbase * p.nct + ct) * 32 + (R & 31)] = zsum;
    }
    float* Prow = p.P + rowbase * p.NB * 32 + (R & 31);
    if constexpr (BS == 4) {   // lane half hi holds blocks kb0 + 8i + 2q + hi
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) Prow[(size_t)(kb0 + 8 * i + 2 * q + hi) * 32] = s[i][q];
    } else if constexpr (BS == 8) {   // block kb0 + 4i + q: sums s[i][q] of both halves
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int qq = 0; qq < 2; ++qq) {
          const float keep = hi ? s[i][2 * qq + 1] : s[i][2 * qq];
          const float give = hi ? s[i][2 * qq] : s[i][2 * qq + 1];
          Prow[(size_t)(kb0 + 4 * i + 2 * qq + hi) * 32] = keep + __shfl_xor(give, 32);
        }
    } else if constexpr (BS == 16) {   // block kb0 + 2i + b: pairs (2b, 2b+1) of both halves
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const float t0 = s[i][0] + s[i][1], t1 = s[i][2] + s[i][3];
        const float keep = hi ? t1 : t0, give = hi ? t0 : t1;
        Prow[(size_t)(kb0 + 2 * i + hi) * 32] = keep + __shfl_xor(give, 32);
      }
    } else {   // BS == 32: block kb0 + i, all four sums of both halves
      float t[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) t[i] = s[i][0] + s[i][1] + s[i][2] + s[i][3];
      const float keep = hi ? t[1] : t[0], give = hi ? t[0] : t[1];
      Prow[(size_t)(kb0 + hi) * 32] = keep + __shfl_xor(give, 32);
    }
  }
}

// Epilogue of a diagonal or ragged 64-column range: columns c > R (causal)
// or c >= Lr are masked to -inf before the range max and sums.
template <int BS, int I0>
__device__ __forceinline__ void epilogue_masked(const GemmParams& p, f32x16_t (&acc)[2][4], int h,
                                                int R_lane0, int cw, int hi) {
  const int Lr = p.Lr;
  const int ct = cw / kRangeCols;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int R = R_lane0 + j * 32;
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int c = cw + i * 32 + 8 * (v >> 2) + 4 * hi + (v & 3);
        float z = acc[I0 + i][j][v] * p.scale_log2;
        if (c >= Lr || (p.causal && c > R)) z = -INFINITY;
        acc[I0 + i][j][v] = z;
        m = fmaxf(m, z);
      }
    m = fmaxf(m, __shfl_xor(m, 32));
    float s[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float acc4 = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float z = acc[I0 + i][j][4 * q + r];
          acc4 += (z == -INFINITY) ? 0.f : fast_exp2(z - m);
        }
        s[i][q] = acc4;
      }
    float zsum = 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) zsum += s[i][q];
    zsum += __shfl_xor(zsum, 32);
    // Stores are guarded rather than branched around so that every lane takes
    // part in the exchanges below.  A range starting at or past Lr (the
    // ragged last tile) owns no snapshot slot.
    const bool row_ok = R < Lr && cw < Lr;
    const size_t rowbase = (size_t)h * p.nR32 + (R >> 5);
    if (row_ok && hi == 0) {
      p.M[(rowbase * p.nct + ct) * 32 + (R & 31)] = m;
      p.Z[(rowbase * p.nct + ct) * 32 + (R & 31)] = zsum;
    }
    float* Prow = p.P + rowbase * p.NB * 32 + (R & 31);
    const int kb0 = cw / BS;
    if constexpr (BS == 4) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int kb = kb0 + 8 * i + 2 * q + hi;
          if (row_ok && kb < p.NB) Prow[(size_t)kb * 32] = s[i][q];
        }
    } else if constexpr (BS == 8) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float tot = s[i][q] + __shfl_xor(s[i][q], 32);
          const int kb = kb0 + 4 * i + q;
          if (row_ok && (q & 1) == hi && kb < p.NB) Prow[(size_t)kb * 32] = tot;
        }
    } else if constexpr (BS == 16) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int q = 0; q < 4; q += 2) {
          float tot = s[i][q] + s[i][q + 1];
          tot += __shfl_xor(tot, 32);
          const int kb = kb0 + 2 * i + q / 2;
          if (row_ok && ((q >> 1) & 1) == hi && kb < p.NB) Prow[(size_t)kb * 32] = tot;
        }
    } else {  // BS == 32
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        float tot = s[i][0] + s[i][1] + s[i][2] + s[i][3];
        tot += __shfl_xor(tot, 32);
        const int kb = kb0 + i;
        if (row_ok && i == hi && kb < p.NB) Prow[(size_t)kb * 32] = tot;
      }
    }
  }
}

// One 64-column range of a wave: the unmasked path where no column can be
// masked, the masked path otherwise.
template <int BS, int I0>
__device__ __forceinline__ void epilogue_range(const GemmParams& p, f32x16_t (&acc)[2][4], int h, int Rw,
                                               int cw, int l32, int hi) {
  if (cw + kRangeCols <= p.Lr && (!p.causal || cw + kRangeCols - 1 <= Rw))
    epilogue_interior<BS, I0>(p, acc, h, Rw + l32, cw, hi);
  else if (!p.causal || cw <= Rw + kWaveR - 1)
    epilogue_masked<BS, I0>(p, acc, h, Rw + l32, cw, hi);
}

// Tile of work item w: work order (kv group, tile, query head within group),
// heads fastest; causal tiles are the lower triangle, row tr holding column
// tiles 0 .. tr.
struct TileItem {
  int h, g, R0, C0;
};

__device__ __forceinline__ TileItem decode_item(const GemmParams& p, int w) {
  const int hh = w % p.group;
  const int t = (w / p.group) % p.tiles_per_head;
  const int g = w / (p.group * p.tiles_per_head);
  int tr, tc;
  if (p.causal) {
    tr = (int)((sqrtf(8.0f * (float)t + 1.0f) - 1.0f) * 0.5f);
    while ((tr + 1) * (tr + 2) / 2 <= t) ++tr;
    while (tr * (tr + 1) / 2 > t) --tr;
    tc = t - tr * (tr + 1) / 2;
  } else {
    tr = t / p.ntc;
    tc = t % p.ntc;
  }
  return TileItem{g * p.group + hh, g, tr * kTileR, tc * kTileC};
}

// Persistent scoring GEMM: one workgroup of eight waves per CU (two per
// SIMD), each wave owning a 64 x 128 block of the 256 x 256 tile (eight MFMA
// accumulators).
//
// Scheduling: workgroups are dealt round-robin to the XCDs, so workgroup b
// runs on XCD b % 8.  The work items are cut into chunks of p.deal
// consecutive items, chunk c going to XCD c % 8, and an XCD's wg_per_xcd
// workgroups take every wg_per_xcd-th of its items, so one XCD's CUs work on
// consecutive items -- a few column tiles of one tile row for all query heads
// of one KV group -- and share Q and K rows in its L2.  With chunks of eight
// tiles x all heads of a group, all XCDs also work through the KV groups
// together, so the misses of their L2s find one group's Q and K in the
// memory-side cache (1-4 % faster from 512 tiles per head on, 1 % slower on
// smaller problems); with p.deal = ceil(items / 8) each XCD takes one
// contiguous range instead.
//
// Data movement: a chunk is 64 elements of S*d (four k-steps of 16), one
// 128-byte segment of each of the tile's 512 reshaped rows -- whole cache
// lines, which the L2 serves at twice the rate of half lines.  Two LDS
// stages of 64 KB: chunk kc+2 is copied into chunk kc's stage once every
// wave has read it, while chunk kc+1 is being multiplied.  The fragments of
// the next k-step are read from LDS while the MFMAs of the current one run,
// also across the chunk barrier, so LDS latency is hidden inside the wave.
// The copy sequence runs across items: an item's last two chunk steps copy
// the next item's first two chunks, which land while its epilogue runs.
template <int D, int BS, bool PATTERN>
__global__ __launch_bounds__(kWaves * 64, 1) void score_gemm(GemmParams p) {
  static_assert(kDmaPerWave == 8 && kDmaK == 4, "copy layout assumes 8 copies per wave per chunk");
  // Two LDS stages as distinct objects (the chunk loop is unrolled by two) so
  // LDS reads of one stage never wait on the direct-to-LDS copies into the other.
  __shared__ __attribute__((aligned(1024))) uint8_t st0[kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t st1[kStageBytes];

  // Chunks of p.deal consecutive work items are dealt to the XCDs in turn
  // (chunk c to XCD c % 8), so all XCDs work through the KV groups together;
  // XCD x's j-th item is w(j) = ((j / deal) * 8 + x) * deal + j % deal, which
  // grows with j, so its items are the j < n_x below.
  const int xcd = blockIdx.x % kNumXcd, slot = blockIdx.x / kNumXcd;
  const int full = p.nwork / p.deal, rem = p.nwork % p.deal;
  int n_x = full > xcd ? ((full - xcd - 1) / kNumXcd + 1) * p.deal : 0;
  if (rem && full >= xcd && (full - xcd) % kNumXcd == 0) n_x += rem;
  if (slot >= n_x) return;
  const int nitems = (n_x - slot + p.wg_per_xcd - 1) / p.wg_per_xcd;
  auto item_at = [&](int k) -> int {
    const int j = slot + k * p.wg_per_xcd;
    return ((j / p.deal) * kNumXcd + xcd) * p.deal + j % p.deal;
  };

  const int F = p.S * D;
  const int Lr = p.Lr;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wc = wave % kWavesC, wr = wave / kWavesC;
  const int l32 = lane & 31, hi = lane >> 5;
  // a sampling pattern's key sub-row for query sub-row a, held in lane a
  // (patterns cover S <= 64), read with one lane read instead of a scalar load
  const int phase_lane = PATTERN ? p.phase.v[lane] : 0;

  // Direct-to-LDS copies through buffer resources (buffer_load ... lds).  A
  // stage holds kTileC key rows then kTileR query rows; copy n (1 KB) fills
  // rows 8n .. 8n+7, lane -> row 8n + lane/8 and 16-byte slot lane % 8, which
  // receives the piece the swizzle places there.  Per lane the byte offset of
  // its row is fixed per item; the chunk moves only the scalar offset.  Rows
  // past Lr (ragged last tile) re-read row Lr-1: finite data whose products
  // are masked or never stored.
  auto row_offsets = [&](const TileItem& t, uint32_t (&off)[kDmaPerWave]) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < kDmaPerWave; ++k) {
      const int n = k * kWaves + wave;
      const int row = n * kRowsPerCopy + (lane >> 3);
      const int piece = piece_slot(row, lane & 7);   // the swizzle is an involution
      if (k < kDmaK) {   // copies 0 .. kDmaK-1 of every wave cover the key rows
        const int C = min(t.C0 + row, Lr - 1);
        off[k] = (uint32_t)(C * F * 2 + piece * 16);
      } else {
        const int R = min(t.R0 + row - kTileC, Lr - 1);
        off[k] = (uint32_t)(R * F * 2 + piece * 16);
      }
    }
  };
  const int nk = F / kKC;
  const int nkp = (nk + 1) & ~1;   // chunk steps per item (a step past nk reloads chunk nk-1)
  auto issue = [&](int h_, int g_, const uint32_t (&off)[kDmaPerWave], int kc, uint8_t* stage)
                   __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.K + (size_t)g_ * p.L * D), (short)0, p.L * D * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.Q + (size_t)h_ * p.L * D), (short)0, p.L * D * 2, 0x00020000);
    kc = min(kc, nk - 1);
    const int f0 = kc * kKC;
    const int a = f0 / D, e0 = f0 % D;
    // key operand: sub-row S-1-a of key group c (the stride reshape, reversed
    // phase), or the sub-row the sampling pattern pairs with query sub-row a
    const int ka = PATTERN ? __builtin_amdgcn_readlane(phase_lane, a) : p.S - 1 - a;
    const uint32_t koff = (uint32_t)((ka * D + e0) * 2);
    const uint32_t qoff = (uint32_t)(f0 * 2);
#pragma unroll
    for (int k = 0; k < kDmaPerWave; ++k) {
      const int n = k * kWaves + wave;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(k < kDmaK ? rk : rq,
                                               (__attribute__((address_space(3))) void*)(stage + n * 1024),
                                               16, off[k], k < kDmaK ? koff : qoff, 0, 0);
    }
  };

  // Fragment offsets: A = key rows 128wc + 32i + l32, B = query rows
  // 128wr + 32j + l32, piece 2ks + hi of the chunk; the swizzle depends on
  // l32 only, so block i (j) adds 32 rows = 4 KB.
  int aoff[4], boff[4];   // per k-step
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    aoff[ks] = (wc * kWaveC + l32) * kRowBytes + piece_slot(l32, 2 * ks + hi) * 16;
    boff[ks] = (kTileC + wr * kWaveR + l32) * kRowBytes + piece_slot(l32, 2 * ks + hi) * 16;
  }

  f32x16_t acc[2][4];
  struct Frags {
    bf16x8_t a[2], b[4];
  };
  auto read = [&](const uint8_t* stage, int ks, Frags& f) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 2; ++i) f.a[i] = as_bf16x8(*(const u32x4_t*)(stage + aoff[ks] + i * 32 * kRowBytes));
#pragma unroll
    for (int j = 0; j < 4; ++j) f.b[j] = as_bf16x8(*(const u32x4_t*)(stage + boff[ks] + j * 32 * kRowBytes));
  };
  auto mma = [&](const Frags& f) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma_32x32x16(f.a[i], f.b[j], acc[i][j]);
  };
  // the six LDS reads of a k-step are spread over its first six MFMAs
  auto interleave = []() __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < 6; ++u) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one DS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
  };

  TileItem it = decode_item(p, item_at(0));
  // the item after this one (or this one again after the last: harmless reloads)
  TileItem nx = nitems > 1 ? decode_item(p, item_at(1)) : it;
  uint32_t cur_off[kDmaPerWave], nxt_off[kDmaPerWave];
  row_offsets(it, cur_off);
  row_offsets(nx, nxt_off);
  int cur_h = it.h, cur_g = it.g, nxt_h = nx.h, nxt_g = nx.g;

  Frags f0, f1;
  // Chunk kc of the current item in stage `cur` (f0 holds its first k-step):
  // k-steps 0..2 with the next k-step's fragments read alongside; then wait
  // until this wave's reads of the stage and copies of chunk kc+1 are done and
  // synchronise; copy chunk kc+2 (of this item, or in its last two steps one
  // of the next item's first two chunks) into `cur`; read chunk kc+1's first
  // k-step from `oth` alongside k-step 3.
  auto chunk = [&](int kc, bool live, bool to_next, uint8_t* cur, const uint8_t* oth)
                   __attribute__((always_inline)) {
    const bool comp = live && kc < nk;
    if (comp) {
      read(cur, 1, f1);
      mma(f0);
      interleave();
      read(cur, 2, f0);
      mma(f1);
      interleave();
      read(cur, 3, f1);
      mma(f0);
      interleave();
    }
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    if (to_next) issue(nxt_h, nxt_g, nxt_off, kc + 2 - nkp, cur);
    else issue(cur_h, cur_g, cur_off, kc + 2, cur);
    read(oth, 0, f0);
    if (comp) {
      mma(f1);
      interleave();
    }
  };
  issue(cur_h, cur_g, cur_off, 0, st0);
  issue(cur_h, cur_g, cur_off, 1, st1);
  asm volatile("s_waitcnt vmcnt(8)" ::: "memory");   // chunk 0 landed
  __builtin_amdgcn_s_barrier();
  read(st0, 0, f0);
  for (int k = 0; k < nitems; ++k) {
    // a wave whose whole column range lies right of its last row is fully masked
    const bool live = !p.causal || (it.C0 + wc * kWaveC <= it.R0 + wr * kWaveR + kWaveR - 1);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x16_t{};
    for (int kc = 0; kc < nkp - 2; kc += 2) {
      chunk(kc, live, false, st0, st1);
      chunk(kc + 1, live, false, st1, st0);
    }
    chunk(nkp - 2, live, true, st0, st1);
    chunk(nkp - 1, live, true, st1, st0);
    if (live) {
      const int cw = it.C0 + wc * kWaveC;   // first column of the wave's two ranges
      const int Rw = it.R0 + wr * kWaveR;   // first row of the wave
      epilogue_range<BS, 0>(p, acc, it.h, Rw, cw, l32, hi);
    }
    it = nx;
    cur_h = nxt_h;
    cur_g = nxt_g;
#pragma unroll
    for (int q = 0; q < kDmaPerWave; ++q) cur_off[q] = nxt_off[q];
    if (k + 2 < nitems) {
      nx = decode_item(p, item_at(k + 2));
      row_offsets(nx, nxt_off);
      nxt_h = nx.h;
      nxt_g = nx.g;
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

struct FixupParams {
  const float* P;
  const float* M;
  const float* Z;
  float* scores;   // [hq][NB][NB]
  int hq, NB, Lr, nR32, nct, bs, causal;
};

// Softmax statistics of reshaped row R (index r within its 32-row group) from
// the 64-column range snapshots M, Z of that group: the row max and 1 / the
// row denominator.  Eight consecutive lanes share a row (sub = lane & 7) and
// combine their partial results with xor shuffles, so every caller computes
// bit-identical values; a whole aligned 8-lane group always calls together.
__device__ __forceinline__ void row_stats(const float* M, const float* Z, int r, int R, int Lr,
                                          int nct, int bs, int causal, int sub, float& m_out,
                                          float& invz_out) {
  int nct_r = nct;
  if (causal) {
    const int last = (R / bs + 1) * bs - 1;   // last row of R's query block
    nct_r = min(nct, last / kRangeCols + 1);
  }
  float m = -INFINITY;
  if (R < Lr) {
#pragma unroll 4
    for (int c = sub; c < nct_r; c += 8) m = fmaxf(m, M[c * 32 + r]);
  }
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
  float z = 0.f;
  if (R < Lr && m != -INFINITY)
#pragma unroll 4
    for (int c = sub; c < nct_r; c += 8) {
      const float mc = M[c * 32 + r];
      if (mc != -INFINITY) z += Z[c * 32 + r] * fast_exp2(mc - m);
    }
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) z += __shfl_xor(z, o);
  m_out = m;
  invz_out = (z > 0.f) ? 1.0f / z : 0.f;
}

// Block score of key block kb for the query block whose reshaped rows are
// r0 .. r0+BS-1 of the group: the rows' partial block sums rescaled to the
// rows' final softmax, summed in row order, divided by BS.
template <int BS>
__device__ __forceinline__ float block_score(const float* P, const float* M, const float* s_mfin,
                                             const float* s_invz, int kb, int r0) {
  const int c = (kb * BS) / kRangeCols;
  // the BS partial sums and range maxima of the block's rows: BS/4 16-byte
  // loads each (r0 is a multiple of BS >= 4, rows of 32 floats)
  f32x4_t pv[BS / 4], mv[BS / 4];
#pragma unroll
  for (int g = 0; g < BS / 4; ++g) {
    pv[g] = *(const f32x4_t*)(P + (size_t)kb * 32 + r0 + 4 * g);
    mv[g] = *(const f32x4_t*)(M + c * 32 + r0 + 4 * g);
  }
  float acc = 0.f;
#pragma unroll
  for (int u = 0; u < BS; ++u) {
    const int r = r0 + u;
    const float mc = mv[u / 4][u % 4];
    if (mc != -INFINITY) acc += pv[u / 4][u % 4] * fast_exp2(mc - s_mfin[r]) * s_invz[r];
  }
  return acc * (1.0f / (float)BS);
}

// One workgroup per (head, 32 reshaped rows); BS = B/S reshaped rows per
// query block.
template <int BS>
__global__ __launch_bounds__(256) void score_fixup(FixupParams p) {
  __shared__ float s_mfin[32];
  __shared__ float s_invz[32];
  const int h = blockIdx.x / p.nR32;
  const int rg = blockIdx.x % p.nR32;
  const int tid = threadIdx.x;
  const size_t rowbase = (size_t)h * p.nR32 + rg;
  const float* M = p.M + rowbase * p.nct * 32;
  const float* Z = p.Z + rowbase * p.nct * 32;
  const float* P = p.P + rowbase * p.NB * 32;

  // 1. per row: softmax max and denominator from the range snapshots
  {
    const int r = tid >> 3, sub = tid & 7;
    float m, invz;
    row_stats(M, Z, r, rg * 32 + r, p.Lr, p.nct, BS, p.causal, sub, m, invz);
    if (sub == 0) {
      s_mfin[r] = m;
      s_invz[r] = invz;
    }
  }
  __syncthreads();

  // 2. block scores for the 32/bs query blocks of this row group
  constexpr int nq = 32 / BS;
  const int qb0 = rg * nq;
#pragma unroll 2
  for (int it = tid; it < nq * p.NB; it += blockDim.x) {
    const int kb = it / nq, q = it % nq;
    const int qb = qb0 + q;
    if (qb >= p.NB) continue;
    const float out = (!p.causal || kb <= qb) ? block_score<BS>(P, M, s_mfin, s_invz, kb, q * BS) : 0.f;
    p.scores[((size_t)h * p.NB + qb) * p.NB + kb] = out;
  }
}

// Fused finishing + threshold selection: one workgroup per (head, 32
// reshaped rows) computes the block scores of the group's 32/bs query blocks
// exactly as score_fixup does -- same helpers, same order, so the same bits
// -- keeps them in LDS, and each wave ranks and cuts whole rows
// (rank_and_cut, as xattn_select).  The [hq][NB][NB] score matrix never
// reaches memory.
struct FusedParams {
  const float* P;
  const float* M;
  const float* Z;
  uint64_t* mask;
  int32_t* idx;
  int32_t* counts;
  int NB, Lr, nR32, nct, bs, causal, nwords;
  TauArray tau;
};

template <int EPL, int BS>
__global__ __launch_bounds__(256) void score_select_fused(FusedParams p) {
  extern __shared__ float s_sc[];   // [32 / BS][NB] block scores of the group's query blocks
  __shared__ float s_mfin[32];
  __shared__ float s_invz[32];
  const int h = blockIdx.x / p.nR32;
  const int rg = blockIdx.x % p.nR32;
  const int tid = threadIdx.x;
  const size_t rowbase = (size_t)h * p.nR32 + rg;
  const float* M = p.M + rowbase * p.nct * 32;
  const float* Z = p.Z + rowbase * p.nct * 32;
  const float* P = p.P + rowbase * p.NB * 32;
  {
    const int r = tid >> 3, sub = tid & 7;
    float m, invz;
    row_stats(M, Z, r, rg * 32 + r, p.Lr, p.nct, BS, p.causal, sub, m, invz);
    if (sub == 0) {
      s_mfin[r] = m;
      s_invz[r] = invz;
    }
  }
  __syncthreads();
  constexpr int nq = 32 / BS;
  const int qb0 = rg * nq;
#pragma unroll 2
  for (int it = tid; it < nq * p.NB; it += blockDim.x) {
    const int kb = it / nq, q = it % nq;
    const int qb = qb0 + q;
    if (qb >= p.NB) continue;
    s_sc[q * p.NB + kb] =
        (!p.causal || kb <= qb) ? block_score<BS>(P, M, s_mfin, s_invz, kb, q * BS) : 0.f;
  }
  __syncthreads();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const CutSpec cut{kThreshold, 0, 0.f, p.tau.v[h]};
  for (int q = wave; q < nq; q += 4) {
    const int qb = qb0 + q;
    if (qb >= p.NB) break;
    const size_t row = (size_t)h * p.NB + qb;
    const float* srow = s_sc + q * p.NB;
    rank_and_cut<EPL>([&](int i) { return srow[i]; }, p.causal ? qb + 1 : p.NB, p.NB, p.nwords,
                      cut, p.mask + row * p.nwords, p.idx + row * p.NB, p.counts + row);
  }
}

template <int D, int BS>
hipError_t launch_gemm(const GemmParams& gp, hipStream_t st) {
  const dim3 grid(gp.wg_per_xcd * kNumXcd), block(kWaves * 64);
  if (gp.phase.custom) hipLaunchKernelGGL((score_gemm<D, BS, true>), grid, block, 0, st, gp);
  else hipLaunchKernelGGL((score_gemm<D, BS, false>), grid, block, 0, st, gp);
  return hipGetLastError();
}

template <int D>
hipError_t launch_gemm_bs(const GemmParams& gp, int bs, hipStream_t st) {
  switch (bs) {
    case 4: return launch_gemm<D, 4>(gp, st);
    case 8: return launch_gemm<D, 8>(gp, st);
    case 16: return launch_gemm<D, 16>(gp, st);
    case 32: return launch_gemm<D, 32>(gp, st);
  }
  return hipErrorInvalidValue;
}

struct WsLayout {
  size_t p_elems, m_elems;
  int Lr, NB, nR32, nct;
};

WsLayout ws_layout(const Shape& s, int S, int B) {
  WsLayout w;
  w.Lr = s.L / S;
  w.NB = s.L / B;
  w.nR32 = (w.Lr + 31) / 32;
  w.nct = (w.Lr + kRangeCols - 1) / kRangeCols;
  w.p_elems = (size_t)s.hq * w.nR32 * w.NB * 32;
  w.m_elems = (size_t)s.hq * w.nR32 * w.nct * 32;
  return w;
}

// Fixed device scratch of the allocation-free scoring entry point: the
// scoring GEMM's partial block sums and range snapshots for shapes whose
// workspace fits.  Each GPU the library runs on holds its own copy until the
// process ends; every call on a GPU shares it.  In host code `scratch` names
// a host-side stand-in, not device memory: its device address comes from
// hipGetSymbolAddress (score_scratch_ptr), per device.
static __device__ __align__(256) unsigned char scratch[kScoreScratchBytes];

}  // namespace

// Compute units per XCD of the current device (the persistent kernels run one
// workgroup per CU).  Cached per device; several host threads may fill an
// entry at once, all with the same value, so relaxed atomics suffice.
int cus_per_xcd() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 32;
  int v = cached[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < kNumXcd)
      n = 256;
    v = n / kNumXcd;
    cached[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

hipError_t score_scratch_ptr(void** out) {
  static std::atomic<void*> cached[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  void* ptr = cached[dev].load(std::memory_order_acquire);
  if (ptr == nullptr) {
    // once per device, with that device current; concurrent first calls all
    // store the same address
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    cached[dev].store(ptr, std::memory_order_release);
  }
  *out = ptr;
  return hipSuccess;
}

size_t score_workspace_bytes(const Shape& s, int S, int B) {
  if (!s.bf16) return 0;
  const WsLayout w = ws_layout(s, S, B);
  return (w.p_elems + 2 * w.m_elems) * sizeof(float);
}

namespace {

// The scoring GEMM into the workspace partials (P, M, Z).
hipError_t run_score_gemm(const Shape& s, const void* Q, const void* K, int S, int B,
                          const PhaseMap& phase, void* ws, const WsLayout& wl, hipStream_t st) {
  float* P = (float*)ws;
  float* M = P + wl.p_elems;
  float* Z = M + wl.m_elems;
  GemmParams gp;
  gp.Q = (const uint16_t*)Q;
  gp.K = (const uint16_t*)K;
  gp.P = P;
  gp.M = M;
  gp.Z = Z;
  gp.L = s.L;
  gp.S = S;
  gp.group = s.hq / s.hkv;
  gp.NB = wl.NB;
  gp.Lr = wl.Lr;
  gp.nR32 = wl.nR32;
  gp.nct = wl.nct;
  gp.causal = s.causal;
  gp.ntr = (wl.Lr + kTileR - 1) / kTileR;
  gp.ntc = (wl.Lr + kTileC - 1) / kTileC;
  gp.tiles_per_head = s.causal ? gp.ntr * (gp.ntr + 1) / 2 : gp.ntr * gp.ntc;
  gp.nwork = gp.tiles_per_head * s.hq;
  const int per_range = (gp.nwork + kNumXcd - 1) / kNumXcd;
  gp.deal = gp.tiles_per_head >= 512 ? 8 * gp.group : per_range;
  {
    const int full = gp.nwork / gp.deal, rem = gp.nwork % gp.deal;
    int n0 = full > 0 ? ((full - 1) / kNumXcd + 1) * gp.deal : 0;   // XCD 0 holds the most
    if (rem && full % kNumXcd == 0) n0 += rem;
    gp.per_xcd = n0;
  }
  gp.wg_per_xcd = std::min(gp.per_xcd, cus_per_xcd());
  gp.scale_log2 = (float)(1.4426950408889634 / __builtin_sqrt((double)s.d * S));
  gp.phase = phase;
  const int bs = B / S;
  return (s.d == 128) ? launch_gemm_bs<128>(gp, bs, st) : launch_gemm_bs<64>(gp, bs, st);
}

template <int EPL>
hipError_t launch_fused(const FusedParams& fp, int groups, hipStream_t st) {
  const dim3 grid(groups), block(256);
  const size_t lds = (size_t)(32 / fp.bs) * fp.NB * sizeof(float);   // <= 8 x 4096 floats
  switch (fp.bs) {
    case 4: hipLaunchKernelGGL((score_select_fused<EPL, 4>), grid, block, lds, st, fp); break;
    case 8: hipLaunchKernelGGL((score_select_fused<EPL, 8>), grid, block, lds, st, fp); break;
    case 16: hipLaunchKernelGGL((score_select_fused<EPL, 16>), grid, block, lds, st, fp); break;
    case 32: hipLaunchKernelGGL((score_select_fused<EPL, 32>), grid, block, lds, st, fp); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_score_bf16(const Shape& s, const void* Q, const void* K, int S, int B,
                             const PhaseMap& phase, float* scores, void* ws, hipStream_t st) {
  const WsLayout wl = ws_layout(s, S, B);
  hipError_t e = run_score_gemm(s, Q, K, S, B, phase, ws, wl, st);
  if (e != hipSuccess) return e;
  FixupParams fp;
  fp.P = (float*)ws;
  fp.M = fp.P + wl.p_elems;
  fp.Z = fp.M + wl.m_elems;
  fp.scores = scores;
  fp.hq = s.hq;
  fp.NB = wl.NB;
  fp.Lr = wl.Lr;
  fp.nR32 = wl.nR32;
  fp.nct = wl.nct;
  fp.bs = B / S;
  fp.causal = s.causal;
  const dim3 grid(s.hq * wl.nR32), block(256);
  switch (fp.bs) {
    case 4: hipLaunchKernelGGL(score_fixup<4>, grid, block, 0, st, fp); break;
    case 8: hipLaunchKernelGGL(score_fixup<8>, grid, block, 0, st, fp); break;
    case 16: hipLaunchKernelGGL(score_fixup<16>, grid, block, 0, st, fp); break;
    case 32: hipLaunchKernelGGL(score_fixup<32>, grid, block, 0, st, fp); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_score_select_bf16(const Shape& s, const void* Q, const void* K, int S, int B,
                                    const TauArray& tau, uint64_t* mask, int32_t* idx,
                                    int32_t* counts, void* ws, hipStream_t st) {
  const WsLayout wl = ws_layout(s, S, B);
  PhaseMap antidiagonal{};
  hipError_t e = run_score_gemm(s, Q, K, S, B, antidiagonal, ws, wl, st);
  if (e != hipSuccess) return e;
  FusedParams fp;
  fp.P = (float*)ws;
  fp.M = fp.P + wl.p_elems;
  fp.Z = fp.M + wl.m_elems;
  fp.mask = mask;
  fp.idx = idx;
  fp.counts = counts;
  fp.NB = wl.NB;
  fp.Lr = wl.Lr;
  fp.nR32 = wl.nR32;
  fp.nct = wl.nct;
  fp.bs = B / S;
  fp.causal = s.causal;
  fp.nwords = (wl.NB + 63) / 64;
  fp.tau = tau;
  const int groups = s.hq * wl.nR32;
  if (wl.NB <= 256) return launch_fused<4>(fp, groups, st);
  if (wl.NB <= 1024) return launch_fused<16>(fp, groups, st);
  return launch_fused<64>(fp, groups, st);
}

}  // namespace xattn
