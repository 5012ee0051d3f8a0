// Block-sparse and dense attention for bf16 on gfx950 ("XAttention: Block
// Sparse Attention with Antidiagonal Scoring", papercache.org summary,
// section 1 step 3: attention computed on the selected blocks only).
//
// One workgroup per (query head, pair of neighbouring query blocks of B rows
// each); each of its 2B/32 waves owns 32 query rows of one of the two
// blocks.  The key/value blocks to visit -- the union of the two blocks'
// selected sets in sparse mode, all causal-visible ones in dense mode --
// stream through LDS one block (B keys) per tile, double buffered: while a tile is
// being used, the next one is copied global -> LDS by direct-to-LDS loads, so
// the copy never passes through registers.  Each tile is copied
// once for both blocks; a wave skips the tiles its own block does not use
// (neighbouring blocks select largely the same keys, so the copy traffic per
// query row falls by about 40 % against one block per workgroup).  K and V
// tiles are stored row-major with an XOR swizzle of their 16-byte chunks
// (conflict-free reads for both access patterns below).
//
// Per tile a wave computes S^T = K Q^T with 32x32x16 bf16 MFMAs (each lane
// then owns one query row), applies the causal mask, an online softmax in the
// exp2 domain (the O rescale is skipped when no row's max moved), rounds P to
// bf16, and accumulates O^T += V^T P^T.  The V^T operand comes from the
// row-major V tile through LDS transpose reads (ds_read_b64_tr_b16).  Query
// head h reads key/value head h / (hq / hkv).
#include <atomic>

#include "common.h"
#include "launch.h"

namespace xattn {
namespace {


typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

struct FlashParams {
  const uint16_t* Q;
  const uint16_t* K;
  const uint16_t* V;
  uint16_t* O;
  const int32_t* idx;      // nullptr: dense
  const int32_t* counts;
  int L, hq, group, NB, causal;
  int nwork, grid, interleave, chunk_pairs;
  float scale_log2;        // log2(e) / sqrt(d)
  unsigned int* queue;     // persistent sparse mode: this launch's per-XCD item counters
};

// XOR swizzle of the 16-byte chunks of a tile row: chunk c of row r sits at
// c ^ swz(r).  gfx950's LDS behaves as 64 four-byte banks (256 bytes per bank
// line), so the bank group of a chunk is its byte offset / 16 mod 16.  For
// d = 128 (one row per bank line) swz(r) = 4(r mod 4) + (r/4 mod 4) makes both
// access patterns conflict-free: K-operand reads (consecutive rows, one chunk
// each) and transposed V reads (4 consecutive rows x 4 neighbouring chunks per
// 32 lanes).  For d = 64 two rows share a bank line and swz(r) =
// 4(r/2 mod 2) + 2(r/4 mod 2) keeps the transposed reads conflict-free.
template <int D>
__device__ __forceinline__ int swz(int row) {
  if constexpr (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
  return (((row >> 1) & 1) << 2) | (((row >> 2) & 1) << 1);
}

// Byte offset of element (row, col) of a swizzled [64][D] bf16 tile.
template <int D>
__device__ __forceinline__ int tile_off(int row, int col) {
  return row * (D * 2) + (((col >> 3) ^ swz<D>(row)) << 4) + ((col & 7) << 1);
}

// Keys per LDS tile: one whole 128-key block per step for B = 128 (half the
// steps, barriers and per-step softmax overhead of 64-key tiles), 64 for B = 64.
template <int BQ>
constexpr int kTileKeys = BQ >= 128 ? 128 : 64;

// Query-block pairs per scheduling chunk (times the heads of a KV group).
// The work-groups of one chunk share their key/value tiles in the XCD's L2,
// so larger chunks fetch fewer bytes beyond it; small chunks keep the work
// per XCD even.  With the alternating deal below, from 512 pairs per head on
// eight pairs fetch 17 % fewer bytes than two (131K tokens: 107 against
// 129 GB per sparse launch, 18.5 against 36 GB dense) in the same time; at 128
// pairs per head eight are 3.5 % slower than two, and sixteen are slower at
// every size measured.
inline int pairs_per_chunk(int npairs) { return npairs >= 512 ? 8 : 2; }

// Copy one KT x D tile (rows key0 .. key0+KT-1 of one KV head's K or V) into
// LDS by direct-to-LDS loads.  Each instruction of a wave fills 1 KB of LDS in
// lane order; lane l fetches the global chunk that the swizzled layout places
// at its position.  The loads go through a buffer resource over the head
// (scalar tile offset, per-lane 32-bit offset fixed for the kernel): the
// compiler counts the global-segment form of these loads as a possible LDS
// access that completes out of order, so after it every wait for a fragment
// read would drain all outstanding LDS reads; the buffer form keeps those
// waits partial.
template <int D, int KT, int NWAVES>
__device__ __forceinline__ void load_tile(__amdgpu_buffer_rsrc_t src, int key0, uint8_t* lds, int wave,
                                          int lane) {
  constexpr int kChunksPerRow = D / 8;
  constexpr int kRowsPerInst = 64 / kChunksPerRow;
  constexpr int kInsts = KT / kRowsPerInst;    // 1 KB instructions per tile
  static_assert(kInsts % NWAVES == 0, "tile instructions must split evenly over waves");
  const uint32_t tile = (uint32_t)key0 * (D * 2);
#pragma unroll
  for (int k = 0; k < kInsts / NWAVES; ++k) {
    const int n = k * NWAVES + wave;               // wave is uniform (scalar)
    const int p = n * 64 + lane;                   // 16-byte chunk position in the tile
    const int row = p / kChunksPerRow;
    const int c = (p % kChunksPerRow) ^ swz<D>(row);
    const uint32_t off = (uint32_t)(row * D * 2 + c * 16);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (__attribute__((address_space(3))) void*)(lds + n * 1024),
                                             16, off, tile, 0, 0);
  }
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// max(x[l], x[l ^ 32]) in every lane l, without the LDS crossbar:
// v_permlane32_swap exchanges the upper half of its first operand with the
// lower half of its second, so two copies of x end up holding x[l] and
// x[l ^ 32] between them.  Written as a VALU asm statement with both
// registers read-write: this hipcc gives the builtin's second result the
// first result's register.  The s_nop covers the wait after the VALU write of
// the operands.
__device__ __forceinline__ float max_with_other_half(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  return fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}

__device__ __forceinline__ uint32_t cvt2_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// One wave's share of a key/value tile: kKT keys from key0 (rows of sK, sV)
// against its 32 query rows (this lane: row qrow; the wave's first row is
// qwave0), folded into the running output o, row max m and denominator
// share lsum.
template <int D, int kKT>
__device__ __forceinline__ void attend_tile(float scale_log2, int causal, const uint8_t* sK, const uint8_t* sV,
                                            const int (&koff)[D / 16], const int (&voff)[D / 32][2],
                                            const bf16x8_t (&qf)[D / 16], f32x16_t (&o)[D / 32],
                                            float& m, float& lsum, int key0, int qrow, int qwave0,
                                            int hi) {
  // S^T (kKT keys x 32 queries) as kNS 32x32 tiles.  K fragments are read
  // kAhead k-steps before their MFMAs so LDS latency overlaps the matrix
  // work instead of stalling each MFMA.
  constexpr int kSteps = D / 16;
  constexpr int kNS = kKT / 32;                // 32-key sub-tiles
  constexpr int kNU = kKT / 16;                // 16-key chunks of P
  constexpr int kAhead = kNS >= 4 ? 2 : 3;
  f32x16_t s[kNS];
#pragma unroll
  for (int i = 0; i < kNS; ++i) s[i] = f32x16_t{};
  bf16x8_t kfr[kAhead + 1][kNS];
#pragma unroll
  for (int t = 0; t < kAhead; ++t)
#pragma unroll
    for (int i = 0; i < kNS; ++i)
      kfr[t][i] = as_bf16x8(*(const u32x4_t*)(sK + koff[t] + i * 32 * D * 2));
#pragma unroll
  for (int t = 0; t < kSteps; ++t) {
    if (t + kAhead < kSteps) {
#pragma unroll
      for (int i = 0; i < kNS; ++i)
        kfr[(t + kAhead) % (kAhead + 1)][i] =
            as_bf16x8(*(const u32x4_t*)(sK + koff[t + kAhead] + i * 32 * D * 2));
    }
#pragma unroll
    for (int i = 0; i < kNS; ++i) s[i] = mfma_32x32x16(kfr[t % (kAhead + 1)][i], qf[t], s[i]);
  }
  // Keep the reads kAhead steps ahead: the scheduler otherwise sinks them
  // next to their MFMAs.  (mask 0x100: DS read, 0x008: MFMA)
  __builtin_amdgcn_sched_group_barrier(0x100, kNS * kAhead, 0);
#pragma unroll
  for (int t = 0; t < kSteps - kAhead; ++t) {
    __builtin_amdgcn_sched_group_barrier(0x008, kNS, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, kNS, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, kNS * kAhead, 0);
  __builtin_amdgcn_sched_barrier(0);
  // V^T fragments (A operand of O^T += V^T P^T) of 16-key chunk u and
  // output column block dt, by transposed LDS reads; chunk 0 is read now
  // so the reads land during the softmax.
  auto read_v = [&](int u, int dt) -> bf16x8_t {
    const uint8_t* vp = sV + 16 * u * D * 2;
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(vp + voff[dt][0]));
    const v4i16 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(vp + voff[dt][1]));
    return as_bf16x8(u32x4_t{__builtin_bit_cast(u32x2_t, lo)[0], __builtin_bit_cast(u32x2_t, lo)[1],
                             __builtin_bit_cast(u32x2_t, hi4)[0], __builtin_bit_cast(u32x2_t, hi4)[1]});
  };
  bf16x8_t vf[2][D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) vf[0][dt] = read_v(0, dt);
  __builtin_amdgcn_sched_barrier(0);
  if (causal && key0 + kKT - 1 > qwave0) {   // tile crosses this wave's diagonal
    // key = key0 + 4 hi + (32 i + 8 (v / 4) + v % 4) is masked when it
    // exceeds qrow: one per-lane bound against compile-time offsets (no
    // per-element key constants held in registers across the loop)
    const int bound = qrow - key0 - 4 * hi;
#pragma unroll
    for (int i = 0; i < kNS; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (32 * i + 8 * (v >> 2) + (v & 3) > bound) s[i][v] = -INFINITY;
  }
  float mloc = -INFINITY;
#pragma unroll
  for (int i = 0; i < kNS; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) mloc = fmaxf(mloc, s[i][v]);
  mloc = max_with_other_half(mloc) * scale_log2;
  // The reference max m of a row only moves when this tile's max exceeds it
  // by more than kSlack (log2 units), so P stays <= 2^kSlack and the O /
  // denominator rescale (a wave-uniform branch) is rare.  The result is
  // unchanged: numerator and denominator share the reference.  A row with
  // nothing visible yet keeps m = -inf and gets p = 0.
  constexpr float kSlack = 8.0f;
  if (__ballot(mloc > m + kSlack)) {
    const float mnew = (mloc > m + kSlack) ? mloc : m;
    const float alpha = fast_exp2(m - mnew);   // m == -inf gives 0; unchanged rows 1
    lsum *= alpha;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) o[dt] *= alpha;
    m = mnew;
  }
  const float mref = (m == -INFINITY) ? 0.f : m;
  // P in bf16 in chunks of 16 keys; the denominator sums the same
  // rounded values (packed dot2, in chunk order).  The MFMAs of chunk u
  // are interleaved with the exponentials and V reads of chunk u + 1
  // (fenced, so the vector and matrix work of one wave overlap).
  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
  float rs0 = 0.f, rs1 = 0.f;
  auto p_pair = [&](int u, int e) -> uint32_t {
    const int i = u >> 1, v0 = (u & 1) * 8;
    const float p0 = fast_exp2(fmaf(s[i][v0 + 2 * e], scale_log2, -mref));
    const float p1 = fast_exp2(fmaf(s[i][v0 + 2 * e + 1], scale_log2, -mref));
    const uint32_t pk = cvt2_bf16(p0, p1);
    if (e & 1) rs1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk), ones, rs1, false);
    else rs0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk), ones, rs0, false);
    return pk;
  };
  constexpr int kDt = D / 32;            // output column blocks
  constexpr int kPairsPerDt = 4 / kDt;   // P pairs of the next chunk per MFMA
  uint32_t pk[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) pk[e] = p_pair(0, e);
  bf16x8_t pcur = as_bf16x8(u32x4_t{pk[0], pk[1], pk[2], pk[3]});
#pragma unroll
  for (int u = 0; u < kNU; ++u) {
#pragma unroll
    for (int dt = 0; dt < kDt; ++dt) {
      o[dt] = mfma_32x32x16(vf[u & 1][dt], pcur, o[dt]);
      if (u < kNU - 1) {
        vf[(u + 1) & 1][dt] = read_v(u + 1, dt);
#pragma unroll
        for (int e = dt * kPairsPerDt; e < (dt + 1) * kPairsPerDt; ++e) pk[e] = p_pair(u + 1, e);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (u < kNU - 1) pcur = as_bf16x8(u32x4_t{pk[0], pk[1], pk[2], pk[3]});
  }
  lsum += rs0 + rs1;
}

// The merged key-block list of a work item from the two blocks' bitmaps
// (s_bits[0 .. nw32) for the first block, s_bits[nw32 .. 2 nw32) for the
// second): entry kb | flagA << 30 | flagB << 31 in ascending kb, written to
// s_list with the per-word offsets in s_off; the entry count is s_off[nw32]
// after the final barrier.  With `clear` the bitmap words are zeroed as they
// are consumed, ready for the next item.  All threads call it (barriers).
template <int kThreads>
__device__ __forceinline__ void finish_list(uint32_t* s_bits, int32_t* s_off, int32_t* s_list, int nw32,
                                            int tid, int wave, int lane, bool clear) {
  // list offsets of the bitmap words: one wave, a few words per lane and a
  // wave-wide inclusive scan of the per-lane counts
  if (wave == 0) {
    const int per = (nw32 + 63) / 64;
    const int w0 = lane * per;
    int c = 0;
    for (int k = 0; k < per; ++k) {
      const int w = w0 + k;
      if (w < nw32) c += __builtin_popcount(s_bits[w] | s_bits[nw32 + w]);
    }
    int incl = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o);
      if (lane >= o) incl += t;
    }
    int acc = incl - c;
    for (int k = 0; k < per; ++k) {
      const int w = w0 + k;
      if (w < nw32) {
        s_off[w] = acc;
        acc += __builtin_popcount(s_bits[w] | s_bits[nw32 + w]);
      }
    }
    if (lane == 63) s_off[nw32] = incl;
  }
  __syncthreads();
  for (int w = tid; w < nw32; w += kThreads) {
    const uint32_t a = s_bits[w], bb = s_bits[nw32 + w];
    if (clear) {
      s_bits[w] = 0u;
      s_bits[nw32 + w] = 0u;
    }
    uint32_t u = a | bb;
    int o = s_off[w];
    while (u) {
      const int bit = __builtin_ctz(u);
      s_list[o++] = (int32_t)((uint32_t)(32 * w + bit) | (((a >> bit) & 1u) << 30) | (((bb >> bit) & 1u) << 31));
      u &= u - 1;
    }
  }
  __syncthreads();
}

template <int D, int BQ>
__global__ __launch_bounds__(BQ * 4, 1) void flash_bf16_kernel(FlashParams p) {
  constexpr int kBlockWaves = BQ / 32;          // waves per query block
  constexpr int kWaves = 2 * kBlockWaves;        // a workgroup covers two query blocks
  constexpr int kThreads = kWaves * 64;
  constexpr int kKT = kTileKeys<BQ>;            // keys per LDS tile
  constexpr int kTilesPerBlock = BQ / kKT;
  constexpr int kTileBytes = kKT * D * 2;
  // Two K/V buffers as distinct objects: with the loop unrolled by two every
  // access names its buffer at compile time, so the compiler can see that LDS
  // reads of one buffer do not wait on the direct-to-LDS copy into the other.
  __shared__ __attribute__((aligned(1024))) uint8_t sK0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t sV0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t sK1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t sV1[kTileBytes];


  // Work order.  A work item is a pair of neighbouring query blocks (2i,
  // 2i+1) of one head.  Items of one KV group are (pair descending, head),
  // cut into chunks of p.chunk_pairs pairs x all heads of the group.
  // Chunks are dealt to the 8 XCDs in rounds of eight, the XCD order
  // reversed every other round, and every XCD runs through the groups in
  // the same order, so (a) all XCDs work on the same KV group at a time --
  // its K/V stays resident in the memory-side cache -- (b) the work-groups
  // on one XCD run all heads of the group on the same query blocks, and (c)
  // the XCDs get equal work: causal pairs shrink along the order, and a
  // plain round-robin deal would give XCD 0 the longest pair of every
  // round.  When the counts do not divide evenly, each XCD takes a
  // contiguous range instead (one KV group per XCD).
  const int npairs = (p.NB + 1) / 2;
  const int per_group = npairs * p.group;
  int g, rem;
  if (p.interleave) {
    const int bid = blockIdx.x;
    const int xcd = bid % kNumXcd, k = bid / kNumXcd;
    const int per_xcd = per_group / kNumXcd;     // items of one group on one XCD
    const int chunk = p.chunk_pairs * p.group;   // items per chunk
    g = k / per_xcd;
    const int kk = k % per_xcd;
    const int r = kk / chunk;                    // round
    rem = (r * kNumXcd + ((r & 1) ? kNumXcd - 1 - xcd : xcd)) * chunk + kk % chunk;
    if (g >= p.hq / p.group) return;
  } else {
    const int w = xcd_swizzle(blockIdx.x, p.grid);
    if (w >= p.nwork) return;
    g = w / per_group;
    rem = w % per_group;
  }
  const int pair = npairs - 1 - rem / p.group;
  const int h = g * p.group + rem % p.group;
  // Waves 0 .. kBlockWaves-1 take query block qbA, the others qbB (== NB when
  // NB is odd and this is the last pair: those waves only help copy).  Wave w
  // runs on SIMD w % 4, so each SIMD holds one wave of each block.
  const int qbA = 2 * pair, qbB = 2 * pair + 1;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int half = wave / kBlockWaves;           // 0: block A, 1: block B
  const int qb = qbA + half;
  const bool rows_valid = qb < p.NB;
  const int wq = wave % kBlockWaves;
  const int qrow = qb * BQ + wq * 32 + l32;      // this lane's query token
  const int qwave0 = qb * BQ + wq * 32;

  // this KV head's K and V as buffer resources (L * D * 2 < 2^31 bytes, checked by the caller)
  const __amdgpu_buffer_rsrc_t Kg = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.K + (size_t)g * p.L * D), (short)0, p.L * D * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t Vg = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.V + (size_t)g * p.L * D), (short)0, p.L * D * 2, 0x00020000);

  // The key blocks the workgroup visits: the union of the two blocks' sets,
  // in ascending order, each with a flag per block.  Sparse mode builds it in
  // LDS from the two lists (as bitmaps: invalid entries dropped, a repeated
  // entry kept once); dense mode visits every causal-visible block.
  //
  // A wave's vector loads complete in order, so the two blocks' counts and
  // index rows are requested together and before the query fragments: the
  // bitmaps then wait for one memory round trip, not for the query loads
  // issued ahead of them.  Rows of up to kRowAhead * threads entries are read
  // whole (entries past the count are read and ignored); longer rows are read
  // in a loop over their counted entries.
  extern __shared__ int32_t s_dyn[];
  const int nw32 = (p.NB + 31) / 32;
  int32_t* s_list = s_dyn;                                  // [NB]: kb | flagA << 30 | flagB << 31
  uint32_t* s_bits = (uint32_t*)(s_dyn + p.NB);             // [2][nw32]
  int32_t* s_off = s_dyn + p.NB + 2 * nw32;                 // [nw32 + 1]
  const bool sparse = p.idx != nullptr;
  constexpr int kRowAhead = 4;
  const bool whole_rows = p.NB <= kRowAhead * kThreads;
  const bool hasB = qbB < p.NB;
  const int32_t* rowA = p.idx + ((size_t)h * p.NB + qbA) * p.NB;
  const int32_t* rowB = rowA + p.NB;
  int cntA = 0, cntB = 0;
  int ea[kRowAhead], eb[kRowAhead];
  if (sparse) {
    for (int i = tid; i < 2 * nw32; i += kThreads) s_bits[i] = 0u;
    cntA = p.counts[(size_t)h * p.NB + qbA];
    cntB = hasB ? p.counts[(size_t)h * p.NB + qbB] : 0;
    if (whole_rows) {
#pragma unroll
      for (int m = 0; m < kRowAhead; ++m) {
        const int j = tid + m * kThreads;
        ea[m] = j < p.NB ? rowA[j] : -1;
        eb[m] = (hasB && j < p.NB) ? rowB[j] : -1;
      }
    }
  }
  asm volatile("" ::: "memory");   // the query loads stay behind the index loads

  // query fragments (B operand of S^T = K Q^T): lane holds Q[qrow][16t + 8hi .. +8]
  bf16x8_t qf[D / 16];
  {
    const uint16_t* qp = p.Q + ((size_t)h * p.L + (rows_valid ? qrow : qrow - BQ)) * D + hi * 8;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) qf[t] = as_bf16x8(*(const u32x4_t*)(qp + 16 * t));
  }

  int nkb;
  if (sparse) {
    cntA = cntA < 0 ? 0 : (cntA > p.NB ? p.NB : cntA);
    cntB = cntB < 0 ? 0 : (cntB > p.NB ? p.NB : cntB);
    __syncthreads();   // bitmaps cleared
    auto mark = [&](int kb, int b, int qbb) __attribute__((always_inline)) {
      if (kb < 0 || kb >= p.NB || (p.causal && kb > qbb)) return;
      atomicOr(&s_bits[b * nw32 + (kb >> 5)], 1u << (kb & 31));
    };
    if (whole_rows) {
#pragma unroll
      for (int m = 0; m < kRowAhead; ++m) {
        const int j = tid + m * kThreads;
        if (j < cntA) mark(ea[m], 0, qbA);
        if (j < cntB) mark(eb[m], 1, qbB);
      }
    } else {
      for (int j = tid; j < cntA; j += kThreads) mark(rowA[j], 0, qbA);
      for (int j = tid; j < cntB; j += kThreads) mark(rowB[j], 1, qbB);
    }
    __syncthreads();
    finish_list<kThreads>(s_bits, s_off, s_list, nw32, tid, wave, lane, false);
    nkb = s_off[nw32];
  } else {
    nkb = p.causal ? min(qbB, p.NB - 1) + 1 : p.NB;
  }
  const int ntiles = nkb * kTilesPerBlock;
  // first key of tile n and whether this wave's query block uses it
  auto tile_info = [&](int n, bool& mine) -> int {
    const int j = n / kTilesPerBlock;
    int kb;
    bool fa, fb;
    if (sparse) {
      const uint32_t e = (uint32_t)__builtin_amdgcn_readfirstlane(s_list[j]);
      kb = (int)(e & 0x3FFFFFFFu);
      fa = (e >> 30) & 1u;
      fb = e >> 31;
    } else {
      kb = j;
      fa = !p.causal || kb <= qbA;
      fb = qbB < p.NB && (!p.causal || kb <= qbB);
    }
    mine = half ? fb : fa;
    return kb * BQ + (n % kTilesPerBlock) * kKT;
  };

  f32x16_t o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) o[i] = f32x16_t{};
  float m = -INFINITY;   // running max (log2 units) of this lane's query row
  float lsum = 0.f;      // this lane's share of the running denominator

  // Per-lane LDS byte offsets.  The swizzle repeats every 16 rows.  K operand:
  // row 32i + l32, chunk 2t + hi -- fixed per lane and t (the i = 1 half is
  // 32 rows further).  V operand (transposed reads): row 16u + 8r + 4hi + i16/4
  // and column 32dt + 16(g16 & 1) + 4(i16 & 3) -- fixed per lane, dt and r;
  // u adds whole 16-row groups.
  int koff[D / 16], voff[D / 32][2];
  {
    const int g16 = lane >> 4, i16 = lane & 15;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) koff[t] = tile_off<D>(l32, 16 * t + 8 * hi);
    const int vrow = 4 * hi + (i16 >> 2);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 2; ++r)
        voff[dt][r] = tile_off<D>(vrow + 8 * r, 32 * dt + 16 * (g16 & 1) + 4 * (i16 & 3));
  }

  bool mine = false;
  int key0 = ntiles > 0 ? tile_info(0, mine) : -1;
  if (key0 >= 0) {
    load_tile<D, kKT, kWaves>(Kg, key0, sK0, wave, lane);
    load_tile<D, kKT, kWaves>(Vg, key0, sV0, wave, lane);
  }
  wait_vmem();
  __syncthreads();

  // One tile: start copying tile n+1 into the other buffer, use tile n, then
  // wait for the copy and synchronise.
  auto step = [&](int n, const uint8_t* sK, const uint8_t* sV, uint8_t* nK,
                  uint8_t* nV) __attribute__((always_inline)) {
    bool mine_next = false;
    const int key0_next = (n + 1 < ntiles) ? tile_info(n + 1, mine_next) : -1;
    if (key0_next >= 0) {
      load_tile<D, kKT, kWaves>(Kg, key0_next, nK, wave, lane);
      load_tile<D, kKT, kWaves>(Vg, key0_next, nV, wave, lane);
    }
    if (key0 >= 0 && mine && !(p.causal && key0 > qwave0 + 31)) {
      attend_tile<D, kKT>(p.scale_log2, p.causal, sK, sV, koff, voff, qf, o, m, lsum, key0, qrow, qwave0, hi);
    }
    key0 = key0_next;
    mine = mine_next;
    wait_vmem();
    __syncthreads();
  };
  for (int n = 0; n < ntiles; n += 2) {
    step(n, sK0, sV0, sK1, sV1);
    if (n + 1 < ntiles) step(n + 1, sK1, sV1, sK0, sV0);
  }

  // normalise and store: lane holds O[qrow][32 dt + 8 gg + 4 hi + r]
  if (!rows_valid) return;
  const float ltot = lsum + __shfl_xor(lsum, 32);
  const float inv = ltot > 0.f ? 1.0f / ltot : 0.f;
  uint16_t* op = p.O + ((size_t)h * p.L + qrow) * D;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) {
      const int col = dt * 32 + 8 * gg + 4 * hi;
      u32x2_t v;
      v[0] = cvt2_bf16(o[dt][4 * gg] * inv, o[dt][4 * gg + 1] * inv);
      v[1] = cvt2_bf16(o[dt][4 * gg + 2] * inv, o[dt][4 * gg + 3] * inv);
      *(u32x2_t*)(op + col) = v;
    }
}

// Work queues of the persistent sparse kernel: kQueueSlots launch slots of
// one counter per XCD, each counter on its own 128-byte line.  A launch takes
// the next slot (round robin on the host) and clears it with a kernel on its
// own stream first, so calls may overlap on one GPU as long as fewer than
// kQueueSlots of them are in flight at once.  In host code `attn_queue` names
// a host-side stand-in; its device address comes from hipGetSymbolAddress,
// per device.
constexpr int kQueueSlots = 64;
constexpr int kQueueStride = 32;   // unsigned ints per counter (128 bytes)
static __device__ __align__(256) unsigned int attn_queue[kQueueSlots * kNumXcd * kQueueStride];

__global__ void queue_reset_kernel(unsigned int* q) {
  if (threadIdx.x < kNumXcd) q[threadIdx.x * kQueueStride] = 0u;
}

// Work item k of XCD xcd in the order the non-persistent grid dispatches
// them: KV group g and the item's index rem within the group.
__device__ __forceinline__ void decode_item(const FlashParams& p, int xcd, int k, int& g, int& rem) {
  const int per_group = ((p.NB + 1) / 2) * p.group;
  if (p.interleave) {
    const int per_xcd = per_group / kNumXcd;
    const int chunk = p.chunk_pairs * p.group;
    g = k / per_xcd;
    const int kk = k % per_xcd;
    const int r = kk / chunk;
    rem = (r * kNumXcd + ((r & 1) ? kNumXcd - 1 - xcd : xcd)) * chunk + kk % chunk;
  } else {
    const int w = xcd * ((p.nwork + kNumXcd - 1) / kNumXcd) + k;
    g = w / per_group;
    rem = w % per_group;
  }
}

// Number of work items of XCD xcd.
__device__ __forceinline__ int items_on_xcd(const FlashParams& p, int xcd) {
  if (p.interleave) return (((p.NB + 1) / 2) * p.group / kNumXcd) * (p.hq / p.group);
  const int per = (p.nwork + kNumXcd - 1) / kNumXcd;
  return max(0, min(per, p.nwork - xcd * per));
}

// Index rows held whole in the persistent kernel's stage: kRowAhead entries
// per thread.
constexpr int kRowAhead = 4;

// A work item of the persistent kernel: (queue << 24) | index in that queue.
constexpr int kNoItem = -1;

// Persistent form of the kernel: dense mode, and sparse mode for index rows
// of at most kRowAhead x threads entries.  One work-group per CU takes the
// work items of its XCD from a counter, in the non-persistent kernel's
// order; once that queue is empty it takes the remaining items of the other
// XCDs' queues, so the load stays balanced as with hardware dispatch.  What
// a work-group otherwise pays at each start is hidden: near the end of item
// i the next item is claimed and (sparse mode) its index rows and counts are
// copied into LDS by direct-to-LDS loads, so between two items only the list
// build from LDS, the query loads and the first tile's copy remain.  Items,
// tiles and arithmetic are those of the non-persistent kernel, which serves
// longer index rows.
template <int D, int BQ, bool SPARSE>
__global__ __launch_bounds__(BQ * 4, 1) void flash_bf16_persistent_kernel(FlashParams p) {
  constexpr int kBlockWaves = BQ / 32;
  constexpr int kWaves = 2 * kBlockWaves;
  constexpr int kThreads = kWaves * 64;
  constexpr int kKT = kTileKeys<BQ>;
  constexpr int kTilesPerBlock = BQ / kKT;
  constexpr int kTileBytes = kKT * D * 2;
  constexpr int kStageInts = 2 * kRowAhead * kThreads;
  __shared__ __attribute__((aligned(1024))) uint8_t sK0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t sV0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t sK1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t sV1[kTileBytes];
  // the next item's two index rows (adjacent in memory, copied as one run)
  // and its two counts; every lane of a copy writes, so the counts take 64
  __shared__ __attribute__((aligned(256))) int32_t s_stage[SPARSE ? kStageInts : 1];
  __shared__ __attribute__((aligned(256))) int32_t s_stage_cnt[SPARSE ? 64 : 1];
  __shared__ int s_next[2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int half = wave / kBlockWaves;           // 0: first block of the pair, 1: second
  const int wq = wave % kBlockWaves;
  const int xcd = blockIdx.x % kNumXcd;
  const int npairs = (p.NB + 1) / 2;

  extern __shared__ int32_t s_dyn[];
  const int nw32 = (p.NB + 31) / 32;
  int32_t* s_list = s_dyn;                                  // [NB]: kb | flagA << 30 | flagB << 31
  uint32_t* s_bits = (uint32_t*)(s_dyn + p.NB);             // [2][nw32]
  int32_t* s_off = s_dyn + p.NB + 2 * nw32;                 // [nw32 + 1]

  int koff[D / 16], voff[D / 32][2];
  {
    const int g16 = lane >> 4, i16 = lane & 15;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) koff[t] = tile_off<D>(l32, 16 * t + 8 * hi);
    const int vrow = 4 * hi + (i16 >> 2);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 2; ++r)
        voff[dt][r] = tile_off<D>(vrow + 8 * r, 32 * dt + 16 * (g16 & 1) + 4 * (i16 & 3));
  }

  // thread 0: the next item of this XCD's queue or, once that is empty, of
  // the other queues in turn, starting from the one the last item came
  // from; kNoItem when every queue is empty.  Every item is handed out by
  // exactly one counter increment.
  int q_from = xcd;
  auto fetch = [&]() __attribute__((always_inline)) -> int {
    for (int t = 0; t < kNumXcd; ++t) {
      const int xq = (q_from + t) % kNumXcd;
      const int k = (int)atomicAdd(p.queue + xq * kQueueStride, 1u);
      if (k < items_on_xcd(p, xq)) {
        q_from = xq;
        return (xq << 24) | k;
      }
    }
    return kNoItem;
  };
  // head and first query block of an item
  auto locate = [&](int item, int& g, int& h, int& qbA) __attribute__((always_inline)) {
    int rem;
    decode_item(p, item >> 24, item & 0xFFFFFF, g, rem);
    qbA = 2 * (npairs - 1 - rem / p.group);
    h = g * p.group + rem % p.group;
  };
  // copy item k's index rows and counts into the stage (sparse mode)
  auto stage = [&](int k) __attribute__((always_inline)) {
    if constexpr (SPARSE) {
      int g, h, qbA;
      locate(k, g, h, qbA);
      const int rows = qbA + 1 < p.NB ? 2 : 1;
      const int n = rows * p.NB;
      const __amdgpu_buffer_rsrc_t ri = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(p.idx + ((size_t)h * p.NB + qbA) * p.NB), (short)0, n * 4, 0x00020000);
      for (int i = wave; i < (n + 63) / 64; i += kWaves)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ri, (__attribute__((address_space(3))) void*)(s_stage + i * 64),
                                                 4, lane * 4, i * 256, 0, 0);
      if (wave == kWaves - 1) {
        const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(p.counts + (size_t)h * p.NB + qbA), (short)0, rows * 4, 0x00020000);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rc, (__attribute__((address_space(3))) void*)s_stage_cnt, 4,
                                                 lane * 4, 0, 0, 0);
      }
    }
  };
  // sparse mode: the merged list of item k from the stage (the bitmaps are
  // clear on entry and cleared again as the list is written); dense mode:
  // every causal-visible key block.  Returns the number of key blocks.
  auto build_list = [&](int k) __attribute__((always_inline)) -> int {
    int g, h, qbA;
    locate(k, g, h, qbA);
    const int qbB = qbA + 1;
    if constexpr (SPARSE) {
      int cntA = s_stage_cnt[0];
      int cntB = qbB < p.NB ? s_stage_cnt[1] : 0;
      cntA = cntA < 0 ? 0 : (cntA > p.NB ? p.NB : cntA);
      cntB = cntB < 0 ? 0 : (cntB > p.NB ? p.NB : cntB);
      auto mark = [&](int kb, int b, int qbb) __attribute__((always_inline)) {
        if (kb < 0 || kb >= p.NB || (p.causal && kb > qbb)) return;
        atomicOr(&s_bits[b * nw32 + (kb >> 5)], 1u << (kb & 31));
      };
#pragma unroll
      for (int m = 0; m < kRowAhead; ++m) {
        const int j = tid + m * kThreads;
        if (j < cntA) mark(s_stage[j], 0, qbA);
        if (j < cntB) mark(s_stage[p.NB + j], 1, qbB);
      }
      __syncthreads();
      finish_list<kThreads>(s_bits, s_off, s_list, nw32, tid, wave, lane, true);
      return s_off[nw32];
    } else {
      return p.causal ? min(qbB, p.NB - 1) + 1 : p.NB;
    }
  };

  // The first item; its number reaches every thread through LDS.  Each later
  // item is claimed kClaimAhead tiles before the current one ends, about
  // when a non-persistent work-group would start on this CU, so items go to
  // whichever CU frees up first; its index rows are copied into the stage
  // during the tile after the claim.
  constexpr int kClaimAhead = 3;
  if (tid == 0) s_next[0] = fetch();
  if constexpr (SPARSE)
    for (int i = tid; i < 2 * nw32; i += kThreads) s_bits[i] = 0u;
  __syncthreads();
  int cur = __builtin_amdgcn_readfirstlane(s_next[0]);
  if (cur == kNoItem) return;
  stage(cur);
  wait_vmem();
  __syncthreads();
  int nkb = build_list(cur);

  for (;;) {
    int g, h, qbA;
    locate(cur, g, h, qbA);
    const int qb = qbA + half;
    const bool rows_valid = qb < p.NB;
    const int qrow = qb * BQ + wq * 32 + l32;
    const int qwave0 = qb * BQ + wq * 32;
    const __amdgpu_buffer_rsrc_t Kg = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.K + (size_t)g * p.L * D), (short)0, p.L * D * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t Vg = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.V + (size_t)g * p.L * D), (short)0, p.L * D * 2, 0x00020000);

    // This wave's 32 query rows (contiguous in memory) by direct-to-LDS
    // copies into its slot of the second buffer pair, which is free until the
    // first tile's barrier, in the key tiles' swizzled layout; the fragments
    // are then read with the key-fragment offsets.  Per-lane fragment loads
    // from memory would touch 32 rows per instruction and hold up the tile
    // copies queued behind them.
    constexpr int kWavesPerBuf = kKT / 32;   // 32-row slots per K or V buffer
    static_assert(2 * kWavesPerBuf >= kWaves && kWavesPerBuf * 32 * D * 2 <= kTileBytes,
                  "query rows fit the second K/V buffer pair");
    const __amdgpu_buffer_rsrc_t Qw = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.Q + ((size_t)h * p.L + (rows_valid ? qwave0 : qwave0 - BQ)) * D), (short)0, 32 * D * 2,
        0x00020000);
    // (The lane index goes through an opaque copy so that the eight per-lane
    // offsets are recomputed per item rather than kept live across the loop,
    // where they would be spilled and reloaded before the copies.)
    int qln = lane;
    asm volatile("" : "+v"(qln));
    if (wave < kWavesPerBuf) load_tile<D, 32, 1>(Qw, 0, sK1 + (wave % kWavesPerBuf) * (32 * D * 2), 0, qln);
    else load_tile<D, 32, 1>(Qw, 0, sV1 + (wave % kWavesPerBuf) * (32 * D * 2), 0, qln);
    bf16x8_t qf[D / 16];

    const int ntiles = nkb * kTilesPerBlock;
    auto tile_info = [&](int n, bool& mine) -> int {
      const int j = n / kTilesPerBlock;
      int kb;
      if constexpr (SPARSE) {
        const uint32_t e = (uint32_t)__builtin_amdgcn_readfirstlane(s_list[j]);
        mine = half ? (e >> 31) : ((e >> 30) & 1u);
        kb = (int)(e & 0x3FFFFFFFu);
      } else {
        kb = j;
        mine = half ? (qbA + 1 < p.NB && (!p.causal || kb <= qbA + 1)) : (!p.causal || kb <= qbA);
      }
      return kb * BQ + (n % kTilesPerBlock) * kKT;
    };

    f32x16_t o[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) o[i] = f32x16_t{};
    float m = -INFINITY;
    float lsum = 0.f;

    // tile n_claim claims the next item (thread 0, at the tile's end), tile
    // n_claim + 1 copies its rows and counts into the stage
    const int n_claim = ntiles > kClaimAhead ? ntiles - kClaimAhead : 0;
    int nxt = kNoItem;
    bool staged = false;

    bool mine = false;
    int key0 = ntiles > 0 ? tile_info(0, mine) : -1;
    if (key0 >= 0) {
      load_tile<D, kKT, kWaves>(Kg, key0, sK0, wave, lane);
      load_tile<D, kKT, kWaves>(Vg, key0, sV0, wave, lane);
    }
    wait_vmem();
    // the wave's own query rows have landed: read its fragments before the
    // barrier, after which tile 1 is copied over them
    auto read_q = [&](const uint8_t* buf) __attribute__((always_inline)) {
      const uint8_t* qs = buf + (wave % kWavesPerBuf) * (32 * D * 2);
#pragma unroll
      for (int t = 0; t < D / 16; ++t) qf[t] = as_bf16x8(*(const u32x4_t*)(qs + koff[t]));
    };
    if (wave < kWavesPerBuf) read_q(sK1);
    else read_q(sV1);
    __syncthreads();

    auto step = [&](int n, const uint8_t* sK, const uint8_t* sV, uint8_t* nK,
                    uint8_t* nV) __attribute__((always_inline)) {
      bool mine_next = false;
      const int key0_next = (n + 1 < ntiles) ? tile_info(n + 1, mine_next) : -1;
      if (key0_next >= 0) {
        load_tile<D, kKT, kWaves>(Kg, key0_next, nK, wave, lane);
        load_tile<D, kKT, kWaves>(Vg, key0_next, nV, wave, lane);
      }
      if (n == n_claim + 1) {
        nxt = __builtin_amdgcn_readfirstlane(s_next[0]);
        if (nxt != kNoItem) stage(nxt);
        staged = true;
      }
      if (key0 >= 0 && mine && !(p.causal && key0 > qwave0 + 31))
        attend_tile<D, kKT>(p.scale_log2, p.causal, sK, sV, koff, voff, qf, o, m, lsum, key0, qrow, qwave0, hi);
      key0 = key0_next;
      mine = mine_next;
      // the compiler waits for an atomic's result at once: here that falls
      // inside the wait for the next tile
      if (n == n_claim && tid == 0) s_next[0] = fetch();
      wait_vmem();
      __syncthreads();
    };
    for (int n = 0; n < ntiles; n += 2) {
      step(n, sK0, sV0, sK1, sV1);
      if (n + 1 < ntiles) step(n + 1, sK1, sV1, sK0, sV0);
    }

    // boundary: claim and stage the next item here if no tile did, build
    // its list (nothing of this item reads LDS any more), then store this
    // item's output, whose writes drain during the next item's first copy
    if (!staged) {
      if (ntiles == 0) {
        if (tid == 0) s_next[0] = fetch();
        __syncthreads();
      }
      nxt = __builtin_amdgcn_readfirstlane(s_next[0]);
      if (nxt != kNoItem) stage(nxt);
      wait_vmem();
      __syncthreads();
    }
    if (nxt != kNoItem) nkb = build_list(nxt);
    if (rows_valid) {
      const float ltot = lsum + __shfl_xor(lsum, 32);
      const float inv = ltot > 0.f ? 1.0f / ltot : 0.f;
      // this wave's 32 x D output through LDS (the second K/V buffer is free
      // here): written in the accumulator layout with 16-byte chunks
      // XOR-swizzled by row, read back row by row, stored as whole rows
      constexpr int kRowB = D * 2;                  // bytes per output row
      constexpr int kChunks = kRowB / 16;
      // a lane index the compiler cannot see through, so the addresses below
      // are formed here rather than held in registers across the item loop
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int r32 = ln & 31, hh = ln >> 5;
      // a K or V buffer holds kKT / 32 waves' 32-row tiles, the two hold all waves
      constexpr int kWavesPerBuf = kKT / 32;
      static_assert(2 * kWavesPerBuf >= kWaves && kWavesPerBuf * 32 * kRowB <= kTileBytes,
                    "output tiles fit the second K/V buffer pair");
      uint8_t* ot = (wave < kWavesPerBuf ? sK1 : sV1) + (wave % kWavesPerBuf) * (32 * kRowB);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
          const int col = dt * 32 + 8 * gg;         // 8-element chunk; this lane holds half 4 hi .. +4
          u32x2_t v;
          v[0] = cvt2_bf16(o[dt][4 * gg] * inv, o[dt][4 * gg + 1] * inv);
          v[1] = cvt2_bf16(o[dt][4 * gg + 2] * inv, o[dt][4 * gg + 3] * inv);
          const int ch = (col / 8) ^ (r32 % kChunks);
          *(u32x2_t*)(ot + r32 * kRowB + ch * 16 + 8 * hh) = v;
        }
      constexpr int kRowsPerInst = 64 / kChunks;
      uint16_t* op = p.O + ((size_t)h * p.L + qwave0) * D;
#pragma unroll
      for (int i = 0; i < 32 / kRowsPerInst; ++i) {
        const int r = i * kRowsPerInst + ln / kChunks, c = ln % kChunks;
        const u32x4_t v = *(const u32x4_t*)(ot + r * kRowB + ((c ^ (r % kChunks)) * 16));
        *(u32x4_t*)(op + (size_t)r * D + c * 8) = v;
      }
    }
    cur = nxt;
    if (cur == kNoItem) break;
  }
}

// dynamic LDS of the sparse mode: the merged block list, two bitmaps, offsets
size_t list_bytes(int NB) {
  const int nw32 = (NB + 31) / 32;
  return (size_t)(NB + 3 * nw32 + 1) * sizeof(int32_t);
}

// This device's address of the work queues, looked up once per device with
// that device current (concurrent first calls all store the same address).
hipError_t queue_base(unsigned int** out) {
  static std::atomic<unsigned int*> cached[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  unsigned int* ptr = cached[dev].load(std::memory_order_acquire);
  if (ptr == nullptr) {
    void* v = nullptr;
    e = hipGetSymbolAddress(&v, HIP_SYMBOL(attn_queue));
    if (e != hipSuccess) return e;
    if (v == nullptr) return hipErrorInvalidSymbol;
    ptr = (unsigned int*)v;
    cached[dev].store(ptr, std::memory_order_release);
  }
  *out = ptr;
  return hipSuccess;
}

// Queue slot of the next persistent launch (shared by every instantiation).
std::atomic<unsigned int> next_queue_slot{0};

// Dense mode, and sparse mode with index rows that fit the stage, run
// persistent (one work-group per CU); longer index rows run one work-group
// per item.
template <int D, int BQ>
hipError_t launch(FlashParams fp, hipStream_t st) {
  const size_t dyn = fp.idx ? list_bytes(fp.NB) : 0;
  if (fp.idx == nullptr || fp.NB <= kRowAhead * BQ * 4) {
    unsigned int* base = nullptr;
    hipError_t e = queue_base(&base);
    if (e != hipSuccess) return e;
    const unsigned int slot = next_queue_slot.fetch_add(1u, std::memory_order_relaxed) % kQueueSlots;
    fp.queue = base + (size_t)slot * kNumXcd * kQueueStride;
    hipLaunchKernelGGL(queue_reset_kernel, dim3(1), dim3(64), 0, st, fp.queue);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (fp.idx != nullptr)
      hipLaunchKernelGGL((flash_bf16_persistent_kernel<D, BQ, true>), dim3(kNumXcd * cus_per_xcd()),
                         dim3(BQ * 4), dyn, st, fp);
    else
      hipLaunchKernelGGL((flash_bf16_persistent_kernel<D, BQ, false>), dim3(kNumXcd * cus_per_xcd()),
                         dim3(BQ * 4), dyn, st, fp);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((flash_bf16_kernel<D, BQ>), dim3(fp.grid), dim3(BQ * 4), dyn, st, fp);
  return hipGetLastError();
}

}  // namespace

size_t flash_bf16_lds_bytes(int d, int B, int NB, bool sparse) {
  const int keys = B >= 128 ? kTileKeys<128> : kTileKeys<64>;
  const size_t tiles = (size_t)4 * keys * d * 2;   // K and V, two stages
  return tiles + (sparse ? list_bytes(NB) : 0);
}

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
  const int npairs = (fp.NB + 1) / 2;
  fp.nwork = npairs * s.hq;
  fp.grid = (fp.nwork + kNumXcd - 1) / kNumXcd * kNumXcd;
  fp.chunk_pairs = pairs_per_chunk(npairs);
  fp.interleave = (npairs * fp.group) % (kNumXcd * fp.chunk_pairs * fp.group) == 0;
  fp.scale_log2 = (float)(1.4426950408889634 / __builtin_sqrt((double)s.d));
  fp.queue = nullptr;
  if (s.d == 128) return B == 128 ? launch<128, 128>(fp, st) : launch<128, 64>(fp, st);
  return B == 128 ? launch<64, 128>(fp, st) : launch<64, 64>(fp, st);
}

}  // namespace xattn
