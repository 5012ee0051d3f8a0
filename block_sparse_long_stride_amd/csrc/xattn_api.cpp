// C-ABI of libxattn: argument validation and dispatch to the gfx950 kernels.
// Every check runs before the first HIP call, so malformed calls return an
// error without touching the device.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <initializer_list>
#include <string>

#include "../../include/xattn.h"
#include "launch.h"

namespace {

thread_local std::string g_last_error;

xattn_status fail(xattn_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
xattn_status fail(xattn_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

xattn_status ok() {
  g_last_error.clear();
  return XATTN_OK;
}

xattn_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(XATTN_EHIP, "%s: %s", what, hipGetErrorString(e));
}

// Every device buffer is read or written with 16-byte vector loads or
// direct-to-LDS copies, so each must start on a 16-byte boundary (a tensor
// view with an odd storage offset would otherwise reach the kernels).
xattn_status check_aligned(std::initializer_list<const void*> ptrs, const char* names) {
  for (const void* p : ptrs)
    if ((uintptr_t)p % 16)
      return fail(XATTN_EINVAL, "device buffers (%s) must be 16-byte aligned; got %p", names, p);
  return XATTN_OK;
}

xattn_status check_shape(const xattn_shape* s, xattn::Shape* out) {
  if (!s) return fail(XATTN_EINVAL, "shape is NULL");
  if (s->hq < 1 || s->hkv < 1 || s->L < 1 || s->d < 1)
    return fail(XATTN_EINVAL, "shape fields must be >= 1 (hq=%d hkv=%d L=%d d=%d)", s->hq, s->hkv,
                s->L, s->d);
  if (s->hq % s->hkv)
    return fail(XATTN_EINVAL, "hq (%d) must be a multiple of hkv (%d)", s->hq, s->hkv);
  if (s->dtype != XATTN_FP32 && s->dtype != XATTN_BF16)
    return fail(XATTN_EINVAL, "dtype %d is neither XATTN_FP32 nor XATTN_BF16", s->dtype);
  if (s->causal != 0 && s->causal != 1) return fail(XATTN_EINVAL, "causal must be 0 or 1");
  const long long elems = (long long)s->hq * s->L * s->d;
  if (elems >= (1ll << 40)) return fail(XATTN_EUNSUPPORTED, "tensor too large");
  out->hq = s->hq;
  out->hkv = s->hkv;
  out->L = s->L;
  out->d = s->d;
  out->causal = s->causal;
  out->bf16 = s->dtype == XATTN_BF16;
  return XATTN_OK;
}

xattn_status check_score_args(const xattn_shape* shape, int S, int B, xattn::Shape* s) {
  xattn_status st = check_shape(shape, s);
  if (st != XATTN_OK) return st;
  if (S < 1 || B < 1) return fail(XATTN_EINVAL, "S (%d) and B (%d) must be >= 1", S, B);
  if (s->L % B) return fail(XATTN_EINVAL, "L (%d) must be a multiple of B (%d)", s->L, B);
  if (B % S) return fail(XATTN_EINVAL, "B (%d) must be a multiple of S (%d)", B, S);
  const int bs = B / S;
  if (s->bf16) {
    if (s->d != 64 && s->d != 128)
      return fail(XATTN_EUNSUPPORTED, "bf16 scoring covers d in {64, 128}, got %d", s->d);
    if (bs != 4 && bs != 8 && bs != 16 && bs != 32)
      return fail(XATTN_EUNSUPPORTED, "bf16 scoring covers B/S in {4, 8, 16, 32}, got %d", bs);
    // one head's Q or K is addressed through a buffer resource of 32-bit size
    if ((long long)s->L * s->d * 2 > 0x7FFFFFFFll)
      return fail(XATTN_EUNSUPPORTED, "bf16 scoring covers L * d * 2 < 2^31 bytes per head, got L=%d d=%d",
                  s->L, s->d);
  } else {
    if (s->d > 1024) return fail(XATTN_EUNSUPPORTED, "fp32 scoring covers d <= 1024");
    if (bs > 256) return fail(XATTN_EUNSUPPORTED, "fp32 scoring covers B/S <= 256");
  }
  return XATTN_OK;
}

xattn_status check_attn_args(const xattn::Shape& s, int B) {
  if (B < 1) return fail(XATTN_EINVAL, "B (%d) must be >= 1", B);
  if (s.L % B) return fail(XATTN_EINVAL, "L (%d) must be a multiple of B (%d)", s.L, B);
  if (s.bf16) {
    if (s.d != 64 && s.d != 128)
      return fail(XATTN_EUNSUPPORTED, "bf16 attention covers d in {64, 128}, got %d", s.d);
    if (B != 64 && B != 128)
      return fail(XATTN_EUNSUPPORTED, "bf16 attention covers B in {64, 128}, got %d", B);
    // one KV head's K or V is addressed through a buffer resource of 32-bit size
    if ((long long)s.L * s.d * 2 > 0x7FFFFFFFll)
      return fail(XATTN_EUNSUPPORTED,
                  "bf16 attention covers L * d * 2 < 2^31 bytes per head, got L=%d d=%d", s.L, s.d);
  } else {
    if (s.d != 32 && s.d != 64 && s.d != 128)
      return fail(XATTN_EUNSUPPORTED, "fp32 attention covers d in {32, 64, 128}, got %d", s.d);
    if (B > 256) return fail(XATTN_EUNSUPPORTED, "fp32 attention covers B <= 256, got %d", B);
  }
  return XATTN_OK;
}

}  // namespace

extern "C" {

size_t xattn_score_workspace_bytes(const xattn_shape* shape, int32_t S, int32_t B) {
  xattn::Shape s;
  std::string saved = g_last_error;
  if (check_score_args(shape, S, B, &s) != XATTN_OK) {
    g_last_error = saved;
    return 0;
  }
  return xattn::score_workspace_bytes(s, S, B);
}

static xattn_status run_score(const xattn_shape* shape, const void* Q, const void* K, int32_t S,
                              int32_t B, const xattn::PhaseMap& phase, float* scores,
                              void* workspace, size_t workspace_bytes, void* stream,
                              const char* what) {
  xattn::Shape s;
  xattn_status st = check_score_args(shape, S, B, &s);
  if (st != XATTN_OK) return st;
  if (!Q || !K || !scores) return fail(XATTN_EINVAL, "Q, K and scores must be non-NULL");
  st = check_aligned({Q, K, scores, workspace}, "Q, K, scores, workspace");
  if (st != XATTN_OK) return st;
  const size_t need = xattn::score_workspace_bytes(s, S, B);
  if (need && !workspace) return fail(XATTN_EINVAL, "workspace is NULL (%zu bytes needed)", need);
  if (workspace_bytes < need)
    return fail(XATTN_EWORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
  hipStream_t hs = (hipStream_t)stream;
  hipError_t e = s.bf16 ? xattn::launch_score_bf16(s, Q, K, S, B, phase, scores, workspace, hs)
                        : xattn::launch_score_fp32(s, Q, K, S, B, phase, scores, hs);
  return hip_status(e, what);
}

xattn_status xattn_score(const xattn_shape* shape, const void* Q, const void* K, int32_t S,
                         int32_t B, float* scores, void* workspace, size_t workspace_bytes,
                         void* stream) {
  xattn::PhaseMap antidiagonal{};
  return run_score(shape, Q, K, S, B, antidiagonal, scores, workspace, workspace_bytes, stream,
                   "xattn_score launch");
}

xattn_status xattn_score_noalloc(const xattn_shape* shape, const void* Q, const void* K,
                                 int32_t S, int32_t B, float* scores, void* stream) {
  static_assert(XATTN_SCORE_SCRATCH_BYTES == xattn::kScoreScratchBytes, "scratch size");
  xattn::Shape s;
  xattn_status st = check_score_args(shape, S, B, &s);
  if (st != XATTN_OK) return st;
  if (!Q || !K || !scores) return fail(XATTN_EINVAL, "Q, K and scores must be non-NULL");
  st = check_aligned({Q, K, scores}, "Q, K, scores");
  if (st != XATTN_OK) return st;
  const size_t need = xattn::score_workspace_bytes(s, S, B);
  if (need > xattn::kScoreScratchBytes)
    return fail(XATTN_EWORKSPACE,
                "xattn_score_noalloc: this shape needs %zu bytes of scoring scratch; the fixed "
                "scratch holds %zu (use xattn_score with a caller workspace)",
                need, xattn::kScoreScratchBytes);
  hipStream_t hs = (hipStream_t)stream;
  void* ws = nullptr;
  if (need) {
    hipError_t e = xattn::score_scratch_ptr(&ws);
    if (e != hipSuccess) return hip_status(e, "xattn_score_noalloc scratch lookup");
  }
  xattn::PhaseMap antidiagonal{};
  hipError_t e = s.bf16 ? xattn::launch_score_bf16(s, Q, K, S, B, antidiagonal, scores, ws, hs)
                        : xattn::launch_score_fp32(s, Q, K, S, B, antidiagonal, scores, hs);
  return hip_status(e, "xattn_score_noalloc launch");
}

xattn_status xattn_score_pattern(const xattn_shape* shape, const void* Q, const void* K,
                                 int32_t S, int32_t B, const int32_t* phase_host, float* scores,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  if (!phase_host) return fail(XATTN_EINVAL, "phase_host must be non-NULL");
  if (S < 1) return fail(XATTN_EINVAL, "S (%d) must be >= 1", S);
  if (S > xattn::kMaxPhase)
    return fail(XATTN_EUNSUPPORTED, "sampling patterns cover S <= %d, got %d", xattn::kMaxPhase, S);
  xattn::PhaseMap ph{};
  ph.custom = 1;
  bool seen[xattn::kMaxPhase] = {};
  for (int a = 0; a < S; ++a) {
    const int32_t v = phase_host[a];
    if (v < 0 || v >= S || seen[v])
      return fail(XATTN_EINVAL, "phase is not a permutation of 0..%d (entry %d = %d)", S - 1, a, v);
    seen[v] = true;
    ph.v[a] = v;
  }
  return run_score(shape, Q, K, S, B, ph, scores, workspace, workspace_bytes, stream,
                   "xattn_score_pattern launch");
}

xattn_status xattn_select(int32_t hq, int32_t NB, int32_t causal, const float* scores,
                          const float* tau_host, uint64_t* mask, int32_t* idx, int32_t* counts,
                          void* stream) {
  if (hq < 1 || NB < 1) return fail(XATTN_EINVAL, "hq (%d) and NB (%d) must be >= 1", hq, NB);
  if (causal != 0 && causal != 1) return fail(XATTN_EINVAL, "causal must be 0 or 1");
  if (!scores || !tau_host || !mask || !idx || !counts)
    return fail(XATTN_EINVAL, "scores, tau_host, mask, idx and counts must be non-NULL");
  if (hq > xattn::kMaxHeads)
    return fail(XATTN_EUNSUPPORTED, "selection covers hq <= %d, got %d", xattn::kMaxHeads, hq);
  if (NB > xattn::kMaxSelectBlocks)
    return fail(XATTN_EUNSUPPORTED, "selection covers NB <= %d, got %d", xattn::kMaxSelectBlocks, NB);
  xattn_status st = check_aligned({scores, mask, idx, counts}, "scores, mask, idx, counts");
  if (st != XATTN_OK) return st;
  xattn::TauArray tau;
  for (int h = 0; h < xattn::kMaxHeads; ++h) tau.v[h] = 1.0f;
  for (int h = 0; h < hq; ++h) {
    const float t = tau_host[h];
    if (!(t > 0.0f && t <= 1.0f))
      return fail(XATTN_EINVAL, "tau[%d] = %g is outside (0, 1]", h, (double)t);
    tau.v[h] = t;
  }
  hipError_t e = xattn::launch_select(hq, NB, causal, scores, tau, mask, idx, counts,
                                      (hipStream_t)stream);
  return hip_status(e, "xattn_select launch");
}

static xattn_status check_select_args(int32_t hq, int32_t NB, int32_t causal, const float* scores,
                                      const void* mask, const void* idx, const void* counts) {
  if (hq < 1 || NB < 1) return fail(XATTN_EINVAL, "hq (%d) and NB (%d) must be >= 1", hq, NB);
  if (causal != 0 && causal != 1) return fail(XATTN_EINVAL, "causal must be 0 or 1");
  if (!scores || !mask || !idx || !counts)
    return fail(XATTN_EINVAL, "scores, mask, idx and counts must be non-NULL");
  if (NB > xattn::kMaxSelectBlocks)
    return fail(XATTN_EUNSUPPORTED, "selection covers NB <= %d, got %d", xattn::kMaxSelectBlocks, NB);
  return check_aligned({scores, mask, idx, counts}, "scores, mask, idx, counts");
}

xattn_status xattn_select_topk(int32_t hq, int32_t NB, int32_t causal, const float* scores,
                               int32_t k_blocks, uint64_t* mask, int32_t* idx, int32_t* counts,
                               void* stream) {
  xattn_status st = check_select_args(hq, NB, causal, scores, mask, idx, counts);
  if (st != XATTN_OK) return st;
  if (k_blocks < 1) return fail(XATTN_EINVAL, "k_blocks = %d must be >= 1", k_blocks);
  hipError_t e = xattn::launch_select_topk(hq, NB, causal, scores, k_blocks, mask, idx, counts,
                                           (hipStream_t)stream);
  return hip_status(e, "xattn_select_topk launch");
}

xattn_status xattn_select_topratio(int32_t hq, int32_t NB, int32_t causal, const float* scores,
                                   float ratio, uint64_t* mask, int32_t* idx, int32_t* counts,
                                   void* stream) {
  xattn_status st = check_select_args(hq, NB, causal, scores, mask, idx, counts);
  if (st != XATTN_OK) return st;
  if (!(ratio > 0.0f && ratio <= 1.0f))
    return fail(XATTN_EINVAL, "ratio = %g is outside (0, 1]", (double)ratio);
  hipError_t e = xattn::launch_select_topratio(hq, NB, causal, scores, ratio, mask, idx, counts,
                                               (hipStream_t)stream);
  return hip_status(e, "xattn_select_topratio launch");
}

xattn_status xattn_sparse_prefill(const xattn_shape* shape, const void* Q, const void* K,
                                  const void* V, int32_t B, const int32_t* idx,
                                  const int32_t* counts, void* O, void* stream) {
  xattn::Shape s;
  xattn_status st = check_shape(shape, &s);
  if (st != XATTN_OK) return st;
  st = check_attn_args(s, B);
  if (st != XATTN_OK) return st;
  if (!Q || !K || !V || !O || !idx || !counts)
    return fail(XATTN_EINVAL, "Q, K, V, O, idx and counts must be non-NULL");
  st = check_aligned({Q, K, V, O, idx, counts}, "Q, K, V, O, idx, counts");
  if (st != XATTN_OK) return st;
  {
    // the work-group keeps its query blocks' block list (bf16: two lists
    // merged; fp32: a bitmap) in LDS beside the K/V tiles
    const int NB = s.L / B;
    const size_t need = s.bf16 ? xattn::flash_bf16_lds_bytes(s.d, B, NB, true)
                               : xattn::flash_fp32_lds_bytes(s.d, NB, true);
    if (need > xattn::kLdsBytesPerCu)
      return fail(XATTN_EUNSUPPORTED,
                  "%s sparse prefill needs %zu bytes of LDS for NB = %d (B = %d, d = %d); "
                  "the limit is %zu",
                  s.bf16 ? "bf16" : "fp32", need, NB, B, s.d, xattn::kLdsBytesPerCu);
  }
  hipStream_t hs = (hipStream_t)stream;
  hipError_t e = s.bf16 ? xattn::launch_flash_bf16(s, Q, K, V, B, idx, counts, O, hs)
                        : xattn::launch_flash_fp32(s, Q, K, V, B, idx, counts, O, hs);
  return hip_status(e, "xattn_sparse_prefill launch");
}

xattn_status xattn_full(const xattn_shape* shape, const void* Q, const void* K, const void* V,
                        void* O, void* stream) {
  xattn::Shape s;
  xattn_status st = check_shape(shape, &s);
  if (st != XATTN_OK) return st;
  if (!Q || !K || !V || !O) return fail(XATTN_EINVAL, "Q, K, V and O must be non-NULL");
  st = check_aligned({Q, K, V, O}, "Q, K, V, O");
  if (st != XATTN_OK) return st;
  int B = 0;
  if (s.bf16) {
    B = (s.L % 128 == 0) ? 128 : (s.L % 64 == 0 ? 64 : 0);
    if (!B) return fail(XATTN_EUNSUPPORTED, "bf16 dense attention needs L %% 64 == 0, got %d", s.L);
  } else {
    for (int b = 128; b >= 1; b >>= 1)
      if (s.L % b == 0) {
        B = b;
        break;
      }
  }
  st = check_attn_args(s, B);
  if (st != XATTN_OK) return st;
  hipStream_t hs = (hipStream_t)stream;
  hipError_t e = s.bf16 ? xattn::launch_flash_bf16(s, Q, K, V, B, nullptr, nullptr, O, hs)
                        : xattn::launch_flash_fp32(s, Q, K, V, B, nullptr, nullptr, O, hs);
  return hip_status(e, "xattn_full launch");
}

// ---- fused scoring + selection, and the video-DiT warm-up policy ----------

static xattn_status check_tau(int32_t hq, const float* tau_host, xattn::TauArray* tau) {
  if (!tau_host) return fail(XATTN_EINVAL, "tau_host must be non-NULL");
  if (hq > xattn::kMaxHeads)
    return fail(XATTN_EUNSUPPORTED, "selection covers hq <= %d, got %d", xattn::kMaxHeads, hq);
  for (int h = 0; h < xattn::kMaxHeads; ++h) tau->v[h] = 1.0f;
  for (int h = 0; h < hq; ++h) {
    const float t = tau_host[h];
    if (!(t > 0.0f && t <= 1.0f))
      return fail(XATTN_EINVAL, "tau[%d] = %g is outside (0, 1]", h, (double)t);
    tau->v[h] = t;
  }
  return XATTN_OK;
}

// Validation shared by the fused path and the warm-up policy's sparse steps.
static xattn_status check_fused_args(const xattn_shape* shape, int32_t S, int32_t B,
                                     const float* tau_host, xattn::Shape* s,
                                     xattn::TauArray* tau) {
  xattn_status st = check_score_args(shape, S, B, s);
  if (st != XATTN_OK) return st;
  if (!s->bf16) return fail(XATTN_EUNSUPPORTED, "the fused scoring + selection path is bf16 only");
  const int NB = s->L / B;
  if (NB > xattn::kMaxSelectBlocks)
    return fail(XATTN_EUNSUPPORTED, "selection covers NB <= %d, got %d", xattn::kMaxSelectBlocks, NB);
  return check_tau(s->hq, tau_host, tau);
}

xattn_status xattn_score_select(const xattn_shape* shape, const void* Q, const void* K, int32_t S,
                                int32_t B, const float* tau_host, uint64_t* mask, int32_t* idx,
                                int32_t* counts, void* workspace, size_t workspace_bytes,
                                void* stream) {
  xattn::Shape s;
  xattn::TauArray tau;
  xattn_status st = check_fused_args(shape, S, B, tau_host, &s, &tau);
  if (st != XATTN_OK) return st;
  if (!Q || !K || !mask || !idx || !counts)
    return fail(XATTN_EINVAL, "Q, K, mask, idx and counts must be non-NULL");
  st = check_aligned({Q, K, mask, idx, counts, workspace}, "Q, K, mask, idx, counts, workspace");
  if (st != XATTN_OK) return st;
  const size_t need = xattn::score_workspace_bytes(s, S, B);
  if (!workspace) return fail(XATTN_EINVAL, "workspace is NULL (%zu bytes needed)", need);
  if (workspace_bytes < need)
    return fail(XATTN_EWORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
  hipError_t e = xattn::launch_score_select_bf16(s, Q, K, S, B, tau, mask, idx, counts, workspace,
                                                 (hipStream_t)stream);
  return hip_status(e, "xattn_score_select launch");
}

namespace {
struct DitLayout {
  size_t score, mask, idx, counts, total;
};
constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
DitLayout dit_layout(const xattn::Shape& s, int S, int B) {
  const size_t NB = (size_t)(s.L / B), rows = (size_t)s.hq * NB;
  DitLayout d;
  d.score = 0;
  d.mask = align_up(xattn::score_workspace_bytes(s, S, B));
  d.idx = d.mask + align_up(rows * ((NB + 63) / 64) * 8);
  d.counts = d.idx + align_up(rows * NB * 4);
  d.total = d.counts + align_up(rows * 4);
  return d;
}
}  // namespace

size_t xattn_dit_workspace_bytes(const xattn_shape* shape, int32_t S, int32_t B) {
  xattn::Shape s;
  std::string saved = g_last_error;
  if (check_score_args(shape, S, B, &s) != XATTN_OK) {
    g_last_error = saved;
    return 0;
  }
  return dit_layout(s, S, B).total;
}

xattn_status xattn_dit_attention(const xattn_shape* shape, const void* Q, const void* K,
                                 const void* V, int32_t S, int32_t B, const float* tau_host,
                                 int32_t step, int32_t warmup_steps, void* O, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  if (step < 0 || warmup_steps < 0)
    return fail(XATTN_EINVAL, "step (%d) and warmup_steps (%d) must be >= 0", step, warmup_steps);
  if (step < warmup_steps) return xattn_full(shape, Q, K, V, O, stream);   // warm-up: dense
  xattn::Shape s;
  xattn::TauArray tau;
  xattn_status st = check_fused_args(shape, S, B, tau_host, &s, &tau);
  if (st != XATTN_OK) return st;
  st = check_attn_args(s, B);
  if (st != XATTN_OK) return st;
  if (!Q || !K || !V || !O) return fail(XATTN_EINVAL, "Q, K, V and O must be non-NULL");
  st = check_aligned({Q, K, V, O, workspace}, "Q, K, V, O, workspace");
  if (st != XATTN_OK) return st;
  const DitLayout d = dit_layout(s, S, B);
  if (!workspace) return fail(XATTN_EINVAL, "workspace is NULL (%zu bytes needed)", d.total);
  if (workspace_bytes < d.total)
    return fail(XATTN_EWORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, d.total);
  char* ws = (char*)workspace;
  uint64_t* mask = (uint64_t*)(ws + d.mask);
  int32_t* idx = (int32_t*)(ws + d.idx);
  int32_t* counts = (int32_t*)(ws + d.counts);
  hipStream_t hs = (hipStream_t)stream;
  hipError_t e = xattn::launch_score_select_bf16(s, Q, K, S, B, tau, mask, idx, counts, ws, hs);
  if (e != hipSuccess) return hip_status(e, "xattn_dit_attention scoring launch");
  e = xattn::launch_flash_bf16(s, Q, K, V, B, idx, counts, O, hs);
  return hip_status(e, "xattn_dit_attention attention launch");
}

// ---- per-head threshold calibration -------------------------------------------

xattn_status xattn_head_error(const xattn_shape* shape, const void* O_sparse, const void* O_dense,
                              double* err, void* stream) {
  xattn::Shape s;
  xattn_status st = check_shape(shape, &s);
  if (st != XATTN_OK) return st;
  if (!O_sparse || !O_dense || !err)
    return fail(XATTN_EINVAL, "O_sparse, O_dense and err must be non-NULL");
  const size_t per_head = (size_t)s.L * s.d, esz = s.bf16 ? 2 : 4;
  if ((per_head * esz) % 16 || ((uintptr_t)O_sparse | (uintptr_t)O_dense) % 16)
    return fail(XATTN_EINVAL, "outputs must be 16-byte aligned with L*d*size a multiple of 16");
  hipError_t e = xattn::launch_head_error(s.hq, per_head, s.bf16, O_sparse, O_dense, err,
                                          (hipStream_t)stream);
  return hip_status(e, "xattn_head_error launch");
}

xattn_status xattn_tau_dp(int32_t hq, int32_t levels, const double* err_host, int32_t steps,
                          int32_t* level_out, double* best_out) {
  if (hq < 1 || levels < 0) return fail(XATTN_EINVAL, "hq (%d) >= 1 and levels (%d) >= 0 required", hq, levels);
  if (!err_host || !level_out) return fail(XATTN_EINVAL, "err_host and level_out must be non-NULL");
  if (steps < 0 || (int64_t)steps > (int64_t)hq * levels)
    return fail(XATTN_EINVAL, "steps = %d is outside [0, hq * levels] = [0, %lld]", steps,
                (long long)hq * levels);
  if ((int64_t)(hq + 1) * (steps + 1) > (int64_t)1 << 26)
    return fail(XATTN_EUNSUPPORTED, "DP table of %d x %d entries is too large", hq + 1, steps + 1);
  for (int64_t i = 0; i < (int64_t)hq * (levels + 1); ++i)
    if (!std::isfinite(err_host[i])) return fail(XATTN_EINVAL, "err_host[%lld] is not finite", (long long)i);
  const double best = xattn::tau_dp(hq, levels, err_host, steps, level_out);
  if (best_out) *best_out = best;
  return ok();
}

const char* xattn_status_str(xattn_status status) {
  switch (status) {
    case XATTN_OK: return "ok";
    case XATTN_EINVAL: return "invalid argument";
    case XATTN_EUNSUPPORTED: return "unsupported shape or parameter";
    case XATTN_EWORKSPACE: return "workspace too small";
    case XATTN_EHIP: return "HIP error";
  }
  return "unknown status";
}

const char* xattn_last_error(void) { return g_last_error.c_str(); }

int32_t xattn_version(void) { return 1; }

}  // extern "C"
