// Host-side driver for the sanitizer build of the C ABI (AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code of libxattn).  Every device call
// below carries at least one argument that validation rejects, so no kernel is
// launched and no GPU is needed; the host-only threshold DP (xattn_tau_dp) is
// run on random inputs and checked against exhaustive enumeration.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "xattn.h"

static int failures = 0;

static void expect(bool ok, const char* what) {
  if (!ok) {
    std::fprintf(stderr, "FAILED: %s (last error: %s)\n", what, xattn_last_error());
    ++failures;
  }
}

// A rejected call: the status is not XATTN_OK and a message was recorded.
static void rejected(xattn_status st, const char* what) {
  expect(st != XATTN_OK, what);
  expect(std::strlen(xattn_last_error()) > 0, what);
}

static xattn_shape shape(int hq, int hkv, int L, int d, int dtype, int causal) {
  xattn_shape s;
  s.hq = hq;
  s.hkv = hkv;
  s.L = L;
  s.d = d;
  s.dtype = dtype;
  s.causal = causal;
  return s;
}

static void device_entry_points() {
  // pointers that validation never dereferences
  void* const p = reinterpret_cast<void*>(0x1000);
  void* const odd = reinterpret_cast<void*>(0x1008);   // not 16-byte aligned
  float* const fp = static_cast<float*>(p);
  uint64_t* const mp = static_cast<uint64_t*>(p);
  int32_t* const ip = static_cast<int32_t*>(p);
  double* const dp = static_cast<double*>(p);
  const xattn_shape ok = shape(4, 2, 4096, 128, XATTN_BF16, 1);
  const xattn_shape bad_heads = shape(3, 2, 4096, 128, XATTN_BF16, 1);
  const xattn_shape bad_dtype = shape(4, 2, 4096, 128, 7, 1);
  const xattn_shape bad_causal = shape(4, 2, 4096, 128, XATTN_BF16, 2);
  const xattn_shape bad_d = shape(4, 2, 4096, 96, XATTN_BF16, 1);
  const xattn_shape huge = shape(1, 1, 1 << 23, 128, XATTN_BF16, 1);
  const float tau[4] = {0.9f, 0.9f, 0.9f, 0.9f};
  const float tau_bad[4] = {0.9f, NAN, 0.9f, 0.9f};
  const float tau_zero[4] = {0.9f, 0.0f, 0.9f, 0.9f};
  const int32_t phase_bad[16] = {0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 14};
  const size_t ws = xattn_score_workspace_bytes(&ok, 16, 128);
  expect(ws > 0, "workspace bytes of a valid shape");
  expect(xattn_score_workspace_bytes(nullptr, 16, 128) == 0, "workspace bytes of a NULL shape");
  expect(xattn_score_workspace_bytes(&bad_d, 16, 128) == 0, "workspace bytes of an unsupported d");
  expect(xattn_dit_workspace_bytes(&ok, 16, 128) >= ws, "DiT workspace covers the scoring one");

  rejected(xattn_score(nullptr, p, p, 16, 128, fp, p, ws, nullptr), "score: NULL shape");
  rejected(xattn_score(&bad_heads, p, p, 16, 128, fp, p, ws, nullptr), "score: hq % hkv");
  rejected(xattn_score(&bad_dtype, p, p, 16, 128, fp, p, ws, nullptr), "score: dtype");
  rejected(xattn_score(&bad_causal, p, p, 16, 128, fp, p, ws, nullptr), "score: causal flag");
  rejected(xattn_score(&ok, p, p, 16, 100, fp, p, ws, nullptr), "score: L % B");
  rejected(xattn_score(&ok, p, p, 0, 128, fp, p, ws, nullptr), "score: S = 0");
  rejected(xattn_score(&ok, p, p, 16, 128, fp, p, ws - 1, nullptr), "score: short workspace");
  rejected(xattn_score(&ok, odd, p, 16, 128, fp, p, ws, nullptr), "score: misaligned Q");
  rejected(xattn_score(&ok, nullptr, p, 16, 128, fp, p, ws, nullptr), "score: NULL Q");
  rejected(xattn_score(&huge, p, p, 16, 128, fp, p, (size_t)1 << 40, nullptr), "score: 2^31-byte head");
  rejected(xattn_score_noalloc(&ok, p, p, 16, 100, fp, nullptr), "score_noalloc: L % B");
  rejected(xattn_score_noalloc(&huge, p, p, 16, 128, fp, nullptr), "score_noalloc: beyond the scratch");
  rejected(xattn_score_pattern(&ok, p, p, 16, 128, phase_bad, fp, p, ws, nullptr),
           "score_pattern: not a permutation");
  rejected(xattn_score_pattern(&ok, p, p, 16, 128, nullptr, fp, p, ws - 16, nullptr),
           "score_pattern: short workspace");

  rejected(xattn_select(4, 32, 1, fp, tau_bad, mp, ip, ip, nullptr), "select: NaN tau");
  rejected(xattn_select(4, 32, 1, fp, tau_zero, mp, ip, ip, nullptr), "select: tau = 0");
  rejected(xattn_select(4, 32, 1, fp, nullptr, mp, ip, ip, nullptr), "select: NULL tau");
  rejected(xattn_select(0, 32, 1, fp, tau, mp, ip, ip, nullptr), "select: hq = 0");
  rejected(xattn_select(4, 32, 1, nullptr, tau, mp, ip, ip, nullptr), "select: NULL scores");
  rejected(xattn_select(1 << 20, 32, 1, fp, tau, mp, ip, ip, nullptr), "select: too many heads");
  rejected(xattn_select(4, 1 << 30, 1, fp, tau, mp, ip, ip, nullptr), "select: too many blocks");
  rejected(xattn_select_topk(4, 32, 1, fp, 0, mp, ip, ip, nullptr), "topk: k = 0");
  rejected(xattn_select_topk(4, 32, 1, fp, 4, mp, nullptr, ip, nullptr), "topk: NULL idx");
  rejected(xattn_select_topratio(4, 32, 1, fp, 1.5f, mp, ip, ip, nullptr), "topratio: ratio > 1");
  rejected(xattn_select_topratio(4, 32, 1, fp, NAN, mp, ip, ip, nullptr), "topratio: NaN ratio");

  rejected(xattn_score_select(&ok, p, p, 16, 128, tau_bad, mp, ip, ip, p, ws, nullptr),
           "score_select: NaN tau");
  rejected(xattn_score_select(&ok, p, p, 16, 128, tau, mp, ip, ip, p, 1, nullptr),
           "score_select: short workspace");
  const size_t dws = xattn_dit_workspace_bytes(&ok, 16, 128);
  rejected(xattn_dit_attention(&ok, p, p, p, 16, 128, tau, -1, 5, p, p, dws, nullptr),
           "dit: negative step");
  rejected(xattn_dit_attention(&ok, p, p, p, 16, 128, tau, 6, 5, p, p, dws - 1, nullptr),
           "dit: short workspace");
  rejected(xattn_dit_attention(&ok, p, p, p, 16, 128, tau, 6, 5, odd, p, dws, nullptr),
           "dit: misaligned O");

  rejected(xattn_sparse_prefill(&ok, p, p, p, 96, ip, ip, p, nullptr), "sparse: unsupported B");
  rejected(xattn_sparse_prefill(&ok, p, p, p, 128, nullptr, ip, p, nullptr), "sparse: NULL idx");
  rejected(xattn_sparse_prefill(&bad_d, p, p, p, 128, ip, ip, p, nullptr), "sparse: unsupported d");
  rejected(xattn_sparse_prefill(&ok, p, p, odd, 128, ip, ip, p, nullptr), "sparse: misaligned V");
  const xattn_shape long_seq = shape(1, 1, 128 * 8192, 128, XATTN_BF16, 1);
  rejected(xattn_sparse_prefill(&long_seq, p, p, p, 128, ip, ip, p, nullptr),
           "sparse: list beyond LDS");
  rejected(xattn_full(&huge, p, p, p, p, nullptr), "full: 2^31-byte head");
  rejected(xattn_full(&ok, p, p, nullptr, p, nullptr), "full: NULL V");
  rejected(xattn_head_error(&ok, p, odd, dp, nullptr), "head_error: misaligned O_dense");
  rejected(xattn_head_error(nullptr, p, p, dp, nullptr), "head_error: NULL shape");
}

static void status_strings() {
  for (int s = 0; s <= 5; ++s) {
    const char* str = xattn_status_str(static_cast<xattn_status>(s));
    expect(str != nullptr && std::strlen(str) > 0, "status string");
  }
  expect(xattn_status_str(static_cast<xattn_status>(-3)) != nullptr, "status string of a bad code");
  expect(xattn_version() >= 1, "version");
}

// xattn_tau_dp against enumeration: the best total over all level vectors
// with exactly `steps` steps is minus the smallest summed error.
static void tau_dp_against_enumeration() {
  std::mt19937 rng(7);
  std::uniform_real_distribution<double> u(0.0, 1.0);
  for (int trial = 0; trial < 200; ++trial) {
    const int hq = 1 + static_cast<int>(rng() % 5);
    const int levels = 1 + static_cast<int>(rng() % 3);
    const int steps = static_cast<int>(rng() % (hq * levels + 1));
    std::vector<double> err(static_cast<size_t>(hq) * (levels + 1));
    for (auto& e : err) e = u(rng);
    std::vector<int32_t> lev(static_cast<size_t>(hq), -1);
    double best = NAN;
    const xattn_status st = xattn_tau_dp(hq, levels, err.data(), steps, lev.data(), &best);
    expect(st == XATTN_OK, "tau_dp on valid input");
    if (st != XATTN_OK) continue;
    int sum = 0;
    double total = 0.0;
    for (int h = 0; h < hq; ++h) {
      expect(lev[h] >= 0 && lev[h] <= levels, "tau_dp level in range");
      sum += lev[h];
      total += err[static_cast<size_t>(h) * (levels + 1) + lev[h]];
    }
    expect(sum == steps, "tau_dp distributes exactly `steps` steps");
    double enum_best = -INFINITY;
    std::vector<int> v(static_cast<size_t>(hq), 0);
    for (;;) {
      int s = 0;
      double e = 0.0;
      for (int h = 0; h < hq; ++h) {
        s += v[h];
        e += err[static_cast<size_t>(h) * (levels + 1) + v[h]];
      }
      if (s == steps && -e > enum_best) enum_best = -e;
      int h = 0;
      while (h < hq && ++v[h] > levels) v[h++] = 0;
      if (h == hq) break;
    }
    expect(std::fabs(best - enum_best) <= 1e-12, "tau_dp best equals enumeration");
    expect(std::fabs(-total - enum_best) <= 1e-12, "tau_dp levels achieve the best");
  }
  std::vector<double> err(8, 0.5);
  std::vector<int32_t> lev(4);
  rejected(xattn_tau_dp(0, 1, err.data(), 0, lev.data(), nullptr), "tau_dp: hq = 0");
  rejected(xattn_tau_dp(4, -1, err.data(), 0, lev.data(), nullptr), "tau_dp: negative levels");
  rejected(xattn_tau_dp(4, 1, err.data(), 5, lev.data(), nullptr), "tau_dp: steps beyond hq * levels");
  rejected(xattn_tau_dp(4, 1, err.data(), -1, lev.data(), nullptr), "tau_dp: negative steps");
  rejected(xattn_tau_dp(4, 1, nullptr, 1, lev.data(), nullptr), "tau_dp: NULL errors");
  rejected(xattn_tau_dp(4, 1, err.data(), 1, nullptr, nullptr), "tau_dp: NULL levels");
  // (hq + 1) x (steps + 1) DP entries beyond 2^26: refused before err_host is read
  rejected(xattn_tau_dp(1 << 13, 1 << 14, err.data(), 1 << 14, lev.data(), nullptr),
           "tau_dp: table too large");
}

int main() {
  device_entry_points();
  status_strings();
  tau_dp_against_enumeration();
  if (failures) {
    std::fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  std::printf("host sanitizer driver: all checks passed\n");
  return 0;
}
