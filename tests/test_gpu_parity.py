"""GPU parity of the HIP path (through the C-ABI) against the fp64 oracle on
small shapes that span several kernel tiles, a ragged tail, every B/S the
bf16 scoring kernel covers, d = 64 and 128, fp32 and bf16, causal and not.
Every stage is compared on every row here; the full-size configs are in
test_gpu_fullsize.py."""
from __future__ import annotations

import functools

import numpy as np
import pytest

import oracle as O
from parity import (assert_outputs_close, assert_scores_close, classify_rows, gpu_selected,
                    mask_bits, out_to_f64, to_device)
from workloads import generate, get_config

pytestmark = pytest.mark.gpu

SMALL = {
    "c1-fp32": get_config(1),
    "llm-S8-B128": get_config(2, hq=4, hkv=2, L=4096),
    "llm-S16-B128-offsets": get_config(3, hq=4, hkv=1, L=8192),
    "llm-bs4-S32": get_config(3, hq=2, hkv=2, L=4096, S=32),
    "llm-bs32-S4": get_config(2, hq=2, hkv=1, L=4096, S=4),
    "llm-d64-B64": get_config(2, hq=2, hkv=1, L=2048, d=64, B=64, S=8),
    "llm-d64-tau-range": get_config(4, hq=4, hkv=2, L=4096, d=64),
    "video-ragged": get_config(5, hq=2, hkv=2, frames=3),
    # causal, odd number of query blocks (33: the last pair of blocks has one)
    # and L/S = 528, a ragged last scoring tile
    "llm-odd-blocks": get_config(2, hq=2, hkv=1, L=4224),
    "noncausal-llm-fp32": get_config(1, causal=False, L=1024),
    # fp32 attention: a block size that is not a multiple of 32 (the SIMT
    # kernel) at d = 32, and one of three 32-row waves (the matrix-core
    # kernel) at d = 128
    "fp32-B48-d32": get_config(1, L=1536, B=48, S=8, d=32),
    "fp32-B96-d128": get_config(1, L=1536, B=96, S=8, d=128),
    # the attention kernel's interleaved XCD work order (pairs of query blocks
    # a multiple of 16), two rounds of chunks per XCD so the alternating deal
    # is used, with one and with eight query heads per KV head
    "llm-mha-interleave": get_config(2, hq=2, hkv=2, L=8192),
    "llm-gqa8-interleave": get_config(3, hq=8, hkv=1, L=8192),
}


@functools.lru_cache(maxsize=None)
def case(name):
    cfg = SMALL[name]
    w = generate(cfg)
    dev = {k: to_device(getattr(w, k), cfg.dtype) for k in ("Q", "K", "V")}
    scores = []
    for h in range(cfg.hq):
        g = h // cfg.group
        scores.append(O.block_scores(w.q64(h), w.k64(g), cfg.S, cfg.B, cfg.causal))
    return cfg, w, dev, np.stack(scores)


def _sync():
    import torch
    torch.cuda.synchronize()


def _gpu_scores(cfg, dev):
    from block_sparse_long_stride_amd import xattn_score
    s = xattn_score(dev["Q"], dev["K"], cfg.S, cfg.B, cfg.causal)
    _sync()
    return s


@pytest.mark.parametrize("name", list(SMALL))
def test_scores_match_oracle(name):
    cfg, w, dev, ora = case(name)
    print(f"[{name}] score", flush=True)
    gpu = _gpu_scores(cfg, dev).cpu().numpy()
    rel = assert_scores_close(gpu, ora)
    print(f"[{name}] max rel score err {rel:.2e}")


def _phase(S, kind, seed=0):
    if kind == "diagonal":
        return list(range(S))
    if kind == "antidiagonal":
        return [S - 1 - a for a in range(S)]
    return [int(x) for x in np.random.default_rng(seed).permutation(S)]


@pytest.mark.parametrize("name", ["c1-fp32", "llm-S8-B128", "llm-S16-B128-offsets", "llm-bs4-S32",
                                  "llm-d64-B64", "video-ragged", "noncausal-llm-fp32"])
@pytest.mark.parametrize("kind", ["diagonal", "random", "antidiagonal"])
def test_pattern_scores_match_oracle(name, kind):
    """Sampling patterns of the pattern ablation through xattn_score_pattern
    against the oracle's pattern sums (the antidiagonal map must reproduce
    xattn_score bit for bit)."""
    from block_sparse_long_stride_amd import xattn_score
    cfg, w, dev, ora = case(name)
    ph = _phase(cfg.S, kind, seed=cfg.S + 17)
    print(f"[{name}] {kind} scores, phase {ph}", flush=True)
    gpu = xattn_score(dev["Q"], dev["K"], cfg.S, cfg.B, cfg.causal, phase=ph)
    _sync()
    gpu = gpu.cpu().numpy()
    want = np.stack([O.block_scores(w.q64(h), w.k64(h // cfg.group), cfg.S, cfg.B, cfg.causal,
                                    phase=ph) for h in range(cfg.hq)])
    rel = assert_scores_close(gpu, want)
    print(f"[{name}] {kind}: max rel score err {rel:.2e}")
    if kind == "antidiagonal":
        np.testing.assert_array_equal(gpu, _gpu_scores(cfg, dev).cpu().numpy())


@pytest.mark.parametrize("name", list(SMALL))
def test_select_matches_oracle_on_same_scores(name):
    """Both sides rank the same fp32 scores: masks, idx and counts are exact."""
    import torch
    from block_sparse_long_stride_amd import xattn_select
    cfg, w, dev, ora = case(name)
    print(f"[{name}] select", flush=True)
    s32 = ora.astype(np.float32)
    mask, idx, counts = xattn_select(torch.from_numpy(s32).cuda(), w.tau, cfg.causal)
    _sync()
    mask, idx, counts = mask.cpu().numpy(), idx.cpu().numpy(), counts.cpu().numpy()
    NB = cfg.nb
    for h in range(cfg.hq):
        for qb in range(NB):
            sel = O.find_blocks(s32[h, qb].astype(np.float64), qb + 1 if cfg.causal else NB,
                                float(w.tau[h]))
            assert counts[h, qb] == sel.kstar, (h, qb)
            assert list(idx[h, qb, :sel.kstar]) == list(sel.selected), (h, qb)
            assert np.all(idx[h, qb, sel.kstar:] == -1), (h, qb)
            np.testing.assert_array_equal(mask[h, qb].view(np.uint64), O.to_mask(sel, NB))


@pytest.mark.parametrize("name", list(SMALL))
def test_cut_rules_match_oracle_on_same_scores(name):
    """Top-K and Top-Ratio on the same fp32 scores: masks, idx and counts are
    exact, for counts below, inside and beyond the valid range."""
    import torch
    from block_sparse_long_stride_amd import xattn_select_topk, xattn_select_topratio
    cfg, w, dev, ora = case(name)
    print(f"[{name}] cut rules", flush=True)
    s32 = ora.astype(np.float32)
    sd = torch.from_numpy(s32).cuda()
    NB = cfg.nb
    runs = [("topk", k) for k in (1, max(1, NB // 4), NB + 5)] + \
           [("ratio", r) for r in (0.27, 1.0, 1e-3)]
    for rule, par in runs:
        if rule == "topk":
            mask, idx, counts = xattn_select_topk(sd, par, cfg.causal)
        else:
            mask, idx, counts = xattn_select_topratio(sd, par, cfg.causal)
        _sync()
        mask, idx, counts = mask.cpu().numpy(), idx.cpu().numpy(), counts.cpu().numpy()
        for h in range(cfg.hq):
            for qb in range(NB):
                nv = qb + 1 if cfg.causal else NB
                row = s32[h, qb].astype(np.float64)
                sel = (O.find_blocks_topk(row, nv, par) if rule == "topk"
                       else O.find_blocks_topratio(row, nv, par))
                assert counts[h, qb] == sel.kstar, (rule, par, h, qb)
                assert list(idx[h, qb, :sel.kstar]) == list(sel.selected), (rule, par, h, qb)
                assert np.all(idx[h, qb, sel.kstar:] == -1), (rule, par, h, qb)
                np.testing.assert_array_equal(mask[h, qb].view(np.uint64), O.to_mask(sel, NB))


@pytest.mark.parametrize("name", list(SMALL))
def test_pipeline_masks_match_oracle(name):
    """GPU score -> GPU select against the oracle's fp64 path, with band counts."""
    from block_sparse_long_stride_amd import xattn_select
    cfg, w, dev, ora = case(name)
    print(f"[{name}] pipeline masks", flush=True)
    scores = _gpu_scores(cfg, dev)
    mask, idx, counts = xattn_select(scores, w.tau, cfg.causal)
    _sync()
    mask, idx, counts = mask.cpu().numpy(), idx.cpu().numpy(), counts.cpu().numpy()
    sels, srts, gsets, taus, labs = [], [], [], [], []
    for h in range(cfg.hq):
        for qb in range(cfg.nb):
            sel = O.find_blocks(ora[h, qb], qb + 1 if cfg.causal else cfg.nb, float(w.tau[h]))
            sels.append(sel)
            srts.append(ora[h, qb][sel.order])
            g = gpu_selected(idx[h, qb], int(counts[h, qb]))
            assert g == mask_bits(mask[h, qb].view(np.uint64), cfg.nb)
            gsets.append(g)
            taus.append(float(w.tau[h]))
            labs.append(f"h{h} qb{qb}")
    rep = classify_rows(sels, srts, gsets, taus, labs)
    print(f"[{name}] {rep.summary()} density "
          f"{sum(len(g) for g in gsets) / sum(s.n_valid for s in sels):.4f}")
    assert not rep.failures, rep.failures[:5]


def _oracle_selections(cfg, w, ora):
    return [[O.find_blocks(ora[h, qb], qb + 1 if cfg.causal else cfg.nb, float(w.tau[h]))
             for qb in range(cfg.nb)] for h in range(cfg.hq)]


def _idx_tensors(cfg, sels):
    import torch
    idx = np.full((cfg.hq, cfg.nb, cfg.nb), -1, dtype=np.int32)
    counts = np.zeros((cfg.hq, cfg.nb), dtype=np.int32)
    for h in range(cfg.hq):
        for qb in range(cfg.nb):
            s = sels[h][qb].selected
            idx[h, qb, :len(s)] = s
            counts[h, qb] = len(s)
    return torch.from_numpy(idx).cuda(), torch.from_numpy(counts).cuda()


@pytest.mark.parametrize("name", list(SMALL))
def test_sparse_prefill_matches_oracle(name):
    from block_sparse_long_stride_amd import xattn_sparse_prefill
    cfg, w, dev, ora = case(name)
    print(f"[{name}] sparse prefill", flush=True)
    sels = _oracle_selections(cfg, w, ora)
    idx, counts = _idx_tensors(cfg, sels)
    out = xattn_sparse_prefill(dev["Q"], dev["K"], dev["V"], cfg.B, idx, counts, cfg.causal)
    _sync()
    got = out_to_f64(out)
    want = np.zeros_like(got)
    for h in range(cfg.hq):
        g = h // cfg.group
        q, k, v = w.q64(h), w.k64(g), w.v64(g)
        for qb in range(cfg.nb):
            want[h, qb * cfg.B:(qb + 1) * cfg.B] = O.block_sparse_attention(
                q, k, v, cfg.B, cfg.causal, qb, sels[h][qb].selected)
    st = assert_outputs_close(got, want, cfg.dtype)
    print(f"[{name}] sparse O {st}")


@pytest.mark.parametrize("name", list(SMALL))
def test_full_matches_oracle(name):
    from block_sparse_long_stride_amd import xattn_full
    cfg, w, dev, ora = case(name)
    print(f"[{name}] full", flush=True)
    out = xattn_full(dev["Q"], dev["K"], dev["V"], cfg.causal)
    _sync()
    got = out_to_f64(out)
    want = np.zeros_like(got)
    for h in range(cfg.hq):
        g = h // cfg.group
        q, k, v = w.q64(h), w.k64(g), w.v64(g)
        for qb in range(cfg.nb):
            want[h, qb * cfg.B:(qb + 1) * cfg.B] = O.full_attention(q, k, v, cfg.B, cfg.causal, qb)
    st = assert_outputs_close(got, want, cfg.dtype)
    print(f"[{name}] full O {st}")


@pytest.mark.parametrize("name", ["c1-fp32", "llm-S8-B128", "video-ragged"])
def test_tau_one_selects_every_block_and_matches_full(name):
    import torch
    from block_sparse_long_stride_amd import xattn_full, xattn_select, xattn_sparse_prefill
    cfg, w, dev, ora = case(name)
    scores = _gpu_scores(cfg, dev)
    mask, idx, counts = xattn_select(scores, np.ones(cfg.hq, np.float32), cfg.causal)
    out_s = xattn_sparse_prefill(dev["Q"], dev["K"], dev["V"], cfg.B, idx, counts, cfg.causal)
    out_f = xattn_full(dev["Q"], dev["K"], dev["V"], cfg.causal)
    _sync()
    c = counts.cpu().numpy()
    want = (np.arange(cfg.nb) + 1) if cfg.causal else np.full(cfg.nb, cfg.nb)
    assert np.all(c == want[None, :])
    # same blocks, same kernels: identical up to the order of key blocks (ascending in both)
    np.testing.assert_array_equal(out_to_f64(out_s), out_to_f64(out_f))


@pytest.mark.parametrize("name", ["llm-S8-B128", "c1-fp32"])
def test_sparse_prefill_edge_lists(name):
    """Empty lists give zeros; invalid entries (-1, >= NB, > qb when causal)
    are ignored; a single block equals attention over that block alone; a list
    is a set (repeated or descending entries give the attention over the
    distinct blocks)."""
    import torch
    from block_sparse_long_stride_amd import xattn_sparse_prefill
    cfg, w, dev, ora = case(name)
    NB = cfg.nb
    idx = np.full((cfg.hq, NB, NB), -1, dtype=np.int32)
    counts = np.zeros((cfg.hq, NB), dtype=np.int32)
    rng = np.random.default_rng(0)
    expect_lists = {}
    for h in range(cfg.hq):
        for qb in range(NB):
            mode = (h * NB + qb) % 5
            if mode == 0:
                lst, cnt = [], 0
            elif mode == 1:
                kb = int(rng.integers(0, qb + 1))
                lst, cnt = [kb], 1
            elif mode == 2:   # junk entries mixed in
                kb = int(rng.integers(0, qb + 1))
                lst = [-5, kb, NB + 3, min(qb + 1, NB - 1) if qb + 1 < NB else -1]
                cnt = len(lst)
            elif mode == 3:   # count larger than NB is clamped; entries after are -1
                lst, cnt = [qb], NB + 7
            else:             # repeats in descending order
                a, b = (int(x) for x in rng.integers(0, qb + 1, size=2))
                lst = [max(a, b), min(a, b), max(a, b), min(a, b)]
                cnt = len(lst)
            idx[h, qb, :len(lst)] = lst
            counts[h, qb] = cnt
            valid = [k for k in lst[:min(cnt, NB)] if 0 <= k < NB and (not cfg.causal or k <= qb)]
            expect_lists[(h, qb)] = valid
    out = xattn_sparse_prefill(dev["Q"], dev["K"], dev["V"], cfg.B, torch.from_numpy(idx).cuda(),
                               torch.from_numpy(counts).cuda(), cfg.causal)
    _sync()
    got = out_to_f64(out)
    want = np.zeros_like(got)
    for h in range(cfg.hq):
        g = h // cfg.group
        q, k, v = w.q64(h), w.k64(g), w.v64(g)
        for qb in range(NB):
            want[h, qb * cfg.B:(qb + 1) * cfg.B] = O.block_sparse_attention(
                q, k, v, cfg.B, cfg.causal, qb, expect_lists[(h, qb)])
    assert_outputs_close(got, want, cfg.dtype)


BF16 = [n for n, c in SMALL.items() if c.dtype == "bf16"]


@pytest.mark.parametrize("name", BF16)
def test_fused_score_select_equals_two_calls(name):
    """xattn_score_select (finishing + selection in one kernel) gives the same
    mask, idx and counts, bit for bit, as xattn_score then xattn_select."""
    from block_sparse_long_stride_amd import xattn_score_select, xattn_select
    cfg, w, dev, ora = case(name)
    print(f"[{name}] fused score+select", flush=True)
    sc = _gpu_scores(cfg, dev)
    m1, i1, c1 = xattn_select(sc, w.tau, cfg.causal)
    m2, i2, c2 = xattn_score_select(dev["Q"], dev["K"], cfg.S, cfg.B, w.tau, cfg.causal)
    _sync()
    for a, b in ((m1, m2), (i1, i2), (c1, c2)):
        np.testing.assert_array_equal(a.cpu().numpy(), b.cpu().numpy())


@pytest.mark.parametrize("name", ["video-ragged", "llm-S8-B128", "llm-d64-B64"])
def test_dit_attention_policy(name):
    """Warm-up steps run dense attention (bit-identical to xattn_full); later
    steps run the fused selection and sparse prefill (bit-identical to those
    calls), and match the oracle's policy output."""
    import torch
    from block_sparse_long_stride_amd import (xattn_dit_attention, xattn_full, xattn_score_select,
                                              xattn_sparse_prefill)
    cfg, w, dev, ora = case(name)
    print(f"[{name}] dit policy", flush=True)
    warm = xattn_dit_attention(dev["Q"], dev["K"], dev["V"], cfg.S, cfg.B, w.tau, step=4,
                               warmup_steps=5, causal=cfg.causal)
    full = xattn_full(dev["Q"], dev["K"], dev["V"], cfg.causal)
    sparse = xattn_dit_attention(dev["Q"], dev["K"], dev["V"], cfg.S, cfg.B, w.tau, step=5,
                                 warmup_steps=5, causal=cfg.causal)
    _, idx, counts = xattn_score_select(dev["Q"], dev["K"], cfg.S, cfg.B, w.tau, cfg.causal)
    ref = xattn_sparse_prefill(dev["Q"], dev["K"], dev["V"], cfg.B, idx, counts, cfg.causal)
    _sync()
    np.testing.assert_array_equal(out_to_f64(warm), out_to_f64(full))
    np.testing.assert_array_equal(out_to_f64(sparse), out_to_f64(ref))
    # against the oracle: dense rows exactly as full attention; sparse rows on the
    # GPU's own selection (isolates the attention from the tau band)
    got_w, got_s = out_to_f64(warm), out_to_f64(sparse)
    idx_np, cnt_np = idx.cpu().numpy(), counts.cpu().numpy()
    want_w, want_s = np.zeros_like(got_w), np.zeros_like(got_s)
    for h in range(cfg.hq):
        g = h // cfg.group
        q, k, v = w.q64(h), w.k64(g), w.v64(g)
        for qb in range(cfg.nb):
            rows = slice(qb * cfg.B, (qb + 1) * cfg.B)
            want_w[h, rows] = O.dit_attention(q, k, v, cfg.S, cfg.B, float(w.tau[h]), 4, 5, qb,
                                              cfg.causal)
            want_s[h, rows] = O.block_sparse_attention(q, k, v, cfg.B, cfg.causal, qb,
                                                       idx_np[h, qb, :cnt_np[h, qb]])
    assert_outputs_close(got_w, want_w, cfg.dtype)
    assert_outputs_close(got_s, want_s, cfg.dtype)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_head_error_matches_oracle(dtype):
    """Per-head relative squared error on the device against the oracle's."""
    import torch
    from block_sparse_long_stride_amd import xattn_head_error
    rng = np.random.default_rng(12)
    hq, L, d = 5, 1536, 64
    b = rng.standard_normal((hq, L, d))
    a = b + rng.standard_normal((hq, L, d)) * np.array([0, 1e-3, 1e-2, 0.3, 1.0])[:, None, None]
    b[4] = 0.0                                        # zero reference: error 0 by definition
    tt = torch.bfloat16 if dtype == "bf16" else torch.float32
    A, Bt = torch.from_numpy(a).to(tt).cuda(), torch.from_numpy(b).to(tt).cuda()
    got = xattn_head_error(A, Bt).cpu().numpy()
    a_r, b_r = A.float().cpu().numpy(), Bt.float().cpu().numpy()   # the values the device sees
    want = np.array([O.head_rel_sq_error(a_r[h], b_r[h]) for h in range(hq)])
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=0)
    assert got[0] == 0.0 and got[4] == 0.0


@pytest.mark.parametrize("name", ["llm-S8-B128", "video-ragged"])
def test_tau_calibration_end_to_end(name):
    """Calibration on the device: dense output once, then per level k the
    threshold tau0 * 0.9^k for every head -> selection -> sparse prefill ->
    head errors; the library DP on those errors equals the oracle DP and the
    errors equal the oracle's on the same outputs."""
    import torch
    from block_sparse_long_stride_amd import (xattn_full, xattn_head_error, xattn_select,
                                              xattn_sparse_prefill, xattn_tau_dp)
    cfg, w, dev, ora = case(name)
    R, tau0 = 2, 0.95
    dense = xattn_full(dev["Q"], dev["K"], dev["V"], cfg.causal)
    sc = _gpu_scores(cfg, dev)
    errs, outs = [], []
    for t in O.tau_levels(tau0, R):
        _, idx, counts = xattn_select(sc, np.full(cfg.hq, t, np.float32), cfg.causal)
        o = xattn_sparse_prefill(dev["Q"], dev["K"], dev["V"], cfg.B, idx, counts, cfg.causal)
        errs.append(xattn_head_error(o, dense).cpu().numpy())
        outs.append(o.float().cpu().numpy())
    _sync()
    err = np.stack(errs, axis=1)                      # [hq][R+1]
    d32 = dense.float().cpu().numpy()
    want = np.array([[O.head_rel_sq_error(outs[k][h], d32[h]) for k in range(R + 1)]
                     for h in range(cfg.hq)])
    np.testing.assert_allclose(err, want, rtol=1e-12, atol=0)
    for steps in range(cfg.hq * R + 1):
        assert xattn_tau_dp(err, steps) == O.tau_dp(err, steps)
