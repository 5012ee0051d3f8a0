"""GPU parity at the full sizes of configs 1-5, in the launch configuration
the bench times.

Per config the whole path runs once on the GPU: score -> select -> sparse
prefill over the GPU's own selection, and dense attention.  The comparison
then runs one chunk of heads at a time (a test per chunk, so progress shows
while the oracle works, its heads spread over the host's cores):

  * every (head, query block) row of the chunk: block scores against the
    oracle, masks under the strict rule of tests/parity.py, and the GPU
    selection (threshold, Top-K, Top-Ratio) on the oracle's own fp32 scores,
    bit for bit.  Heads: all of configs 1, 2, 3 and 5; KV groups 0 and 7
    (query heads 0-3 and 28-31) of config 4.
  * outputs of the path itself: sparse prefill over the GPU's selection
    against oracle attention over the same blocks, and dense attention --
    every row of configs 1 and 2; at configs 3-5 both query blocks of
    sampled pairs (the attention kernel's unit of work, so its merge of two
    real lists runs), 8 pairs per chunk, always including the last pair.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle as O
from parity import (assert_outputs_close, assert_scores_close, classify_rows, mask_bits,
                    out_to_f64, to_device)
from workloads import generate, get_config

pytestmark = pytest.mark.gpu

CIDS = [1, 2, 3, 4, 5]
PAIRS_PER_CHUNK = 8


def head_chunks(cid):
    cfg = get_config(cid)
    if cid == 4:
        return [list(range(0, 4)), list(range(28, 32))]
    n = max(1, min(8, cfg.hq))
    per = cfg.hq // n
    return [list(range(k * per, (k + 1) * per)) for k in range(n)]


def every_row_outputs(cid):
    return cid in (1, 2)


def _workers(n):
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    return max(1, min(n, cores, 16))


def _parallel(fn, items):
    """fn over items on host threads, one BLAS thread each (numpy releases
    the GIL in its loops, so heads proceed in parallel)."""
    from threadpoolctl import threadpool_limits
    items = list(items)
    with threadpool_limits(1):
        with ThreadPoolExecutor(_workers(len(items))) as ex:
            return list(ex.map(fn, items))


def pytest_generate_tests(metafunc):
    if "fullsize" not in metafunc.fixturenames:
        return
    if "chunk" in metafunc.fixturenames:
        params = [(c, k) for c in CIDS for k in range(len(head_chunks(c)))]
        ids = [f"config{c}-heads{head_chunks(c)[k][0]}-{head_chunks(c)[k][-1]}" for c, k in params]
        metafunc.parametrize(("fullsize", "chunk"), params, indirect=["fullsize"], ids=ids,
                             scope="module")
    else:
        metafunc.parametrize("fullsize", CIDS, indirect=True, ids=[f"config{c}" for c in CIDS],
                             scope="module")


def _sync():
    import torch
    torch.cuda.synchronize()


def run(cid):
    """Generate config `cid`, run the GPU path once, keep its results on the
    host (and Q, K on the device for the extra scoring calls)."""
    import torch
    from block_sparse_long_stride_amd import (xattn_full, xattn_score, xattn_select,
                                              xattn_sparse_prefill)
    cfg = get_config(cid)
    print(f"[config {cid}] generating", flush=True)
    w = generate(cfg)
    dev = {k: to_device(getattr(w, k), cfg.dtype) for k in ("Q", "K", "V")}
    print(f"[config {cid}] GPU path", flush=True)
    scores = xattn_score(dev["Q"], dev["K"], cfg.S, cfg.B, cfg.causal)
    mask, idx, counts = xattn_select(scores, w.tau, cfg.causal)
    out_s = xattn_sparse_prefill(dev["Q"], dev["K"], dev["V"], cfg.B, idx, counts, cfg.causal)
    out_f = xattn_full(dev["Q"], dev["K"], dev["V"], cfg.causal)
    _sync()
    res = {
        "scores": scores.cpu().numpy(),
        "mask": mask.cpu().numpy().view(np.uint64),
        "idx": idx.cpu().numpy(),
        "counts": counts.cpu().numpy(),
        "out_s": out_s.cpu(),
        "out_f": out_f.cpu(),
        "gpu_sel": (mask, idx, counts),
    }
    del scores, out_s, out_f
    valid = cfg.hq * (cfg.nb * (cfg.nb + 1) // 2 if cfg.causal else cfg.nb * cfg.nb)
    res["density"] = float(res["counts"].astype(np.int64).sum()) / valid
    return cfg, w, dev, res


@pytest.fixture(scope="module")
def fullsize(request):
    """One config at a time: pytest groups the tests by this module-scoped
    parameter, so each config is generated and run once."""
    import torch
    out = run(request.param)
    yield out
    del out
    torch.cuda.empty_cache()


def _oracle_head(cfg, w, h):
    """Every query-block row of head h: fp64 block scores and find_blocks."""
    sc = O.block_scores(w.q64(h), w.k64(h // cfg.group), cfg.S, cfg.B, cfg.causal)
    sels = O.select_all(sc, cfg.causal, float(w.tau[h]))
    return sc, sels


def test_fullsize_rows(fullsize, chunk):
    """Scores and masks of every row of the chunk's heads, and the GPU cut
    rules on the oracle's fp32 scores of those rows."""
    import torch
    from block_sparse_long_stride_amd import (xattn_select, xattn_select_topk,
                                              xattn_select_topratio)
    cfg, w, dev, r = fullsize
    heads = head_chunks(cfg.cid)[chunk]
    ora = dict(zip(heads, _parallel(lambda h: _oracle_head(cfg, w, h), heads)))

    rel = 0.0
    for h in heads:
        rel = max(rel, assert_scores_close(r["scores"][h], ora[h][0], f"scores h{h}"))

    sels, srts, gsets, taus, labs = [], [], [], [], []
    for h in heads:
        for qb in range(cfg.nb):
            sel = ora[h][1][qb]
            n = int(r["counts"][h, qb])
            g = [int(x) for x in r["idx"][h, qb, :n]]
            assert np.all(r["idx"][h, qb, n:] == -1), (h, qb)
            assert g == mask_bits(r["mask"][h, qb], cfg.nb), (h, qb)
            sels.append(sel)
            srts.append(ora[h][0][qb][sel.order])
            gsets.append(g)
            taus.append(float(w.tau[h]))
            labs.append(f"h{h} qb{qb}")
    rep = classify_rows(sels, srts, gsets, taus, labs)
    print(f"[config {cfg.cid} heads {heads[0]}-{heads[-1]}] {rep.summary()} "
          f"max rel score err {rel:.2e} layer density {r['density']:.4f}")
    assert not rep.failures, rep.failures[:5]

    # the cut rules on the oracle's fp32 scores: bit-exact on every row
    s = torch.zeros((cfg.hq, cfg.nb, cfg.nb), dtype=torch.float32)
    rows32 = {h: ora[h][0].astype(np.float32) for h in heads}
    for h in heads:
        s[h] = torch.from_numpy(rows32[h])
    s = s.cuda()
    kblk = max(1, 8192 // cfg.B)
    rules = {
        "threshold": (lambda: xattn_select(s, w.tau, cfg.causal),
                      lambda row, nv, h: O.find_blocks(row, nv, float(w.tau[h]))),
        "topk": (lambda: xattn_select_topk(s, kblk, cfg.causal),
                 lambda row, nv, h: O.find_blocks_topk(row, nv, kblk)),
        "topratio": (lambda: xattn_select_topratio(s, 0.27, cfg.causal),
                     lambda row, nv, h: O.find_blocks_topratio(row, nv, 0.27)),
    }
    for rule, (gpu_fn, ora_fn) in rules.items():
        mask, idx, counts = gpu_fn()
        _sync()
        mask = mask.cpu().numpy().view(np.uint64)
        idx, counts = idx.cpu().numpy(), counts.cpu().numpy()
        for h in heads:
            for qb in range(cfg.nb):
                nv = qb + 1 if cfg.causal else cfg.nb
                sel = ora_fn(rows32[h][qb].astype(np.float64), nv, h)
                assert int(counts[h, qb]) == sel.kstar, (rule, h, qb)
                assert list(idx[h, qb, :sel.kstar]) == list(sel.selected), (rule, h, qb)
                assert np.all(idx[h, qb, sel.kstar:] == -1), (rule, h, qb)
                np.testing.assert_array_equal(mask[h, qb], O.to_mask(sel, cfg.nb))


def _output_rows(cfg, heads, chunk):
    """(head, query block) rows whose outputs are checked."""
    if every_row_outputs(cfg.cid):
        return [(h, qb) for h in heads for qb in range(cfg.nb)]
    npairs = (cfg.nb + 1) // 2
    rng = np.random.default_rng(4321 + 97 * cfg.cid + chunk)
    pairs = set(int(p) for p in rng.integers(0, npairs, size=PAIRS_PER_CHUNK - 1))
    pairs.add(npairs - 1)
    rows = []
    for p in sorted(pairs):
        h = heads[p % len(heads)]
        rows += [(h, qb) for qb in (2 * p, 2 * p + 1) if qb < cfg.nb]
    return rows


def test_fullsize_outputs(fullsize, chunk):
    """Sparse prefill over the GPU's own selection and dense attention: the
    path's actual outputs against the oracle, row by row."""
    cfg, w, dev, r = fullsize
    heads = head_chunks(cfg.cid)[chunk]
    rows = _output_rows(cfg, heads, chunk)

    def one(hq):
        h, qb = hq
        g = h // cfg.group
        q, k, v = w.q64(h), w.k64(g), w.v64(g)
        n = int(r["counts"][h, qb])
        sel = [int(x) for x in r["idx"][h, qb, :n]]
        return (O.block_sparse_attention(q, k, v, cfg.B, cfg.causal, qb, sel),
                O.full_attention(q, k, v, cfg.B, cfg.causal, qb))

    if every_row_outputs(cfg.cid):
        # one task per head (its 64-bit copies are made once)
        def per_head(h):
            g = h // cfg.group
            q, k, v = w.q64(h), w.k64(g), w.v64(g)
            out = []
            for qb in range(cfg.nb):
                n = int(r["counts"][h, qb])
                sel = [int(x) for x in r["idx"][h, qb, :n]]
                out.append((O.block_sparse_attention(q, k, v, cfg.B, cfg.causal, qb, sel),
                            O.full_attention(q, k, v, cfg.B, cfg.causal, qb)))
            return out
        want = [x for head in _parallel(per_head, heads) for x in head]
    else:
        want = _parallel(one, rows)
    got_s = np.stack([out_to_f64(r["out_s"][h, qb * cfg.B:(qb + 1) * cfg.B]) for h, qb in rows])
    got_f = np.stack([out_to_f64(r["out_f"][h, qb * cfg.B:(qb + 1) * cfg.B]) for h, qb in rows])
    st_s = assert_outputs_close(got_s, np.stack([a for a, _ in want]), cfg.dtype, "sparse O")
    st_f = assert_outputs_close(got_f, np.stack([b for _, b in want]), cfg.dtype, "full O")
    both = sum(1 for h, qb in rows if qb % 2 == 0 and (h, qb + 1) in set(rows)
               and r["counts"][h, qb] > 0 and r["counts"][h, qb + 1] > 0)
    print(f"[config {cfg.cid} heads {heads[0]}-{heads[-1]}] rows {len(rows)} "
          f"(pairs with two lists {both}) sparse O {st_s} full O {st_f}")


def test_fullsize_pattern_scores(fullsize):
    """Diagonal and random sampling patterns at full size: sampled rows
    against the oracle's pattern sums."""
    from block_sparse_long_stride_amd import xattn_score
    cfg, w, dev, r = fullsize
    rng = np.random.default_rng(77 + cfg.cid)
    hs = sorted({0, cfg.hq - 1, int(rng.integers(0, cfg.hq))})
    for kind, ph in (("diagonal", list(range(cfg.S))),
                     ("random", [int(x) for x in rng.permutation(cfg.S)])):
        sc = xattn_score(dev["Q"], dev["K"], cfg.S, cfg.B, cfg.causal, phase=ph)
        _sync()
        rel = 0.0
        for h in hs:
            qbs = sorted({0, cfg.nb - 1} | {int(x) for x in rng.integers(0, cfg.nb, size=4)})
            want = O.block_scores(w.q64(h), w.k64(h // cfg.group), cfg.S, cfg.B, cfg.causal,
                                  qblocks=qbs, phase=ph)
            got = sc[h, qbs].cpu().numpy()
            rel = max(rel, assert_scores_close(got, want, f"{kind} h{h}"))
        del sc
        print(f"[config {cfg.cid}] {kind} pattern: max rel score err {rel:.2e}")


def test_fullsize_fused_score_select(fullsize):
    """The fused scoring + selection path equals the two-call path bit for bit
    on the whole layer (bf16 configs)."""
    import torch
    from block_sparse_long_stride_amd import xattn_score_select
    cfg, w, dev, r = fullsize
    if cfg.dtype != "bf16":
        pytest.skip("the fused path is bf16 only")
    mask, idx, counts = xattn_score_select(dev["Q"], dev["K"], cfg.S, cfg.B, w.tau, cfg.causal)
    _sync()
    m2, i2, c2 = r["gpu_sel"]
    assert torch.equal(counts, c2)
    assert torch.equal(idx, i2)
    assert torch.equal(mask, m2)
    del mask, idx, counts
