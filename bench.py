"""Benchmark of the XAttention prefill path on one MI355X.

One step = xattn_score + xattn_select + xattn_sparse_prefill over the whole
L=131072, 32 query / 8 KV head, d=128, bf16, causal layer (S=16, B=128,
tau=0.95), inputs already resident in HBM.  `value` is dense-equivalent
TFLOP/s: the FLOPs of exact causal attention over the layer (4*d*hq*L(L+1)/2)
divided by the measured time per step.

Prints one JSON line.  Per-call times come from HIP events recorded on the
stream the library launches on; the roofline object is for the dominant
kernel (sparse prefill), priced by its algorithmic FLOPs (4*d per selected
causal query-key pair) against the bf16 dense MFMA peak.  The CPU baseline
times the fp64 oracle on a bounded sample of (head, query block) rows of the
same workload and scales it to the full layer.

    python bench.py [--steps K] [--warmup W] [--config 3] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-full", action="store_true", help="skip timing xattn_full")
    ap.add_argument("--cpu-sample-seconds", type=float, default=20.0)
    ap.add_argument("--no-next", action="store_true",
                    help="skip the measurements beside the headline step (Top-K / Top-Ratio "
                         "selection, sampling patterns, fused scoring + selection, tau "
                         "calibration, DiT warm-up policy)")
    ap.add_argument("--no-dit", dest="next_dit", action="store_false",
                    help="skip the video-DiT warm-up policy measurement (config 5)")
    ap.add_argument("--only", choices=["score", "select", "sparse", "full", "copy"],
                    help="profiling mode: run only this call `--steps` times (after one "
                         "untimed pass of the path), print nothing but a short summary; "
                         "`copy` copies a 1 GiB device buffer, the reference for scaling "
                         "the HBM byte counters")
    return ap.parse_args()


def kernel_source_hash(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "block_sparse_long_stride_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None if absent or taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != kernel_source_hash(rec.get("sources", [])):
        return None
    return rec.get("bytes_per_launch")


def cpu_model():
    """The host CPU's model name from /proc/cpuinfo (None if unreadable)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(cfg, w, seconds):
    """Time the oracle (score rows, find_blocks, block-sparse attention) on a
    random sample of (head, query block) rows until `seconds` have elapsed,
    then scale to all hq * NB rows."""
    import numpy as np
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    rng = np.random.default_rng(7)
    heads = sorted(int(h) for h in rng.choice(cfg.hq, size=min(2, cfg.hq), replace=False))
    per_head = {}
    for h in heads:   # exact fp64 copies of the inputs (input preparation, not timed)
        g = h // cfg.group
        per_head[h] = (w.q64(h), w.k64(g), w.v64(g))
    spent, rows = 0.0, 0
    while spent < seconds:
        h = heads[rows % len(heads)]
        qb = int(rng.integers(0, cfg.nb))
        q, k, v = per_head[h]
        t0 = time.perf_counter()
        sc = O.block_scores(q, k, cfg.S, cfg.B, cfg.causal, qblocks=[qb])
        sel = O.find_blocks(sc[0], qb + 1 if cfg.causal else cfg.nb, float(w.tau[h]))
        O.block_sparse_attention(q, k, v, cfg.B, cfg.causal, qb, sel.selected)
        spent += time.perf_counter() - t0
        rows += 1
    ms_full = spent / rows * cfg.hq * cfg.nb * 1e3
    return ms_full, rows, threads


def dit_policy_rows(timed, stream, steps=50, warmup=5):
    """Warm-up policy of the video-DiT experiment on the config-5 workload:
    one dense (warm-up) step and one sparse step are timed; the 50-step run
    is their weighted sum."""
    import numpy as np
    import torch
    from block_sparse_long_stride_amd import xattn
    from workloads import generate, get_config
    cfg = get_config(5)
    w = generate(cfg)
    dev = "cuda"
    Q, K, V = (torch.from_numpy(np.ascontiguousarray(getattr(w, k)).view(np.int16))
               .view(torch.bfloat16).to(dev) for k in ("Q", "K", "V"))
    out = torch.empty_like(Q)
    sh = xattn.shape_of(Q, K, cfg.causal)
    ws = torch.empty(xattn.xattn_dit_workspace_bytes(sh, cfg.S, cfg.B), dtype=torch.uint8,
                     device=dev)
    run = lambda t: xattn.xattn_dit_attention(Q, K, V, cfg.S, cfg.B, w.tau, step=t,
                                              warmup_steps=warmup, causal=cfg.causal, out=out,
                                              workspace=ws, stream=stream)
    ms_dense = timed(lambda: run(0), reps=2)
    ms_sparse = timed(lambda: run(warmup), reps=2)
    NB = cfg.L // cfg.B
    counts = ws[xattn_counts_offset(ws.numel(), cfg.hq, NB):].view(torch.int32)[:cfg.hq * NB]
    dens = int(counts.to(torch.int64).sum()) / (cfg.hq * NB * NB)
    n_dense = sum(1 for t in range(steps) if t < warmup)
    total = n_dense * ms_dense + (steps - n_dense) * ms_sparse
    res = {"workload": f"config5 {cfg.name}: L={cfg.L}, hq=hkv={cfg.hq}, d={cfg.d}, bf16, "
                       f"non-causal, S={cfg.S}, B={cfg.B}, tau={cfg.tau}",
           "steps": steps, "warmup_steps": warmup, "dense_step_ms": round(ms_dense, 3),
           "sparse_step_ms": round(ms_sparse, 3), "sparse_step_density": round(dens, 5),
           "run_ms_from_step_times": round(total, 1),
           "run_ms_all_dense": round(steps * ms_dense, 1),
           "run_density": round((n_dense + (steps - n_dense) * dens) / steps, 5)}
    del Q, K, V, out, ws
    torch.cuda.empty_cache()
    return res


def xattn_counts_offset(ws_bytes, hq, NB):
    """Byte offset of the counts array at the end of the DiT workspace."""
    return ws_bytes - (hq * NB * 4 + 255) // 256 * 256


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(--gpus must be 1)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    from block_sparse_long_stride_amd import xattn
    from workloads import generate, get_config

    cfg = get_config(args.config)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    xattn.lib()
    if args.only == "copy":
        nbytes = 1 << 30
        src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"only": "copy", "bytes_read": nbytes, "bytes_written": nbytes,
                          "steps": args.steps}))
        return
    t0 = time.perf_counter()
    w = generate(cfg)
    print(f"# generated config {cfg.cid} in {time.perf_counter() - t0:.1f}s", file=sys.stderr,
          flush=True)

    def up(a):
        if cfg.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    Q, K, V = up(w.Q), up(w.K), up(w.V)
    hq, NB, L, d = cfg.hq, cfg.nb, cfg.L, cfg.d
    sh = xattn.shape_of(Q, K, cfg.causal)
    ws = torch.empty(xattn.xattn_score_workspace_bytes(sh, cfg.S, cfg.B), dtype=torch.uint8, device=dev)
    scores = torch.empty((hq, NB, NB), dtype=torch.float32, device=dev)
    mask = torch.empty((hq, NB, (NB + 63) // 64), dtype=torch.int64, device=dev)
    idx = torch.empty((hq, NB, NB), dtype=torch.int32, device=dev)
    counts = torch.empty((hq, NB), dtype=torch.int32, device=dev)
    out = torch.empty_like(Q)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        xattn.xattn_score(Q, K, cfg.S, cfg.B, cfg.causal, scores=scores, workspace=ws, stream=stream)
        if ev:
            ev[1].record(stream)
        xattn.xattn_select(scores, w.tau, cfg.causal, mask=mask, idx=idx, counts=counts, stream=stream)
        if ev:
            ev[2].record(stream)
        xattn.xattn_sparse_prefill(Q, K, V, cfg.B, idx, counts, cfg.causal, out=out, stream=stream)
        if ev:
            ev[3].record(stream)

    if args.only:
        step()
        torch.cuda.synchronize()
        for _ in range(args.steps):
            if args.only == "score":
                xattn.xattn_score(Q, K, cfg.S, cfg.B, cfg.causal, scores=scores, workspace=ws,
                                  stream=stream)
            elif args.only == "select":
                xattn.xattn_select(scores, w.tau, cfg.causal, mask=mask, idx=idx, counts=counts,
                                   stream=stream)
            elif args.only == "sparse":
                xattn.xattn_sparse_prefill(Q, K, V, cfg.B, idx, counts, cfg.causal, out=out,
                                           stream=stream)
            else:
                xattn.xattn_full(Q, K, V, cfg.causal, out=out, stream=stream)
        torch.cuda.synchronize()
        print(json.dumps({"only": args.only, "config": cfg.cid, "steps": args.steps,
                          "density": float(counts.to(torch.int64).sum()) /
                          (hq * (NB * (NB + 1) // 2 if cfg.causal else NB * NB))}))
        return
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    per = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(3)] for e in evs])
    score_ms, select_ms, sparse_ms = [float(np.median(per[:, j])) for j in range(3)]
    ev_step_ms = float(np.median(per.sum(axis=1)))

    # algorithmic work
    F_full = 4.0 * d * hq * (L * (L + 1) / 2 if cfg.causal else float(L) * L)
    Lr = L // cfg.S
    F_score = 2.0 * cfg.S * d * hq * (Lr * (Lr + 1) / 2 if cfg.causal else float(Lr) * Lr)
    c = counts.to(torch.int64)
    n_sel = int(c.sum())
    valid = hq * (NB * (NB + 1) // 2 if cfg.causal else NB * NB)
    if cfg.causal:
        diag = int(((mask[:, torch.arange(NB, device=dev), torch.arange(NB, device=dev) // 64]
                     >> (torch.arange(NB, device=dev) % 64)) & 1).sum())
        pairs = (n_sel - diag) * cfg.B * cfg.B + diag * cfg.B * (cfg.B + 1) / 2
    else:
        pairs = float(n_sel) * cfg.B * cfg.B
    F_sparse = 4.0 * d * pairs
    # select: 4 B per valid score read + mask + idx (counts entries + -1 padding) + counts
    sel_bytes = 4.0 * valid + mask.numel() * 8 + 4.0 * hq * NB * NB + 4.0 * hq * NB

    full_ms = None
    if not args.no_full:
        ef = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        xattn.xattn_full(Q, K, V, cfg.causal, out=out, stream=stream)
        ef[0].record(stream)
        xattn.xattn_full(Q, K, V, cfg.causal, out=out, stream=stream)
        ef[1].record(stream)
        torch.cuda.synchronize()
        full_ms = ef[0].elapsed_time(ef[1])

    # variants measured beside the headline (not part of the timed step)
    variants = {}
    if not args.no_next:
        def timed(fn, reps=5):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            fn()
            e[0].record(stream)
            for _ in range(reps):
                fn()
            e[1].record(stream)
            torch.cuda.synchronize()
            return e[0].elapsed_time(e[1]) / reps

        kblk = max(1, 8192 // cfg.B)
        for name, fn in (
                ("select_topk", lambda: xattn.xattn_select_topk(scores, kblk, cfg.causal, mask=mask,
                                                                idx=idx, counts=counts, stream=stream)),
                ("select_topratio", lambda: xattn.xattn_select_topratio(
                    scores, 0.27, cfg.causal, mask=mask, idx=idx, counts=counts, stream=stream))):
            ms_r = timed(fn)
            n_r = int(counts.to(torch.int64).sum())
            b_r = 4.0 * valid + mask.numel() * 8 + 4.0 * hq * NB * NB + 4.0 * hq * NB
            variants[name] = {
                "param": f"K={kblk * cfg.B} tokens ({kblk} blocks)" if name == "select_topk"
                         else "ratio=0.27",
                "ms": round(ms_r, 3), "gbs": round(b_r / (ms_r * 1e-3) / 1e9, 1),
                "density": round(n_r / valid, 5)}
        # sampling patterns of the pattern ablation: same scoring kernel, another
        # key sub-row per query sub-row; density of the threshold selection
        rng_p = np.random.default_rng(2024)
        for name, ph in (("diagonal", list(range(cfg.S))),
                         ("random", [int(x) for x in rng_p.permutation(cfg.S)])):
            ms_p = timed(lambda: xattn.xattn_score(Q, K, cfg.S, cfg.B, cfg.causal, scores=scores,
                                                   workspace=ws, stream=stream, phase=ph))
            xattn.xattn_select(scores, w.tau, cfg.causal, mask=mask, idx=idx, counts=counts,
                               stream=stream)
            torch.cuda.synchronize()
            n_p = int(counts.to(torch.int64).sum())
            variants["score_" + name] = {
                "phase": ph, "ms": round(ms_p, 3),
                "tflops": round(F_score / (ms_p * 1e-3) / 1e12, 1),
                "frac_bf16_peak": round(F_score / (ms_p * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                "density_threshold_select": round(n_p / valid, 5)}
        xattn.xattn_score(Q, K, cfg.S, cfg.B, cfg.causal, scores=scores, workspace=ws, stream=stream)
        # fused scoring + selection against the two calls, same workload
        if cfg.dtype == "bf16":
            ms_f = timed(lambda: xattn.xattn_score_select(Q, K, cfg.S, cfg.B, w.tau, cfg.causal,
                                                          mask=mask, idx=idx, counts=counts,
                                                          workspace=ws, stream=stream))
            variants["score_select_fused"] = {
                "ms": round(ms_f, 3), "two_calls_ms": round(score_ms + select_ms, 3),
                "density": round(int(counts.to(torch.int64).sum()) / valid, 5)}
        # per-head threshold calibration: tau0 * 0.9^k (k = 0 .. 2) for every head,
        # errors of the sparse outputs against the dense one, DP over hq steps
        if cfg.dtype == "bf16":
            R_lv, t0c = 2, float(np.max(w.tau))
            dense = torch.empty_like(Q)
            spo = torch.empty_like(Q)
            torch.cuda.synchronize()
            tc0 = time.perf_counter()
            xattn.xattn_full(Q, K, V, cfg.causal, out=dense, stream=stream)
            xattn.xattn_score(Q, K, cfg.S, cfg.B, cfg.causal, scores=scores, workspace=ws,
                              stream=stream)
            errs = []
            for t in [t0c * 0.9 ** k for k in range(R_lv + 1)]:
                xattn.xattn_select(scores, [t] * hq, cfg.causal, mask=mask, idx=idx,
                                   counts=counts, stream=stream)
                xattn.xattn_sparse_prefill(Q, K, V, cfg.B, idx, counts, cfg.causal, out=spo,
                                           stream=stream)
                errs.append(xattn.xattn_head_error(spo, dense, stream=stream).cpu().numpy())
            err = np.stack(errs, axis=1)
            levels, best = xattn.xattn_tau_dp(err, hq)
            torch.cuda.synchronize()
            calib_ms = (time.perf_counter() - tc0) * 1e3
            tau_h = [t0c * 0.9 ** k for k in levels]
            xattn.xattn_select(scores, tau_h, cfg.causal, mask=mask, idx=idx, counts=counts,
                               stream=stream)
            torch.cuda.synchronize()
            d_cal = int(counts.to(torch.int64).sum()) / valid
            variants["tau_calibration"] = {
                "tau0": t0c, "levels": R_lv, "steps": hq, "calibration_ms": round(calib_ms, 1),
                "mean_tau": round(float(np.mean(tau_h)), 4),
                "heads_per_level": [levels.count(k) for k in range(R_lv + 1)],
                "proxy_error_sum": round(-best, 6),
                "density_calibrated": round(d_cal, 5), "density_uniform_tau0": round(n_sel / valid, 5)}
            del dense, spo
        # video-DiT warm-up policy on the config-5 workload (non-causal video tokens)
        if args.next_dit:
            variants["dit_warmup_policy"] = dit_policy_rows(timed, stream)
        # restore the threshold selection for anything that follows
        xattn.xattn_select(scores, w.tau, cfg.causal, mask=mask, idx=idx, counts=counts,
                           stream=stream)
        torch.cuda.synchronize()

    tflops = F_full / (wall_ms * 1e-3) / 1e12
    achieved = F_sparse / (sparse_ms * 1e-3) / 1e12
    # the library runs bf16 sparse prefill persistent while an index row has at
    # most four entries per thread (NB <= 16 B), one work-group per item beyond
    if cfg.dtype == "bf16":
        sparse_kernel = "flash_bf16_persistent_kernel" if NB <= 16 * cfg.B else "flash_bf16_kernel"
    else:
        sparse_kernel = "flash_fp32_mfma_kernel" if cfg.B % 32 == 0 else "flash_fp32_kernel"
    res = {
        "metric": "score+select+sparse-prefill ms and dense-equiv TFLOP/s at L=128K, 32/8 heads",
        "value": round(tflops, 2),
        "unit": "TFLOP/s (dense-equivalent)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded RoPE'd Gaussians + shared c + sink columns; no dataset)",
        "config": {"workload": f"config{cfg.cid} {cfg.name}: L={L}, hq={hq}, hkv={cfg.hkv}, d={d}, "
                               f"{cfg.dtype}, {'causal' if cfg.causal else 'non-causal'}, S={cfg.S}, "
                               f"B={cfg.B}, tau={cfg.tau if cfg.tau is not None else list(cfg.tau_range)}",
                   "L": L, "hq": hq, "hkv": cfg.hkv, "d": d, "S": cfg.S, "B": cfg.B,
                   "parallelism": "single GPU"},
        "ms": {"score": round(score_ms, 3), "select": round(select_ms, 3),
               "sparse_prefill": round(sparse_ms, 3), "events_step": round(ev_step_ms, 3),
               "full": None if full_ms is None else round(full_ms, 3)},
        "density": round(n_sel / valid, 5),
        "speedup_vs_full": None if full_ms is None else round(full_ms / wall_ms, 3),
        "kernels": {
            "score": {"tflops": round(F_score / (score_ms * 1e-3) / 1e12, 1),
                      "frac_bf16_peak": round(F_score / (score_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                      "flops": F_score},
            "select": {"gbs": round(sel_bytes / (select_ms * 1e-3) / 1e9, 1),
                       "frac_hbm_peak": round(sel_bytes / (select_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                       "bytes": sel_bytes},
            "sparse_prefill": {"tflops": round(achieved, 1),
                               "frac_bf16_peak": round(achieved / PEAK_BF16_TFLOPS, 4),
                               "flops": F_sparse},
            "full": None if full_ms is None else {
                "tflops": round(F_full / (full_ms * 1e-3) / 1e12, 1),
                "frac_bf16_peak": round(F_full / (full_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)},
        },
        "roofline": {"bound": "mfma", "kernel": f"{sparse_kernel} (xattn_sparse_prefill)",
                     "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic("flash_bf16", f"config{cfg.cid}")},
        "cpu_baseline": None,
        "variants": variants or None,
    }
    if not args.no_cpu_baseline:
        ms_cpu, rows, threads = cpu_baseline(cfg, w, args.cpu_sample_seconds)
        res["cpu_baseline"] = {"value": round(F_full / (ms_cpu * 1e-3) / 1e12, 6),
                               "unit": "TFLOP/s (dense-equivalent)", "cores": threads,
                               "cpu_model": cpu_model(), "kind": "oracle", "ms_per_step": round(ms_cpu, 1),
                               "sample": f"{rows} random (head, query block) rows of the same "
                                         f"workload through oracle score, find_blocks and "
                                         f"block-sparse attention (fp64 numpy), scaled to "
                                         f"{hq * NB} rows"}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
