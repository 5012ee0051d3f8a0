"""The work-item counters of the persistent bf16 sparse-attention kernel.

Sparse prefill in bf16 with NB <= 16 B (index rows of at most four entries
per thread) runs one work-group per CU that takes work items from counters
in a static device array of 64 launch slots (a slot per launch, round robin,
cleared by a kernel on the launch's stream).  These tests run
that path in the ways a slot could be misused: launches of two different
inputs on two streams at once, and more consecutive launches than there are
slots.  Every output must equal, bit for bit, the output of a single launch
on the default stream (whose agreement with the oracle is checked in
test_gpu_parity.py and test_gpu_fullsize.py).
"""
from __future__ import annotations

import pytest

from parity import to_device
from workloads import generate, get_config

pytestmark = pytest.mark.gpu


def _inputs(cid, **kw):
    import torch
    from block_sparse_long_stride_amd import xattn_score, xattn_select
    cfg = get_config(cid, **kw)
    assert cfg.dtype == "bf16" and cfg.nb <= 16 * cfg.B   # the persistent kernel's range
    w = generate(cfg)
    dev = {k: to_device(getattr(w, k), cfg.dtype) for k in ("Q", "K", "V")}
    scores = xattn_score(dev["Q"], dev["K"], cfg.S, cfg.B, cfg.causal)
    _, idx, counts = xattn_select(scores, w.tau, cfg.causal)
    torch.cuda.synchronize()
    return cfg, dev, idx, counts


def _launch(inp, out=None, stream=None):
    from block_sparse_long_stride_amd import xattn_sparse_prefill
    cfg, dev, idx, counts = inp
    return xattn_sparse_prefill(dev["Q"], dev["K"], dev["V"], cfg.B, idx, counts, cfg.causal,
                                out=out, stream=stream)


def _bits(t):
    import torch
    return t.view(torch.int16)


def test_launches_on_two_streams_at_once_match_single_launches():
    import torch
    inputs = [_inputs(2, hq=4, hkv=2, L=4096),          # causal GQA, interleaved work order
              _inputs(5, hq=2, hkv=2, frames=3)]        # non-causal, contiguous ranges
    ref = [_launch(inp).clone() for inp in inputs]
    torch.cuda.synchronize()
    reps = 8
    outs = [[torch.empty_like(r) for _ in range(reps)] for r in ref]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    print("two streams: launching", flush=True)
    for it in range(reps):
        for j, inp in enumerate(inputs):
            with torch.cuda.stream(streams[j]):
                _launch(inp, out=outs[j][it], stream=streams[j])
    torch.cuda.synchronize()
    for j in range(len(inputs)):
        for it in range(reps):
            assert torch.equal(_bits(outs[j][it]), _bits(ref[j])), f"input {j}, launch {it}"


def test_more_launches_than_counter_slots_match_the_first():
    import torch
    inp = _inputs(3, hq=4, hkv=1, L=8192)
    ref = _launch(inp).clone()
    torch.cuda.synchronize()
    out = torch.empty_like(ref)
    print("70 consecutive launches", flush=True)
    for i in range(70):
        out.zero_()
        _launch(inp, out=out)
        if i % 10 == 9:
            torch.cuda.synchronize()
            assert torch.equal(_bits(out), _bits(ref)), f"launch {i}"
