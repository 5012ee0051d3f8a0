"""The allocation-free scoring entry point, xattn_score_noalloc (for callers
that cannot allocate: its partials live in the library's fixed device
scratch), called through the C-ABI against xattn_score with a caller
workspace on the same seeded inputs: bit-identical scores on two calls in a
row, the second with a smaller input (the scratch still holds the first
call's partials), then the first shape again."""
import ctypes

import numpy as np
import pytest

from parity import to_device
from workloads import generate, get_config

pytestmark = pytest.mark.gpu

# (config recipe, overrides): 50 MiB of scratch, then 0.9 MiB
CASES = [(2, dict(hq=32, hkv=8, L=16384)), (3, dict(hq=4, hkv=1, L=4096))]


def _noalloc_c_abi(Q, K, S, B, causal, scores):
    import block_sparse_long_stride_amd.xattn as X
    sh = X.shape_of(Q, K, causal)
    st = X.lib().xattn_score_noalloc(ctypes.byref(sh), ctypes.c_void_p(Q.data_ptr()),
                                     ctypes.c_void_p(K.data_ptr()), S, B,
                                     ctypes.c_void_p(scores.data_ptr()), None)
    assert st == X.XATTN_OK, X.lib().xattn_last_error()


def test_noalloc_scores_equal_the_workspace_path_on_consecutive_calls():
    import torch
    from block_sparse_long_stride_amd import xattn_score, xattn_score_workspace_bytes
    import block_sparse_long_stride_amd.xattn as X
    for cid, kw in CASES + CASES[:1]:
        cfg = get_config(cid, **kw)
        print(f"[no-alloc] hq={cfg.hq} hkv={cfg.hkv} L={cfg.L} S={cfg.S} B={cfg.B}", flush=True)
        w = generate(cfg)
        Q, K = to_device(w.Q, cfg.dtype), to_device(w.K, cfg.dtype)
        need = xattn_score_workspace_bytes(X.shape_of(Q, K, cfg.causal), cfg.S, cfg.B)
        assert 0 < need <= X.XATTN_SCORE_SCRATCH_BYTES
        want = xattn_score(Q, K, cfg.S, cfg.B, cfg.causal)
        got = torch.full_like(want, float("nan"))
        _noalloc_c_abi(Q, K, cfg.S, cfg.B, cfg.causal, got)
        torch.cuda.synchronize()
        assert torch.equal(got, want), float((got - want).abs().max())
        rows = got.sum(dim=2).cpu().numpy()
        assert np.allclose(rows, 1.0, atol=1e-4)
