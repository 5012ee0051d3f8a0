"""Launch shapes at the top of the block-count range, on seeded inputs of the
long-context recipe (one head, S = 16 or 32, B = 128):

  * the fused scoring + selection path at B/S = 4 and NB = 4096 (its largest
    LDS block-score buffer) equals the two calls bit for bit, and sampled
    block-score rows of the two-call path match the oracle;
  * sparse prefill over every causal block equals dense attention bit for
    bit at NB = 4096 and at NB = 7488 (the largest block list that fits in
    LDS beside the 128-key tiles), and sampled query blocks of both match
    oracle attention (first, middle and last block: the last one attends to
    all 958464 keys at NB = 7488)."""
import numpy as np
import pytest

import oracle as O
from parity import assert_outputs_close, assert_scores_close, out_to_f64, to_device
from workloads import generate, get_config

pytestmark = pytest.mark.gpu


def _workload(L, S):
    cfg = get_config(3, hq=1, hkv=1, L=L, S=S, rope_offset_max=0, extra_sinks=8)
    return cfg, generate(cfg)


def test_fused_equals_two_calls_at_nb_4096_bs4():
    import torch
    import block_sparse_long_stride_amd as xa
    S, B = 32, 128
    L = 4096 * B
    print(f"[large-nb] fused vs two calls L={L} S={S} B={B}", flush=True)
    cfg, w = _workload(L, S)
    Q, K = to_device(w.Q, "bf16"), to_device(w.K, "bf16")
    sc = xa.xattn_score(Q, K, S, B, True)
    m1, i1, c1 = xa.xattn_select(sc, [0.9], True)
    m2, i2, c2 = xa.xattn_score_select(Q, K, S, B, [0.9], True)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2) and torch.equal(i1, i2) and torch.equal(m1, m2)
    assert int(c1.min()) >= 1
    qbs = [0, 1, 2047, 4094, 4095]
    want = O.block_scores(w.q64(0), w.k64(0), S, B, True, qblocks=qbs)
    rel = assert_scores_close(sc[0, qbs].cpu().numpy(), want, "scores at NB=4096")
    print(f"[large-nb] NB=4096 sampled score rows max rel err {rel:.2e}")


@pytest.mark.parametrize("NB", [4096, 7488])
def test_sparse_over_every_block_equals_dense_at_large_nb(NB):
    import torch
    import block_sparse_long_stride_amd as xa
    B = 128
    L = NB * B
    print(f"[large-nb] sparse (all causal blocks) vs dense L={L} NB={NB}", flush=True)
    cfg, w = _workload(L, 16)
    Q, K, V = (to_device(getattr(w, k), "bf16") for k in ("Q", "K", "V"))
    kb = torch.arange(NB, device="cuda", dtype=torch.int32)
    idx = torch.where(kb[None, :] <= kb[:, None], kb[None, :], torch.full_like(kb[None, :], -1))
    idx = idx[None].contiguous()
    counts = (kb + 1)[None].contiguous()
    out_s = xa.xattn_sparse_prefill(Q, K, V, B, idx, counts, True)
    out_f = xa.xattn_full(Q, K, V, True)
    torch.cuda.synchronize()
    assert torch.equal(out_s, out_f)
    assert bool(torch.isfinite(out_s.float()).all())
    q, k, v = w.q64(0), w.k64(0), w.v64(0)
    got, want = [], []
    for qb in (0, NB // 2, NB - 1):
        got.append(out_to_f64(out_f[0, qb * B:(qb + 1) * B]))
        want.append(O.full_attention(q, k, v, B, True, qb))
    st = assert_outputs_close(np.stack(got), np.stack(want), "bf16", f"dense O at NB={NB}")
    print(f"[large-nb] NB={NB} sampled rows vs oracle {st}")
