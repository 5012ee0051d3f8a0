"""The Python binding refuses caller-supplied device buffers whose shape,
dtype or layout differs from what the kernels index (no kernel is launched
for a refused call)."""
import pytest

pytestmark = pytest.mark.gpu


def test_binding_checks_output_buffers():
    import torch
    import block_sparse_long_stride_amd.xattn as X
    dev = "cuda"
    hq, hkv, L, d, S, B = 2, 1, 1024, 64, 8, 64
    NB = L // B
    Q = torch.zeros((hq, L, d), dtype=torch.bfloat16, device=dev)
    K = torch.zeros((hkv, L, d), dtype=torch.bfloat16, device=dev)
    sc = torch.zeros((hq, NB, NB), dtype=torch.float32, device=dev)
    print("[binding] output buffer checks", flush=True)
    with pytest.raises(ValueError):   # scores one row short
        X.xattn_score(Q, K, S, B, True, scores=torch.zeros((hq, NB - 1, NB), device=dev))
    with pytest.raises(ValueError):   # idx of the wrong dtype
        X.xattn_select(sc, [0.9] * hq, True, idx=torch.zeros((hq, NB, NB), dtype=torch.int64,
                                                            device=dev))
    with pytest.raises(ValueError):   # mask with too few words
        X.xattn_select_topratio(sc, 0.5, True, mask=torch.zeros((hq, NB, 0), dtype=torch.int64,
                                                               device=dev))
    with pytest.raises(ValueError):   # counts not contiguous
        X.xattn_score_select(Q, K, S, B, [0.9] * hq, True,
                             counts=torch.zeros((NB, hq), dtype=torch.int32, device=dev).t())
    idx = torch.zeros((hq, NB, NB), dtype=torch.int32, device=dev)
    cnt = torch.zeros((hq, NB), dtype=torch.int32, device=dev)
    with pytest.raises(ValueError):   # idx for another B
        X.xattn_sparse_prefill(Q, K, K, B, idx[:, :, :NB // 2].contiguous(), cnt, True)
    with pytest.raises(ValueError):   # out of the wrong shape
        X.xattn_full(Q, K, K, True, out=torch.zeros((hq, L, d + 1), dtype=torch.bfloat16,
                                                    device=dev))
    # well-formed buffers pass and the call runs
    m, i, c = X.xattn_select(sc, [0.9] * hq, True)
    torch.cuda.synchronize()
    assert m.shape == (hq, NB, 1) and i.shape == (hq, NB, NB) and c.shape == (hq, NB)
