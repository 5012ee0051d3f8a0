"""The C-ABI library loads without a GPU, exports every entry point that
include/xattn.h declares, and rejects malformed arguments before any HIP
call (so these checks run on the CPU)."""
import ctypes
import os
import re

import numpy as np
import pytest

import block_sparse_long_stride_amd.xattn as X

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "xattn.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(xattn_[a-z_]+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert _declared() == sorted(X.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = X.lib()
    for name in _declared():
        assert hasattr(lib, name), name
    assert lib.xattn_version() == 1


def _shape(**kw):
    d = dict(hq=4, hkv=2, L=4096, d=128, dtype=X.XATTN_BF16, causal=1)
    d.update(kw)
    return X.Shape(d["hq"], d["hkv"], d["L"], d["d"], d["dtype"], d["causal"])


DUMMY = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first


def _score(sh, S=16, B=128, ws_bytes=1 << 40):
    lib = X.lib()
    return lib.xattn_score(ctypes.byref(sh), DUMMY, DUMMY, S, B, DUMMY, DUMMY, ws_bytes, None)


@pytest.mark.parametrize("kw,S,B,status", [
    (dict(hq=3, hkv=2), 16, 128, X.XATTN_EINVAL),          # hq % hkv
    (dict(L=4000), 16, 128, X.XATTN_EINVAL),               # L % B
    (dict(), 24, 128, X.XATTN_EINVAL),                     # B % S
    (dict(dtype=7), 16, 128, X.XATTN_EINVAL),
    (dict(causal=2), 16, 128, X.XATTN_EINVAL),
    (dict(L=0), 16, 128, X.XATTN_EINVAL),
    (dict(), 0, 128, X.XATTN_EINVAL),
    (dict(d=96), 16, 128, X.XATTN_EUNSUPPORTED),           # bf16 d
    (dict(), 2, 128, X.XATTN_EUNSUPPORTED),                # B/S = 64
    (dict(), 16, 32, X.XATTN_EUNSUPPORTED),                # B/S = 2
])
def test_score_rejects(kw, S, B, status):
    assert _score(_shape(**kw), S, B) == status
    assert X.lib().xattn_last_error()


def test_score_rejects_heads_beyond_32_bit_buffers():
    lib = X.lib()
    sh = _shape(hq=1, hkv=1, L=1 << 23, d=128)   # 2^31 bytes per head
    assert lib.xattn_score(ctypes.byref(sh), DUMMY, DUMMY, 16, 128, DUMMY, DUMMY, 1 << 40,
                           None) == X.XATTN_EUNSUPPORTED
    assert b"2^31" in lib.xattn_last_error()


def test_attention_rejects_heads_beyond_32_bit_buffers():
    lib = X.lib()
    sh = _shape(hq=1, hkv=1, L=1 << 23, d=128)   # 2^31 bytes per KV head
    assert lib.xattn_full(ctypes.byref(sh), DUMMY, DUMMY, DUMMY, DUMMY, None) == X.XATTN_EUNSUPPORTED
    assert b"2^31" in lib.xattn_last_error()


def test_score_workspace_checks():
    lib = X.lib()
    sh = _shape()
    need = lib.xattn_score_workspace_bytes(ctypes.byref(sh), 16, 128)
    Lr, NB = 4096 // 16, 4096 // 128
    assert need == 4 * (sh.hq * (Lr // 32) * NB * 32 + 2 * sh.hq * (Lr // 32) * ((Lr + 63) // 64) * 32)
    assert _score(sh, ws_bytes=need - 1) == X.XATTN_EWORKSPACE
    assert lib.xattn_score(ctypes.byref(sh), DUMMY, DUMMY, 16, 128, DUMMY, None, need, None) == X.XATTN_EINVAL
    assert lib.xattn_score(ctypes.byref(sh), None, DUMMY, 16, 128, DUMMY, DUMMY, need, None) == X.XATTN_EINVAL
    assert lib.xattn_score_workspace_bytes(ctypes.byref(_shape(hq=3)), 16, 128) == 0
    fp32 = _shape(dtype=X.XATTN_FP32)
    assert lib.xattn_score_workspace_bytes(ctypes.byref(fp32), 16, 128) == 0


def test_score_pattern_rejects():
    lib = X.lib()
    sh = _shape()

    def call(ph, S=16):
        arr = (ctypes.c_int32 * max(1, len(ph)))(*ph) if ph is not None else None
        return lib.xattn_score_pattern(ctypes.byref(sh), DUMMY, DUMMY, S, 128, arr, DUMMY, DUMMY,
                                       1 << 40, None)

    assert call(None) == X.XATTN_EINVAL
    assert call([0] * 16) == X.XATTN_EINVAL                          # repeated entry
    assert call(list(range(15)) + [16]) == X.XATTN_EINVAL            # out of range
    assert call(list(range(15)) + [-1]) == X.XATTN_EINVAL
    assert b"permutation" in lib.xattn_last_error()
    assert call(list(range(128)), S=128) == X.XATTN_EUNSUPPORTED     # S > 64
    # a valid permutation still goes through the shape checks
    sh.L = 4000
    assert call(list(range(16))) == X.XATTN_EINVAL


def test_fused_and_dit_reject():
    lib = X.lib()
    sh = _shape()
    tau = np.full(4, 0.9, dtype=np.float32)
    tp = tau.ctypes.data_as(ctypes.c_void_p)
    need = lib.xattn_score_workspace_bytes(ctypes.byref(sh), 16, 128)
    fused = lambda **kw: lib.xattn_score_select(
        ctypes.byref(kw.get("sh", sh)), DUMMY, DUMMY, 16, 128, kw.get("tau", tp), DUMMY, DUMMY,
        DUMMY, kw.get("ws", DUMMY), kw.get("bytes", need), None)
    assert fused(bytes=need - 1) == X.XATTN_EWORKSPACE
    assert fused(ws=None) == X.XATTN_EINVAL
    assert fused(tau=None) == X.XATTN_EINVAL
    bad = np.array([0.9, 0.9, 1.5, 0.9], dtype=np.float32)
    assert fused(tau=bad.ctypes.data_as(ctypes.c_void_p)) == X.XATTN_EINVAL
    assert fused(sh=_shape(dtype=X.XATTN_FP32)) == X.XATTN_EUNSUPPORTED
    dneed = lib.xattn_dit_workspace_bytes(ctypes.byref(sh), 16, 128)
    assert dneed > need
    dit = lambda step, warm=5, bytes=dneed, ws=DUMMY: lib.xattn_dit_attention(
        ctypes.byref(sh), DUMMY, DUMMY, DUMMY, 16, 128, tp, step, warm, DUMMY, ws, bytes, None)
    assert dit(-1) == X.XATTN_EINVAL
    assert dit(7, warm=-2) == X.XATTN_EINVAL
    assert dit(7, bytes=dneed - 1) == X.XATTN_EWORKSPACE
    assert dit(7, ws=None) == X.XATTN_EINVAL
    assert lib.xattn_dit_workspace_bytes(ctypes.byref(_shape(L=4000)), 16, 128) == 0


def test_select_rejects():
    lib = X.lib()

    def call(hq=2, NB=8, causal=1, tau=(0.9, 0.9), null=False):
        t = np.asarray(tau, dtype=np.float32)
        return lib.xattn_select(hq, NB, causal, DUMMY, t.ctypes.data_as(ctypes.c_void_p),
                                None if null else DUMMY, DUMMY, DUMMY, None)

    assert call(tau=(0.9, 0.0)) == X.XATTN_EINVAL
    assert call(tau=(1.5, 0.9)) == X.XATTN_EINVAL
    assert call(tau=(float("nan"), 0.9)) == X.XATTN_EINVAL
    assert call(NB=0) == X.XATTN_EINVAL
    assert call(causal=3) == X.XATTN_EINVAL
    assert call(null=True) == X.XATTN_EINVAL
    assert call(NB=4097) == X.XATTN_EUNSUPPORTED
    assert call(hq=129, tau=np.full(129, 0.9)) == X.XATTN_EUNSUPPORTED


def test_select_cut_rules_reject():
    lib = X.lib()

    def topk(hq=2, NB=8, causal=1, k=4, null=False):
        return lib.xattn_select_topk(hq, NB, causal, DUMMY, k, None if null else DUMMY, DUMMY,
                                     DUMMY, None)

    def ratio(hq=2, NB=8, causal=1, r=0.27, null=False):
        return lib.xattn_select_topratio(hq, NB, causal, DUMMY, r, DUMMY, DUMMY,
                                         None if null else DUMMY, None)

    assert topk(k=0) == X.XATTN_EINVAL
    assert topk(k=-3) == X.XATTN_EINVAL
    assert topk(NB=0) == X.XATTN_EINVAL
    assert topk(causal=2) == X.XATTN_EINVAL
    assert topk(null=True) == X.XATTN_EINVAL
    assert topk(NB=4097) == X.XATTN_EUNSUPPORTED
    assert ratio(r=0.0) == X.XATTN_EINVAL
    assert ratio(r=1.01) == X.XATTN_EINVAL
    assert ratio(r=float("nan")) == X.XATTN_EINVAL
    assert ratio(hq=0) == X.XATTN_EINVAL
    assert ratio(null=True) == X.XATTN_EINVAL
    assert ratio(NB=5000) == X.XATTN_EUNSUPPORTED
    assert b"k_blocks" in lib.xattn_last_error() or b"NB" in lib.xattn_last_error()


def test_attention_rejects():
    lib = X.lib()
    sh = _shape()
    assert lib.xattn_sparse_prefill(ctypes.byref(sh), DUMMY, DUMMY, DUMMY, 256, DUMMY, DUMMY, DUMMY,
                                    None) == X.XATTN_EUNSUPPORTED
    assert lib.xattn_sparse_prefill(ctypes.byref(sh), DUMMY, DUMMY, DUMMY, 100, DUMMY, DUMMY, DUMMY,
                                    None) == X.XATTN_EINVAL
    assert lib.xattn_sparse_prefill(ctypes.byref(sh), DUMMY, DUMMY, DUMMY, 128, None, DUMMY, DUMMY,
                                    None) == X.XATTN_EINVAL
    # bf16, B = 128, d = 128: the merged block list of NB = 7489 blocks no
    # longer fits in LDS beside the K/V tiles (7488 does)
    big = _shape(hq=1, hkv=1, L=7489 * 128)
    assert lib.xattn_sparse_prefill(ctypes.byref(big), DUMMY, DUMMY, DUMMY, 128, DUMMY, DUMMY,
                                    DUMMY, None) == X.XATTN_EUNSUPPORTED
    assert b"LDS" in lib.xattn_last_error()
    assert lib.xattn_full(ctypes.byref(_shape(L=4000)), DUMMY, DUMMY, DUMMY, DUMMY,
                          None) == X.XATTN_EUNSUPPORTED
    assert lib.xattn_full(ctypes.byref(_shape(d=80)), DUMMY, DUMMY, DUMMY, DUMMY,
                          None) == X.XATTN_EUNSUPPORTED
    assert lib.xattn_full(None, DUMMY, DUMMY, DUMMY, DUMMY, None) == X.XATTN_EINVAL


def test_status_strings():
    lib = X.lib()
    for s in range(5):
        assert lib.xattn_status_str(s)


def test_binding_rejects_host_tensors_before_any_library_call():
    """The Python layer hands the kernels device pointers only: host tensors
    are refused before the library is called."""
    import torch
    Q = torch.zeros((2, 256, 64), dtype=torch.bfloat16)
    K = torch.zeros((1, 256, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        X.xattn_score(Q, K, 8, 64, True)
    with pytest.raises(ValueError):
        X.xattn_select(torch.zeros((2, 4, 4), dtype=torch.float32), [0.9, 0.9], True)
    with pytest.raises(ValueError):
        X.xattn_select_topk(torch.zeros((2, 4, 4), dtype=torch.float32), 2, True)
    with pytest.raises(ValueError):
        X.xattn_sparse_prefill(Q, K, K, 64, None, None, True)
    with pytest.raises(ValueError):
        X.xattn_full(Q, K, K, True)
    with pytest.raises(ValueError):
        X.xattn_select(torch.zeros((2, 4, 5), dtype=torch.float32), [0.9, 0.9], True)


MIS = ctypes.c_void_p(0x1008)   # 8-byte aligned only


def test_every_entry_point_rejects_misaligned_device_buffers():
    """The kernels read and write through 16-byte vector and direct-to-LDS
    accesses: a device pointer off a 16-byte boundary is refused up front."""
    lib = X.lib()
    sh = _shape()
    tau = (ctypes.c_float * 4)(0.9, 0.9, 0.9, 0.9)
    phase = (ctypes.c_int32 * 16)(*range(16))
    E = X.XATTN_EINVAL
    for i in range(4):
        a = [MIS if j == i else DUMMY for j in range(4)]
        assert lib.xattn_score(ctypes.byref(sh), a[0], a[1], 16, 128, a[2], a[3], 1 << 40, None) == E
        assert b"16-byte" in lib.xattn_last_error()
        assert lib.xattn_score_pattern(ctypes.byref(sh), a[0], a[1], 16, 128, phase, a[2], a[3],
                                       1 << 40, None) == E
        assert lib.xattn_select(4, 32, 1, a[0], tau, a[1], a[2], a[3], None) == E
        assert lib.xattn_select_topk(4, 32, 1, a[0], 2, a[1], a[2], a[3], None) == E
        assert lib.xattn_select_topratio(4, 32, 1, a[0], 0.27, a[1], a[2], a[3], None) == E
        assert lib.xattn_full(ctypes.byref(sh), a[0], a[1], a[2], a[3], None) == E
    for i in range(6):
        a = [MIS if j == i else DUMMY for j in range(6)]
        assert lib.xattn_sparse_prefill(ctypes.byref(sh), a[0], a[1], a[2], 128, a[4], a[5], a[3],
                                        None) == E
        assert lib.xattn_score_select(ctypes.byref(sh), a[0], a[1], 16, 128, tau, a[2], a[3], a[4],
                                      a[5], 1 << 40, None) == E
    for i in range(5):
        a = [MIS if j == i else DUMMY for j in range(5)]
        assert lib.xattn_dit_attention(ctypes.byref(sh), a[0], a[1], a[2], 16, 128, tau, 7, 5, a[3],
                                       a[4], 1 << 40, None) == E
    assert lib.xattn_head_error(ctypes.byref(sh), MIS, DUMMY, DUMMY, None) == E


def test_fp32_sparse_prefill_bounds_its_lds_bitmap():
    """fp32 sparse prefill keeps a bitmap of NB bits beside its key/value
    tiles: a block count whose bitmap no longer fits in one CU's LDS is
    refused before any launch."""
    lib = X.lib()
    big = _shape(hq=1, hkv=1, L=1 << 21, d=128, dtype=X.XATTN_FP32)
    # B = 1: NB = 2^21 blocks, a 256 KB bitmap beside 32 KB of tiles: too much
    assert lib.xattn_sparse_prefill(ctypes.byref(big), DUMMY, DUMMY, DUMMY, 1, DUMMY, DUMMY, DUMMY,
                                    None) == X.XATTN_EUNSUPPORTED
    assert b"LDS" in lib.xattn_last_error()


def test_noalloc_score_refuses_shapes_beyond_its_scratch():
    """xattn_score_noalloc works in a fixed 64 MiB device array: a shape whose
    scoring workspace is larger is refused before any device work."""
    lib = X.lib()
    big = _shape(hq=32, hkv=8, L=32768)
    need = lib.xattn_score_workspace_bytes(ctypes.byref(big), 8, 128)
    assert need > 64 << 20
    assert lib.xattn_score_noalloc(ctypes.byref(big), DUMMY, DUMMY, 8, 128, DUMMY,
                                   None) == X.XATTN_EWORKSPACE
    assert b"scratch" in lib.xattn_last_error()
    fits = _shape(hq=32, hkv=8, L=16384)
    assert lib.xattn_score_workspace_bytes(ctypes.byref(fits), 8, 128) <= 64 << 20
    assert lib.xattn_score_noalloc(ctypes.byref(fits), MIS, DUMMY, 8, 128, DUMMY,
                                   None) == X.XATTN_EINVAL
    assert lib.xattn_score_noalloc(ctypes.byref(fits), DUMMY, DUMMY, 8, 100, DUMMY,
                                   None) == X.XATTN_EINVAL
    assert lib.xattn_score_noalloc(ctypes.byref(fits), DUMMY, None, 8, 128, DUMMY,
                                   None) == X.XATTN_EINVAL
