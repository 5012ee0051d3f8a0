"""Python binding of libxattn (ctypes).

Argument marshalling only: torch tensors supply device pointers, the current
HIP stream supplies the stream, and every step of the path runs in the
library's HIP kernels.  Functions keep the C names.  If libxattn.so is missing
the functions raise; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libxattn.so")

XATTN_OK, XATTN_EINVAL, XATTN_EUNSUPPORTED, XATTN_EWORKSPACE, XATTN_EHIP = range(5)
XATTN_FP32, XATTN_BF16 = 0, 1
XATTN_SCORE_SCRATCH_BYTES = 64 << 20   # fixed scratch of xattn_score_noalloc (include/xattn.h)

# every entry point declared in include/xattn.h
EXPORTS = ("xattn_score_workspace_bytes", "xattn_score", "xattn_score_noalloc",
           "xattn_score_pattern", "xattn_select",
           "xattn_select_topk",
           "xattn_select_topratio", "xattn_score_select", "xattn_sparse_prefill", "xattn_full",
           "xattn_dit_workspace_bytes", "xattn_dit_attention", "xattn_head_error", "xattn_tau_dp",
           "xattn_status_str",
           "xattn_last_error", "xattn_version")


class XattnError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where} failed with status {status}: {detail}")
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [("hq", ctypes.c_int32), ("hkv", ctypes.c_int32), ("L", ctypes.c_int32),
                ("d", ctypes.c_int32), ("dtype", ctypes.c_int32), ("causal", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libxattn.so (built in-tree by block_sparse_long_stride_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m block_sparse_long_stride_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    SP = ctypes.POINTER(Shape)
    L.xattn_score_workspace_bytes.argtypes = [SP, I32, I32]
    L.xattn_score_workspace_bytes.restype = SZ
    L.xattn_score.argtypes = [SP, P, P, I32, I32, P, P, SZ, P]
    L.xattn_score.restype = I32
    L.xattn_score_noalloc.argtypes = [SP, P, P, I32, I32, P, P]
    L.xattn_score_noalloc.restype = I32
    L.xattn_score_pattern.argtypes = [SP, P, P, I32, I32, P, P, P, SZ, P]
    L.xattn_score_pattern.restype = I32
    L.xattn_select.argtypes = [I32, I32, I32, P, P, P, P, P, P]
    L.xattn_select.restype = I32
    L.xattn_select_topk.argtypes = [I32, I32, I32, P, I32, P, P, P, P]
    L.xattn_select_topk.restype = I32
    L.xattn_select_topratio.argtypes = [I32, I32, I32, P, ctypes.c_float, P, P, P, P]
    L.xattn_select_topratio.restype = I32
    L.xattn_score_select.argtypes = [SP, P, P, I32, I32, P, P, P, P, P, SZ, P]
    L.xattn_score_select.restype = I32
    L.xattn_dit_workspace_bytes.argtypes = [SP, I32, I32]
    L.xattn_dit_workspace_bytes.restype = SZ
    L.xattn_dit_attention.argtypes = [SP, P, P, P, I32, I32, P, I32, I32, P, P, SZ, P]
    L.xattn_dit_attention.restype = I32
    L.xattn_head_error.argtypes = [SP, P, P, P, P]
    L.xattn_head_error.restype = I32
    L.xattn_tau_dp.argtypes = [I32, I32, P, I32, P, P]
    L.xattn_tau_dp.restype = I32
    L.xattn_sparse_prefill.argtypes = [SP, P, P, P, I32, P, P, P, P]
    L.xattn_sparse_prefill.restype = I32
    L.xattn_full.argtypes = [SP, P, P, P, P, P]
    L.xattn_full.restype = I32
    L.xattn_status_str.argtypes = [I32]
    L.xattn_status_str.restype = ctypes.c_char_p
    L.xattn_last_error.argtypes = []
    L.xattn_last_error.restype = ctypes.c_char_p
    L.xattn_version.argtypes = []
    L.xattn_version.restype = I32
    _lib = L
    return L


def _check(status: int, where: str) -> None:
    if status != XATTN_OK:
        raise XattnError(status, where, lib().xattn_last_error().decode())


def _torch():
    import torch
    return torch


def _stream(stream) -> int:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(getattr(stream, "cuda_stream", stream))


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _device_buffer(t, name: str, shape, dtype, device) -> None:
    """A caller-supplied buffer must be exactly what the kernels index: a
    contiguous tensor of this shape and dtype on the inputs' device."""
    if not (t.is_cuda and t.device == device and t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous tensor on {device}")
    if t.dtype != dtype or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be {dtype} of shape {tuple(shape)}, "
                         f"got {t.dtype} {tuple(t.shape)}")


def _byte_buffer(t, name: str, device) -> int:
    if not (t.is_cuda and t.device == device and t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous tensor on {device}")
    return t.numel() * t.element_size()


def shape_of(Q, K, causal: bool) -> Shape:
    torch = _torch()
    if Q.dim() != 3 or K.dim() != 3:
        raise ValueError("Q must be [hq][L][d] and K [hkv][L][d]")
    if Q.dtype == torch.bfloat16:
        dt = XATTN_BF16
    elif Q.dtype == torch.float32:
        dt = XATTN_FP32
    else:
        raise ValueError(f"unsupported dtype {Q.dtype}")
    if K.dtype != Q.dtype or Q.shape[1:] != K.shape[1:]:
        raise ValueError("Q and K must share dtype, L and d")
    for t in (Q, K):
        if not (t.is_cuda and t.device == Q.device and t.is_contiguous()):
            raise ValueError("Q and K must be contiguous tensors on one device")
    return Shape(Q.shape[0], K.shape[0], Q.shape[1], Q.shape[2], dt, int(bool(causal)))


def xattn_score_workspace_bytes(shape: Shape, S: int, B: int) -> int:
    return int(lib().xattn_score_workspace_bytes(ctypes.byref(shape), S, B))


def xattn_score(Q, K, S: int, B: int, causal: bool, scores=None, workspace=None, stream=None,
                phase: Optional[Sequence[int]] = None):
    """Block scores, fp32 [hq][NB][NB].  `phase` (a permutation of 0..S-1)
    selects another sampling pattern through xattn_score_pattern; None is the
    antidiagonal (xattn_score)."""
    torch = _torch()
    import numpy as np
    sh = shape_of(Q, K, causal)
    NB = sh.L // B if B > 0 else 0
    if scores is None:
        scores = torch.empty((sh.hq, NB, NB), dtype=torch.float32, device=Q.device)
    else:
        _device_buffer(scores, "scores", (sh.hq, NB, NB), torch.float32, Q.device)
    need = xattn_score_workspace_bytes(sh, S, B)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=Q.device)
    ws_bytes = 0 if workspace is None else _byte_buffer(workspace, "workspace", Q.device)
    if phase is None:
        _check(lib().xattn_score(ctypes.byref(sh), _ptr(Q), _ptr(K), S, B, _ptr(scores),
                                 _ptr(workspace), ws_bytes, _stream(stream)), "xattn_score")
    else:
        ph = np.ascontiguousarray(np.asarray(phase, dtype=np.int32))
        if ph.shape != (S,):
            raise ValueError(f"phase must hold S = {S} entries")
        _check(lib().xattn_score_pattern(ctypes.byref(sh), _ptr(Q), _ptr(K), S, B,
                                         ph.ctypes.data_as(ctypes.c_void_p), _ptr(scores),
                                         _ptr(workspace), ws_bytes, _stream(stream)),
               "xattn_score_pattern")
    return scores


def xattn_score_noalloc(Q, K, S: int, B: int, causal: bool, scores=None, stream=None):
    """Block scores through the library's fixed scratch (no workspace; the
    caller may pass a preallocated `scores` to allocate nothing at all)."""
    torch = _torch()
    sh = shape_of(Q, K, causal)
    NB = sh.L // B if B > 0 else 0
    if scores is None:
        scores = torch.empty((sh.hq, NB, NB), dtype=torch.float32, device=Q.device)
    else:
        _device_buffer(scores, "scores", (sh.hq, NB, NB), torch.float32, Q.device)
    _check(lib().xattn_score_noalloc(ctypes.byref(sh), _ptr(Q), _ptr(K), S, B, _ptr(scores),
                                     _stream(stream)), "xattn_score_noalloc")
    return scores


def xattn_select(scores, tau: Sequence[float], causal: bool, mask=None, idx=None, counts=None,
                 stream=None) -> Tuple:
    """(mask uint64-as-int64 [hq][NB][words], idx int32 [hq][NB][NB], counts int32 [hq][NB])."""
    hq, NB, mask, idx, counts = _select_outputs(scores, mask, idx, counts)
    tau_np = _tau_host(tau, hq)
    _check(lib().xattn_select(hq, NB, int(bool(causal)), _ptr(scores),
                              tau_np.ctypes.data_as(ctypes.c_void_p), _ptr(mask), _ptr(idx),
                              _ptr(counts), _stream(stream)), "xattn_select")
    return mask, idx, counts


def _mask_idx_counts(hq, NB, mask, idx, counts, device):
    """Selection outputs: allocated when None, else checked against the
    layout the kernels write."""
    torch = _torch()
    words = (NB + 63) // 64
    outs = []
    for t, name, shp, dt in ((mask, "mask", (hq, NB, words), torch.int64),
                             (idx, "idx", (hq, NB, NB), torch.int32),
                             (counts, "counts", (hq, NB), torch.int32)):
        if t is None:
            t = torch.empty(shp, dtype=dt, device=device)
        else:
            _device_buffer(t, name, shp, dt, device)
        outs.append(t)
    return outs


def _select_outputs(scores, mask, idx, counts):
    torch = _torch()
    if scores.dim() != 3 or scores.shape[1] != scores.shape[2]:
        raise ValueError("scores must be [hq][NB][NB]")
    hq, NB = scores.shape[0], scores.shape[1]
    if not (scores.is_cuda and scores.is_contiguous() and scores.dtype == torch.float32):
        raise ValueError("scores must be a contiguous fp32 device tensor")
    mask, idx, counts = _mask_idx_counts(hq, NB, mask, idx, counts, scores.device)
    return hq, NB, mask, idx, counts


def xattn_select_topk(scores, k_blocks: int, causal: bool, mask=None, idx=None, counts=None,
                      stream=None) -> Tuple:
    """Top-K cut (k_blocks blocks per query block) of the selection ranking."""
    hq, NB, mask, idx, counts = _select_outputs(scores, mask, idx, counts)
    _check(lib().xattn_select_topk(hq, NB, int(bool(causal)), _ptr(scores), int(k_blocks),
                                   _ptr(mask), _ptr(idx), _ptr(counts), _stream(stream)),
           "xattn_select_topk")
    return mask, idx, counts


def xattn_select_topratio(scores, ratio: float, causal: bool, mask=None, idx=None, counts=None,
                          stream=None) -> Tuple:
    """Top-Ratio cut (nearest integer to ratio x valid blocks) of the selection ranking."""
    hq, NB, mask, idx, counts = _select_outputs(scores, mask, idx, counts)
    _check(lib().xattn_select_topratio(hq, NB, int(bool(causal)), _ptr(scores), float(ratio),
                                       _ptr(mask), _ptr(idx), _ptr(counts), _stream(stream)),
           "xattn_select_topratio")
    return mask, idx, counts


def _tau_host(tau, hq):
    import numpy as np
    return np.ascontiguousarray(np.broadcast_to(np.asarray(tau, dtype=np.float32), (hq,)))


def xattn_score_select(Q, K, S: int, B: int, tau: Sequence[float], causal: bool, mask=None,
                       idx=None, counts=None, workspace=None, stream=None) -> Tuple:
    """Fused scoring + threshold selection (no score matrix): (mask, idx, counts)."""
    torch = _torch()
    sh = shape_of(Q, K, causal)
    NB = sh.L // B if B > 0 else 0
    mask, idx, counts = _mask_idx_counts(sh.hq, NB, mask, idx, counts, Q.device)
    need = xattn_score_workspace_bytes(sh, S, B)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=Q.device)
    ws_bytes = _byte_buffer(workspace, "workspace", Q.device)
    t = _tau_host(tau, sh.hq)
    _check(lib().xattn_score_select(ctypes.byref(sh), _ptr(Q), _ptr(K), S, B,
                                    t.ctypes.data_as(ctypes.c_void_p), _ptr(mask), _ptr(idx),
                                    _ptr(counts), _ptr(workspace), ws_bytes, _stream(stream)),
           "xattn_score_select")
    return mask, idx, counts


def xattn_dit_workspace_bytes(sh: Shape, S: int, B: int) -> int:
    return int(lib().xattn_dit_workspace_bytes(ctypes.byref(sh), S, B))


def xattn_dit_attention(Q, K, V, S: int, B: int, tau: Sequence[float], step: int,
                        warmup_steps: int = 5, causal: bool = False, out=None, workspace=None,
                        stream=None):
    """One denoising step's attention under the full-attention warm-up policy."""
    torch = _torch()
    sh = shape_of(Q, K, causal)
    _check_v(V, K)
    out = _attn_out(out, Q)
    if workspace is None and step >= warmup_steps:
        workspace = torch.empty(max(xattn_dit_workspace_bytes(sh, S, B), 1), dtype=torch.uint8,
                                device=Q.device)
    ws_bytes = 0 if workspace is None else _byte_buffer(workspace, "workspace", Q.device)
    t = _tau_host(tau, sh.hq)
    _check(lib().xattn_dit_attention(ctypes.byref(sh), _ptr(Q), _ptr(K), _ptr(V), S, B,
                                     t.ctypes.data_as(ctypes.c_void_p), int(step),
                                     int(warmup_steps), _ptr(out), _ptr(workspace), ws_bytes,
                                     _stream(stream)), "xattn_dit_attention")
    return out


def xattn_head_error(O_sparse, O_dense, err=None, stream=None):
    """Per-head relative squared error of two [hq][L][d] outputs (float64 [hq])."""
    torch = _torch()
    if O_sparse.shape != O_dense.shape or O_sparse.dtype != O_dense.dtype or O_sparse.dim() != 3:
        raise ValueError("O_sparse and O_dense must be [hq][L][d] tensors of one dtype")
    for t in (O_sparse, O_dense):
        if not (t.is_cuda and t.device == O_dense.device and t.is_contiguous()):
            raise ValueError("outputs must be contiguous tensors on one device")
    hq, L, d = O_dense.shape
    dt = XATTN_BF16 if O_dense.dtype == torch.bfloat16 else XATTN_FP32
    sh = Shape(hq, hq, L, d, dt, 0)
    if err is None:
        err = torch.empty(hq, dtype=torch.float64, device=O_dense.device)
    else:
        _device_buffer(err, "err", (hq,), torch.float64, O_dense.device)
    _check(lib().xattn_head_error(ctypes.byref(sh), _ptr(O_sparse), _ptr(O_dense), _ptr(err),
                                  _stream(stream)), "xattn_head_error")
    return err


def xattn_tau_dp(err, steps: int) -> Tuple[list, float]:
    """Host DP over threshold-reduction steps: err[h][k] (k = 0 .. levels)."""
    import numpy as np
    e = np.ascontiguousarray(np.asarray(err, dtype=np.float64))
    if e.ndim != 2:
        raise ValueError("err must be [hq][levels + 1]")
    hq, r1 = e.shape
    out = np.zeros(hq, dtype=np.int32)
    best = ctypes.c_double(0.0)
    _check(lib().xattn_tau_dp(hq, r1 - 1, e.ctypes.data_as(ctypes.c_void_p), int(steps),
                              out.ctypes.data_as(ctypes.c_void_p), ctypes.byref(best)),
           "xattn_tau_dp")
    return [int(x) for x in out], float(best.value)


def _check_v(V, K) -> None:
    if V.shape != K.shape or V.dtype != K.dtype or not (V.is_cuda and V.device == K.device
                                                         and V.is_contiguous()):
        raise ValueError("V must match K (shape, dtype, device) and be contiguous")


def _attn_out(out, Q):
    if out is None:
        return _torch().empty_like(Q)
    _device_buffer(out, "out", tuple(Q.shape), Q.dtype, Q.device)
    return out


def xattn_sparse_prefill(Q, K, V, B: int, idx, counts, causal: bool, out=None, stream=None):
    torch = _torch()
    sh = shape_of(Q, K, causal)
    _check_v(V, K)
    if B < 1 or sh.L % B:
        raise ValueError(f"L = {sh.L} must be a positive multiple of B = {B}")
    NB = sh.L // B
    _device_buffer(idx, "idx", (sh.hq, NB, NB), torch.int32, Q.device)
    _device_buffer(counts, "counts", (sh.hq, NB), torch.int32, Q.device)
    out = _attn_out(out, Q)
    _check(lib().xattn_sparse_prefill(ctypes.byref(sh), _ptr(Q), _ptr(K), _ptr(V), B, _ptr(idx),
                                      _ptr(counts), _ptr(out), _stream(stream)),
           "xattn_sparse_prefill")
    return out


def xattn_full(Q, K, V, causal: bool, out=None, stream=None):
    sh = shape_of(Q, K, causal)
    _check_v(V, K)
    out = _attn_out(out, Q)
    _check(lib().xattn_full(ctypes.byref(sh), _ptr(Q), _ptr(K), _ptr(V), _ptr(out),
                            _stream(stream)), "xattn_full")
    return out
