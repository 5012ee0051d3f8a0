"""The library's per-head threshold DP (a host routine of libxattn, no device
work) against the oracle's DP: identical levels and value on the same
errors, including exact ties; and its argument checks."""
import math

import numpy as np
import pytest

import block_sparse_long_stride_amd.xattn as X
import oracle as O


@pytest.mark.parametrize("trial", range(40))
def test_library_dp_equals_oracle(trial):
    rng = np.random.default_rng(5000 + trial)
    H, R = int(rng.integers(1, 40)), int(rng.integers(0, 4))
    inc = rng.exponential(1.0, size=(H, R + 1))
    err = np.cumsum(inc, axis=1)
    if trial % 4 == 0:
        err = np.round(err * 2) / 2          # exact ties exercise the tie rule
    for steps in sorted({0, H * R, int(rng.integers(0, H * R + 1))}):
        lv_lib, best_lib = X.xattn_tau_dp(err, steps)
        lv_ora, best_ora = O.tau_dp(err, steps)
        assert lv_lib == lv_ora
        assert best_lib == best_ora          # same operations in the same order


def test_library_dp_rejects():
    lib = X.lib()
    import ctypes
    e = np.zeros((4, 3))
    ep = e.ctypes.data_as(ctypes.c_void_p)
    out = np.zeros(4, dtype=np.int32)
    op = out.ctypes.data_as(ctypes.c_void_p)
    assert lib.xattn_tau_dp(4, 2, ep, 9, op, None) == X.XATTN_EINVAL     # > hq * levels
    assert lib.xattn_tau_dp(4, 2, ep, -1, op, None) == X.XATTN_EINVAL
    assert lib.xattn_tau_dp(0, 2, ep, 0, op, None) == X.XATTN_EINVAL
    assert lib.xattn_tau_dp(4, -1, ep, 0, op, None) == X.XATTN_EINVAL
    assert lib.xattn_tau_dp(4, 2, None, 0, op, None) == X.XATTN_EINVAL
    e[1, 1] = math.nan
    assert lib.xattn_tau_dp(4, 2, ep, 2, op, None) == X.XATTN_EINVAL
    assert lib.xattn_tau_dp(100000, 1000, ep, 100000, op, None) == X.XATTN_EUNSUPPORTED
