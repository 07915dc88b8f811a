"""Shared helpers of the GPU parity tests: device transfer, the attention
tolerance and the boundary-mismatch rule for codes (see test_gpu_parity)."""
import math

import numpy as np
import torch

from oracle import iqref as R

DEV = "cuda"
C32, T32, _ = R.codebook()
SCALE = 1.0 / math.sqrt(128)


def _t(a, dtype=None):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV) if dtype is None else \
        torch.from_numpy(np.ascontiguousarray(a)).to(DEV, dtype)


def _np(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _assert_attention_close(got, ref, what="", v_scale=1.0):
    """max-abs <= 2e-3 and rel-L2 <= 1e-3. The max-abs bound is stated for V of unit scale; the
    output is linear in V, so for V scaled by v_scale it is 2e-3 * v_scale (rel-L2 is scale-free)."""
    err = np.abs(got - ref)
    max_abs = float(err.max()) if err.size else 0.0
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    print(f"[{what}] max_abs={max_abs:.3e} rel_l2={rel:.3e}", flush=True)
    assert max_abs <= 2e-3 * v_scale and rel <= 1e-3, (what, max_abs, rel)


def _boundary_mismatch_ok(codes_gpu, codes_ref, y_ref, n_ref, thresholds=None):
    """Mismatched codes must sit within 1e-6 of a boundary (in y/n units) and be < 1e-5 of all."""
    diff = codes_gpu != codes_ref
    nd = int(diff.sum())
    if nd:
        u = y_ref[diff].astype(np.float64) / np.broadcast_to(n_ref[..., None], y_ref.shape)[diff].astype(np.float64)
        thr = T32 if thresholds is None else thresholds
        gap = np.min(np.abs(u[:, None] - thr.astype(np.float64)[None, :]), axis=1)
        assert np.all(gap <= 1e-6), gap.max()
        assert np.all(np.abs(codes_gpu[diff].astype(int) - codes_ref[diff].astype(int)) == 1)
    assert nd < 1e-5 * codes_ref.size, (nd, codes_ref.size)
    return nd


