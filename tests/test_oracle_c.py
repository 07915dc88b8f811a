"""The plain C oracle (oracle/iqoracle.c) against the pinned numpy oracle (oracle/iqref.py).

The numpy oracle is pinned to the pages and to closed forms in
test_oracle_pins.py; the C oracle, which the benchmark times as the CPU
baseline, must compute the same things: the same codes (bit for bit, except
where rounding order moves a rotated coordinate across a cell boundary, as
for the GPU) and norms (to one float ulp), and the same decode outputs to
1e-12 relative.
"""
import math

import numpy as np
import pytest

import iqinputs
from oracle import iqoracle_c as C
from oracle import iqref as R

C32, T32, _ = R.codebook()
C16, T16, _ = R.codebook(levels=16)
SCALE = 1.0 / math.sqrt(128)


@pytest.mark.parametrize("levels", [8, 16])
def test_c_encode_equals_numpy_oracle(levels):
    thr = T32 if levels == 8 else T16
    rot = iqinputs.rotation_params(3, 0, 1)[0]
    x = iqinputs.kv(3, 0, "k", 3000, 1, "fixed_x8", "f32")[:, 0]
    x = (x.astype(np.float64) * np.random.default_rng(1).uniform(1e-3, 1e3, (3000, 1))).astype(np.float32)
    rows, norms = C.encode(x, rot, thr)
    ref_rows, ref_norms, y = R.rotate_quantize(x, rot, thr)
    assert np.all(np.abs(norms.view(np.int32).astype(np.int64) - ref_norms.view(np.int32)) <= 1)
    got, ref = R.unpack(rows), R.unpack(ref_rows)
    diff = got != ref
    if diff.any():   # only where y / n sits on a cell boundary to rounding order
        u = (y.astype(np.float64) / ref_norms[:, None].astype(np.float64))[diff]
        assert np.min(np.abs(u[:, None] - thr.astype(np.float64)[None, :]), axis=1).max() <= 1e-6
    assert diff.sum() < 1e-5 * diff.size


def test_c_encode_special_vectors():
    rot = iqinputs.rotation_params(4, 0, 1)[0]
    x = np.zeros((3, 128), np.float32)
    x[1, 5] = 2.0
    x[2, :] = np.nan
    rows, norms = C.encode(x, rot, T32)
    ref_rows, ref_norms, _ = R.rotate_quantize(x, rot, T32)
    assert np.array_equal(rows, ref_rows)
    assert norms[0] == 0 and np.isnan(norms[2]) and not rows[2].any()
    assert norms[1] == ref_norms[1]


def _cache(seed, hkv, total, k_bits=3):
    cap = -(-total // 32) * 32
    rot = iqinputs.rotation_params(seed, 0, hkv)
    k = np.zeros((cap, hkv, 128), np.float16)
    v = np.zeros_like(k)
    k[:total] = iqinputs.kv(seed, 0, "k", total, hkv, "student_t6", "f16")
    v[:total] = iqinputs.kv(seed, 0, "v", total, hkv, "student_t6", "f16")
    kr, kn = R.encode_tokens(k, rot, T16 if k_bits == 4 else T32)
    vt, vn = R.encode_tokens_v(v, rot, T32)
    return rot, kr, kn, vt, vn


@pytest.mark.parametrize("hq,hkv,lens,k_bits", [(8, 2, [300, 0, 77], 3), (4, 4, [513], 3), (16, 1, [129, 31], 4)])
def test_c_decode_equals_numpy_oracle(hq, hkv, lens, k_bits):
    lens = np.array(lens, np.int32)
    starts = (np.concatenate([[0], np.cumsum(lens)[:-1]]) + 5).astype(np.int32)
    rot, kr, kn, vt, vn = _cache(hq + hkv, hkv, int(starts[-1] + lens[-1]) + 1, k_bits)
    q = iqinputs.queries(hq, 0, len(lens), hq)
    kc = C16 if k_bits == 4 else C32
    got = C.decode(q, kr, kn, vt, vn, rot, kc, C32, starts, lens, SCALE)
    ref = R.decode_attention(q, kr, kn, vt, vn, rot, starts, lens, SCALE, C32, k_centroids32=kc)
    assert np.max(np.abs(got - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))
    part = C.decode(q, kr, kn, vt, vn, rot, kc, C32, starts, lens, SCALE, heads=[hkv - 1])
    g = hq // hkv
    assert np.array_equal(part[:, (hkv - 1) * g:], got[:, (hkv - 1) * g:]) and np.isnan(part[:, :(hkv - 1) * g]).all()


def test_c_oracle_reports_threads():
    assert C.threads() >= 1
