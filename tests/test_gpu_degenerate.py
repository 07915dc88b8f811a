"""Degenerate inputs of the decode (MI355X only), against the oracle.

The method is defined for every input; these are the cases where the
attention reduces to something simple and where the kernel's scaling steps
meet zeros: a query head that is all zero (every score 0, so attention is the
plain mean of the reconstructed V), a softmax scale of 0 and a negative scale,
sequences of one token, K rows of norm 0 (all codes 0, every score 0), V of
norm 0 (output 0), and a sequence whose tokens are all the same (output = that
token's V). Tolerances as in test_gpu_parity (max-abs 2e-3, relative L2 1e-3)."""
import numpy as np
import pytest

import iqinputs
import quantized_kv_cache_wht_amd as iq
from oracle import iqref as R

pytestmark = pytest.mark.gpu
from parity_util import C32, T32, SCALE, _t, _np, _assert_attention_close  # noqa: E402


def _cache(rot, k, v):
    kr, kn = R.encode_tokens(k, rot, T32)
    vt, vn = R.encode_tokens_v(v, rot, T32)
    hkv, cap = kr.shape[:2]
    c = iq.PackedKVCache.allocate(hkv, cap, _t(rot))
    c.k_codes.copy_(_t(kr))
    c.v_codes.copy_(_t(vt))
    c.k_norms.copy_(_t(kn))
    c.v_norms.copy_(_t(vn))
    return c, (kr, kn, vt, vn)


def _kv(seed, cap, hkv):
    k = np.zeros((cap, hkv, 128), np.float16)
    v = np.zeros_like(k)
    k[:] = iqinputs.kv(seed, 0, "k", cap, hkv, "student_t6", "f16")
    v[:] = iqinputs.kv(seed, 0, "v", cap, hkv, "student_t6", "f16")
    return k, v


@pytest.mark.parametrize("hq,hkv", [(8, 1), (32, 4)])
@pytest.mark.parametrize("scale", [SCALE, 0.0, -SCALE])
def test_zero_queries_and_degenerate_scales(hq, hkv, scale):
    cap = 2048
    rot = iqinputs.rotation_params(61, 0, hkv)
    k, v = _kv(61, cap, hkv)
    cache, (kr, kn, vt, vn) = _cache(rot, k, v)
    lens = np.array([1500, 1, 37], np.int32)
    starts = np.array([0, 1600, 1700], np.int32)
    q = iqinputs.queries(61, 1, len(lens), hq)
    q[:, 0] = 0.0          # the first query head of every sequence is zero
    q[1, hq - 1] = 0.0
    out = _np(iq.iq_decode_attention(cache, _t(q), _t(starts), _t(lens), 1500, scale=scale))
    ref = R.decode_attention(q, kr, kn, vt, vn, rot, starts, lens, scale, C32)
    _assert_attention_close(out, ref, f"zero query heads, scale={scale:+.3f} hq={hq} hkv={hkv}")
    # a zero query (or scale 0) weighs every token alike: the plain mean of the reconstructed V
    s, a, n = 0, 0, 1500
    mean = R.dequantize_codes(R.v_codes_range(vt[0], a, n), vn[0, a:a + n], rot[0], C32).mean(axis=0)
    _assert_attention_close(out[s, 0], mean, "zero query = mean of V")
    if scale == 0.0:
        for h in range(hkv):
            mean_h = R.dequantize_codes(R.v_codes_range(vt[h], a, n), vn[h, a:a + n], rot[h], C32).mean(axis=0)
            g = hq // hkv
            _assert_attention_close(out[s, h * g:(h + 1) * g], np.broadcast_to(mean_h, (g, 128)), "scale 0")


def test_zero_norm_rows_and_identical_tokens():
    hkv, hq = 2, 8
    cap = 1024
    rot = iqinputs.rotation_params(62, 0, hkv)
    k, v = _kv(62, cap, hkv)
    k[100:400] = 0.0                     # K rows of norm 0: all codes 0, every score 0
    v[500:700] = 0.0                     # V rows of norm 0: output 0
    k[800:1000] = k[800]                 # one token repeated
    v[800:1000] = v[800]
    cache, (kr, kn, vt, vn) = _cache(rot, k, v)
    assert np.all(kn[:, 100:400] == 0) and np.all(kr[:, 100:400] == 0)
    lens = np.array([300, 200, 200, 600], np.int32)
    starts = np.array([100, 500, 800, 50], np.int32)   # the last one mixes zero-norm K rows with others
    q = iqinputs.queries(62, 1, len(lens), hq)
    out = _np(iq.iq_decode_attention(cache, _t(q), _t(starts), _t(lens), 600))
    ref = R.decode_attention(q, kr, kn, vt, vn, rot, starts, lens, SCALE, C32)
    _assert_attention_close(out, ref, "zero-norm rows and identical tokens")
    assert np.all(out[1] == 0)           # every V of sequence 1 has norm 0
    for h in range(hkv):                 # identical tokens: the output is that token's V
        v1 = R.dequantize_codes(R.v_codes_range(vt[h], 800, 1), vn[h, 800:801], rot[h], C32)[0]
        g = hq // hkv
        _assert_attention_close(out[2, h * g:(h + 1) * g], np.broadcast_to(v1, (g, 128)), "identical tokens")
