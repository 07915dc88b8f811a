"""GPU parity of the decode paths over the range of V and K magnitudes.

Attention is defined for any real K and V (zhichai.net essay, section
"为什么压缩 KV 缓存这么难？": softmax(Q K^T / sqrt(d)) V), so the packed
decode must hold the tolerance whatever the scale of the norms, not only for
the unit-scale synthetic data of the other tests:
  * every V norm scaled by 1e-6 .. 1e6 (the output scales with it);
  * V norms that differ by eight orders of magnitude within one sequence;
  * a sharp softmax (scale 10/sqrt(128), and K norms x 8);
  * a planted needle key whose V norm is 1e-5 of its neighbours' (the token
    that dominates the softmax carries the smallest V);
and the same through the fused decode step, the deferred (fp16 prefix +
packed suffix) decode, the fp16 decode and 4-bit K.

The caches are encoded by the oracle and their norms then scaled in float32;
both sides read the same codes and norms. Tolerance: rel-L2 <= 1e-3, and
max-abs <= 2e-3 times the scale of V (the output is linear in V).
"""
import math

import numpy as np
import pytest

import iqinputs
import quantized_kv_cache_wht_amd as iq
from oracle import iqref as R
from parity_util import C32, T32, SCALE, _t, _np, _assert_attention_close

pytestmark = pytest.mark.gpu

C16, T16, _ = R.codebook(levels=16)


def _oracle_cache(seed, hkv, total, k_bits=3, outliers="student_t6"):
    """Oracle-encoded cache of ``total`` slots (rounded up to 32; padding slots encode zeros)."""
    cap = -(-max(total, 1) // 32) * 32
    rot = iqinputs.rotation_params(seed, 0, hkv)
    k = np.zeros((cap, hkv, 128), np.float16)
    v = np.zeros_like(k)
    k[:total] = iqinputs.kv(seed, 0, "k", total, hkv, outliers, "f16")
    v[:total] = iqinputs.kv(seed, 0, "v", total, hkv, outliers, "f16")
    kr, kn = R.encode_tokens(k, rot, T16 if k_bits == 4 else T32)
    vt, vn = R.encode_tokens_v(v, rot, T32)
    return rot, kr, kn, vt, vn


def _upload(rot, kr, kn, vt, vn, k_bits=3):
    hkv, cap, _ = kr.shape
    cache = iq.PackedKVCache.allocate(hkv, cap, _t(rot), k_bits=k_bits)
    cache.k_codes.copy_(_t(kr))
    cache.v_codes.copy_(_t(vt))
    cache.k_norms.copy_(_t(kn))
    cache.v_norms.copy_(_t(vn))
    return cache


def _layout(lens, pad=3):
    lens = np.array(lens, np.int32)
    starts = (np.concatenate([[0], np.cumsum(lens)[:-1]]) + pad).astype(np.int32)
    return starts, lens, int(starts[-1] + lens[-1]) + 1


GROUPS = [(4, 4), (32, 4), (16, 1)]    # (Hq, Hkv): G = 1, 8, 16


@pytest.mark.parametrize("hq,hkv", GROUPS)
@pytest.mark.parametrize("vs", [1e-6, 1e-3, 1e3, 1e6])
def test_decode_v_scaled(hq, hkv, vs):
    starts, lens, total = _layout([3000, 77])
    rot, kr, kn, vt, vn = _oracle_cache(hq + 3 * hkv, hkv, total)
    vn = (vn * np.float32(vs)).astype(np.float32)
    cache = _upload(rot, kr, kn, vt, vn)
    q = iqinputs.queries(hq, 7, len(lens), hq)
    out = _np(iq.iq_decode_attention(cache, _t(q), _t(starts), _t(lens), int(lens.max())))
    ref = R.decode_attention(q, kr, kn, vt, vn, rot, starts, lens, SCALE, C32)
    _assert_attention_close(out, ref, f"V x {vs:g} hq={hq} hkv={hkv}", v_scale=vs)


@pytest.mark.parametrize("hq,hkv", GROUPS)
def test_decode_v_norms_spanning_eight_decades(hq, hkv):
    """Per-token V norms scaled by 10^u, u ~ U(-4, 4): within one 32-slot block the largest V norm
    is ~1e8 times the smallest, so the softmax reference must follow them token by token."""
    starts, lens, total = _layout([2500, 600])
    rot, kr, kn, vt, vn = _oracle_cache(hq * 5 + hkv, hkv, total)
    f = 10.0 ** np.random.default_rng(hq + hkv).uniform(-4, 4, vn.shape)
    vn = (vn * f).astype(np.float32)
    cache = _upload(rot, kr, kn, vt, vn)
    q = iqinputs.queries(hq, 8, len(lens), hq)
    out = _np(iq.iq_decode_attention(cache, _t(q), _t(starts), _t(lens), int(lens.max())))
    ref = R.decode_attention(q, kr, kn, vt, vn, rot, starts, lens, SCALE, C32)
    _assert_attention_close(out, ref, f"V norms 1e-4..1e4 hq={hq} hkv={hkv}", v_scale=float(np.abs(ref).max()))


@pytest.mark.parametrize("hq,hkv", GROUPS)
@pytest.mark.parametrize("k_scale,scale", [(1.0, 10.0 / math.sqrt(128)), (8.0, 1.0 / math.sqrt(128)),
                                           (8.0, 10.0 / math.sqrt(128))])
def test_decode_sharp_softmax(hq, hkv, k_scale, scale):
    starts, lens, total = _layout([2100, 300])
    rot, kr, kn, vt, vn = _oracle_cache(hq * 11 + hkv, hkv, total)
    kn = (kn * np.float32(k_scale)).astype(np.float32)
    cache = _upload(rot, kr, kn, vt, vn)
    q = iqinputs.queries(hq, 9, len(lens), hq)
    out = _np(iq.iq_decode_attention(cache, _t(q), _t(starts), _t(lens), int(lens.max()), scale=scale))
    ref = R.decode_attention(q, kr, kn, vt, vn, rot, starts, lens, scale, C32)
    _assert_attention_close(out, ref, f"sharp K x {k_scale:g} scale {scale:.3f} hq={hq} hkv={hkv}")


@pytest.mark.parametrize("hq,hkv", GROUPS)
def test_decode_needle_with_tiny_v(hq, hkv):
    """The needle key K[p] = 4 q (first query head of each group) dominates the softmax while its V
    norm is 1e-5 of the others': the output mixes that tiny V with the small weights of the rest."""
    T = 4000
    hkv_rot = iqinputs.rotation_params(hq + 17, 0, hkv)
    k = iqinputs.kv(hq + 17, 0, "k", T, hkv, "fixed_x8", "f16")
    v = iqinputs.kv(hq + 17, 0, "v", T, hkv, "fixed_x8", "f16")
    q = iqinputs.queries(hq, 10, 1, hq)
    p = 1234
    iqinputs.plant_needle(k, q[0], p, hq // hkv)
    kr, kn = R.encode_tokens(k, hkv_rot, T32)
    vt, vn = R.encode_tokens_v(v, hkv_rot, T32)
    vn[:, p] *= np.float32(1e-5)
    cache = _upload(hkv_rot, kr, kn, vt, vn)
    st, ln = np.array([0], np.int32), np.array([T], np.int32)
    out = _np(iq.iq_decode_attention(cache, _t(q), _t(st), _t(ln), T))
    ref = R.decode_attention(q, kr, kn, vt, vn, hkv_rot, st, ln, SCALE, C32)
    _assert_attention_close(out, ref, f"needle with V x 1e-5 hq={hq} hkv={hkv}")


@pytest.mark.parametrize("vs", [1e-5, 1e5])
@pytest.mark.parametrize("hq,hkv", [(32, 4), (16, 1)])
def test_append_decode_v_scaled_end_to_end(vs, hq, hkv):
    """fp32 K/V with V scaled by vs, encoded by the GPU (bulk append) and one fused decode step; the
    oracle encodes the same inputs and attends over the grown cache."""
    lens = np.array([1500, 41], np.int32)
    starts = (np.concatenate([[0], np.cumsum(lens + 1)[:-1]]) + 2).astype(np.int32)
    cap = -(-(int(starts[-1] + lens[-1]) + 1) // 32) * 32
    seed = 600 + hq
    rot = iqinputs.rotation_params(seed, 0, hkv)
    k = iqinputs.kv(seed, 0, "k", cap, hkv, "student_t6", "f32")
    v = (iqinputs.kv(seed, 0, "v", cap, hkv, "student_t6", "f32").astype(np.float64) * vs).astype(np.float32)
    new_slots = starts + lens
    q = iqinputs.queries(seed, 1, len(lens), hq)
    cache = iq.PackedKVCache.allocate(hkv, cap, _t(rot))
    iq.iq_rotate_quantize_append(cache, _t(k), _t(v), first_slot=0)
    out = _np(iq.iq_append_decode_attention(cache, _t(k[new_slots]), _t(v[new_slots]), _t(q), _t(starts),
                                            _t(lens), int(lens.max())))
    kr, kn = R.encode_tokens(k, rot, T32)
    vt, vn = R.encode_tokens_v(v, rot, T32)
    ref = R.decode_attention(q, kr, kn, vt, vn, rot, starts, lens + 1, SCALE, C32)
    _assert_attention_close(out, ref, f"fused step, V x {vs:g} hq={hq} hkv={hkv}", v_scale=vs)


@pytest.mark.parametrize("vs", [1e-3, 1e2])
def test_deferred_decode_v_scaled(vs):
    """fp16 prefix V scaled by vs (in fp16) and packed suffix V norms scaled by vs."""
    hq, hkv = 32, 4
    pre, suf = np.array([1500, 40], np.int32), np.array([700, 300], np.int32)
    pst = (np.concatenate([[0], np.cumsum(pre)[:-1]]) + 5).astype(np.int32)
    sst = (np.concatenate([[0], np.cumsum(suf)[:-1]]) + 1).astype(np.int32)
    cap16 = -(-(int(pst[-1] + pre[-1]) + 1) // 32) * 32
    seed = 700
    rot, kr, kn, vt, vn = _oracle_cache(seed, hkv, int(sst[-1] + suf[-1]) + 1)
    vn = (vn * np.float32(vs)).astype(np.float32)
    k16 = iqinputs.kv(seed, 1, "k", cap16, hkv, "student_t6", "f16")
    v16 = (iqinputs.kv(seed, 1, "v", cap16, hkv, "student_t6", "f32").astype(np.float64) * vs).astype(np.float16)
    cache = _upload(rot, kr, kn, vt, vn)
    q = iqinputs.queries(seed, 3, len(pre), hq)
    out = _np(iq.iq_decode_attention_deferred(cache, _t(sst), _t(suf), int(suf.max()), _t(k16), _t(v16), _t(pst),
                                              _t(pre), int(pre.max()), _t(q)))
    ref = R.decode_attention_deferred(q, k16, v16, pst, pre, kr, kn, vt, vn, rot, sst, suf, SCALE, C32)
    _assert_attention_close(out, ref, f"deferred V x {vs:g}", v_scale=vs)


@pytest.mark.parametrize("vs,scale", [(1e-3, 1.0 / math.sqrt(128)), (1.0, 10.0 / math.sqrt(128))])
def test_f16_decode_v_scaled_and_sharp(vs, scale):
    hq, hkv = 32, 8
    starts, lens, total = _layout([2000, 500])
    cap = -(-total // 32) * 32
    k = iqinputs.kv(801, 0, "k", cap, hkv, "student_t6", "f16")
    v = (iqinputs.kv(801, 0, "v", cap, hkv, "student_t6", "f32").astype(np.float64) * vs).astype(np.float16)
    q = iqinputs.queries(801, 1, len(lens), hq)
    out = _np(iq.iq_decode_attention_f16(_t(k), _t(v), _t(q), _t(starts), _t(lens), int(lens.max()), scale=scale))
    g = hq // hkv
    ref = np.zeros_like(out, dtype=np.float64)
    for s in range(len(lens)):
        a, n = int(starts[s]), int(lens[s])
        for h in range(hkv):
            ref[s, h * g:(h + 1) * g] = R.attention(q[s, h * g:(h + 1) * g], k[a:a + n, h].astype(np.float64),
                                                    v[a:a + n, h].astype(np.float64), scale)
    _assert_attention_close(out, ref, f"fp16 decode V x {vs:g} scale {scale:.3f}", v_scale=vs)


@pytest.mark.parametrize("vs", [1e-5, 1e4])
def test_decode_k4_v_scaled(vs):
    hq, hkv = 32, 4
    starts, lens, total = _layout([2200, 15])
    rot, kr, kn, vt, vn = _oracle_cache(901, hkv, total, k_bits=4)
    vn = (vn * np.float32(vs)).astype(np.float32)
    cache = _upload(rot, kr, kn, vt, vn, k_bits=4)
    q = iqinputs.queries(901, 1, len(lens), hq)
    out = _np(iq.iq_decode_attention(cache, _t(q), _t(starts), _t(lens), int(lens.max())))
    ref = R.decode_attention(q, kr, kn, vt, vn, rot, starts, lens, SCALE, C32, k_centroids32=C16)
    _assert_attention_close(out, ref, f"4-bit K, V x {vs:g}", v_scale=vs)
