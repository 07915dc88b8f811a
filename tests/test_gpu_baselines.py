"""GPU parity of the comparison paths: decode over a plain fp16 cache (the
FP16-KV baseline) and the unfused path (iq_dequantize, then that decode).
The oracle is the definition of attention in float64 on the same fp16 K/V
(or, for the unfused path, on the oracle's own reconstruction of the packed
cache). Tolerances as in test_gpu_parity."""
import numpy as np
import pytest
import torch

import iqinputs
import quantized_kv_cache_wht_amd as iq
from oracle import iqref as R
from parity_util import C32, T32, SCALE, _t, _np, _assert_attention_close

pytestmark = pytest.mark.gpu


def _ref_f16(q, k, v, starts, lens, hkv):
    """float64 attention of every (seq, query head) over fp16 K/V [cap][Hkv][128]."""
    n_seqs, hq, _ = q.shape
    g = hq // hkv
    out = np.zeros((n_seqs, hq, 128))
    for s in range(n_seqs):
        a, n = int(starts[s]), int(lens[s])
        for h in range(hkv):
            if n == 0:
                continue
            out[s, h * g:(h + 1) * g] = R.attention(q[s, h * g:(h + 1) * g], k[a:a + n, h].astype(np.float64),
                                                    v[a:a + n, h].astype(np.float64), SCALE)
    return out


@pytest.mark.parametrize("hq,hkv,lens,token_major", [
    (1, 1, [512], True),
    (8, 2, [0, 700, 1300], True),
    (32, 4, [2100], False),
    (16, 1, [513, 3], False),
    (32, 8, [1024, 77, 4000], True),
    (32, 4, [13, 4096], True),
])
def test_f16_decode_matches_oracle(hq, hkv, lens, token_major):
    lens = np.array(lens, np.int32)
    starts = (np.concatenate([[0], np.cumsum(lens)[:-1]]) + 3).astype(np.int32)   # misaligned starts
    cap = -(-(int(starts[-1] + lens[-1]) + 1) // 32) * 32
    k = iqinputs.kv(hq + hkv, 0, "k", cap, hkv, "student_t6", "f16")
    v = iqinputs.kv(hq + hkv, 0, "v", cap, hkv, "student_t6", "f16")
    q = iqinputs.queries(hq, 1, len(lens), hq)
    ref = _ref_f16(q, k, v, starts, lens, hkv)
    kt, vt = (_t(k), _t(v)) if token_major else (_t(k.transpose(1, 0, 2)), _t(v.transpose(1, 0, 2)))
    out = _np(iq.iq_decode_attention_f16(kt, vt, _t(q), _t(starts), _t(lens), int(lens.max()),
                                         token_major=token_major))
    _assert_attention_close(out, ref, f"f16 hq={hq} hkv={hkv} lens={list(lens)} token_major={token_major}")
    for s in np.nonzero(lens == 0)[0]:
        assert np.all(out[s] == 0)


def test_f16_decode_invalid_ranges_give_nan():
    hkv, hq = 2, 4
    k = iqinputs.kv(7, 0, "k", 320, hkv, "fixed_x8", "f16")
    q = iqinputs.queries(7, 0, 3, hq)
    starts = np.array([0, 250, -1], np.int32)
    lens = np.array([100, 100, 5], np.int32)
    out = _np(iq.iq_decode_attention_f16(_t(k), _t(k), _t(q), _t(starts), _t(lens), 150))
    assert np.all(np.isnan(out[1])) and np.all(np.isnan(out[2]))
    _assert_attention_close(out[0], _ref_f16(q[:1], k, k, starts[:1], lens[:1], hkv)[0], "valid beside invalid")


def test_unfused_path_matches_fused_and_oracle():
    """iq_dequantize (fp16) + fp16 decode against the fused packed decode and the oracle's packed attention."""
    w = iqinputs.WORKLOADS["dense8b_gqa_t8192"]
    inp = iqinputs.layer_inputs(w, 2, n_tokens=3000)
    cap = 3008
    cache = iq.PackedKVCache.allocate(w.num_kv_heads, cap, _t(inp["rot"]))
    iq.iq_rotate_quantize_append(cache, _t(inp["k"]), _t(inp["v"]))
    st, ln = _t(inp["seq_start"]), _t(inp["seq_len"])
    fused = _np(iq.iq_decode_attention(cache, _t(inp["q"]), st, ln, 3000))
    k16, v16 = iq.iq_dequantize(cache, 0, cap, torch.float16)
    unfused = _np(iq.iq_decode_attention_f16(k16, v16, _t(inp["q"]), st, ln, 3000, token_major=True))
    k = np.zeros((cap, w.num_kv_heads, 128), np.float16)
    v = np.zeros_like(k)
    k[:3000], v[:3000] = inp["k"], inp["v"]
    kr, kn = R.encode_tokens(k, inp["rot"], T32)
    vt, vn = R.encode_tokens_v(v, inp["rot"], T32)
    ref = R.decode_attention(inp["q"], kr, kn, vt, vn, inp["rot"], inp["seq_start"], inp["seq_len"], SCALE, C32)
    _assert_attention_close(fused, ref, "fused packed decode")
    # the unfused path rounds the reconstruction to fp16 first: its error is that rounding's
    _assert_attention_close(unfused, ref, "unfused: dequantize to fp16 + fp16 decode")


# ------------------------------------------------- deferred quantization ----
@pytest.mark.parametrize("kind,k_bits", [("wht_so4", 3), ("planar", 3), ("wht_so4", 4)])
@pytest.mark.parametrize("pre,suf", [([700, 0, 33], [40, 1, 0]), ([0, 0], [300, 12]), ([2100], [0]),
                                     ([3000, 5], [257, 64])])
def test_deferred_decode_matches_oracle(kind, k_bits, pre, suf):
    hq, hkv = 32, 4
    pre, suf = np.array(pre, np.int32), np.array(suf, np.int32)
    n_seqs = len(pre)
    pst = (np.concatenate([[0], np.cumsum(pre)[:-1]]) + 7).astype(np.int32)
    sst = (np.concatenate([[0], np.cumsum(suf)[:-1]]) + 3).astype(np.int32)
    cap16 = -(-(int(pst[-1] + pre[-1]) + 1) // 32) * 32
    cap = -(-(int(sst[-1] + suf[-1]) + 1) // 32) * 32
    seed = int(pre.sum() + suf.sum())
    rot = iqinputs.rotation_params_kind(seed, 0, hkv, kind)
    k16 = iqinputs.kv(seed, 1, "k", cap16, hkv, "student_t6", "f16")
    v16 = iqinputs.kv(seed, 1, "v", cap16, hkv, "student_t6", "f16")
    k = iqinputs.kv(seed, 2, "k", cap, hkv, "student_t6", "f16")
    v = iqinputs.kv(seed, 2, "v", cap, hkv, "student_t6", "f16")
    c_k, t_k, _ = R.codebook(levels=16 if k_bits == 4 else 8)
    kr, kn = R.encode_tokens(k, rot, t_k)
    vt, vn = R.encode_tokens_v(v, rot, T32)
    cache = iq.PackedKVCache.allocate(hkv, cap, _t(rot), k_bits=k_bits)
    cache.k_codes.copy_(_t(kr))
    cache.v_codes.copy_(_t(vt))
    cache.k_norms.copy_(_t(kn))
    cache.v_norms.copy_(_t(vn))
    q = iqinputs.queries(seed, 3, n_seqs, hq)
    out = _np(iq.iq_decode_attention_deferred(cache, _t(sst), _t(suf), int(suf.max()), _t(k16), _t(v16), _t(pst),
                                              _t(pre), int(pre.max()), _t(q)))
    ref = R.decode_attention_deferred(q, k16, v16, pst, pre, kr, kn, vt, vn, rot, sst, suf, SCALE, C32,
                                      k_centroids32=c_k)
    _assert_attention_close(out, ref, f"deferred {kind} k_bits={k_bits} prefix={list(pre)} suffix={list(suf)}")
    for s in np.nonzero((pre + suf) == 0)[0]:
        assert np.all(out[s] == 0)
