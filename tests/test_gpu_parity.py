"""GPU parity of the HIP path against the CPU oracle (MI355X only).

Tolerances (stated by the method's spec and restated here):
  * codes and norms: bit-exact when both sides quantize the same float32
    rotated vectors (``iq_quantize_pack``); through the full encode
    (``iq_rotate_quantize_append``, where the GPU rotates in float32) a code
    may differ only where the oracle's y/n lies within 1e-6 of a cell
    boundary, and such codes must be fewer than 1e-5 of all codes;
  * attention outputs: max-abs error <= 2e-3 and relative L2 error <= 1e-3.
"""
import math

import numpy as np
import pytest
import torch

import iqinputs
import quantized_kv_cache_wht_amd as iq
from oracle import iqref as R

pytestmark = pytest.mark.gpu
from parity_util import C32, T32, SCALE, DEV, _t, _np, _assert_attention_close, _boundary_mismatch_ok  # noqa: E402


# ------------------------------------------------------------- rotation ----
@pytest.mark.parametrize("kind", iqinputs.ROTATION_KINDS)
@pytest.mark.parametrize("n_tok,heads", [(1, 1), (300, 3), (4096, 8)])
def test_rotate_matches_oracle(n_tok, heads, kind):
    rot = iqinputs.rotation_params_kind(101, n_tok, heads, kind)
    x = np.random.default_rng(n_tok).standard_normal((n_tok, heads, 128)).astype(np.float32) * 5
    y = _np(iq.iq_rotate(_t(rot), _t(x)))
    ref = np.stack([R.rotate(x[:, h].astype(np.float64), rot[h]) for h in range(heads)], axis=1)
    scale = np.linalg.norm(x.astype(np.float64), axis=-1, keepdims=True)
    assert np.max(np.abs(y - ref) / scale) < 2e-6
    back = _np(iq.iq_rotate(_t(rot), _t(y), inverse=True))
    assert np.max(np.abs(back - x) / scale) < 4e-6


# ------------------------------------------------------ quantize + pack ----
def test_quantize_pack_bit_exact_on_same_rotated_input():
    g = np.random.default_rng(5)
    rot = iqinputs.rotation_params(5, 0, 1)[0]
    x = iqinputs.kv(5, 0, "k", 6000, 1, "fixed_x8", "f32")[:, 0].astype(np.float64)
    x *= g.uniform(1e-3, 1e3, (6000, 1))
    y = R.rotate(x, rot).astype(np.float32)
    extra = np.zeros((9, 128), np.float32)
    extra[1, 7] = 2.5                                     # single nonzero: zeros land on the tie at 0
    extra[2] = np.nan
    extra[3] = np.float32(1e-20) * np.ones(128, np.float32)
    extra[4, :] = -1.0
    # non-finite norms: one NaN dim; a norm past the fp32 range; single +inf and -inf dims
    extra[5, :] = 1.0
    extra[5, 9] = np.nan
    extra[6, :] = 1e38
    extra[7, :] = -0.5
    extra[7, 3] = np.inf
    extra[8, :] = 0.25
    extra[8, 100] = -np.inf
    # exact ties at the positive and negative boundaries (norm fixed to 1)
    ties = []
    for k in range(7):
        a = np.float32(T32[k])
        b = np.float32(np.sqrt(1.0 - float(a) ** 2))
        v = np.zeros(128, np.float32)
        v[0], v[1] = b, a
        ties.append(v)
    y = np.concatenate([y, extra, np.array(ties)], axis=0)
    codes_ref, n_ref = R.quantize(y, T32)
    rows_ref = R.pack(codes_ref)
    codes, norms = iq.iq_quantize_pack(_t(y))
    codes, norms = _np(codes), _np(norms)
    assert np.array_equal(codes, rows_ref)
    nan = np.isnan(n_ref)
    assert np.array_equal(np.isnan(norms), nan)
    assert np.array_equal(norms[~nan].view(np.uint32), n_ref[~nan].view(np.uint32))


# --------------------------------------------------------------- append ----
def _encode_ref(x, rot):
    """Oracle encode of [n][Hkv][128]: codes [Hkv][n][128], norms, y32."""
    hkv = x.shape[1]
    out_c, out_n, out_y = [], [], []
    for h in range(hkv):
        y32 = R.rotate(x[:, h].astype(np.float64), rot[h]).astype(np.float32)
        c, n = R.quantize(y32, T32)
        out_c.append(c), out_n.append(n), out_y.append(y32)
    return np.stack(out_c), np.stack(out_n), np.stack(out_y)


@pytest.mark.parametrize("wname,n_tok,first", [("single_head_t512", 512, 0), ("dense8b_gqa_t8192", 1000, 37),
                                               ("moe30b_gqa_t32768", 333, 5),
                                               # short appends (the 16-lane kernel)
                                               ("single_head_t512", 1, 511), ("dense8b_gqa_t8192", 5, 35),
                                               ("moe30b_gqa_t32768", 64, 3), ("dense8b_gqa_t8192", 65, 8)])
def test_append_matches_oracle(wname, n_tok, first):
    w = iqinputs.WORKLOADS[wname]
    rot = iqinputs.rotation_params(w.seed, 0, w.num_kv_heads)
    k = iqinputs.kv(w.seed, 0, "k", n_tok, w.num_kv_heads, w.outliers, w.dtype)
    v = iqinputs.kv(w.seed, 0, "v", n_tok, w.num_kv_heads, w.outliers, w.dtype)
    cache = iq.PackedKVCache.allocate(w.num_kv_heads, first + n_tok + 3, _t(rot))
    iq.iq_rotate_quantize_append(cache, _t(k), _t(v), first_slot=first)
    total = 0
    cap = cache.capacity
    for name, x in (("k", k), ("v", v)):
        codes_ref, n_ref, y_ref = _encode_ref(x, rot)
        if name == "k":
            all_codes = R.unpack(_np(cache.k_codes))
        else:
            all_codes = R.unpack_tiles(_np(cache.v_codes))
        assert all_codes.shape == (w.num_kv_heads, cap, 128)
        norms = _np(getattr(cache, f"{name}_norms"))[:, first:first + n_tok]
        total += _boundary_mismatch_ok(all_codes[:, first:first + n_tok], codes_ref, y_ref, n_ref)
        assert np.max(np.abs(norms - n_ref) / n_ref) < 2e-6
        assert not all_codes[:, :first].any() and not all_codes[:, first + n_tok:].any()
    print(f"boundary mismatches: {total}")


def test_append_v_tiles_keep_neighbours():
    """Appends that start and end inside V tiles leave the other slots of those tiles intact, and
    the short-append and bulk kernels encode identically."""
    hkv = 2
    rot = iqinputs.rotation_params(21, 0, hkv)
    x = iqinputs.kv(21, 0, "v", 224, hkv, "student_t6", "f16")
    cache = iq.PackedKVCache.allocate(hkv, 224, _t(rot))
    # calls covering slots 0..223: short ones [0, 13), [13, 14), [150, 151), [151, 224), a bulk one [14, 150)
    for a0, a1 in [(0, 13), (13, 14), (14, 150), (150, 151), (151, 224)]:
        iq.iq_rotate_quantize_append(cache, _t(x[a0:a1]), _t(x[a0:a1]), first_slot=a0)
    one = iq.PackedKVCache.allocate(hkv, 224, _t(rot))
    iq.iq_rotate_quantize_append(one, _t(x), _t(x), first_slot=0)
    assert torch.equal(cache.v_codes, one.v_codes) and torch.equal(cache.k_codes, one.k_codes)
    assert torch.equal(cache.v_norms, one.v_norms)


@pytest.mark.parametrize("n", [70, 40])     # bulk kernel, short-append kernel
def test_append_with_slot_list_and_out_of_range_slots(n):
    hkv = 2
    rot = iqinputs.rotation_params(9, 0, hkv)
    k = iqinputs.kv(9, 0, "k", n, hkv, "student_t6", "f16")
    v = iqinputs.kv(9, 0, "v", n, hkv, "student_t6", "f16")
    slots = np.random.default_rng(1).permutation(100)[:n].astype(np.int32)
    slots[3] = -1
    slots[10] = 100                       # == capacity: skipped
    cache = iq.PackedKVCache.allocate(hkv, 100, _t(rot))
    iq.iq_rotate_quantize_append(cache, _t(k), _t(v), slots=_t(slots))
    assert cache.capacity == 128
    slots[10] = 128                       # beyond the rounded-up capacity: skipped
    cache = iq.PackedKVCache.allocate(hkv, 100, _t(rot))
    iq.iq_rotate_quantize_append(cache, _t(k), _t(v), slots=_t(slots))
    good = (slots >= 0) & (slots < 128)
    written = np.zeros(128, bool)
    written[slots[good]] = True
    for name, x, codes_all in (("k", k, R.unpack(_np(cache.k_codes))), ("v", v, R.unpack_tiles(_np(cache.v_codes)))):
        codes_ref, n_ref, y_ref = _encode_ref(x, rot)
        _boundary_mismatch_ok(codes_all[:, slots[good]], codes_ref[:, good], y_ref[:, good], n_ref[:, good])
        assert not codes_all[:, ~written].any()


# ------------------------------------------------------------ dequantize ----
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.float16])
def test_dequantize_matches_oracle(out_dtype):
    hkv, n = 3, 800
    rot = iqinputs.rotation_params(3, 1, hkv)
    x = iqinputs.kv(3, 1, "k", n, hkv, "fixed_x8", "f32")
    codes, norms = R.encode_codes(x, rot, T32)
    vcodes = codes[:, ::-1].copy()
    vnorms = norms[:, ::-1].copy()
    cache = iq.PackedKVCache.allocate(hkv, n, _t(rot))
    cache.k_codes.copy_(_t(R.pack(codes)))
    cache.v_codes.copy_(_t(R.pack_tiles(vcodes)))
    cache.k_norms.copy_(_t(norms))
    cache.v_norms.copy_(_t(vnorms))
    k_out, v_out = iq.iq_dequantize(cache, 101, 600, out_dtype)
    k_out, v_out = _np(k_out).astype(np.float64), _np(v_out).astype(np.float64)
    tol = 2e-6 if out_dtype == torch.float32 else 1e-3
    for h in range(hkv):
        ref_k = R.dequantize_codes(codes[h, 101:701], norms[h, 101:701], rot[h], C32)
        ref_v = R.dequantize_codes(vcodes[h, 101:701], vnorms[h, 101:701], rot[h], C32)
        assert np.max(np.abs(k_out[:, h] - ref_k) / norms[h, 101:701, None]) < tol
        assert np.max(np.abs(v_out[:, h] - ref_v) / vnorms[h, 101:701, None]) < tol


# ---------------------------------------------------------------- decode ----
def _oracle_cache(seed, hkv, total, outliers="student_t6", dtype="f16", kind="wht_so4"):
    """Oracle-encoded cache of ``total`` slots rounded up to a multiple of 32 (padding slots encode zeros)."""
    cap = -(-max(total, 1) // 32) * 32
    rot = iqinputs.rotation_params_kind(seed, 0, hkv, kind)
    k = np.zeros((cap, hkv, 128), np.float16 if dtype == "f16" else np.float32)
    v = np.zeros_like(k)
    k[:total] = iqinputs.kv(seed, 0, "k", total, hkv, outliers, dtype)
    v[:total] = iqinputs.kv(seed, 0, "v", total, hkv, outliers, dtype)
    kr, kn = R.encode_tokens(k, rot, T32)
    vt, vn = R.encode_tokens_v(v, rot, T32)
    return rot, kr, kn, vt, vn


def _upload(rot, kr, kn, vt, vn):
    hkv, cap, _ = kr.shape
    cache = iq.PackedKVCache.allocate(hkv, cap, _t(rot))
    assert cache.capacity == cap
    cache.k_codes.copy_(_t(kr))
    cache.v_codes.copy_(_t(vt))
    cache.k_norms.copy_(_t(kn))
    cache.v_norms.copy_(_t(vn))
    return cache


@pytest.mark.parametrize("hq,hkv,lens", [
    (1, 1, [512]),
    (2, 1, [1, 255, 256, 257]),
    (8, 2, [0, 700, 1300]),
    (32, 4, [2100]),
    (16, 1, [513, 3]),
    (32, 8, [1024, 77, 4000]),
    (32, 4, [13, 4096]),          # start 13: one block more than an aligned start, taken by the last split
    (4, 1, [31, 1024, 1]),
])
def test_decode_matches_oracle(hq, hkv, lens):
    lens = np.array(lens, np.int32)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int32)
    total = int(lens.sum())
    rot, kr, kn, vr, vn = _oracle_cache(hq * 100 + hkv, hkv, total + 5)
    cache = _upload(rot, kr, kn, vr, vn)
    q = iqinputs.queries(hq, 0, len(lens), hq)
    out = _np(iq.iq_decode_attention(cache, _t(q), _t(starts), _t(lens), int(lens.max())))
    ref = R.decode_attention(q, kr, kn, vr, vn, rot, starts, lens, SCALE, C32)
    _assert_attention_close(out, ref, f"hq={hq} hkv={hkv} lens={list(lens)}")
    for s in np.nonzero(lens == 0)[0]:
        assert np.all(out[s] == 0)


@pytest.mark.parametrize("hq,hkv,start,n", [
    (32, 4, 31, 2100),     # last start whose row still begins in block 0
    (32, 4, 32, 2100),     # first start that does not
    (32, 4, 100, 1),
    (8, 8, 5000, 700),     # fewer live blocks than splits times waves
    (16, 1, 3000, 9000),
    (4, 1, 60, 65),
])
def test_decode_single_sequence_at_any_start(hq, hkv, start, n):
    """One sequence per launch: a row that does not begin at slot 0 of its cache row, in a cache with
    more slots before and after it."""
    total = start + n + 40
    rot, kr, kn, vr, vn = _oracle_cache(start + n, hkv, total)
    cache = _upload(rot, kr, kn, vr, vn)
    starts, lens = np.array([start], np.int32), np.array([n], np.int32)
    q = iqinputs.queries(hq, 2, 1, hq)
    out = _np(iq.iq_decode_attention(cache, _t(q), _t(starts), _t(lens), n))
    ref = R.decode_attention(q, kr, kn, vr, vn, rot, starts, lens, SCALE, C32)
    _assert_attention_close(out, ref, f"hq={hq} hkv={hkv} start={start} len={n}")


def test_decode_invalid_ranges_give_nan_and_no_fault():
    hkv, hq = 2, 4
    rot, kr, kn, vr, vn = _oracle_cache(77, hkv, 300)
    cache = _upload(rot, kr, kn, vr, vn)
    starts = np.array([0, 250, -1, 10], np.int32)
    lens = np.array([100, 100, 5, 200], np.int32)       # seq 1 runs past capacity (320), seq 2 negative start
    assert cache.capacity == 320
    q = iqinputs.queries(3, 0, 4, hq)
    out = _np(iq.iq_decode_attention(cache, _t(q), _t(starts), _t(lens), 150))   # seq 3 exceeds max_seq_len
    assert np.all(np.isnan(out[1])) and np.all(np.isnan(out[2])) and np.all(np.isnan(out[3]))
    ref = R.decode_attention(q, kr, kn, vr, vn, rot, starts, lens, SCALE, C32, seqs=[0])
    _assert_attention_close(out[0], ref[0], "valid seq beside invalid ones")


def test_decode_is_deterministic():
    hkv, hq = 4, 32
    rot, kr, kn, vr, vn = _oracle_cache(5, hkv, 5000)
    cache = _upload(rot, kr, kn, vr, vn)
    q = _t(iqinputs.queries(5, 0, 1, hq))
    st, ln = _t(np.array([0], np.int32)), _t(np.array([5000], np.int32))
    a = _np(iq.iq_decode_attention(cache, q, st, ln, 5000))
    b = _np(iq.iq_decode_attention(cache, q, st, ln, 5000))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_decode_reuses_one_workspace_across_shapes():
    """One uninitialised workspace serves calls of different shapes."""
    hkv, hq = 4, 32
    rot, kr, kn, vr, vn = _oracle_cache(41, hkv, 9000)
    cache = _upload(rot, kr, kn, vr, vn)
    q = iqinputs.queries(41, 0, 3, hq)
    ws = iq.decode_workspace(3, hq, hkv, 9000)
    ws.fill_(0xFF)                                       # NaN bit patterns: nothing may depend on the contents
    for lens, ml in [([9000], 9000), ([100, 5000, 1], 9000), ([40, 40, 40], 64), ([9000], 9000), ([3000, 0, 2999], 3000)]:
        lens = np.array(lens, np.int32)
        starts = np.array([0, 3000, 6000][:len(lens)], np.int32) if len(lens) > 1 else np.array([0], np.int32)
        qq = q[:len(lens)]
        got = _np(iq.iq_decode_attention(cache, _t(qq), _t(starts), _t(lens), ml, workspace=ws))
        fresh = _np(iq.iq_decode_attention(cache, _t(qq), _t(starts), _t(lens), ml))
        assert np.array_equal(got.view(np.uint32), fresh.view(np.uint32)), list(lens)
        ref = R.decode_attention(qq, kr, kn, vr, vn, rot, starts, lens, SCALE, C32)
        _assert_attention_close(got, ref, f"reused workspace lens={list(lens)}")


def test_single_head_workload_end_to_end():
    """512 fp32 tokens, one head: GPU encode + GPU decode vs the oracle's encode + attention."""
    w = iqinputs.WORKLOADS["single_head_t512"]
    inp = iqinputs.layer_inputs(w, 0)
    cache = iq.PackedKVCache.allocate(1, 512, _t(inp["rot"]))
    iq.iq_rotate_quantize_append(cache, _t(inp["k"]), _t(inp["v"]))
    out = _np(iq.iq_decode_attention(cache, _t(inp["q"]), _t(inp["seq_start"]), _t(inp["seq_len"]), 512))
    kr, kn = R.encode_tokens(inp["k"], inp["rot"], T32)
    vr, vn = R.encode_tokens_v(inp["v"], inp["rot"], T32)
    ref = R.decode_attention(inp["q"], kr, kn, vr, vn, inp["rot"], inp["seq_start"], inp["seq_len"], SCALE, C32)
    _assert_attention_close(out, ref, "single_head_t512 end to end")


# ------------------------------------------------------ rotation variants ----
@pytest.mark.parametrize("kind", ["iso", "planar"])
@pytest.mark.parametrize("n_tok,first", [(700, 13), (1, 500), (40, 21)])   # bulk and short appends
def test_append_variants_match_oracle(kind, n_tok, first):
    hkv = 4
    rot = iqinputs.rotation_params_kind(17, 0, hkv, kind)
    k = iqinputs.kv(17, 0, "k", n_tok, hkv, "fixed_x8", "f16")
    v = iqinputs.kv(17, 0, "v", n_tok, hkv, "fixed_x8", "f16")
    cache = iq.PackedKVCache.allocate(hkv, first + n_tok, _t(rot))
    iq.iq_rotate_quantize_append(cache, _t(k), _t(v), first_slot=first)
    for name, x, unpack in (("k", k, R.unpack), ("v", v, R.unpack_tiles)):
        codes_ref, n_ref, y_ref = _encode_ref(x, rot)
        got = unpack(_np(getattr(cache, f"{name}_codes")))
        _boundary_mismatch_ok(got[:, first:first + n_tok], codes_ref, y_ref, n_ref)
        norms = _np(getattr(cache, f"{name}_norms"))[:, first:first + n_tok]
        assert np.max(np.abs(norms - n_ref) / n_ref) < 2e-6


@pytest.mark.parametrize("kind", ["iso", "planar"])
@pytest.mark.parametrize("hq,hkv,lens", [(32, 4, [2100]), (8, 2, [0, 700, 1300]), (32, 8, [13, 4096])])
def test_decode_variants_match_oracle(kind, hq, hkv, lens):
    lens = np.array(lens, np.int32)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int32)
    rot, kr, kn, vr, vn = _oracle_cache(hq * 7 + hkv, hkv, int(lens.sum()) + 3, kind=kind)
    cache = _upload(rot, kr, kn, vr, vn)
    q = iqinputs.queries(hq, 2, len(lens), hq)
    out = _np(iq.iq_decode_attention(cache, _t(q), _t(starts), _t(lens), int(lens.max())))
    ref = R.decode_attention(q, kr, kn, vr, vn, rot, starts, lens, SCALE, C32)
    _assert_attention_close(out, ref, f"{kind} hq={hq} hkv={hkv} lens={list(lens)}")


@pytest.mark.parametrize("kind", ["iso", "planar"])
def test_dequantize_variants_match_oracle(kind):
    hkv, n = 2, 256
    rot = iqinputs.rotation_params_kind(23, 0, hkv, kind)
    x = iqinputs.kv(23, 0, "k", n, hkv, "fixed_x8", "f32")
    codes, norms = R.encode_codes(x, rot, T32)
    cache = iq.PackedKVCache.allocate(hkv, n, _t(rot))
    cache.k_codes.copy_(_t(R.pack(codes)))
    cache.v_codes.copy_(_t(R.pack_tiles(codes)))
    cache.k_norms.copy_(_t(norms))
    cache.v_norms.copy_(_t(norms))
    k_out, v_out = iq.iq_dequantize(cache, 0, n)
    k_out, v_out = _np(k_out).astype(np.float64), _np(v_out).astype(np.float64)
    for h in range(hkv):
        ref = R.dequantize_codes(codes[h], norms[h], rot[h], C32)
        assert np.max(np.abs(k_out[:, h] - ref) / norms[h, :, None]) < 2e-6
        assert np.max(np.abs(v_out[:, h] - ref) / norms[h, :, None]) < 2e-6


# -------------------------------------------------- 4-bit K, 3-bit V ----
C16, T16, _ = R.codebook(levels=16)


def _encode_ref_thr(x, rot, thr):
    hkv = x.shape[1]
    out_c, out_n, out_y = [], [], []
    for h in range(hkv):
        y32 = R.rotate(x[:, h].astype(np.float64), rot[h]).astype(np.float32)
        c, n = R.quantize(y32, thr)
        out_c.append(c), out_n.append(n), out_y.append(y32)
    return np.stack(out_c), np.stack(out_n), np.stack(out_y)


@pytest.mark.parametrize("k_bits", [3, 4])
@pytest.mark.parametrize("n_tok", [70, 5])     # bulk kernel, short-append kernel
def test_append_nonfinite_inputs_give_code_zero(k_bits, n_tok):
    """A NaN anywhere in a new K or V vector makes its norm NaN, so every one of its codes is 0 (the
    definition compares with NaN thresholds); its neighbours are encoded as usual."""
    hkv = 2
    rot = iqinputs.rotation_params(41, 0, hkv)
    x = iqinputs.kv(41, 0, "k", n_tok, hkv, "fixed_x8", "f32")
    x[1, 0, 17] = np.nan
    x[3, 1, :] = np.nan
    cache = iq.PackedKVCache.allocate(hkv, 96, _t(rot), k_bits=k_bits)
    iq.iq_rotate_quantize_append(cache, _t(x), _t(x), first_slot=8)
    thr = T16 if k_bits == 4 else T32
    codes_ref, n_ref, y_ref = _encode_ref_thr(x, rot, thr)
    got = R.unpack(_np(cache.k_codes))[:, 8:8 + n_tok]
    gv = R.unpack_tiles(_np(cache.v_codes))[:, 8:8 + n_tok]
    for g in (got, gv):
        assert not g[0, 1].any() and not g[1, 3].any()
    assert np.isnan(_np(cache.k_norms)[0, 9]) and np.isnan(_np(cache.v_norms)[1, 11])
    finite = np.isfinite(n_ref)
    _boundary_mismatch_ok(np.where(finite[..., None], got, 0), np.where(finite[..., None], codes_ref, 0),
                          np.nan_to_num(y_ref), np.where(finite, n_ref, 1.0), thr)


@pytest.mark.parametrize("kind", ["wht_so4", "iso"])
@pytest.mark.parametrize("n_tok,first", [(700, 13), (1, 500), (40, 21)])   # bulk and short appends
def test_append_k4_matches_oracle(kind, n_tok, first):
    hkv = 4
    rot = iqinputs.rotation_params_kind(31, 0, hkv, kind)
    k = iqinputs.kv(31, 0, "k", n_tok, hkv, "student_t6", "f16")
    v = iqinputs.kv(31, 0, "v", n_tok, hkv, "student_t6", "f16")
    cache = iq.PackedKVCache.allocate(hkv, first + n_tok, _t(rot), k_bits=4)
    assert cache.k_codes.shape[2] == 64
    iq.iq_rotate_quantize_append(cache, _t(k), _t(v), first_slot=first)
    codes_ref, n_ref, y_ref = _encode_ref_thr(k, rot, T16)
    got = R.unpack(_np(cache.k_codes))
    assert got.max() <= 15
    _boundary_mismatch_ok(got[:, first:first + n_tok], codes_ref, y_ref, n_ref, T16)
    assert not got[:, :first].any() and not got[:, first + n_tok:].any()
    norms = _np(cache.k_norms)[:, first:first + n_tok]
    assert np.max(np.abs(norms - n_ref) / n_ref) < 2e-6
    vref, vn_ref, vy = _encode_ref_thr(v, rot, T32)
    _boundary_mismatch_ok(R.unpack_tiles(_np(cache.v_codes))[:, first:first + n_tok], vref, vy, vn_ref)


def test_dequantize_k4_matches_oracle():
    hkv, n = 2, 256
    rot = iqinputs.rotation_params(29, 0, hkv)
    x = iqinputs.kv(29, 0, "k", n, hkv, "fixed_x8", "f32")
    k16, kn = R.encode_codes(x, rot, T16)
    v8, vn = R.encode_codes(x, rot, T32)
    cache = iq.PackedKVCache.allocate(hkv, n, _t(rot), k_bits=4)
    cache.k_codes.copy_(_t(R.pack(k16, 4)))
    cache.v_codes.copy_(_t(R.pack_tiles(v8)))
    cache.k_norms.copy_(_t(kn))
    cache.v_norms.copy_(_t(vn))
    k_out, v_out = iq.iq_dequantize(cache, 0, n)
    k_out, v_out = _np(k_out).astype(np.float64), _np(v_out).astype(np.float64)
    for h in range(hkv):
        assert np.max(np.abs(k_out[:, h] - R.dequantize_codes(k16[h], kn[h], rot[h], C16)) / kn[h, :, None]) < 2e-6
        assert np.max(np.abs(v_out[:, h] - R.dequantize_codes(v8[h], vn[h], rot[h], C32)) / vn[h, :, None]) < 2e-6


@pytest.mark.parametrize("kind", ["wht_so4", "planar"])
@pytest.mark.parametrize("hq,hkv,lens", [(32, 4, [2100]), (8, 2, [0, 700, 1300]), (16, 1, [513, 3]),
                                         (32, 8, [13, 4096]), (4, 4, [300])])
def test_decode_k4_matches_oracle(kind, hq, hkv, lens):
    lens = np.array(lens, np.int32)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int32)
    total = int(lens.sum()) + 3
    cap = -(-total // 32) * 32
    rot = iqinputs.rotation_params_kind(hq + 5 * hkv, 0, hkv, kind)
    k = np.zeros((cap, hkv, 128), np.float16)
    v = np.zeros_like(k)
    k[:total] = iqinputs.kv(hq, 3, "k", total, hkv, "student_t6", "f16")
    v[:total] = iqinputs.kv(hq, 3, "v", total, hkv, "student_t6", "f16")
    kr, kn = R.encode_tokens(k, rot, T16)
    vt, vn = R.encode_tokens_v(v, rot, T32)
    cache = iq.PackedKVCache.allocate(hkv, cap, _t(rot), k_bits=4)
    cache.k_codes.copy_(_t(kr))
    cache.v_codes.copy_(_t(vt))
    cache.k_norms.copy_(_t(kn))
    cache.v_norms.copy_(_t(vn))
    q = iqinputs.queries(hq, 4, len(lens), hq)
    out = _np(iq.iq_decode_attention(cache, _t(q), _t(starts), _t(lens), int(lens.max())))
    ref = R.decode_attention(q, kr, kn, vt, vn, rot, starts, lens, SCALE, C32, k_centroids32=C16)
    _assert_attention_close(out, ref, f"4-bit K {kind} hq={hq} hkv={hkv} lens={list(lens)}")


# ---------------------------------------------- fused decode step ----
@pytest.mark.parametrize("hq,hkv,lens,k_bits,kind,f16", [
    (32, 4, [2100], 3, "wht_so4", True),
    (8, 2, [0, 700, 1300], 3, "planar", False),
    (16, 1, [513, 3], 4, "wht_so4", True),
    (32, 8, [13, 4096, 31], 4, "iso", True),
    (4, 4, [300, 7], 3, "wht_so4", False),
    # full occupancy with 4-bit K (two work-groups per CU): the plain plan's 512 splits and the 4
    # new-token work-groups do not fit at once, so the plan leaves them room (the 3-bit case at this
    # shape keeps the plain plan: test_gpu_fullsize's decode step)
    (32, 4, [32767], 4, "wht_so4", True),
])
def test_append_decode_equals_append_then_decode(hq, hkv, lens, k_bits, kind, f16):
    """The fused step writes the same codes and norms as iq_rotate_quantize_append and returns the
    decode over the grown cache (checked against the oracle too)."""
    _check_append_decode(hq, hkv, lens, k_bits, kind, f16, 5)


@pytest.mark.parametrize("hq,hkv,n,first", [(32, 4, 2100, 32), (32, 4, 700, 4133), (8, 8, 90, 31)])
def test_append_decode_single_sequence_at_any_start(hq, hkv, n, first):
    """One sequence per launch whose row does not begin at slot 0 of its cache row (and one that
    begins in the row's first block)."""
    _check_append_decode(hq, hkv, [n], 3, "wht_so4", True, first)


def _check_append_decode(hq, hkv, lens, k_bits, kind, f16, first):
    lens = np.array(lens, np.int32)
    n_seqs = len(lens)
    starts = (np.concatenate([[0], np.cumsum(lens + 1)[:-1]]) + first).astype(np.int32)   # room for each new token
    cap = -(-(int(starts[-1] + lens[-1]) + 1) // 32) * 32
    seed = int(lens.sum()) + hq
    rot = iqinputs.rotation_params_kind(seed, 0, hkv, kind)
    dt = "f16" if f16 else "f32"
    x_k = iqinputs.kv(seed, 0, "k", cap, hkv, "student_t6", dt)
    x_v = iqinputs.kv(seed, 0, "v", cap, hkv, "student_t6", dt)
    new_slots = starts + lens
    k_new, v_new = x_k[new_slots], x_v[new_slots]
    q = iqinputs.queries(seed, 1, n_seqs, hq)
    caches = []
    for _ in range(2):
        c = iq.PackedKVCache.allocate(hkv, cap, _t(rot), k_bits=k_bits)
        iq.iq_rotate_quantize_append(c, _t(x_k), _t(x_v), first_slot=0)   # every slot, then
        caches.append(c)
    # ... the new tokens' slots are overwritten by the step under test (reference: the append call)
    iq.iq_rotate_quantize_append(caches[0], _t(k_new), _t(v_new), slots=_t(new_slots.astype(np.int32)))
    ref_out = _np(iq.iq_decode_attention(caches[0], _t(q), _t(starts), _t(lens + 1), int(lens.max()) + 1))
    got = _np(iq.iq_append_decode_attention(caches[1], _t(k_new), _t(v_new), _t(q), _t(starts), _t(lens),
                                            int(lens.max())))
    for name in ("k_codes", "v_codes", "k_norms", "v_norms"):
        assert torch.equal(getattr(caches[0], name), getattr(caches[1], name)), name
    _assert_attention_close(got, ref_out, f"fused step vs append + decode hq={hq} hkv={hkv} lens={list(lens)}")
    c_k, t_k, _ = R.codebook(levels=16 if k_bits == 4 else 8)
    kr = _np(caches[1].k_codes)
    ref = R.decode_attention(q, kr, _np(caches[1].k_norms), _np(caches[1].v_codes), _np(caches[1].v_norms), rot,
                             starts, lens + 1, SCALE, C32, k_centroids32=c_k)
    _assert_attention_close(got, ref, f"fused step vs oracle hq={hq} hkv={hkv} lens={list(lens)} k_bits={k_bits}")


def test_append_decode_new_slot_outside_cache_gives_nan_and_writes_nothing():
    hkv, hq = 2, 4
    rot = iqinputs.rotation_params(3, 0, hkv)
    cache = iq.PackedKVCache.allocate(hkv, 64, _t(rot))
    x = iqinputs.kv(3, 0, "k", 64, hkv, "fixed_x8", "f16")
    iq.iq_rotate_quantize_append(cache, _t(x), _t(x))
    before = [getattr(cache, n).clone() for n in ("k_codes", "v_codes", "k_norms", "v_norms")]
    q = iqinputs.queries(3, 0, 2, hq)
    starts, lens = np.array([0, 32], np.int32), np.array([10, 32], np.int32)   # seq 1's new slot = 64: outside
    new = iqinputs.kv(4, 0, "k", 2, hkv, "fixed_x8", "f16")
    out = _np(iq.iq_append_decode_attention(cache, _t(new), _t(new), _t(q), _t(starts), _t(lens), 32))
    assert np.all(np.isnan(out[1])) and np.all(np.isfinite(out[0]))
    after = [getattr(cache, n) for n in ("k_codes", "v_codes", "k_norms", "v_norms")]
    # only slot 10 (sequence 0's new token) was written: K rows and norms of every other slot, and
    # every V tile but slot 10's (tile 1, slots 8..15), are unchanged
    others = [i for i in range(64) if i != 10]
    for i in (0, 2, 3):
        assert torch.equal(before[i][:, others], after[i][:, others]), i
    tiles = [t for t in range(64 // 8) if t != 1]
    assert torch.equal(before[1][:, tiles], after[1][:, tiles])
    assert not torch.equal(before[2][:, 10], after[2][:, 10])   # the new K norm landed
