"""Seeded random decode configurations against the oracle (MI355X only).

Each case draws its own mix of what the fixed cases in test_gpu_parity.py
vary one or two at a time: group size, KV heads, K width, rotation kind, batch
size, empty sequences, starts that are not multiples of 32, gaps between the
sequences' rows, lengths that straddle split boundaries, a max_seq_len bound
larger than the longest sequence (which changes the split plan), and now and
then a sequence whose length exceeds that bound (its output must be NaN).
Both the decode alone and the fused decode step are checked, to the same
tolerances as the fixed cases (max-abs 2e-3, relative L2 1e-3); and random
appends (short and bulk kernels, contiguous or listed slots) to the encode's
bar: codes equal up to cell-boundary ties, norms to 2e-6, every slot not
written unchanged; and the deferred decode (fp16 prefix, packed suffix) and
the FP16-KV baseline decode at random shapes in either fp16 layout."""
import numpy as np
import pytest
import torch

import iqinputs
import quantized_kv_cache_wht_amd as iq
from oracle import iqref as R

pytestmark = pytest.mark.gpu
from parity_util import C32, T32, SCALE, _t, _np, _assert_attention_close, _boundary_mismatch_ok  # noqa: E402

C16, T16, _ = R.codebook(levels=16)
CASES = 16


def _draw(case):
    g = np.random.default_rng(7000 + case)
    hkv = int(g.choice([1, 2, 4, 8]))
    group = int(g.choice([1, 2, 4, 8, 16]))
    k_bits = int(g.choice([3, 4]))
    kind = str(g.choice(iqinputs.ROTATION_KINDS))
    n_seqs = int(g.integers(1, 6))
    lens = []
    for _ in range(n_seqs):
        r = g.random()
        lens.append(0 if r < 0.12 else int(g.integers(1, 40)) if r < 0.35 else int(g.integers(40, 3000)))
    budget = max(1, 6000 // max(1, hkv // 2))   # keeps the oracle's encode within seconds
    scale_down = max(1.0, sum(lens) / budget)
    lens = np.array([int(x / scale_down) for x in lens], np.int32)
    gaps = g.integers(0, 40, n_seqs)
    starts = (np.concatenate([[0], np.cumsum(lens + gaps)[:-1]]) + gaps[0]).astype(np.int32)
    max_len = int(lens.max()) + int(g.integers(0, 200))
    bad = int(g.integers(0, n_seqs)) if (n_seqs > 1 and g.random() < 0.3) else -1
    return hkv, group, k_bits, kind, lens, starts, max_len, bad


def _label(case, hkv, group, k_bits, kind, lens, starts, max_len, bad):
    return (f"case {case}: hkv={hkv} G={group} k_bits={k_bits} {kind} lens={[int(x) for x in lens]} "
            f"starts={[int(x) for x in starts]} max_seq_len={max_len} over-bound seq={bad}")


@pytest.mark.parametrize("case", range(CASES))
def test_decode_random_configuration(case):
    hkv, group, k_bits, kind, lens, starts, max_len, bad = _draw(case)
    label = _label(case, hkv, group, k_bits, kind, lens, starts, max_len, bad)
    print(label, flush=True)
    hq = hkv * group
    lens_call = lens.copy()
    if bad >= 0:
        lens_call[bad] = max_len + 1    # beyond the launch's bound: NaN, and nothing read out of bounds
    total = int((starts + lens_call).max()) + 5
    cap = -(-total // 32) * 32
    rot = iqinputs.rotation_params_kind(case, 0, hkv, kind)
    k = np.zeros((cap, hkv, 128), np.float16)
    v = np.zeros_like(k)
    k[:total] = iqinputs.kv(case, 1, "k", total, hkv, "student_t6", "f16")
    v[:total] = iqinputs.kv(case, 1, "v", total, hkv, "student_t6", "f16")
    kr, kn = R.encode_tokens(k, rot, T16 if k_bits == 4 else T32)
    vt, vn = R.encode_tokens_v(v, rot, T32)
    cache = iq.PackedKVCache.allocate(hkv, cap, _t(rot), k_bits=k_bits)
    cache.k_codes.copy_(_t(kr))
    cache.v_codes.copy_(_t(vt))
    cache.k_norms.copy_(_t(kn))
    cache.v_norms.copy_(_t(vn))
    q = iqinputs.queries(case, 2, len(lens), hq)
    out = _np(iq.iq_decode_attention(cache, _t(q), _t(starts), _t(lens_call), max_len))
    good = [s for s in range(len(lens)) if s != bad]
    ref = R.decode_attention(q, kr, kn, vt, vn, rot, starts, lens_call, SCALE, C32,
                             k_centroids32=C16 if k_bits == 4 else None, seqs=good)
    _assert_attention_close(out[good], ref[good], label)
    for s in good:
        if lens[s] == 0:
            assert np.all(out[s] == 0), label
    if bad >= 0:
        assert np.all(np.isnan(out[bad])), label


@pytest.mark.parametrize("case", range(CASES // 2))
def test_append_decode_random_configuration(case):
    """The fused step at the same random shapes: the cache it leaves equals iq_rotate_quantize_append's,
    and its output equals iq_decode_attention over the grown cache."""
    hkv, group, k_bits, kind, lens, starts, max_len, _ = _draw(100 + case)
    label = _label(100 + case, hkv, group, k_bits, kind, lens, starts, max_len, -1)
    print(label, flush=True)
    hq = hkv * group
    starts = (starts + np.arange(len(lens), dtype=np.int32)).astype(np.int32)   # room for each new token
    cap = -(-(int((starts + lens).max()) + 1 + 5) // 32) * 32
    rot = iqinputs.rotation_params_kind(case, 0, hkv, kind)
    x_k = iqinputs.kv(case, 4, "k", cap, hkv, "student_t6", "f16")
    x_v = iqinputs.kv(case, 4, "v", cap, hkv, "student_t6", "f16")
    new_slots = starts + lens
    q = iqinputs.queries(case, 5, len(lens), hq)
    caches = []
    for _ in range(2):
        c = iq.PackedKVCache.allocate(hkv, cap, _t(rot), k_bits=k_bits)
        iq.iq_rotate_quantize_append(c, _t(x_k), _t(x_v), first_slot=0)
        caches.append(c)
    k_new, v_new = x_k[new_slots], x_v[new_slots]
    iq.iq_rotate_quantize_append(caches[0], _t(k_new), _t(v_new), slots=_t(new_slots.astype(np.int32)))
    ref = _np(iq.iq_decode_attention(caches[0], _t(q), _t(starts), _t(lens + 1), max_len + 1))
    got = _np(iq.iq_append_decode_attention(caches[1], _t(k_new), _t(v_new), _t(q), _t(starts), _t(lens), max_len))
    for name in ("k_codes", "v_codes", "k_norms", "v_norms"):
        assert torch.equal(getattr(caches[0], name), getattr(caches[1], name)), (name, label)
    _assert_attention_close(got, ref, label)


def _encode_ref(x, rot, thr):
    """Oracle codes [Hkv][n][128], norms [Hkv][n] and the float32 rotated vectors of x [n][Hkv][128]."""
    out_c, out_n, out_y = [], [], []
    for h in range(x.shape[1]):
        y32 = R.rotate(x[:, h].astype(np.float64), rot[h]).astype(np.float32)
        c, n = R.quantize(y32, thr)
        out_c.append(c), out_n.append(n), out_y.append(y32)
    return np.stack(out_c), np.stack(out_n), np.stack(out_y)


@pytest.mark.parametrize("case", range(12))
def test_append_random_configuration(case):
    """Random appends into a cache that already holds other tokens: the short-append (<= 64 tokens)
    and bulk kernels, contiguous slots from any first slot or a slot list with entries outside the
    cache, fp16 or fp32 input, every rotation kind and K width. Written slots match the oracle (codes
    up to cell-boundary ties, norms to 2e-6); every other slot, including the other slots of V tiles
    the append only partly covers, keeps its previous contents bit for bit."""
    g = np.random.default_rng(9000 + case)
    hkv = int(g.choice([1, 2, 4, 8]))
    kind = str(g.choice(iqinputs.ROTATION_KINDS))
    k_bits = int(g.choice([3, 4]))
    dt = str(g.choice(["f16", "f32"]))
    r = g.random()
    n_tok = int(g.integers(1, 17)) if r < 0.3 else int(g.integers(17, 101)) if r < 0.6 else int(g.integers(101, 3000))
    use_slots = bool(g.random() < 0.4)
    label = f"case {case}: hkv={hkv} {kind} k_bits={k_bits} {dt} n_tok={n_tok} slot_list={use_slots}"
    print(label, flush=True)
    rot = iqinputs.rotation_params_kind(50 + case, 0, hkv, kind)
    if use_slots:
        cap = -(-(2 * n_tok + 8) // 32) * 32
        slots = g.permutation(cap)[:n_tok].astype(np.int32)
        k_out = g.random(n_tok) < 0.1
        slots[k_out] = np.where(g.random(int(k_out.sum())) < 0.5, -1 - g.integers(0, 5, int(k_out.sum())),
                                cap + g.integers(0, 5, int(k_out.sum())))
        written = slots[(slots >= 0) & (slots < cap)]
        sel = np.nonzero((slots >= 0) & (slots < cap))[0]
    else:
        first = int(g.integers(0, 100))
        cap = -(-(first + n_tok + int(g.integers(0, 40))) // 32) * 32
        written = np.arange(first, first + n_tok)
        sel = np.arange(n_tok)
    x_bg = iqinputs.kv(60 + case, 0, "k", cap, hkv, "student_t6", "f16")
    k = iqinputs.kv(70 + case, 0, "k", n_tok, hkv, "student_t6", dt)
    v = iqinputs.kv(70 + case, 0, "v", n_tok, hkv, "student_t6", dt)
    cache = iq.PackedKVCache.allocate(hkv, cap, _t(rot), k_bits=k_bits)
    assert cache.capacity == cap
    iq.iq_rotate_quantize_append(cache, _t(x_bg), _t(x_bg), first_slot=0)   # every slot holds a token first
    before = {n: getattr(cache, n).clone() for n in ("k_codes", "v_codes", "k_norms", "v_norms")}
    if use_slots:
        iq.iq_rotate_quantize_append(cache, _t(k), _t(v), slots=_t(slots))
    else:
        iq.iq_rotate_quantize_append(cache, _t(k), _t(v), first_slot=first)
    thr_k = T16 if k_bits == 4 else T32
    kc, kn, ky = _encode_ref(k[sel], rot, thr_k)
    vc, vn, vy = _encode_ref(v[sel], rot, T32)
    got_k = R.unpack(_np(cache.k_codes))
    got_v = R.unpack_tiles(_np(cache.v_codes))
    _boundary_mismatch_ok(got_k[:, written], kc, ky, kn, thr_k)
    _boundary_mismatch_ok(got_v[:, written], vc, vy, vn)
    for name, ref in (("k_norms", kn), ("v_norms", vn)):
        assert np.max(np.abs(_np(getattr(cache, name))[:, written] - ref) / ref) < 2e-6, (name, label)
    others = np.setdiff1d(np.arange(cap), written)
    old_k, old_v = R.unpack(_np(before["k_codes"])), R.unpack_tiles(_np(before["v_codes"]))
    assert np.array_equal(got_k[:, others], old_k[:, others]), label
    assert np.array_equal(got_v[:, others], old_v[:, others]), label
    for name in ("k_norms", "v_norms"):
        assert np.array_equal(_np(getattr(cache, name))[:, others], _np(before[name])[:, others]), (name, label)


def _ragged(g, n_seqs, budget, p_empty=0.2):
    lens = np.array([0 if g.random() < p_empty else int(g.integers(1, 2500)) for _ in range(n_seqs)], np.int64)
    if lens.sum() > budget:
        lens = (lens * budget // lens.sum())
    lens = lens.astype(np.int32)
    gaps = g.integers(0, 40, n_seqs)
    starts = (np.concatenate([[0], np.cumsum(lens + gaps)[:-1]]) + gaps[0]).astype(np.int32)
    return lens, starts


@pytest.mark.parametrize("case", range(8))
def test_deferred_and_f16_decode_random_configuration(case):
    """The deferred decode (fp16 prefix, then the packed suffix) and the FP16-KV baseline decode at random
    shapes, either fp16 layout, against attention from the definition over the same K/V."""
    g = np.random.default_rng(11000 + case)
    hkv = int(g.choice([1, 2, 4, 8]))
    group = int(g.choice([1, 2, 4, 8, 16]))
    kind = str(g.choice(iqinputs.ROTATION_KINDS))
    k_bits = int(g.choice([3, 4]))
    token_major = bool(g.random() < 0.5)
    n_seqs = int(g.integers(1, 5))
    budget = max(64, 5000 // max(1, hkv // 2))
    pre, pst = _ragged(g, n_seqs, budget // 2)
    suf, sst = _ragged(g, n_seqs, budget // 2)
    hq = hkv * group
    label = (f"case {case}: hkv={hkv} G={group} {kind} k_bits={k_bits} token_major={token_major} "
             f"prefix={[int(x) for x in pre]} at {[int(x) for x in pst]} suffix={[int(x) for x in suf]} "
             f"at {[int(x) for x in sst]}")
    print(label, flush=True)
    cap16 = -(-(int((pst + pre).max()) + 1) // 32) * 32
    cap = -(-(int((sst + suf).max()) + 1) // 32) * 32
    rot = iqinputs.rotation_params_kind(80 + case, 0, hkv, kind)
    k16 = iqinputs.kv(90 + case, 1, "k", cap16, hkv, "student_t6", "f16")
    v16 = iqinputs.kv(90 + case, 1, "v", cap16, hkv, "student_t6", "f16")
    k = iqinputs.kv(90 + case, 2, "k", cap, hkv, "student_t6", "f16")
    v = iqinputs.kv(90 + case, 2, "v", cap, hkv, "student_t6", "f16")
    c_k, t_k, _ = R.codebook(levels=16 if k_bits == 4 else 8)
    kr, kn = R.encode_tokens(k, rot, t_k)
    vt, vn = R.encode_tokens_v(v, rot, T32)
    cache = iq.PackedKVCache.allocate(hkv, cap, _t(rot), k_bits=k_bits)
    cache.k_codes.copy_(_t(kr))
    cache.v_codes.copy_(_t(vt))
    cache.k_norms.copy_(_t(kn))
    cache.v_norms.copy_(_t(vn))
    q = iqinputs.queries(95 + case, 3, n_seqs, hq)
    lay = (lambda a: _t(a)) if token_major else (lambda a: _t(np.ascontiguousarray(a.transpose(1, 0, 2))))
    max_pre, max_suf = int(pre.max()) + int(g.integers(0, 50)), int(suf.max()) + int(g.integers(0, 50))
    out = _np(iq.iq_decode_attention_deferred(cache, _t(sst), _t(suf), max_suf, lay(k16), lay(v16), _t(pst), _t(pre),
                                              max_pre, _t(q), token_major=token_major))
    ref = R.decode_attention_deferred(q, k16, v16, pst, pre, kr, kn, vt, vn, rot, sst, suf, SCALE, C32,
                                      k_centroids32=c_k)
    _assert_attention_close(out, ref, "deferred " + label)
    for s in np.nonzero((pre + suf) == 0)[0]:
        assert np.all(out[s] == 0), label
    # the FP16-KV baseline over the prefix alone
    out16 = _np(iq.iq_decode_attention_f16(lay(k16), lay(v16), _t(q), _t(pst), _t(pre), max_pre,
                                           token_major=token_major))
    ref16 = np.zeros_like(out16, dtype=np.float64)
    for s in range(n_seqs):
        a, n = int(pst[s]), int(pre[s])
        for h in range(hkv):
            if n:
                ref16[s, h * group:(h + 1) * group] = R.attention(q[s, h * group:(h + 1) * group],
                                                                   k16[a:a + n, h].astype(np.float64),
                                                                   v16[a:a + n, h].astype(np.float64), SCALE)
    _assert_attention_close(out16, ref16, "f16 " + label)
