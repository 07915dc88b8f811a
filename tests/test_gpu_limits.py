"""The decode at the limits of its launch (MI355X only).

* The largest batch the grid allows (65,535 sequences, many of them empty),
  for the decode and for the fused decode step. The cache is written by the
  library's encode and read back; the oracle decodes a sample of sequences from
  that same cache (encode parity is covered elsewhere).
* One sequence longer than the split plan's cap (2,048 splits of 64 blocks):
  the plan then lengthens its splits. With a periodic cache (64 distinct rows
  repeated), attention over the sequence equals attention over the 64 rows,
  each weighted by how often it occurs in the sequence: the oracle computes
  that from the definition, exactly, at a size it could not take token by
  token.
* A head whose K codes pass 2^31 bytes (48M slots): encode, decode and the
  fused step where every byte offset needs 64-bit arithmetic.
Tolerances as in test_gpu_parity (max-abs 2e-3, relative L2 1e-3)."""
import numpy as np
import pytest
import torch

import iqinputs
import quantized_kv_cache_wht_amd as iq
from oracle import iqref as R

pytestmark = pytest.mark.gpu
from parity_util import C32, T32, SCALE, DEV, _t, _np, _assert_attention_close, _boundary_mismatch_ok  # noqa: E402


def test_decode_and_step_at_the_largest_batch():
    n, hkv, group = 65535, 1, 2
    hq = hkv * group
    g = np.random.default_rng(65535)
    lens = g.integers(0, 41, n).astype(np.int32)
    lens[g.random(n) < 0.1] = 0
    starts = np.concatenate([[3], 3 + np.cumsum(lens + 1 + g.integers(0, 3, n))[:-1]]).astype(np.int32)
    cap = -(-(int(starts[-1] + lens[-1]) + 2) // 32) * 32
    rot = iqinputs.rotation_params(5, 0, hkv)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(5)
    xk = torch.randn((cap, hkv, 128), generator=gen, device=DEV).half()
    xv = torch.randn((cap, hkv, 128), generator=gen, device=DEV).half()
    caches = []
    for _ in range(2):
        c = iq.PackedKVCache.allocate(hkv, cap, _t(rot))
        iq.iq_rotate_quantize_append(c, xk, xv, first_slot=0)
        caches.append(c)
    q = iqinputs.queries(7, 0, n, hq)
    out = _np(iq.iq_decode_attention(caches[0], _t(q), _t(starts), _t(lens), 40))
    sample = sorted({0, 1, n - 2, n - 1, int(np.argmax(lens == 0)), *g.integers(0, n, 200).tolist()})
    kr, kn = _np(caches[0].k_codes), _np(caches[0].k_norms)
    vt, vn = _np(caches[0].v_codes), _np(caches[0].v_norms)
    ref = R.decode_attention(q, kr, kn, vt, vn, rot, starts, lens, SCALE, C32, seqs=sample)
    _assert_attention_close(out[sample], ref[sample], f"{n} sequences, sampled")
    assert np.all(out[lens == 0] == 0)
    # the fused step over the same batch: one new token per sequence
    new_slots = (starts + lens).astype(np.int32)
    kn_new = torch.randn((n, hkv, 128), generator=gen, device=DEV).half()
    vn_new = torch.randn((n, hkv, 128), generator=gen, device=DEV).half()
    iq.iq_rotate_quantize_append(caches[0], kn_new, vn_new, slots=_t(new_slots))
    want = iq.iq_decode_attention(caches[0], _t(q), _t(starts), _t(lens + 1), 41)
    got = iq.iq_append_decode_attention(caches[1], kn_new, vn_new, _t(q), _t(starts), _t(lens), 40)
    for name in ("k_codes", "v_codes", "k_norms", "v_norms"):
        assert torch.equal(getattr(caches[0], name), getattr(caches[1], name)), name
    _assert_attention_close(_np(got), _np(want), f"fused step, {n} sequences")


def test_decode_beyond_the_split_cap_periodic():
    hkv, group, period = 1, 8, 64
    hq = hkv * group
    n_tok = 2048 * 64 * 32 + 4096 + 5      # past 2,048 splits of 64 blocks
    start = 13
    cap = -(-(start + n_tok + 1) // period) * period
    rot = iqinputs.rotation_params(9, 0, hkv)
    x = iqinputs.kv(9, 0, "k", period, hkv, "student_t6", "f16")
    y = iqinputs.kv(9, 0, "v", period, hkv, "student_t6", "f16")
    kr_p, kn_p = R.encode_tokens(x, rot, T32)            # [1][64][48], [1][64]
    vt_p, vn_p = R.encode_tokens_v(y, rot, T32)          # [1][8][384], [1][64]
    cache = iq.PackedKVCache.allocate(hkv, cap, _t(rot))
    reps = cap // period
    cache.k_codes.copy_(_t(kr_p).repeat(1, reps, 1))
    cache.v_codes.copy_(_t(vt_p).repeat(1, reps, 1))
    cache.k_norms.copy_(_t(kn_p).repeat(1, reps))
    cache.v_norms.copy_(_t(vn_p).repeat(1, reps))
    q = iqinputs.queries(9, 1, 1, hq)
    out = _np(iq.iq_decode_attention(cache, _t(q), _t(np.array([start], np.int32)),
                                     _t(np.array([n_tok], np.int32)), n_tok))
    # attention over the multiset of the period's rows: row i occurs count_i times
    slots = np.arange(period)
    first = (slots - start) % period                      # offset of row i's first occurrence
    count = np.where(first < n_tok, (n_tok - 1 - first) // period + 1, 0).astype(np.float64)
    assert count.sum() == n_tok
    k_hat = R.dequantize(kr_p[0], kn_p[0], rot[0], C32)
    v_hat = R.dequantize_codes(R.unpack_tiles(vt_p[0]), vn_p[0], rot[0], C32)
    s = SCALE * (q[0].astype(np.float64) @ k_hat.T)       # [hq][64]
    w = count[None, :] * np.exp(s - s.max(axis=1, keepdims=True))
    ref = (w @ v_hat) / w.sum(axis=1, keepdims=True)
    _assert_attention_close(out[0], ref, f"{n_tok} tokens, periodic cache")


def test_cache_past_two_gib_per_head():
    """A head whose K rows reach past 2^31 bytes (48M slots x 48 B): the encode, the decode and the
    fused step in the cache's far end, where every byte offset needs more than 31 bits."""
    hkv, group = 1, 4
    hq = hkv * group
    cap = 48 * 2 ** 20
    n_tok, first = 3000, cap - 3200                     # rows past byte 2^31 of the head's K codes
    assert first * 48 > 2 ** 31
    rot = iqinputs.rotation_params(13, 0, hkv)
    cache = iq.PackedKVCache.allocate(hkv, cap, _t(rot))
    assert cache.capacity == cap
    k = iqinputs.kv(13, 0, "k", n_tok, hkv, "student_t6", "f16")
    v = iqinputs.kv(13, 0, "v", n_tok, hkv, "student_t6", "f16")
    iq.iq_rotate_quantize_append(cache, _t(k), _t(v), first_slot=first)
    # slots written one by one through a slot list, at both ends of the head
    far = np.array([7, cap - 1, cap - 9, 100], np.int32)
    kf = iqinputs.kv(14, 0, "k", len(far), hkv, "student_t6", "f16")
    iq.iq_rotate_quantize_append(cache, _t(kf), _t(kf), slots=_t(far))
    a0 = first - 32                                     # read back a window (tile-aligned)
    kr = _np(cache.k_codes[:, a0:])
    kn = _np(cache.k_norms[:, a0:])
    vt = _np(cache.v_codes[:, a0 // 8:])
    vn = _np(cache.v_norms[:, a0:])
    for x, got_c, got_n, rows in ((k, R.unpack(kr), kn, np.arange(32, 32 + n_tok)),
                                  (v, R.unpack_tiles(vt), vn, np.arange(32, 32 + n_tok))):
        y = R.rotate(x[:, 0].astype(np.float64), rot[0]).astype(np.float32)
        c_ref, n_ref = R.quantize(y, T32)
        _boundary_mismatch_ok(got_c[0, rows], c_ref, y, n_ref)
        assert np.max(np.abs(got_n[0, rows] - n_ref) / n_ref) < 2e-6
    y = R.rotate(kf[:, 0].astype(np.float64), rot[0]).astype(np.float32)
    c_ref, n_ref = R.quantize(y, T32)
    ends = [cap - 1 - a0, cap - 9 - a0]
    _boundary_mismatch_ok(R.unpack(kr)[0, ends], c_ref[[1, 2]], y[[1, 2]], n_ref[[1, 2]])
    # decode over the far sequence, and the fused step appending right after it
    q = iqinputs.queries(13, 1, 1, hq)
    st, ln = np.array([first], np.int32), np.array([n_tok], np.int32)
    out = _np(iq.iq_decode_attention(cache, _t(q), _t(st), _t(ln), n_tok))
    ref = R.decode_attention(q, kr, kn, vt, vn, rot, st - a0, ln, SCALE, C32)
    _assert_attention_close(out, ref, "decode past 2 GiB")
    k_new = iqinputs.kv(15, 0, "k", 1, hkv, "student_t6", "f16")
    got = _np(iq.iq_append_decode_attention(cache, _t(k_new), _t(k_new), _t(q), _t(st), _t(ln), n_tok))
    want = _np(iq.iq_decode_attention(cache, _t(q), _t(st), _t(ln + 1), n_tok + 1))
    _assert_attention_close(got, want, "fused step past 2 GiB")
