"""GPU parity at the workloads' full sizes and launch configurations.

The GPU encodes the whole layer itself (bulk ``iq_rotate_quantize_append``)
and decodes with the same launch configuration as bench.py or the workload
(same n_seqs, heads and max_seq_len, hence the same split-K plan); the oracle
encodes the same seeded inputs independently and computes the outputs that
are compared (all of them where it finishes in seconds, a sample of KV heads
or sequences otherwise). Tolerances are those of test_gpu_parity.
"""
import math

import numpy as np
import pytest
import torch

import iqinputs
import quantized_kv_cache_wht_amd as iq
from oracle import iqref as R
from parity_util import C32, T32, SCALE, _t, _np, _assert_attention_close, _boundary_mismatch_ok

pytestmark = pytest.mark.gpu


def _gpu_encode(k, v, rot, capacity):
    cache = iq.PackedKVCache.allocate(k.shape[1], capacity, _t(rot))
    iq.iq_rotate_quantize_append(cache, _t(k), _t(v), first_slot=0)
    return cache


def _oracle_heads(k, v, rot, heads):
    """Oracle encode of the given KV heads: (rot, k rows, k norms, v tiles, v norms) restricted to them."""
    hs = list(heads)
    kr, kn = R.encode_tokens(k[:, hs], rot[hs], T32)
    vt, vn = R.encode_tokens_v(v[:, hs], rot[hs], T32)
    return rot[hs], kr, kn, vt, vn


def _check_codes(cache, heads, kr, kn, vt, vn, k, v, rot, n_tok):
    """GPU codes of the sampled heads vs the oracle's, under the boundary rule."""
    hs = list(heads)
    nd = 0
    for name, x, ref_packed, ref_norms, unpack in (("k", k, kr, kn, R.unpack), ("v", v, vt, vn, R.unpack_tiles)):
        got = unpack(_np(getattr(cache, f"{name}_codes"))[hs])[:, :n_tok]
        ref = unpack(ref_packed)[:, :n_tok]
        y = np.stack([R.rotate(x[:n_tok, h].astype(np.float64), rot[h]).astype(np.float32) for h in hs])
        nd += _boundary_mismatch_ok(got, ref, y, ref_norms[:, :n_tok])
        norms = _np(getattr(cache, f"{name}_norms"))[hs][:, :n_tok]
        assert np.max(np.abs(norms - ref_norms[:, :n_tok]) / ref_norms[:, :n_tok]) < 2e-6
    return nd


def test_moe30b_full_layer_encode_decode_and_needle():
    """32768 tokens, Hq 32 / Hkv 4, batch 1: bench.py's decode launch. Every code, every output,
    and the planted needle of each KV head."""
    w = iqinputs.WORKLOADS["moe30b_gqa_t32768"]
    print(f"[{w.name}] full layer", flush=True)
    inp = iqinputs.layer_inputs(w, 0)
    k, v, q, rot = inp["k"], inp["v"], inp["q"], inp["rot"]
    T = w.seq_len
    cache = _gpu_encode(k, v, rot, T)
    ws = iq.decode_workspace(1, w.num_q_heads, w.num_kv_heads, T)
    out = _np(iq.iq_decode_attention(cache, _t(q), _t(inp["seq_start"]), _t(inp["seq_len"]), T, workspace=ws))

    heads = range(w.num_kv_heads)
    rot_s, kr, kn, vt, vn = _oracle_heads(k, v, rot, heads)
    nd = _check_codes(cache, heads, kr, kn, vt, vn, k, v, rot, T)
    ref = R.decode_attention(q, kr, kn, vt, vn, rot_s, inp["seq_start"], inp["seq_len"], SCALE, C32)
    _assert_attention_close(out, ref, f"{w.name} all heads, {nd} boundary codes")

    # needle: query head h*G attends almost only to the planted key, so its output is that
    # slot's reconstructed V
    p = int(inp["needle_slot"][0])
    for h in heads:
        kh = R.dequantize(kr[h], kn[h], rot_s[h], C32)
        wts = R.softmax(kh @ q[0, h * w.group].astype(np.float64) * SCALE)
        assert int(np.argmax(wts)) == p and wts[p] > 0.99, (h, int(np.argmax(wts)), float(wts[p]))
        v_p = R.dequantize_codes(R.v_codes_range(vt[h], p, 1), vn[h, p:p + 1], rot_s[h], C32)[0]
        assert np.max(np.abs(out[0, h * w.group] - v_p)) < 2e-3 + (1 - wts[p]) * np.max(np.abs(v_p)) * 4


def test_moe30b_decode_step_bench_launch():
    """bench.py's timed call: 32767 tokens encoded in bulk, then one iq_append_decode_attention that
    appends token 32767 and attends to all 32768 (the split plan with the new token's work-groups).
    Every code and norm of the grown cache, and every output, against the oracle."""
    w = iqinputs.WORKLOADS["moe30b_gqa_t32768"]
    print(f"[{w.name}] decode step", flush=True)
    inp = iqinputs.layer_inputs(w, 1)
    k, v, q, rot = inp["k"], inp["v"], inp["q"], inp["rot"]
    T = w.seq_len
    cache = iq.PackedKVCache.allocate(k.shape[1], T, _t(rot))
    iq.iq_rotate_quantize_append(cache, _t(k[:T - 1]), _t(v[:T - 1]), first_slot=0)
    start = np.zeros(1, np.int32)
    cached = np.full(1, T - 1, np.int32)
    ws = iq.decode_workspace(1, w.num_q_heads, w.num_kv_heads, T - 1)
    out = _np(iq.iq_append_decode_attention(cache, _t(k[T - 1:]), _t(v[T - 1:]), _t(q), _t(start), _t(cached),
                                            T - 1, workspace=ws))
    heads = range(w.num_kv_heads)
    rot_s, kr, kn, vt, vn = _oracle_heads(k, v, rot, heads)
    nd = _check_codes(cache, heads, kr, kn, vt, vn, k, v, rot, T)
    ref = R.decode_attention(q, kr, kn, vt, vn, rot_s, start, np.full(1, T, np.int32), SCALE, C32)
    _assert_attention_close(out, ref, f"{w.name} decode step, {nd} boundary codes")


def test_dense8b_full_layer():
    """8192 tokens, Hq 32 / Hkv 8, batch 1, Student-t outlier channels: all heads."""
    w = iqinputs.WORKLOADS["dense8b_gqa_t8192"]
    print(f"[{w.name}] full layer", flush=True)
    inp = iqinputs.layer_inputs(w, 5)
    k, v, q, rot = inp["k"], inp["v"], inp["q"], inp["rot"]
    cache = _gpu_encode(k, v, rot, w.seq_len)
    out = _np(iq.iq_decode_attention(cache, _t(q), _t(inp["seq_start"]), _t(inp["seq_len"]), w.seq_len))
    heads = range(w.num_kv_heads)
    rot_s, kr, kn, vt, vn = _oracle_heads(k, v, rot, heads)
    nd = _check_codes(cache, heads, kr, kn, vt, vn, k, v, rot, w.seq_len)
    ref = R.decode_attention(q, kr, kn, vt, vn, rot_s, inp["seq_start"], inp["seq_len"], SCALE, C32)
    _assert_attention_close(out, ref, f"{w.name}, {nd} boundary codes")


def test_long_context_131072_sampled_heads():
    """131072 tokens, Hq 32 / Hkv 8: bulk encode of the whole layer on the GPU, one decode over it;
    the oracle checks KV heads 2 and 7 (codes, norms and their 8 query heads each)."""
    w = iqinputs.WORKLOADS["long_t131072"]
    print(f"[{w.name}] full layer, sampled heads", flush=True)
    inp = iqinputs.layer_inputs(w, 0)
    k, v, q, rot = inp["k"], inp["v"], inp["q"], inp["rot"]
    T = w.seq_len
    cache = _gpu_encode(k, v, rot, T)
    out = _np(iq.iq_decode_attention(cache, _t(q), _t(inp["seq_start"]), _t(inp["seq_len"]), T))
    heads = [2, 7]
    rot_s, kr, kn, vt, vn = _oracle_heads(k, v, rot, heads)
    nd = _check_codes(cache, heads, kr, kn, vt, vn, k, v, rot, T)
    g = w.group
    q_s = np.concatenate([q[:, h * g:(h + 1) * g] for h in heads], axis=1)
    ref = R.decode_attention(q_s, kr, kn, vt, vn, rot_s, inp["seq_start"], inp["seq_len"], SCALE, C32)
    got = np.concatenate([out[:, h * g:(h + 1) * g] for h in heads], axis=1)
    _assert_attention_close(got, ref, f"{w.name} heads {heads}, {nd} boundary codes")


def test_ragged32_launch_configuration():
    """The batched workload's launch: 32 sequences, Hq 32 / Hkv 8, max_seq_len 32768 (so the same
    split-K plan as the full batch). One sequence has the full 32768 tokens; the others are
    seeded lengths in [1, 2048] (whole-batch inputs would be 4 GB of host float64), which leaves
    most of their splits empty, as short sequences of the full batch do."""
    w = iqinputs.WORKLOADS["ragged32_gqa"]
    print(f"[{w.name}] launch configuration", flush=True)
    rng = np.random.default_rng(w.seed)
    lens = rng.integers(1, 2049, size=w.n_seqs).astype(np.int32)
    lens[11] = w.seq_len
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int32) + 5   # flat cache, offset 5
    total = int(starts[-1] + lens[-1])
    cap = -(-total // 32) * 32
    rot = iqinputs.rotation_params(w.seed, 0, w.num_kv_heads)
    k = np.zeros((cap, w.num_kv_heads, 128), np.float16)
    v = np.zeros_like(k)
    k[5:total] = iqinputs.kv(w.seed, 0, "k", total - 5, w.num_kv_heads, w.outliers, w.dtype)
    v[5:total] = iqinputs.kv(w.seed, 0, "v", total - 5, w.num_kv_heads, w.outliers, w.dtype)
    q = iqinputs.queries(w.seed, 0, w.n_seqs, w.num_q_heads)
    cache = _gpu_encode(k, v, rot, cap)
    out = _np(iq.iq_decode_attention(cache, _t(q), _t(starts), _t(lens), w.seq_len))
    heads = [0, 3, 6]
    rot_s, kr, kn, vt, vn = _oracle_heads(k, v, rot, heads)
    seqs = [0, 11, 17, 31]
    g = w.group
    q_s = np.concatenate([q[:, h * g:(h + 1) * g] for h in heads], axis=1)
    ref = R.decode_attention(q_s, kr, kn, vt, vn, rot_s, starts, lens, SCALE, C32, seqs=seqs)
    got = np.concatenate([out[:, h * g:(h + 1) * g] for h in heads], axis=1)
    _assert_attention_close(got[seqs], ref[seqs], f"{w.name} seqs {seqs} heads {heads}")
    assert np.all(np.isfinite(out))


def test_ragged32_batch_at_workload_lengths():
    """The batched workload as bench.py launches it: 32 sequences with the workload's seeded
    lengths (uniform in [1024, 32768]) back to back in one flat cache, Hq 32 / Hkv 8, max_seq_len =
    the longest. Every sequence is encoded by the GPU's bulk append; the sampled ones (the shortest,
    the longest, and those whose last split holds the fewest and the most 32-slot blocks) from their
    seeded inputs, which the oracle encodes too, the others from device random numbers (their
    outputs are not checked; they make the launch the real one). Codes of the sampled sequences and
    the outputs of two KV heads' query heads against the oracle."""
    w = iqinputs.WORKLOADS["ragged32_gqa"]
    print(f"[{w.name}] workload lengths", flush=True)
    lens = iqinputs.seq_lengths(w)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int32)
    total, hkv, hq, g = int(lens.sum()), w.num_kv_heads, w.num_q_heads, w.group
    ml = int(lens.max())
    # the plan of this batch: splits of 64 blocks (its cap), as many as the longest sequence needs
    n_splits = iq.iq_decode_workspace_bytes(w.n_seqs, hq, hkv, ml) // (w.n_seqs * hq * 132 * 4) - 1
    assert n_splits == -(-(-(-ml // 32)) // 64)
    nblk = (starts % 32 + lens + 31) // 32
    tail = nblk % 64
    order = np.argsort(tail)
    sampled = sorted({int(np.argmin(lens)), int(np.argmax(lens)), int(order[0]), int(order[1]), int(order[-1]),
                      int(order[-2])})
    assert len(sampled) >= 5
    rot = iqinputs.rotation_params(w.seed, 0, hkv)
    cache = iq.PackedKVCache.allocate(hkv, total, _t(rot))
    gen = torch.Generator(device="cuda")
    gen.manual_seed(w.seed)
    inputs = {}
    for s in range(w.n_seqs):
        n = int(lens[s])
        if s in sampled:
            k = iqinputs.kv_seq(w.seed, 0, "k", s, n, hkv, w.outliers, w.dtype)
            v = iqinputs.kv_seq(w.seed, 0, "v", s, n, hkv, w.outliers, w.dtype)
            inputs[s] = (k, v)
            kt, vt = _t(k), _t(v)
        else:
            kt = torch.randn((n, hkv, 128), generator=gen, device="cuda").half()
            vt = torch.randn((n, hkv, 128), generator=gen, device="cuda").half()
        iq.iq_rotate_quantize_append(cache, kt, vt, first_slot=int(starts[s]))
    q = iqinputs.queries(w.seed, 0, w.n_seqs, hq)
    out = _np(iq.iq_decode_attention(cache, _t(q), _t(starts), _t(lens), ml))
    assert np.all(np.isfinite(out))
    heads = [1, 6]
    kc, vc = _np(cache.k_codes)[heads], _np(cache.v_codes)[heads]
    kn_gpu, vn_gpu = _np(cache.k_norms)[heads], _np(cache.v_norms)[heads]
    nd = 0
    for s in sampled:
        a, n = int(starts[s]), int(lens[s])
        k, v = inputs[s]
        pad = -(-n // 8) * 8
        kp = np.zeros((pad, hkv, 128), k.dtype)
        vp = np.zeros_like(kp)
        kp[:n], vp[:n] = k, v
        rot_s, kr, kn, vt, vn = _oracle_heads(kp, vp, rot, heads)
        # codes and norms the GPU wrote for this sequence
        for x, ref_codes, ref_norms, got_codes, got_norms in (
                (k, R.unpack(kr)[:, :n], kn[:, :n], R.unpack(kc[:, a:a + n]), kn_gpu[:, a:a + n]),
                (v, R.unpack_tiles(vt)[:, :n], vn[:, :n],
                 R.unpack_tiles(vc[:, a // 8:(a + n + 7) // 8])[:, a % 8:a % 8 + n], vn_gpu[:, a:a + n])):
            y = np.stack([R.rotate(x[:, h].astype(np.float64), rot[h]).astype(np.float32) for h in heads])
            nd += _boundary_mismatch_ok(got_codes, ref_codes, y, ref_norms)
            assert np.max(np.abs(got_norms - ref_norms) / ref_norms) < 2e-6
        q_s = np.concatenate([q[s:s + 1, h * g:(h + 1) * g] for h in heads], axis=1)
        ref = R.decode_attention(q_s, kr, kn, vt, vn, rot_s, np.zeros(1, np.int32), np.full(1, n, np.int32), SCALE,
                                 C32)
        got = np.concatenate([out[s:s + 1, h * g:(h + 1) * g] for h in heads], axis=1)
        _assert_attention_close(got, ref, f"{w.name} seq {s} (len {n}, start {a}, {int(nblk[s])} blocks) "
                                          f"heads {heads}")
    print(f"[{w.name}] sampled {sampled}, {nd} boundary codes", flush=True)
