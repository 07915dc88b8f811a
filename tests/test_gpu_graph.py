"""The library's launches captured in a HIP graph (torch.cuda.CUDAGraph) give, on every replay,
exactly what the same calls give when launched one by one.

The captured sequence covers the entry points a serving step would put in a graph: a bulk encode
into a slot list, the fused append + decode, a decode over the grown cache, the 4-bit-K decode and
the explicit dequantize. Between replays the test runs unrelated eager work on the same stream,
clears every output, and synchronises; each replay is compared bit for bit with the eager run.
"""
import numpy as np
import pytest
import torch

import iqinputs
import quantized_kv_cache_wht_amd as iq
from parity_util import _t

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager_calls():
    hkv, hq = 2, 8
    lens = np.array([700, 1500], np.int32)            # tokens already cached per sequence
    starts = np.array([3, 800], np.int32)             # misaligned starts, room for each new token
    cap = 2336
    n_seqs = len(lens)
    rot = _t(iqinputs.rotation_params(41, 0, hkv))
    x_k = iqinputs.kv(41, 0, "k", cap, hkv, "student_t6", "f16")
    x_v = iqinputs.kv(41, 0, "v", cap, hkv, "student_t6", "f16")
    extra_slots = np.array([2320, 2321, 2330], np.int32)   # a few rows written by slot list
    extra_k = _t(iqinputs.kv(42, 0, "k", 3, hkv, "student_t6", "f16"))
    extra_v = _t(iqinputs.kv(42, 0, "v", 3, hkv, "student_t6", "f16"))
    new_k = _t(iqinputs.kv(43, 0, "k", n_seqs, hkv, "student_t6", "f16"))
    new_v = _t(iqinputs.kv(43, 0, "v", n_seqs, hkv, "student_t6", "f16"))
    q = _t(iqinputs.queries(41, 1, n_seqs, hq))
    st, ln, ln1 = _t(starts), _t(lens), _t(lens + 1)
    mx = int(lens.max()) + 1

    def fresh(k_bits):
        c = iq.PackedKVCache.allocate(hkv, cap, rot, k_bits=k_bits)
        iq.iq_rotate_quantize_append(c, _t(x_k), _t(x_v), first_slot=0)
        return c

    c3, c4 = fresh(3), fresh(4)
    ws = iq.decode_workspace(n_seqs, hq, hkv, mx)
    outs = {name: torch.empty((n_seqs, hq, 128), dtype=torch.float32, device="cuda")
            for name in ("step", "decode", "decode_k4")}
    deq_k = torch.empty((64, hkv, 128), dtype=torch.float16, device="cuda")
    deq_v = torch.empty_like(deq_k)
    slots = _t(extra_slots)

    def calls(stream):
        iq.iq_rotate_quantize_append(c3, extra_k, extra_v, slots=slots, stream=stream)
        iq.iq_append_decode_attention(c3, new_k, new_v, q, st, ln, mx - 1, out=outs["step"], workspace=ws,
                                      stream=stream)
        iq.iq_decode_attention(c3, q, st, ln1, mx, out=outs["decode"], workspace=ws, stream=stream)
        iq.iq_decode_attention(c4, q, st, ln1, mx, out=outs["decode_k4"], workspace=ws, stream=stream)
        iq.iq_dequantize(c3, 690, 64, torch.float16, k_out=deq_k, v_out=deq_v, stream=stream)

    def state():
        return [t.clone() for t in (*outs.values(), deq_k, deq_v, c3.k_codes, c3.v_codes, c3.k_norms,
                                    c3.v_norms)]

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        calls(stream)
    torch.cuda.synchronize()
    eager = state()
    # the captured calls write the same rows again, so a replay must reproduce this state exactly
    graph = torch.cuda.CUDAGraph()
    cap_stream = torch.cuda.Stream()
    cap_stream.wait_stream(stream)
    with torch.cuda.stream(cap_stream):
        with torch.cuda.graph(graph, stream=cap_stream):
            calls(cap_stream)
    torch.cuda.synchronize()
    names = ["out step", "out decode", "out decode_k4", "dequant k", "dequant v", "k_codes", "v_codes",
             "k_norms", "v_norms"]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    for replay in range(3):
        with torch.cuda.stream(stream):
            # unrelated eager work between replays, then every output cleared
            a = torch.randn((256, 256), generator=gen, device="cuda")
            (a @ a).sum().item()
            for t in (*outs.values(), deq_k, deq_v):
                t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, e, g in zip(names, eager, state()):
            assert torch.equal(e, g), f"replay {replay}: {name} differs from the eager calls"


def test_graph_replays_of_the_other_decodes():
    """The no-allocation decode step (the entry point for callers under graph capture), the deferred
    decode (fp16 prefix, packed suffix) and the FP16-KV decode, captured together: every replay equals
    the eager calls bit for bit."""
    hkv, hq = 4, 32
    lens = np.array([900, 33, 0], np.int32)
    starts = np.array([5, 1000, 1100], np.int32)
    pre = np.array([300, 0, 77], np.int32)
    pst = np.array([0, 320, 640], np.int32)
    cap, cap16 = 1184, 736
    n_seqs = len(lens)
    rot = _t(iqinputs.rotation_params(51, 0, hkv))
    x_k = _t(iqinputs.kv(51, 0, "k", cap, hkv, "student_t6", "f16"))
    x_v = _t(iqinputs.kv(51, 0, "v", cap, hkv, "student_t6", "f16"))
    k16 = _t(iqinputs.kv(52, 0, "k", cap16, hkv, "student_t6", "f16"))
    v16 = _t(iqinputs.kv(52, 0, "v", cap16, hkv, "student_t6", "f16"))
    new_k = _t(iqinputs.kv(53, 0, "k", n_seqs, hkv, "student_t6", "f16"))
    new_v = _t(iqinputs.kv(53, 0, "v", n_seqs, hkv, "student_t6", "f16"))
    q = _t(iqinputs.queries(51, 1, n_seqs, hq))
    st, ln, ln1, pst_t, pre_t = _t(starts), _t(lens), _t(lens + 1), _t(pst), _t(pre)
    mx, mx16 = int(lens.max()), int(pre.max())
    cache = iq.PackedKVCache.allocate(hkv, cap, rot)
    iq.iq_rotate_quantize_append(cache, x_k, x_v, first_slot=0)
    outs = {name: torch.empty((n_seqs, hq, 128), dtype=torch.float32, device="cuda")
            for name in ("noalloc step", "deferred", "f16")}
    ws_def = torch.empty(max(iq.iq_decode_deferred_workspace_bytes(n_seqs, hq, hkv, mx16, mx + 1), 16),
                         dtype=torch.uint8, device="cuda")
    ws16 = iq.decode_workspace(n_seqs, hq, hkv, mx16)

    def calls(stream):
        iq.iq_append_decode_attention_noalloc(cache, new_k, new_v, q, st, ln, mx, out=outs["noalloc step"],
                                              stream=stream)
        iq.iq_decode_attention_deferred(cache, st, ln1, mx + 1, k16, v16, pst_t, pre_t, mx16, q,
                                        out=outs["deferred"], workspace=ws_def, stream=stream)
        iq.iq_decode_attention_f16(k16, v16, q, pst_t, pre_t, mx16, out=outs["f16"], workspace=ws16,
                                   stream=stream)

    def state():
        return [t.clone() for t in (*outs.values(), cache.k_codes, cache.v_codes, cache.k_norms, cache.v_norms)]

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        calls(stream)
    torch.cuda.synchronize()
    eager = state()
    graph = torch.cuda.CUDAGraph()
    cap_stream = torch.cuda.Stream()
    cap_stream.wait_stream(stream)
    with torch.cuda.stream(cap_stream):
        with torch.cuda.graph(graph, stream=cap_stream):
            calls(cap_stream)
    torch.cuda.synchronize()
    names = [*outs.keys(), "k_codes", "v_codes", "k_norms", "v_norms"]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(8)
    for replay in range(3):
        with torch.cuda.stream(stream):
            a = torch.randn((256, 256), generator=gen, device="cuda")
            (a @ a).sum().item()
            for t in outs.values():
                t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, e, g in zip(names, eager, state()):
            assert torch.equal(e, g), f"replay {replay}: {name} differs from the eager calls"
