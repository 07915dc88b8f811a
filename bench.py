"""Benchmark: packed 3-bit KV decode on one MI355X.

Workload (default): the 30B-A3B-MoE-shaped GQA decode at 32768 tokens of
context, 48 layers, 32 query heads, 4 KV heads, head dim 128, batch 1, K/V
fp16 with four fixed outlier channels x8 (synthetic, seeded). Untimed set-up
fills every layer's packed cache with 32767 tokens through the library's own
bulk encode. One timed step = for each of the 48 layers: encode and append
one new token (K and V) at slot 32767 and run decode attention over all 32768
packed tokens, as one iq_append_decode_attention call (a split-K launch whose
extra work-groups encode the new token beside the splits, then the merge). The 96 launches of a step are
captured once as a HIP graph and replayed per step (--eager launches them one
by one); every warm-up replay and the last timed one are compared bit for bit
with an eager step.

Printed JSON line: value = packed K/V bytes of the attended tokens per step /
step time (GB/s); roofline = the step's launch pair (split + merge kernels;
HIP events on the launch stream around runs of back-to-back launches) against
the 8 TB/s HBM peak, with the HBM traffic per launch from the committed
counter summary when it matches the decode sources; valu_roof = the same
launch pair's VALU instructions (same summary) against the chip's VALU issue
rate; comparisons = decode
alone, append + decode as two calls, the FP16-KV and unfused paths, the
rotation variants and 4-bit K; cpu_baseline = the plain C oracle's decode (and
encode) on a bounded sample of the same workload, on the host's cores;
append_roofline = the long-context bulk encode (131072 tokens x 8 KV heads)
against the VALU issue roof and the HBM roof, with the one-token append's
latency.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# VALU issue roof: one wave64 VALU instruction per clock per CU (4 SIMDs x 16
# lanes; fp32 without packed math), 256 CUs at 2.4 GHz, in G instructions/s
VALU_PEAK_GINST = 256 * 2.4
ROW_BYTES = 48 + 4          # packed codes + fp32 norm, one (token, KV head, K or V)
SPIN_CYCLES_PER_LAUNCH = 200_000   # ~80 us of GPU clock per queued launch: more than the host needs


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="moe30b_gqa_t32768")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the CPU oracle sample")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--eager", action="store_true", help="launch the step's kernels one by one instead of a graph")
    p.add_argument("--no-compare", action="store_true", help="skip the FP16-KV and unfused comparison timings")
    p.add_argument("--copy-calibration-mib", type=int, default=0,
                   help="finish with 3 device-to-device copies of this many MiB (reference for HBM counters)")
    p.add_argument("--profile-append", action="store_true",
                   help="only the bulk encode of the append roofline (and the calibration copies), for counter runs")
    p.add_argument("--profile-decode", choices=("long_t131072", "ragged32_gqa"), default=None,
                   help="only this workload's decode launches (and the calibration copies), for counter runs")
    return p.parse_args()


def calibration_copies(torch, mib: int):
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


DECODE_SOURCES = ("iq_decode.hip", "iq_decode_common.h", "iq_decode_packed.h", "iq_decode_packed_body.inc",
                  "iq_decode_new_token.h", "iq_device.h", "iq_launch.h")
ENCODE_SOURCES = ("iq_encode.hip", "iq_device.h", "iq_launch.h")


def source_digest(names=DECODE_SOURCES) -> str:
    """sha256 over the given kernel sources (counter figures belong to one version of them)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "quantized_kv_cache_wht_amd", "csrc")
    for name in names:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def decode_source_digest() -> str:
    return source_digest(DECODE_SOURCES)


def encode_source_digest() -> str:
    return source_digest(ENCODE_SOURCES)


def read_counters(path: str, digest: str) -> dict:
    """The per-launch counter figures of a committed summary (HBM bytes, VALU and MFMA
    instructions), if it was taken on the sources with this digest; else {}."""
    if not os.path.exists(path):
        return {}
    fields = {}
    with open(path) as f:
        for line in f:
            if line.startswith("- ") and ": " in line:
                k, v = line[2:].strip().split(": ", 1)
                fields[k.strip("`")] = v.strip().strip("`")
    if fields.get("source_sha256", fields.get("decode_source_sha256")) != digest:
        return {}
    out = {}
    for k in ("hbm_bytes_per_launch", "valu_insts_per_launch", "mfma_insts_per_launch"):
        try:
            out[k] = float(fields[k])
        except (KeyError, ValueError):
            pass
    return out


def measured_counters(workload: str) -> dict:
    """Counter figures of the decode step's launch pair (profiles/decode_<workload>_traffic.md)."""
    return read_counters(os.path.join(ROOT, "profiles", f"decode_{workload}_traffic.md"), decode_source_digest())


def measured_traffic(workload: str):
    """HBM bytes per decode launch from the committed counter summary, or None."""
    return measured_counters(workload).get("hbm_bytes_per_launch")


APPEND_WORKLOAD = "long_t131072"


def append_counters() -> dict:
    """Counter figures of the bulk encode (profiles/append_<workload>_traffic.md)."""
    return read_counters(os.path.join(ROOT, "profiles", f"append_{APPEND_WORKLOAD}_traffic.md"),
                         encode_source_digest())


def time_per_call(torch, fn, n_calls, stream):
    """GPU time per call of fn(i), i = 0 .. n_calls - 1, back to back on one stream."""
    for i in range(n_calls):
        fn(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(SPIN_CYCLES_PER_LAUNCH * 2 * n_calls)
    e0.record(stream)
    for i in range(n_calls):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / n_calls


def comparisons(iq, caches, qs, seq_start, seq_len, ws, outs, stream, synth_kv, T, hkv, fused_us, new_k, new_v,
                n_layers=8):
    """The pages' comparisons on this workload's decode: the same decode over an fp16 K/V cache
    (FP16-KV baseline, K/V of the same shape and value model) and the unfused path (iq_dequantize
    of the packed cache to fp16, then that decode), over n_layers layers' caches in turn (fp16
    caches of that many layers exceed the last-level cache); the decode alone and the step as two
    calls over all of the step's packed caches, as the fused step runs."""
    import torch
    k16 = [synth_kv(T, 30_000 + l).transpose(0, 1).contiguous() for l in range(n_layers)]   # [Hkv][T][128]
    v16 = [synth_kv(T, 40_000 + l).transpose(0, 1).contiguous() for l in range(n_layers)]
    dk = torch.empty((T, hkv, 128), dtype=torch.float16, device=k16[0].device)
    dv = torch.empty_like(dk)

    def fp16_decode(i):
        l = i % n_layers
        iq.iq_decode_attention_f16(k16[l], v16[l], qs[l], seq_start, seq_len, T, token_major=False, out=outs[l],
                                   workspace=ws, stream=stream)

    def dequantize(i):
        iq.iq_dequantize(caches[i % n_layers], 0, T, torch.float16, k_out=dk, v_out=dv, stream=stream)

    def unfused(i):
        l = i % n_layers
        dequantize(i)
        iq.iq_decode_attention_f16(dk, dv, qs[l], seq_start, seq_len, T, token_major=True, out=outs[l],
                                   workspace=ws, stream=stream)

    n = 4 * n_layers
    n_packed = len(caches)

    def decode_only(i):
        l = i % n_packed
        iq.iq_decode_attention(caches[l], qs[l], seq_start, seq_len, T, out=outs[l], workspace=ws, stream=stream)

    def append_then_decode(i):
        l = i % n_packed
        iq.iq_rotate_quantize_append(caches[l], new_k[l], new_v[l], first_slot=T - 1, stream=stream)
        decode_only(i)

    variants = rotation_variants(iq, caches, qs, seq_start, seq_len, ws, outs, stream, synth_kv, T, hkv)
    k4 = k4_decode(iq, qs, seq_start, seq_len, ws, outs, stream, synth_kv, T, hkv)
    r = {"layers_cycled": n_layers,
         "packed_layers_cycled": n_packed,
         "fused_step_us": round(fused_us, 3),
         "decode_only_us": round(time_per_call(torch, decode_only, 2 * n_packed, stream), 3),
         "append_then_decode_us": round(time_per_call(torch, append_then_decode, 2 * n_packed, stream), 3),
         "packed_bytes_per_launch": hkv * T * 2 * ROW_BYTES,
         "fp16_kv_decode_us": round(time_per_call(torch, fp16_decode, n, stream), 3),
         "fp16_kv_bytes_per_launch": hkv * T * 2 * 256,
         "dequantize_to_fp16_us": round(time_per_call(torch, dequantize, n, stream), 3),
         "unfused_decode_us": round(time_per_call(torch, unfused, n, stream), 3),
         "rotation_variants": variants,
         "k4_v3": k4}
    del k16, v16, dk, dv
    return r


def rotation_variants(iq, caches, qs, seq_start, seq_len, ws, outs, stream, synth_kv, T, hkv, n_layers=24):
    """Decode and one-token append per rotation kind, each over n_layers caches of this workload's
    shape (more bytes than the last-level cache holds), the default kind's being the main caches."""
    import torch
    import iqinputs
    res = {}
    for kind in iqinputs.ROTATION_KINDS:
        if kind == "wht_so4":
            cs = caches[:n_layers]
        else:
            cs = []
            for l in range(n_layers):
                rot = torch.from_numpy(iqinputs.rotation_params_kind(7, l, hkv, kind)).to(caches[0].k_codes.device)
                c = iq.PackedKVCache.allocate(hkv, T, rot, device=rot.device)
                iq.iq_rotate_quantize_append(c, synth_kv(T, 50_000 + l), synth_kv(T, 60_000 + l), first_slot=0,
                                             stream=stream)
                cs.append(c)
        k1, v1 = synth_kv(1, 70_000), synth_kv(1, 70_001)

        def dec(i, cs=cs):
            l = i % n_layers
            iq.iq_decode_attention(cs[l], qs[l], seq_start, seq_len, T, out=outs[l], workspace=ws, stream=stream)

        def app(i, cs=cs):
            iq.iq_rotate_quantize_append(cs[i % n_layers], k1, v1, first_slot=T - 1, stream=stream)
        res[kind] = {"decode_us": round(time_per_call(torch, dec, 2 * n_layers, stream), 3),
                     "append_1_token_us": round(time_per_call(torch, app, 2 * n_layers, stream), 3)}
    return res


def k4_decode(iq, qs, seq_start, seq_len, ws, outs, stream, synth_kv, T, hkv, n_layers=24):
    """Decode with 4-bit K and 3-bit V (120 B per token and KV head) over n_layers caches."""
    import torch
    import iqinputs
    cs = []
    for l in range(n_layers):
        rot = torch.from_numpy(iqinputs.rotation_params(9, l, hkv)).to(qs[0].device)
        c = iq.PackedKVCache.allocate(hkv, T, rot, device=rot.device, k_bits=4)
        iq.iq_rotate_quantize_append(c, synth_kv(T, 80_000 + l), synth_kv(T, 90_000 + l), first_slot=0,
                                     stream=stream)
        cs.append(c)

    def dec(i):
        l = i % n_layers
        iq.iq_decode_attention(cs[l], qs[l], seq_start, seq_len, T, out=outs[l], workspace=ws, stream=stream)
    return {"decode_us": round(time_per_call(torch, dec, 2 * n_layers, stream), 3),
            "bytes_per_launch": hkv * T * (64 + 4 + 48 + 4)}


def append_bulk(iq, stream, reps=6):
    """The long-context workload's bulk encode (prefill-style compression): 131072 fp16 tokens of
    K and V, 8 KV heads, into three layers' caches in turn (inputs and caches exceed the last-level
    cache). One iq_rotate_quantize_append call is one launch of the bulk kernel (grid z: K and V).
    Returns (us per call, tokens, KV heads)."""
    import torch
    import iqinputs
    dev = torch.device("cuda")
    gen = torch.Generator(device=dev)
    gen.manual_seed(20260819)
    w = iqinputs.WORKLOADS[APPEND_WORKLOAD]
    T, hkv = w.seq_len, w.num_kv_heads
    k = torch.randn((T, hkv, 128), generator=gen, device=dev).half()
    v = torch.randn((T, hkv, 128), generator=gen, device=dev).half()
    rot = torch.from_numpy(iqinputs.rotation_params(12, 0, hkv)).to(dev)
    cs = [iq.PackedKVCache.allocate(hkv, T, rot, device=dev) for _ in range(3)]
    us = time_per_call(torch, lambda i: iq.iq_rotate_quantize_append(cs[i % 3], k, v, first_slot=0, stream=stream),
                       reps, stream)
    del k, v, cs
    torch.cuda.empty_cache()
    return us, T, hkv


def append_roofline(us: float, T: int, hkv: int, one_token_us: float | None) -> dict:
    """The bulk encode against the VALU issue roof (its bound: the counters read its loop at the
    issue rate) and the HBM roof. Algorithmic bytes per vector (token, KV head, K or V): 256 B of
    fp16 in, 48 B of codes and a 4 B norm out."""
    nbytes = T * hkv * 2 * (256 + ROW_BYTES)
    gbps = nbytes / us / 1e3
    c = append_counters()
    valu = c.get("valu_insts_per_launch")
    traffic = c.get("hbm_bytes_per_launch")
    hbm = {"achieved": round(gbps, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBS, 4),
           "traffic": None if traffic is None else round(traffic), "algorithmic_bytes": nbytes}
    r = {"kernel": "append_kernel<_Float16, false, false>",
         "launch": f"{T} tokens x {hkv} KV heads, K and V (fp16 in)",
         "launch_us": round(us, 2), "token_layers_per_s": round(T / (us * 1e-6)),
         "one_token_append_us": None if one_token_us is None else round(one_token_us, 3)}
    if valu is not None:
        gi = valu / (us * 1e-6) / 1e9
        r.update({"bound": "alu", "achieved": round(gi, 2), "peak": VALU_PEAK_GINST, "unit": "Ginst/s",
                  "frac": round(gi / VALU_PEAK_GINST, 4), "valu_insts_per_launch": round(valu), "hbm": hbm})
    else:
        r.update({"bound": "hbm", **{k: hbm[k] for k in ("achieved", "peak", "unit", "frac", "traffic")}})
    return r


def long_decode(iq, stream, gen, timing_cache, calls=12):
    """The 131072-token decode (32 query heads, 8 KV heads) over three layers' caches in turn, back
    to back; returns (us per call, packed bytes per call)."""
    import torch
    import iqinputs
    dev = torch.device("cuda")
    w = iqinputs.WORKLOADS["long_t131072"]
    T, hkv, hq = w.seq_len, w.num_kv_heads, w.num_q_heads
    cs = [timing_cache(hkv, T) for _ in range(3)]
    ql = torch.randn((1, hq, 128), generator=gen, device=dev)
    stl = torch.zeros(1, dtype=torch.int32, device=dev)
    lnl = torch.full((1,), T, dtype=torch.int32, device=dev)
    wsl = iq.decode_workspace(1, hq, hkv, T, device=dev)
    outl = torch.empty_like(ql)
    us = time_per_call(torch, lambda i: iq.iq_decode_attention(cs[i % 3], ql, stl, lnl, T, out=outl,
                                                               workspace=wsl, stream=stream), calls, stream)
    del cs
    return us, hkv * T * 2 * ROW_BYTES


def ragged_decode(iq, stream, gen, timing_cache, calls=10):
    """The 32-sequence ragged batch (seeded lengths in [1024, 32768], 32 query heads, 8 KV heads) on
    one layer's cache, back to back; returns (us per call, packed bytes per call)."""
    import numpy as np
    import torch
    import iqinputs
    dev = torch.device("cuda")
    w = iqinputs.WORKLOADS["ragged32_gqa"]
    lens = np.asarray(iqinputs.seq_lengths(w), np.int32)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int32)
    total, hkv, hq = int(lens.sum()), w.num_kv_heads, w.num_q_heads
    cap = -(-total // 32) * 32
    c = timing_cache(hkv, cap)
    qb = torch.randn((len(lens), hq, 128), generator=gen, device=dev)
    stb, lnb = torch.from_numpy(starts).to(dev), torch.from_numpy(lens).to(dev)
    ml = int(lens.max())
    wsb = iq.decode_workspace(len(lens), hq, hkv, ml, device=dev)
    outb = torch.empty_like(qb)
    us = time_per_call(torch, lambda i: iq.iq_decode_attention(c, qb, stb, lnb, ml, out=outb, workspace=wsb,
                                                                stream=stream), calls, stream)
    del c, wsb
    return us, hkv * total * 2 * ROW_BYTES


def random_code_cache(iq, gen):
    """A cache factory for timing: random codes and norms (the decode's work does not depend on the
    values; parity at these shapes is tested separately)."""
    import torch
    import iqinputs
    dev = torch.device("cuda")

    def timing_cache(hkv, cap):
        rot = torch.from_numpy(iqinputs.rotation_params(11, 0, hkv)).to(dev)
        c = iq.PackedKVCache.allocate(hkv, cap, rot, device=dev)
        c.k_codes.random_(0, 256, generator=gen)
        c.v_codes.random_(0, 256, generator=gen)
        c.k_norms.uniform_(5.0, 15.0, generator=gen)
        c.v_norms.uniform_(5.0, 15.0, generator=gen)
        return c
    return timing_cache


def other_workloads(iq, stream):
    """The other measured configurations, timed like the main one (HIP events around back-to-back
    calls). Their caches hold random codes and norms (the decode's work does not depend on the
    values; parity at these shapes is tested separately); the bulk encode runs on seeded N(0,1) fp16
    K/V. Also a device-to-device copy, the streaming peak measured on this GPU."""
    import torch
    import iqinputs
    dev = torch.device("cuda")
    gen = torch.Generator(device=dev)
    gen.manual_seed(20260818)
    timing_cache = random_code_cache(iq, gen)

    res = {}
    # 8B dense shape: Hq 32, Hkv 8, 8191 cached tokens, 32 layers, one decode step per layer
    w = iqinputs.WORKLOADS["dense8b_gqa_t8192"]
    T, hkv, hq, L = w.seq_len, w.num_kv_heads, w.num_q_heads, w.n_layers
    cs = [timing_cache(hkv, T) for _ in range(L)]
    q = torch.randn((1, hq, 128), generator=gen, device=dev)
    kn = torch.randn((1, hkv, 128), generator=gen, device=dev).half()
    vn = torch.randn((1, hkv, 128), generator=gen, device=dev).half()
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    cached = torch.full((1,), T - 1, dtype=torch.int32, device=dev)
    ws = iq.decode_workspace(1, hq, hkv, T, device=dev)
    out = torch.empty((1, hq, 128), device=dev)

    def step8b(i):
        iq.iq_append_decode_attention(cs[i % L], kn, vn, q, st, cached, T - 1, out=out, workspace=ws, stream=stream)
    us = time_per_call(torch, step8b, 2 * L, stream)
    nbytes = hkv * T * 2 * ROW_BYTES
    res[w.name] = {"step_per_layer_us": round(us, 3), "ms_per_step": round(us * L / 1e3, 4),
                   "GBps": round(nbytes / us / 1e3, 1),
                   "note": "the 32 layers' packed caches (218 MB) fit the 256 MB last-level cache"}
    del cs

    # batched: 32 sequences with seeded lengths in [1024, 32768], Hkv 8, one layer (over 400 MB)
    us, nbytes = ragged_decode(iq, stream, gen, timing_cache)
    res["ragged32_gqa"] = {"decode_us": round(us, 1), "bytes": nbytes, "GBps": round(nbytes / us / 1e3, 1),
                           "frac_hbm_peak": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4)}

    # long context: decode over three layers' caches of 131072 tokens
    us_dec, dec_bytes = long_decode(iq, stream, gen, timing_cache)
    res["long_t131072"] = {"decode_us": round(us_dec, 2), "decode_GBps": round(dec_bytes / us_dec / 1e3, 1),
                           "frac_hbm_peak": round(dec_bytes / us_dec / 1e3 / HBM_PEAK_GBS, 4),
                           "note": "the bulk encode of this workload is append_roofline"}

    # streaming peak on this GPU: device-to-device copy of 1 GiB (read + write bytes)
    a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    us = time_per_call(torch, lambda i: b.copy_(a), 5, stream)
    res["copy_1GiB"] = {"us": round(us, 1), "GBps": round(2 * (1 << 30) / us / 1e3, 1)}
    del a, b
    torch.cuda.empty_cache()
    return res


def cpu_baseline(w, budget_s: float):
    """The plain C oracle (oracle/iqoracle.c: double precision, OpenMP over tokens) on the host's
    cores: decodes of (layer 0, KV head h) over the workload's packed tokens, cycling through the
    heads, for about 80% of budget_s, then the encode (rotate + quantize + pack, K and V of every
    KV head) of the layer's tokens for the rest. The cache it decodes is encoded by the numpy oracle
    (untimed)."""
    import numpy as np
    import iqinputs
    from oracle import iqoracle_c as C
    from oracle import iqref as R

    c32, t32, _ = R.codebook()
    T, hkv = w.seq_len, w.num_kv_heads
    rot = iqinputs.rotation_params(w.seed, 0, hkv)
    k = iqinputs.kv(w.seed, 0, "k", T, hkv, w.outliers, w.dtype)
    v = iqinputs.kv(w.seed, 0, "v", T, hkv, w.outliers, w.dtype)
    q = iqinputs.queries(w.seed, 0, 1, w.num_q_heads)
    kr, kn = R.encode_tokens(k, rot, t32)
    vr, vn = R.encode_tokens_v(v, rot, t32)
    st, ln = np.array([0], np.int32), np.array([T], np.int32)
    threads = C.threads()
    C.decode(q, kr, kn, vr, vn, rot, c32, c32, st, ln, 1.0 / math.sqrt(128), heads=[0])   # warm-up
    done, t0 = 0, time.perf_counter()
    while True:
        C.decode(q, kr, kn, vr, vn, rot, c32, c32, st, ln, 1.0 / math.sqrt(128), heads=[done % hkv])
        done += 1
        el = time.perf_counter() - t0
        if el >= 0.8 * budget_s:
            break
    dec_gbps = done * T * 2 * ROW_BYTES / el / 1e9
    kf, vf = k.astype(np.float32), v.astype(np.float32)
    layers, t1 = 0, time.perf_counter()
    while True:
        for h in range(hkv):
            C.encode(kf[:, h], rot[h], t32)
            C.encode(vf[:, h], rot[h], t32)
        layers += 1
        el_enc = time.perf_counter() - t1
        if el_enc >= 0.2 * budget_s:
            break
    return {"value": round(dec_gbps, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} decodes of (layer 0, one KV head) over {T} packed tokens x {w.group} query heads, "
                      f"{el:.1f} s; plain C oracle (double, OpenMP over tokens, {threads} threads; "
                      f"host reports {os.cpu_count()} CPUs)",
            "quantize_append_token_layers_per_s": round(layers * T / el_enc, 1),
            "quantize_append_sample": f"{layers} encodes of the layer's {T} tokens (K and V of {hkv} KV heads), "
                                      f"{el_enc:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)

    import numpy as np
    import torch
    import iqinputs
    import quantized_kv_cache_wht_amd as iq

    w = iqinputs.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.profile_decode:
        gen = torch.Generator(device=dev)
        gen.manual_seed(20260818)
        run = long_decode if args.profile_decode == "long_t131072" else ragged_decode
        us, nbytes = run(iq, torch.cuda.current_stream(), gen, random_code_cache(iq, gen), calls=6)
        if args.copy_calibration_mib > 0:
            calibration_copies(torch, args.copy_calibration_mib)
        print(json.dumps({"profile_decode_us": round(us, 2), "workload": args.profile_decode, "bytes": nbytes}),
              flush=True)
        return
    if args.profile_append:
        us, T_a, hkv_a = append_bulk(iq, torch.cuda.current_stream())
        if args.copy_calibration_mib > 0:
            calibration_copies(torch, args.copy_calibration_mib)
        print(json.dumps({"profile_append_us": round(us, 2), "tokens": T_a, "num_kv_heads": hkv_a}), flush=True)
        return
    T, L, hq, hkv = w.seq_len, w.n_layers, w.num_q_heads, w.num_kv_heads
    fdt = torch.float16 if w.dtype == "f16" else torch.float32
    stream = torch.cuda.current_stream()
    gen = torch.Generator(device=dev)

    def synth_kv(n, seed):
        gen.manual_seed(seed)
        x = torch.randn((n, hkv, 128), generator=gen, device=dev, dtype=torch.float32)
        if w.outliers == "fixed_x8":
            x[:, :, list(iqinputs.FIXED_OUTLIER_CHANNELS)] *= iqinputs.FIXED_OUTLIER_SCALE
        else:
            tdist = torch.distributions.StudentT(torch.tensor(3.0, device=dev))
            for h in range(hkv):
                ch = torch.randperm(128, generator=gen, device=dev)[:6]
                x[:, h, ch] = tdist.sample((n, 6))
        return x.to(fdt).contiguous()

    # ---- set-up: fill the caches (untimed except the bulk-encode rate) ----
    caches, qs = [], []
    enc_ms = []
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for l in range(L):
        rot = torch.from_numpy(iqinputs.rotation_params(w.seed, l, hkv)).to(dev)
        c = iq.PackedKVCache.allocate(hkv, T, rot, device=dev)
        k, v = synth_kv(T - 1, 2 * l), synth_kv(T - 1, 2 * l + 1)
        ev0.record(stream)
        iq.iq_rotate_quantize_append(c, k, v, first_slot=0)
        ev1.record(stream)
        torch.cuda.synchronize()
        enc_ms.append(ev0.elapsed_time(ev1))
        del k, v
        caches.append(c)
        qs.append(torch.from_numpy(iqinputs.queries(w.seed, l, 1, hq)).to(dev))
    enc_ms = sorted(enc_ms)[len(enc_ms) // 2]
    append_tok_layers_per_s = (T - 1) / (enc_ms * 1e-3)

    new_k = [synth_kv(1, 10_000 + l) for l in range(L)]
    new_v = [synth_kv(1, 20_000 + l) for l in range(L)]
    seq_start = torch.zeros(1, dtype=torch.int32, device=dev)
    seq_len = torch.full((1,), T, dtype=torch.int32, device=dev)          # after the step's append
    cached = torch.full((1,), T - 1, dtype=torch.int32, device=dev)       # before it
    ws = iq.decode_workspace(1, hq, hkv, T, device=dev)
    outs = [torch.empty((1, hq, 128), dtype=torch.float32, device=dev) for _ in range(L)]

    def step_layer(l, st):
        # append the new token at slot T - 1 and attend to all T tokens (split + merge launches)
        iq.iq_append_decode_attention(caches[l], new_k[l], new_v[l], qs[l], seq_start, cached, T - 1, out=outs[l],
                                      workspace=ws, stream=st)

    def step(st):
        for l in range(L):
            step_layer(l, st)

    # eager reference of one step
    step(stream)
    torch.cuda.synchronize()
    eager = torch.stack(outs).clone()

    # the whole step (48 x (append + decode)) is one HIP graph, replayed per step
    graph = None
    if not args.eager:
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            with torch.cuda.graph(graph, stream=cap):
                step(cap)
        stream.wait_stream(cap)
        torch.cuda.synchronize()
    run = (lambda: graph.replay()) if graph is not None else (lambda: step(stream))

    replays_match = True
    for _ in range(args.warmup):
        for o in outs:
            o.fill_(float("nan"))
        run()
        torch.cuda.synchronize()
        replays_match &= bool(torch.equal(torch.stack(outs), eager))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        run()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    replays_match &= bool(torch.equal(torch.stack(outs), eager))
    ms_per_step = el * 1e3 / args.steps
    bytes_per_launch = hkv * T * 2 * ROW_BYTES
    bytes_per_step = L * bytes_per_launch
    value = bytes_per_step / (ms_per_step * 1e-3) / 1e9

    # decode-step launches (split kernel with the new token's work-groups, then
    # the merge) timed with HIP events on their stream: each pair of events
    # brackets one launch pair per layer, back to back,
    # and a spin kernel queued first keeps the GPU busy while the host enqueues
    # them, so the events time the GPU, not the host's calls.
    reps = max(2, args.steps // 4)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    torch.cuda._sleep(SPIN_CYCLES_PER_LAUNCH * reps * L)
    evs[0].record(stream)
    for r in range(reps):
        for l in range(L):
            step_layer(l, stream)
        evs[r + 1].record(stream)
    torch.cuda.synchronize()
    dec_us = np.array([evs[r].elapsed_time(evs[r + 1]) * 1e3 / L for r in range(reps)])
    achieved = bytes_per_launch / (dec_us.mean() * 1e-6) / 1e9
    counters = measured_counters(w.name)
    traffic = counters.get("hbm_bytes_per_launch")
    valu = counters.get("valu_insts_per_launch")
    comp = None if args.no_compare else comparisons(iq, caches, qs, seq_start, seq_len, ws, outs, stream, synth_kv,
                                                     T, hkv, float(dec_us.mean()), new_k, new_v)
    others = None if args.no_compare else other_workloads(iq, stream)

    # quantize-append: the one-token append of the step's shape (latency) over the step's caches, and
    # the long-context bulk encode against its roofs
    one_tok_us = time_per_call(torch, lambda i: iq.iq_rotate_quantize_append(
        caches[i % L], new_k[i % L], new_v[i % L], first_slot=T - 1, stream=stream), 2 * L, stream)
    app_us, app_T, app_hkv = append_bulk(iq, stream)
    app_roof = append_roofline(app_us, app_T, app_hkv, one_tok_us)

    if args.copy_calibration_mib > 0:
        calibration_copies(torch, args.copy_calibration_mib)

    res = {
        "metric": "packed-KV decode attention GB/s & % HBM peak; quantize-append tokens/s",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # the contractions run on fp16 MFMA with fp32 accumulation; scores and queries in hi/lo fp16
        # pairs (fp32-level products), V centroids as fp16 hi halves (within 2e-5); softmax in fp32
        "dtype": "f16 hi/lo MFMA, f32 accumulate",
        "data": "synthetic",
        "config": {"workload": w.name, "context": T, "layers": L, "num_q_heads": hq, "num_kv_heads": hkv,
                   "head_dim": 128, "batch": 1, "kv_input": w.dtype,
                   "step": "per layer: append 1 token (K,V) + decode over the packed cache",
                   "launch": "eager" if graph is None else "hip_graph"},
        "graph_replays_match_eager": replays_match,
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "decode_launch_us": {"mean": round(float(dec_us.mean()), 3), "median": round(float(np.median(dec_us)), 3),
                             "min": round(float(dec_us.min()), 3)},
        "quantize_append_token_layers_per_s": app_roof["token_layers_per_s"],
        "quantize_append": {"bulk_131072x8_token_layers_per_s": app_roof["token_layers_per_s"],
                            "setup_bulk_32767x4_token_layers_per_s": round(append_tok_layers_per_s, 1),
                            "setup_bulk_32767x4_ms": round(enc_ms, 4),
                            "one_token_append_us": app_roof["one_token_append_us"]},
        "append_roofline": app_roof,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else round(traffic)},
        # the same launch pair against the VALU issue roof (instruction count from the
        # committed counter summary, time from the events above; null when stale)
        "valu_roof": None if valu is None else {
            "bound": "alu", "achieved": round(valu / (dec_us.mean() * 1e-6) / 1e9, 2), "peak": VALU_PEAK_GINST,
            "unit": "Ginst/s", "frac": round(valu / (dec_us.mean() * 1e-6) / 1e9 / VALU_PEAK_GINST, 4),
            "valu_insts_per_launch": round(valu), "mfma_insts_per_launch": round(counters.get("mfma_insts_per_launch", 0))},
        "comparisons": comp,
        "other_workloads": others,
    }
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
