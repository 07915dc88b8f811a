"""Host-side checks of libiq's C ABI: it loads, exports what include/iq.h
declares, computes the same codebook as the oracle, and rejects invalid
arguments before launching anything. No GPU is needed."""
import ctypes
import os
import re

import numpy as np
import pytest

import quantized_kv_cache_wht_amd as iq
from oracle import iqref

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "iq.h")).read()
    return sorted(set(re.findall(r"IQ_API\s+[\w\s\*]+?\b(iq_\w+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert len(names) == 14, names
    h = ctypes.CDLL(iq.library_path())
    for n in names:
        assert hasattr(h, n), n
    assert set(names) == set(iq._SIGNATURES)


def test_codebook_matches_oracle_bit_for_bit():
    c, t = iq.iq_codebook()
    oc, ot, _ = iqref.codebook()
    assert np.array_equal(c.view(np.uint32), oc.view(np.uint32))
    assert np.array_equal(t.view(np.uint32), ot.view(np.uint32))


def test_codebook16_matches_oracle_bit_for_bit():
    c, t = iq.iq_codebook(16)
    oc, ot, _ = iqref.codebook(levels=16)
    assert np.array_equal(c.view(np.uint32), oc.view(np.uint32))
    assert np.array_equal(t.view(np.uint32), ot.view(np.uint32))
    L = iq.lib()
    buf = np.zeros(16, np.float32)
    assert L.iq_codebook_levels(12, buf.ctypes.data, buf.ctypes.data) == -1


def test_status_strings():
    for s in (0, -1, -2, -3, -4, -5):
        assert iq.status_string(s)
    assert iq.status_string(-99) == "unknown status"


def _view(head_dim=128, hkv=2, cap=128, ptr=0x10000, rotation=0, k_bits=3):
    return iq.CacheView(head_dim, hkv, cap, ptr, ptr + 0x1000, ptr + 0x2000, ptr + 0x3000, ptr + 0x4000, rotation,
                        k_bits)


def test_append_validation():
    L = iq.lib()
    v = _view()
    p = ctypes.c_void_p(0x20000)
    assert L.iq_rotate_quantize_append(None, p, p, 1, 4, 0, None, None) == -1
    assert L.iq_rotate_quantize_append(ctypes.byref(_view(head_dim=64)), p, p, 1, 4, 0, None, None) == -2
    assert L.iq_rotate_quantize_append(ctypes.byref(v), p, p, 7, 4, 0, None, None) == -1      # dtype
    assert L.iq_rotate_quantize_append(ctypes.byref(v), p, p, 1, -1, 0, None, None) == -1     # n_tokens
    assert L.iq_rotate_quantize_append(ctypes.byref(v), p, p, 1, 4, 125, None, None) == -3    # past capacity
    assert L.iq_rotate_quantize_append(ctypes.byref(_view(cap=100)), p, p, 1, 4, 0, None, None) == -1  # cap % 32
    assert L.iq_rotate_quantize_append(ctypes.byref(v), p, p, 1, 4, -1, None, None) == -3
    assert L.iq_rotate_quantize_append(ctypes.byref(v), None, p, 1, 4, 0, None, None) == -1
    assert L.iq_rotate_quantize_append(ctypes.byref(v), ctypes.c_void_p(0x20004), p, 1, 4, 0, None, None) == -1
    assert L.iq_rotate_quantize_append(ctypes.byref(v), p, p, 1, 0, 0, None, None) == 0       # no-op
    bad = _view(ptr=0x10008)                                                                # misaligned arrays
    assert L.iq_rotate_quantize_append(ctypes.byref(bad), p, p, 1, 4, 0, None, None) == -1
    assert L.iq_rotate_quantize_append(ctypes.byref(_view(rotation=3)), p, p, 1, 4, 0, None, None) == -1
    assert L.iq_rotate_quantize_append(ctypes.byref(_view(rotation=2)), p, p, 1, 0, 0, None, None) == 0
    assert L.iq_rotate_quantize_append(ctypes.byref(_view(k_bits=5)), p, p, 1, 4, 0, None, None) == -1
    assert L.iq_rotate_quantize_append(ctypes.byref(_view(k_bits=4)), p, p, 1, 0, 0, None, None) == 0


def test_decode_validation():
    L = iq.lib()
    v = _view(hkv=2)
    p = ctypes.c_void_p(0x30000)
    need = L.iq_decode_workspace_bytes(1, 8, 2, 100)
    assert need > 0
    args = lambda hq=8, ws=need, n=1, ml=100: (ctypes.byref(v), p, hq, p, p, n, ml, 0.1, p, p, ws, None)
    assert L.iq_decode_attention(*args(hq=7)) == -1          # Hq % Hkv
    assert L.iq_decode_attention(*args(hq=6)) == -2          # group 3 unsupported
    assert L.iq_decode_attention(*args(hq=64)) == -2         # group 32 unsupported
    assert L.iq_decode_attention(*args(ws=need - 1)) == -4
    assert L.iq_decode_attention(*args(n=-1)) == -1
    assert L.iq_decode_attention(*args(n=0)) == 0
    assert L.iq_decode_attention(*args(n=65536, ws=1 << 40)) == -2   # grid limit
    assert L.iq_decode_workspace_bytes(-1, 8, 2, 100) == 0
    # workspace grows with context and shrinks to one split for short contexts
    assert L.iq_decode_workspace_bytes(1, 32, 4, 32768) >= L.iq_decode_workspace_bytes(1, 32, 4, 1024)
    # per query head: one split record, and the decode step's new token's
    assert L.iq_decode_workspace_bytes(1, 32, 8, 1) == 2 * 32 * 132 * 4


def test_decode_f16_validation():
    L = iq.lib()
    p = ctypes.c_void_p(0x50000)
    need = L.iq_decode_workspace_bytes(1, 8, 2, 100)

    def call(k=p, ts=256, hs=128, hkv=2, cap=128, hq=8, n=1, ws=need, wsp=p):
        return L.iq_decode_attention_f16(k, p, ts, hs, hkv, cap, p, hq, p, p, n, 100, 0.1, p, wsp, ws, None)
    assert call(cap=100) == -1                 # capacity % 32
    assert call(ts=12) == -1                   # stride % 8
    assert call(ts=0) == -1
    assert call(hq=7) == -1                    # Hq % Hkv
    assert call(hq=6) == -2                    # group 3
    assert call(ws=need - 1) == -4
    assert call(k=ctypes.c_void_p(0x50008)) == -1   # alignment
    assert call(k=None) == -1
    assert call(n=0) == 0
    assert call(hkv=0) == -1


def test_append_decode_validation():
    L = iq.lib()
    v = _view(hkv=2)
    p = ctypes.c_void_p(0x70000)
    need = L.iq_decode_workspace_bytes(1, 8, 2, 100)

    def call(dt=1, hq=8, ws=need, n=1, kn=p):
        return L.iq_append_decode_attention(ctypes.byref(v), kn, p, dt, p, hq, p, p, n, 100, 0.1, p, p, ws, None)
    assert call(dt=5) == -1
    assert call(hq=6) == -2
    assert call(ws=need - 1) == -4
    assert call(kn=None) == -1
    assert call(kn=ctypes.c_void_p(0x70004)) == -1
    assert call(n=0) == 0


def test_append_decode_noalloc_validation():
    """The no-allocation step checks the records' size against the scratch array on the host: a call
    whose records would not fit is refused before anything reaches a GPU."""
    L = iq.lib()
    v = _view(hkv=4)
    p = ctypes.c_void_p(0x90000)

    def call(hq=32, n=1, ml=100, kn=p):
        return L.iq_append_decode_attention_noalloc(ctypes.byref(v), kn, p, 1, p, hq, p, p, n, ml, 0.1, p, None)
    big = L.iq_decode_workspace_bytes(64, 32, 4, 32768)
    assert big > iq.NOALLOC_SCRATCH_BYTES
    assert call(n=64, ml=32768) == -4
    assert L.iq_decode_workspace_bytes(1, 32, 4, 32768) <= iq.NOALLOC_SCRATCH_BYTES
    assert L.iq_decode_workspace_bytes(32, 32, 8, 32768) <= iq.NOALLOC_SCRATCH_BYTES   # the ragged batch's
    assert call(hq=12) == -2        # group 3
    assert call(hq=6) == -1         # Hq % Hkv
    assert call(kn=None) == -1
    assert call(n=-1) == -1
    assert call(n=0) == 0


def test_noalloc_scratch_size_matches_header():
    src = open(os.path.join(ROOT, "include", "iq.h")).read()
    m = re.search(r"#define IQ_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == iq.NOALLOC_SCRATCH_BYTES


def test_decode_deferred_validation():
    L = iq.lib()
    v = _view(hkv=2)
    p = ctypes.c_void_p(0x60000)
    need = L.iq_decode_deferred_workspace_bytes(1, 8, 2, 300, 100)
    assert need >= L.iq_decode_workspace_bytes(1, 8, 2, 100)

    def call(hq=8, ws=need, cap16=320, ts=256, n=1):
        return L.iq_decode_attention_deferred(ctypes.byref(v), p, p, 100, p, p, ts, 128, cap16, p, p, 300,
                                              p, hq, n, 0.1, p, p, ws, None)
    assert call(ws=need - 1) == -4
    assert call(cap16=300) == -1
    assert call(ts=4) == -1
    assert call(hq=6) == -2
    assert call(n=0) == 0
    assert L.iq_decode_deferred_workspace_bytes(1, 8, 2, -1, 100) == 0


def test_dequant_and_rotate_validation():
    L = iq.lib()
    v = _view()
    p = ctypes.c_void_p(0x40000)
    assert L.iq_dequantize(ctypes.byref(v), 120, 20, 0, p, p, None) == -3
    assert L.iq_dequantize(ctypes.byref(v), 0, 20, 3, p, p, None) == -1
    assert L.iq_dequantize(ctypes.byref(v), 0, 20, 0, None, None, None) == 0
    assert L.iq_rotate(None, 0, 1, p, p, 4, 0, None) == -1
    assert L.iq_rotate(p, 0, 1, p, p, 4, 2, None) == -1
    assert L.iq_rotate(p, 0, 0, p, p, 4, 0, None) == -1
    assert L.iq_rotate(p, 3, 1, p, p, 4, 0, None) == -1        # unknown rotation kind
    assert L.iq_rotate(p, 2, 1, p, p, 0, 0, None) == 0
    assert L.iq_quantize_pack(p, -1, p, p, None) == -1
    assert L.iq_quantize_pack(p, 0, p, p, None) == 0


def test_binding_rotation_kinds_follow_parameter_shapes():
    import torch
    assert iq.rotation_kind(torch.zeros(3, 32, 8)) == iq.IQ_ROT_WHT_SO4
    assert iq.rotation_kind(torch.zeros(3, 32, 4)) == iq.IQ_ROT_ISO
    assert iq.rotation_kind(torch.zeros(3, 64, 2)) == iq.IQ_ROT_PLANAR
    with pytest.raises(ValueError):
        iq.rotation_kind(torch.zeros(3, 16, 8))


def test_binding_refuses_host_tensors():
    import torch
    with pytest.raises(TypeError):
        iq.iq_quantize_pack(torch.zeros(4, 128))
