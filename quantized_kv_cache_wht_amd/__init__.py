"""IsoQuant packed 3-bit KV cache for AMD MI355X (gfx950).

Thin Python binding over the C ABI of ``libiq.so`` (declared in
``include/iq.h``). Every step of the method runs in the library's HIP
kernels; this module only checks tensor shapes and dtypes, passes device
pointers and the current HIP stream, and turns error codes into exceptions.
PyTorch supplies device memory and streams. There is no CPU fallback: if the
library has not been built, importing the binding's functions raises.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os

import numpy as np
import torch

HEAD_DIM = 128
ROW_BYTES = 48
TILE = 8                    # V tiles: 8 slots, dim-major
TILE_BYTES = TILE * ROW_BYTES
CAPACITY_MULTIPLE = 32      # cache capacity must be a multiple of this
ROT_PARAMS_PER_HEAD = 256
# iq_rotation: the kind follows from the parameters' per-head shape
IQ_ROT_WHT_SO4, IQ_ROT_ISO, IQ_ROT_PLANAR = 0, 1, 2
_ROT_SHAPES = {(32, 8): IQ_ROT_WHT_SO4, (32, 4): IQ_ROT_ISO, (64, 2): IQ_ROT_PLANAR}


def rotation_kind(rot: torch.Tensor) -> int:
    """iq_rotation of per-head parameters [Hkv][32][8] (WHT + SO(4)), [Hkv][32][4] (one quaternion per
    block) or [Hkv][64][2] (one Givens rotation per dim pair)."""
    kind = _ROT_SHAPES.get(tuple(rot.shape[-2:]))
    if kind is None or rot.dim() != 3:
        raise ValueError(f"rotation parameters of shape {tuple(rot.shape)} match no rotation kind")
    return kind

IQ_OK = 0
IQ_F32 = 0
IQ_F16 = 1

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libiq.so")
_lib = None


class IqError(RuntimeError):
    """A libiq call returned a non-OK status."""

    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {status_string(status)} (status {status})")


class CacheView(ctypes.Structure):
    """Mirror of ``iq_cache_view``."""
    _fields_ = [
        ("head_dim", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("capacity", ctypes.c_int32),
        ("k_codes", ctypes.c_void_p),
        ("v_codes", ctypes.c_void_p),
        ("k_norms", ctypes.c_void_p),
        ("v_norms", ctypes.c_void_p),
        ("rot", ctypes.c_void_p),
        ("rotation", ctypes.c_int32),
        ("k_bits", ctypes.c_int32),
    ]


_SIGNATURES = {
    "iq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "iq_codebook": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p]),
    "iq_codebook_levels": (ctypes.c_int, [ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]),
    "iq_rotate": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                 ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]),
    "iq_quantize_pack": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p]),
    "iq_rotate_quantize_append": (ctypes.c_int, [ctypes.POINTER(CacheView), ctypes.c_void_p, ctypes.c_void_p,
                                                 ctypes.c_int, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                                 ctypes.c_void_p]),
    "iq_dequantize": (ctypes.c_int, [ctypes.POINTER(CacheView), ctypes.c_int32, ctypes.c_int32, ctypes.c_int,
                                     ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "iq_decode_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                    ctypes.c_int32]),
    "iq_decode_attention": (ctypes.c_int, [ctypes.POINTER(CacheView), ctypes.c_void_p, ctypes.c_int32,
                                           ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                           ctypes.c_void_p]),
    "iq_decode_deferred_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                             ctypes.c_int32, ctypes.c_int32]),
    "iq_decode_attention_deferred": (ctypes.c_int, [ctypes.POINTER(CacheView), ctypes.c_void_p, ctypes.c_void_p,
                                                    ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                                    ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                                    ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                                    ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p,
                                                    ctypes.c_size_t, ctypes.c_void_p]),
    "iq_append_decode_attention": (ctypes.c_int, [ctypes.POINTER(CacheView), ctypes.c_void_p, ctypes.c_void_p,
                                                  ctypes.c_int, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                                  ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_float,
                                                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                                  ctypes.c_void_p]),
    "iq_append_decode_attention_noalloc": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                                          ctypes.c_int, ctypes.c_void_p, ctypes.c_int32,
                                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                                          ctypes.c_int32, ctypes.c_float, ctypes.c_void_p,
                                                          ctypes.c_void_p]),
    "iq_decode_attention_f16": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                               ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
                                               ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                               ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                               ctypes.c_void_p]),
}


def library_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """The loaded libiq (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"libiq.so not found at {_LIB_PATH}; build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        h = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            f = getattr(h, name)
            f.restype, f.argtypes = res, args
        _lib = h
    return _lib


def status_string(status: int) -> str:
    return lib().iq_status_string(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != IQ_OK:
        raise IqError(fn, status)


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(t: torch.Tensor, dtype: torch.dtype, name: str) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


# --------------------------------------------------------------------------
def iq_codebook(levels: int = 8):
    """(centroids float32[L], thresholds float32[L-1]) as the library computes them (host call);
    L = 8 (3-bit) or 16 (4-bit K)."""
    c = np.zeros(levels, np.float32)
    t = np.zeros(levels - 1, np.float32)
    if levels == 8:
        _check("iq_codebook", lib().iq_codebook(c.ctypes.data, t.ctypes.data))
    else:
        _check("iq_codebook_levels", lib().iq_codebook_levels(levels, c.ctypes.data, t.ctypes.data))
    return c, t


@dataclasses.dataclass
class PackedKVCache:
    """Device buffers of one layer of the packed cache (allocated with torch).

    K is stored as one row per slot (48 bytes, or 64 for 4-bit K); V as 384-byte tiles of 8 slots
    (dim-major: code of dim j of the slot at tile position r at bits 24j + 3r).
    """
    k_codes: torch.Tensor     # uint8 [Hkv][capacity][16 * k_bits]
    v_codes: torch.Tensor     # uint8 [Hkv][capacity / 8][384]
    k_norms: torch.Tensor     # float32 [Hkv][capacity]
    v_norms: torch.Tensor
    rot: torch.Tensor         # float32 [Hkv][32][8], [Hkv][32][4] or [Hkv][64][2] (see rotation_kind)

    @classmethod
    def allocate(cls, num_kv_heads: int, capacity: int, rot: torch.Tensor, device="cuda",
                 k_bits: int = 3) -> "PackedKVCache":
        """Zeroed cache with at least ``capacity`` slots (rounded up to a multiple of 32)."""
        cap = -(-capacity // CAPACITY_MULTIPLE) * CAPACITY_MULTIPLE
        zf = lambda: torch.zeros((num_kv_heads, cap), dtype=torch.float32, device=device)
        rot = rot.to(device=device, dtype=torch.float32).contiguous()
        rotation_kind(rot)
        if rot.shape[0] != num_kv_heads:
            raise ValueError("rot must hold num_kv_heads heads")
        if k_bits not in (3, 4):
            raise ValueError("k_bits must be 3 or 4")
        return cls(torch.zeros((num_kv_heads, cap, 16 * k_bits), dtype=torch.uint8, device=device),
                   torch.zeros((num_kv_heads, cap // TILE, TILE_BYTES), dtype=torch.uint8, device=device),
                   zf(), zf(), rot)

    @property
    def num_kv_heads(self) -> int:
        return self.k_codes.shape[0]

    @property
    def capacity(self) -> int:
        return self.k_codes.shape[1]

    @property
    def k_bits(self) -> int:
        return self.k_codes.shape[2] // 16

    def view(self) -> CacheView:
        for name in ("k_codes", "v_codes"):
            _dev(getattr(self, name), torch.uint8, name)
        for name in ("k_norms", "v_norms", "rot"):
            _dev(getattr(self, name), torch.float32, name)
        return CacheView(HEAD_DIM, self.num_kv_heads, self.capacity, self.k_codes.data_ptr(),
                         self.v_codes.data_ptr(), self.k_norms.data_ptr(), self.v_norms.data_ptr(),
                         self.rot.data_ptr(), rotation_kind(self.rot), self.k_bits)


def iq_rotate(rot: torch.Tensor, x: torch.Tensor, inverse: bool = False, out: torch.Tensor | None = None,
              stream=None) -> torch.Tensor:
    """y = R x (or R^-1 x) for x float32 [n_tokens][num_heads][128]; the kind of R follows from rot's shape."""
    n_tok, heads, d = x.shape
    out = torch.empty_like(x) if out is None else out
    _check("iq_rotate", lib().iq_rotate(_dev(rot, torch.float32, "rot"), rotation_kind(rot), heads,
                                        _dev(x, torch.float32, "x"),
                                        _dev(out, torch.float32, "out"), n_tok, int(bool(inverse)),
                                        _stream(stream)))
    return out


def iq_quantize_pack(y: torch.Tensor, stream=None):
    """Codes uint8 [n][48] and norms float32 [n] of rotated vectors y float32 [n][128]."""
    n = y.shape[0]
    codes = torch.empty((n, ROW_BYTES), dtype=torch.uint8, device=y.device)
    norms = torch.empty((n,), dtype=torch.float32, device=y.device)
    _check("iq_quantize_pack", lib().iq_quantize_pack(_dev(y, torch.float32, "y"), n, codes.data_ptr(),
                                                      norms.data_ptr(), _stream(stream)))
    return codes, norms


def _in_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return IQ_F32
    if t.dtype == torch.float16:
        return IQ_F16
    raise TypeError("K/V must be float32 or float16")


def iq_rotate_quantize_append(cache: PackedKVCache, k: torch.Tensor, v: torch.Tensor, first_slot: int = 0,
                              slots: torch.Tensor | None = None, stream=None) -> None:
    """Encode new tokens k, v [n_tokens][Hkv][128] into the cache rows."""
    n_tok = k.shape[0]
    dt = _in_dtype(k)
    if v.dtype != k.dtype or v.shape != k.shape:
        raise ValueError("k and v must match")
    sp = _dev(slots, torch.int32, "slots") if slots is not None else None
    view = cache.view()
    _check("iq_rotate_quantize_append",
           lib().iq_rotate_quantize_append(ctypes.byref(view), _dev(k, k.dtype, "k"), _dev(v, v.dtype, "v"), dt,
                                           n_tok, first_slot, sp, _stream(stream)))


def iq_dequantize(cache: PackedKVCache, first_slot: int, n_tokens: int, out_dtype=torch.float32,
                  k_out: torch.Tensor | None = None, v_out: torch.Tensor | None = None, stream=None):
    """Explicit reconstruction of K and V rows: two tensors [n_tokens][Hkv][128] (given or new)."""
    dt = {torch.float32: IQ_F32, torch.float16: IQ_F16}[out_dtype]
    shape = (n_tokens, cache.num_kv_heads, HEAD_DIM)
    dev = cache.k_codes.device
    k_out = torch.empty(shape, dtype=out_dtype, device=dev) if k_out is None else k_out
    v_out = torch.empty(shape, dtype=out_dtype, device=dev) if v_out is None else v_out
    for name, t in (("k_out", k_out), ("v_out", v_out)):
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} must have shape {shape}")
    view = cache.view()
    _check("iq_dequantize", lib().iq_dequantize(ctypes.byref(view), first_slot, n_tokens, dt,
                                                _dev(k_out, out_dtype, "k_out"), _dev(v_out, out_dtype, "v_out"),
                                                _stream(stream)))
    return k_out, v_out


def iq_decode_workspace_bytes(n_seqs: int, num_q_heads: int, num_kv_heads: int, max_seq_len: int) -> int:
    return int(lib().iq_decode_workspace_bytes(n_seqs, num_q_heads, num_kv_heads, max_seq_len))


def decode_workspace(n_seqs: int, num_q_heads: int, num_kv_heads: int, max_seq_len: int, device="cuda"):
    """A decode workspace for these sizes (its contents need no initialisation)."""
    need = iq_decode_workspace_bytes(n_seqs, num_q_heads, num_kv_heads, max_seq_len)
    return torch.empty(max(need, 16), dtype=torch.uint8, device=device)


def iq_decode_attention(cache: PackedKVCache, q: torch.Tensor, seq_start: torch.Tensor, seq_len: torch.Tensor,
                        max_seq_len: int, scale: float | None = None, out: torch.Tensor | None = None,
                        workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Decode attention on the packed cache: q float32 [n_seqs][Hq][128] -> out [n_seqs][Hq][128]."""
    n_seqs, hq, _ = q.shape
    scale = 1.0 / math.sqrt(HEAD_DIM) if scale is None else float(scale)
    out = torch.empty_like(q) if out is None else out
    need = iq_decode_workspace_bytes(n_seqs, hq, cache.num_kv_heads, max_seq_len)
    if workspace is None:
        workspace = decode_workspace(n_seqs, hq, cache.num_kv_heads, max_seq_len, q.device)
    view = cache.view()
    _check("iq_decode_attention",
           lib().iq_decode_attention(ctypes.byref(view), _dev(q, torch.float32, "q"), hq,
                                     _dev(seq_start, torch.int32, "seq_start"), _dev(seq_len, torch.int32, "seq_len"),
                                     n_seqs, max_seq_len, scale, _dev(out, torch.float32, "out"),
                                     _dev(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream)))
    return out


def iq_decode_attention_f16(k: torch.Tensor, v: torch.Tensor, q: torch.Tensor, seq_start: torch.Tensor,
                            seq_len: torch.Tensor, max_seq_len: int, token_major: bool = True,
                            scale: float | None = None, out: torch.Tensor | None = None,
                            workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Decode attention over a plain fp16 cache.

    k, v float16, contiguous: [capacity][Hkv][128] when ``token_major`` (the
    layout iq_dequantize writes), else [Hkv][capacity][128].
    """
    if k.shape != v.shape or k.dim() != 3 or k.shape[2] != HEAD_DIM:
        raise ValueError("k and v must be matching [.., .., 128] tensors")
    for name, t in (("k", k), ("v", v)):
        _dev(t, torch.float16, name)
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if token_major:
        cap, hkv = k.shape[0], k.shape[1]
        ts, hs = hkv * HEAD_DIM, HEAD_DIM
    else:
        hkv, cap = k.shape[0], k.shape[1]
        ts, hs = HEAD_DIM, cap * HEAD_DIM
    n_seqs, hq, _ = q.shape
    scale = 1.0 / math.sqrt(HEAD_DIM) if scale is None else float(scale)
    out = torch.empty_like(q) if out is None else out
    if workspace is None:
        workspace = decode_workspace(n_seqs, hq, hkv, max_seq_len, q.device)
    _check("iq_decode_attention_f16",
           lib().iq_decode_attention_f16(k.data_ptr(), v.data_ptr(), ts, hs, hkv, cap, _dev(q, torch.float32, "q"),
                                         hq, _dev(seq_start, torch.int32, "seq_start"),
                                         _dev(seq_len, torch.int32, "seq_len"), n_seqs, max_seq_len, scale,
                                         _dev(out, torch.float32, "out"), _dev(workspace, torch.uint8, "workspace"),
                                         workspace.numel(), _stream(stream)))
    return out


def _f16_strides(k: torch.Tensor, v: torch.Tensor, token_major: bool):
    if k.shape != v.shape or k.dim() != 3 or k.shape[2] != HEAD_DIM:
        raise ValueError("k and v must be matching [.., .., 128] tensors")
    for name, t in (("k", k), ("v", v)):
        _dev(t, torch.float16, name)
    if token_major:
        cap, hkv = k.shape[0], k.shape[1]
        return cap, hkv, hkv * HEAD_DIM, HEAD_DIM
    hkv, cap = k.shape[0], k.shape[1]
    return cap, hkv, HEAD_DIM, cap * HEAD_DIM


def iq_decode_deferred_workspace_bytes(n_seqs: int, num_q_heads: int, num_kv_heads: int, max_prefix_len: int,
                                       max_seq_len: int) -> int:
    return int(lib().iq_decode_deferred_workspace_bytes(n_seqs, num_q_heads, num_kv_heads, max_prefix_len,
                                                        max_seq_len))


def iq_decode_attention_deferred(cache: PackedKVCache, seq_start: torch.Tensor, seq_len: torch.Tensor,
                                 max_seq_len: int, k16: torch.Tensor, v16: torch.Tensor, prefix_start: torch.Tensor,
                                 prefix_len: torch.Tensor, max_prefix_len: int, q: torch.Tensor,
                                 token_major: bool = True, scale: float | None = None,
                                 out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                                 stream=None) -> torch.Tensor:
    """Decode over an fp16 prefix (k16/v16, layout as for iq_decode_attention_f16) followed by the
    packed suffix in ``cache``."""
    cap16, hkv, ts, hs = _f16_strides(k16, v16, token_major)
    if hkv != cache.num_kv_heads:
        raise ValueError("the fp16 prefix and the packed cache must have the same KV heads")
    n_seqs, hq, _ = q.shape
    scale = 1.0 / math.sqrt(HEAD_DIM) if scale is None else float(scale)
    out = torch.empty_like(q) if out is None else out
    if workspace is None:
        need = iq_decode_deferred_workspace_bytes(n_seqs, hq, hkv, max_prefix_len, max_seq_len)
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    view = cache.view()
    _check("iq_decode_attention_deferred",
           lib().iq_decode_attention_deferred(ctypes.byref(view), _dev(seq_start, torch.int32, "seq_start"),
                                              _dev(seq_len, torch.int32, "seq_len"), max_seq_len, k16.data_ptr(),
                                              v16.data_ptr(), ts, hs, cap16,
                                              _dev(prefix_start, torch.int32, "prefix_start"),
                                              _dev(prefix_len, torch.int32, "prefix_len"), max_prefix_len,
                                              _dev(q, torch.float32, "q"), hq, n_seqs, scale,
                                              _dev(out, torch.float32, "out"),
                                              _dev(workspace, torch.uint8, "workspace"), workspace.numel(),
                                              _stream(stream)))
    return out


def iq_append_decode_attention(cache: PackedKVCache, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor,
                               seq_start: torch.Tensor, seq_len: torch.Tensor, max_seq_len: int,
                               scale: float | None = None, out: torch.Tensor | None = None,
                               workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """One decode step: token s of k_new/v_new [n_seqs][Hkv][128] goes to slot seq_start[s] + seq_len[s]
    (seq_len = tokens already cached) and the attention covers seq_len[s] + 1 slots."""
    n_seqs, hq, _ = q.shape
    dt = _in_dtype(k_new)
    if v_new.dtype != k_new.dtype or v_new.shape != k_new.shape or k_new.shape[0] != n_seqs:
        raise ValueError("k_new and v_new must be matching [n_seqs][Hkv][128] tensors")
    scale = 1.0 / math.sqrt(HEAD_DIM) if scale is None else float(scale)
    out = torch.empty_like(q) if out is None else out
    if workspace is None:
        workspace = decode_workspace(n_seqs, hq, cache.num_kv_heads, max_seq_len, q.device)
    view = cache.view()
    _check("iq_append_decode_attention",
           lib().iq_append_decode_attention(ctypes.byref(view), _dev(k_new, k_new.dtype, "k_new"),
                                            _dev(v_new, v_new.dtype, "v_new"), dt, _dev(q, torch.float32, "q"), hq,
                                            _dev(seq_start, torch.int32, "seq_start"),
                                            _dev(seq_len, torch.int32, "seq_len"), n_seqs, max_seq_len, scale,
                                            _dev(out, torch.float32, "out"),
                                            _dev(workspace, torch.uint8, "workspace"), workspace.numel(),
                                            _stream(stream)))
    return out


NOALLOC_SCRATCH_BYTES = 16 << 20   # IQ_NOALLOC_SCRATCH_BYTES


def iq_append_decode_attention_noalloc(cache: PackedKVCache, k_new: torch.Tensor, v_new: torch.Tensor,
                                       q: torch.Tensor, seq_start: torch.Tensor, seq_len: torch.Tensor,
                                       max_seq_len: int, out: torch.Tensor, scale: float | None = None,
                                       stream=None) -> torch.Tensor:
    """iq_append_decode_attention with the library's own scratch array in place of a workspace:
    allocates nothing (``out`` is the caller's). Calls overlapping on one GPU must be serialised."""
    n_seqs, hq, _ = q.shape
    dt = _in_dtype(k_new)
    if v_new.dtype != k_new.dtype or v_new.shape != k_new.shape or k_new.shape[0] != n_seqs:
        raise ValueError("k_new and v_new must be matching [n_seqs][Hkv][128] tensors")
    scale = 1.0 / math.sqrt(HEAD_DIM) if scale is None else float(scale)
    view = cache.view()
    _check("iq_append_decode_attention_noalloc",
           lib().iq_append_decode_attention_noalloc(ctypes.byref(view), _dev(k_new, k_new.dtype, "k_new"),
                                                    _dev(v_new, v_new.dtype, "v_new"), dt,
                                                    _dev(q, torch.float32, "q"), hq,
                                                    _dev(seq_start, torch.int32, "seq_start"),
                                                    _dev(seq_len, torch.int32, "seq_len"), n_seqs, max_seq_len, scale,
                                                    _dev(out, torch.float32, "out"), _stream(stream)))
    return out
