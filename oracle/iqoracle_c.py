"""Loader of the plain C oracle (iqoracle.c) -- TEST INFRASTRUCTURE ONLY.

Only the test suite and the benchmark's CPU-baseline leg use this module. The
C oracle restates the definitions of iqref.py in C (double precision,
OpenMP over tokens and vectors) and is pinned against iqref.py by the tests;
its library is compiled here with gcc on first use when it has not been
built yet.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "iqoracle.c")
LIB = os.path.join(HERE, "libiqoracle.so")
GCC_FLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-shared", "-fPIC", "-Wall"]

_lib = None


def build() -> str:
    tmp = LIB + ".tmp"
    subprocess.run(["gcc", *GCC_FLAGS, "-o", tmp, SOURCE, "-lm"], check=True)
    os.replace(tmp, LIB)
    return LIB


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SOURCE):
            build()
        h = ctypes.CDLL(LIB)
        p = ctypes.c_void_p
        h.iqo_threads.restype, h.iqo_threads.argtypes = ctypes.c_int, []
        h.iqo_encode.restype = ctypes.c_int
        h.iqo_encode.argtypes = [p, ctypes.c_int64, p, p, ctypes.c_int, p, p]
        h.iqo_decode.restype = ctypes.c_int
        h.iqo_decode.argtypes = [p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, p, p, p, p,
                                 p, p, p, p, p, p, ctypes.c_int, ctypes.c_double, p]
        _lib = h
    return _lib


def threads() -> int:
    """OpenMP threads the C oracle's parallel loops use."""
    return int(lib().iqo_threads())


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def encode(x: np.ndarray, rot_head: np.ndarray, thresholds: np.ndarray):
    """x [n][128] (converted to float32) -> packed rows [n][48 or 64] uint8, norms float32 [n]."""
    x = np.ascontiguousarray(x, np.float32)
    rot_head = np.ascontiguousarray(rot_head, np.float32)
    thr = np.ascontiguousarray(thresholds, np.float32)
    levels = len(thr) + 1
    n = x.shape[0]
    rows = np.zeros((n, 16 * (3 if levels == 8 else 4)), np.uint8)
    norms = np.zeros(n, np.float32)
    st = lib().iqo_encode(_ptr(x), n, _ptr(rot_head), _ptr(thr), levels, _ptr(rows), _ptr(norms))
    if st != 0:
        raise ValueError("iqo_encode: unsupported level count")
    return rows, norms


def decode(q, k_rows, k_norms, v_tiles, v_norms, rot, k_cent, v_cent, seq_start, seq_len, scale, heads=None):
    """Decode attention (float64 [n_seqs][Hq][128]); with ``heads``, only those KV heads' query heads are
    computed and the other rows are NaN."""
    q = np.ascontiguousarray(q, np.float32)
    k_rows = np.ascontiguousarray(k_rows, np.uint8)
    v_tiles = np.ascontiguousarray(v_tiles, np.uint8)
    k_norms = np.ascontiguousarray(k_norms, np.float32)
    v_norms = np.ascontiguousarray(v_norms, np.float32)
    rot = np.ascontiguousarray(rot, np.float32)
    k_cent = np.ascontiguousarray(k_cent, np.float32)
    v_cent = np.ascontiguousarray(v_cent, np.float32)
    st = np.ascontiguousarray(seq_start, np.int32)
    ln = np.ascontiguousarray(seq_len, np.int32)
    n_seqs, hq, _ = q.shape
    hkv, cap, row_bytes = k_rows.shape
    k_bits = row_bytes // 16
    hs = None if heads is None else np.ascontiguousarray(heads, np.int32)
    out = np.full((n_seqs, hq, 128), np.nan)
    rc = lib().iqo_decode(_ptr(q), n_seqs, hq, hkv, cap, k_bits, _ptr(k_rows), _ptr(k_norms), _ptr(v_tiles),
                          _ptr(v_norms), _ptr(rot), _ptr(k_cent), _ptr(v_cent), _ptr(st), _ptr(ln),
                          None if hs is None else _ptr(hs), 0 if hs is None else len(hs), float(scale), _ptr(out))
    if rc != 0:
        raise ValueError("iqo_decode: invalid sizes")
    return out
