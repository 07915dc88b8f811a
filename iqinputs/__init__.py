"""Seeded synthetic inputs for the IsoQuant packed 3-bit KV cache.

This module is shared by the tests, the benchmark and the oracle checks. It
holds no arithmetic of the method itself: it only draws random numbers
(keys, values, queries, rotation quaternions, sequence lengths, needle
positions) with numpy's PCG64 keyed by a seed and a tuple of indices.

The shapes mirror the model shapes the RotaryQuant pages talk about (an 8B
dense GQA model, a 30B-A3B MoE, batched ragged decode and a 131072-token
context); no model weights or corpora exist here, so these synthetic tensors
stand in for real activations.

Outlier models:
  * ``fixed_x8``   -- i.i.d. N(0,1) with four fixed channels {5, 42, 77, 120}
                      scaled by 8 (the same channels for every head);
  * ``student_t6`` -- i.i.d. N(0,1) where, per (layer, KV head), six seeded
                      channels are replaced by Student-t(3) samples.
"""
from __future__ import annotations

import dataclasses
import numpy as np

HEAD_DIM = 128
N_BLOCKS = 32               # SO(4) blocks per head vector (128 / 4)
ROT_PARAMS_PER_HEAD = 256   # 32 blocks x 2 unit quaternions x 4 numbers
FIXED_OUTLIER_CHANNELS = (5, 42, 77, 120)
FIXED_OUTLIER_SCALE = 8.0
N_STUDENT_T_CHANNELS = 6
BASE_SEED = 20260814

# tensor ids used as part of the RNG key
_T_K, _T_V, _T_Q, _T_ROT, _T_CHAN, _T_NEEDLE, _T_LEN = range(7)


def rng(seed: int, *keys: int) -> np.random.Generator:
    """A numpy Generator keyed by (seed, *keys)."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed)] + [int(k) for k in keys])))


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int              # position in the workload table (seed offset)
    num_q_heads: int
    num_kv_heads: int
    n_layers: int
    n_seqs: int
    seq_len: int            # context length (max length for ragged batches)
    dtype: str              # "f32" or "f16" K/V input
    outliers: str           # "fixed_x8" or "student_t6"
    ragged: tuple | None = None   # (lo, hi) inclusive uniform length range
    needle: bool = False

    @property
    def seed(self) -> int:
        return BASE_SEED + self.index

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


WORKLOADS = {
    w.name: w
    for w in [
        Workload("single_head_t512", 0, 1, 1, 1, 1, 512, "f32", "fixed_x8"),
        Workload("dense8b_gqa_t8192", 1, 32, 8, 32, 1, 8192, "f16", "student_t6"),
        Workload("moe30b_gqa_t32768", 2, 32, 4, 48, 1, 32768, "f16", "fixed_x8", needle=True),
        Workload("ragged32_gqa", 3, 32, 8, 32, 32, 32768, "f16", "student_t6", ragged=(1024, 32768)),
        Workload("long_t131072", 4, 32, 8, 32, 1, 131072, "f16", "student_t6"),
    ]
}


def rotation_params(seed: int, layer: int, num_kv_heads: int) -> np.ndarray:
    """Random rotation parameters, float32 [num_kv_heads][32][8].

    Each 4-dim block gets two independent Haar-random unit quaternions
    (qL, qR), stored (w, x, y, z) each: four N(0,1) draws normalised in
    float64, then stored as float32.
    """
    g = rng(seed, _T_ROT, layer)
    q = g.standard_normal((num_kv_heads, N_BLOCKS, 2, 4))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    return q.reshape(num_kv_heads, N_BLOCKS, 8).astype(np.float32)


ROTATION_KINDS = ("wht_so4", "iso", "planar")


def rotation_params_kind(seed: int, layer: int, num_kv_heads: int, kind: str) -> np.ndarray:
    """Random parameters of one rotation kind, float32:
    ``wht_so4`` [Hkv][32][8] (as ``rotation_params``); ``iso`` [Hkv][32][4], one
    Haar-random unit quaternion per 4-dim block; ``planar`` [Hkv][64][2], one
    uniformly random unit vector (cos, sin) per dim pair (two N(0,1) draws
    normalised in float64)."""
    if kind == "wht_so4":
        return rotation_params(seed, layer, num_kv_heads)
    g = rng(seed, _T_ROT, layer, 1 + ROTATION_KINDS.index(kind))
    shape = {"iso": (num_kv_heads, N_BLOCKS, 4), "planar": (num_kv_heads, HEAD_DIM // 2, 2)}[kind]
    x = g.standard_normal(shape)
    x /= np.linalg.norm(x, axis=-1, keepdims=True)
    return x.astype(np.float32)


def _as_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return x.astype(np.float32)
    if dtype == "f16":
        return x.astype(np.float16)   # round-to-nearest-even
    raise ValueError(dtype)


def kv(seed: int, layer: int, which: str, n_tokens: int, num_kv_heads: int,
       outliers: str, dtype: str) -> np.ndarray:
    """Synthetic K or V for one layer: [n_tokens][num_kv_heads][128]."""
    tid = {"k": _T_K, "v": _T_V}[which]
    g = rng(seed, tid, layer)
    x = g.standard_normal((n_tokens, num_kv_heads, HEAD_DIM))
    if outliers == "fixed_x8":
        x[:, :, list(FIXED_OUTLIER_CHANNELS)] *= FIXED_OUTLIER_SCALE
    elif outliers == "student_t6":
        gc = rng(seed, _T_CHAN, layer, tid)
        for h in range(num_kv_heads):
            ch = gc.choice(HEAD_DIM, N_STUDENT_T_CHANNELS, replace=False)
            x[:, h, ch] = gc.standard_t(3, size=(n_tokens, N_STUDENT_T_CHANNELS))
    else:
        raise ValueError(outliers)
    return _as_dtype(x, dtype)


def kv_seq(seed: int, layer: int, which: str, seq: int, n_tokens: int, num_kv_heads: int,
           outliers: str, dtype: str) -> np.ndarray:
    """Synthetic K or V of one sequence of a ragged batch, [n_tokens][num_kv_heads][128], keyed by
    (seed, tensor, layer, seq): any sequence can be drawn alone. Same value model as ``kv`` (the
    Student-t channels of a KV head are the layer's, shared by all sequences)."""
    tid = {"k": _T_K, "v": _T_V}[which]
    g = rng(seed, tid, layer, 1 + seq)
    x = g.standard_normal((n_tokens, num_kv_heads, HEAD_DIM))
    if outliers == "fixed_x8":
        x[:, :, list(FIXED_OUTLIER_CHANNELS)] *= FIXED_OUTLIER_SCALE
    elif outliers == "student_t6":
        gc = rng(seed, _T_CHAN, layer, tid)
        for h in range(num_kv_heads):
            ch = gc.choice(HEAD_DIM, N_STUDENT_T_CHANNELS, replace=False)
            x[:, h, ch] = g.standard_t(3, size=(n_tokens, N_STUDENT_T_CHANNELS))
    else:
        raise ValueError(outliers)
    return _as_dtype(x, dtype)


def queries(seed: int, layer: int, n_seqs: int, num_q_heads: int) -> np.ndarray:
    """Decode queries, float32 [n_seqs][num_q_heads][128], i.i.d. N(0,1)."""
    return rng(seed, _T_Q, layer).standard_normal((n_seqs, num_q_heads, HEAD_DIM)).astype(np.float32)


def seq_lengths(w: Workload) -> np.ndarray:
    """Per-sequence context lengths (int32)."""
    if w.ragged is None:
        return np.full(w.n_seqs, w.seq_len, dtype=np.int32)
    lo, hi = w.ragged
    return rng(w.seed, _T_LEN).integers(lo, hi + 1, size=w.n_seqs).astype(np.int32)


def needle_position(seed: int, layer: int, seq_len: int) -> int:
    """Seeded slot (within one sequence) that receives the planted needle key."""
    return int(rng(seed, _T_NEEDLE, layer).integers(0, seq_len))


def plant_needle(k: np.ndarray, q: np.ndarray, pos: int, group: int, scale: float = 4.0) -> None:
    """In place: K[pos, h] = scale * q[h*group] for every KV head h.

    ``k`` is [n_tokens][Hkv][128] for one sequence, ``q`` is [Hq][128].
    """
    for h in range(k.shape[1]):
        k[pos, h] = (scale * q[h * group].astype(np.float64)).astype(k.dtype)


def layer_inputs(w: Workload, layer: int, n_tokens: int | None = None):
    """All inputs of one layer of workload ``w``.

    Returns dict with k, v ([total_tokens][Hkv][128], ragged sequences laid
    out back to back), q ([n_seqs][Hq][128]), rot, seq_start, seq_len and,
    for the needle workload, the needle slot of each sequence.
    """
    lens = seq_lengths(w) if n_tokens is None else np.full(w.n_seqs, n_tokens, np.int32)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int32)
    total = int(lens.sum())
    k = kv(w.seed, layer, "k", total, w.num_kv_heads, w.outliers, w.dtype)
    v = kv(w.seed, layer, "v", total, w.num_kv_heads, w.outliers, w.dtype)
    q = queries(w.seed, layer, w.n_seqs, w.num_q_heads)
    out = dict(k=k, v=v, q=q, rot=rotation_params(w.seed, layer, w.num_kv_heads),
               seq_start=starts, seq_len=lens.astype(np.int32))
    if w.needle:
        pos = []
        for s in range(w.n_seqs):
            p = needle_position(w.seed, layer * 1000003 + s, int(lens[s]))
            seg = k[starts[s]:starts[s] + lens[s]]
            plant_needle(seg, q[s], p, w.group)
            pos.append(int(starts[s]) + p)
        out["needle_slot"] = np.array(pos, dtype=np.int64)
    return out
