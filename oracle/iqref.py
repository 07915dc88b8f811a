"""CPU oracle for the IsoQuant packed 3-bit KV cache (TEST INFRASTRUCTURE ONLY).

Only the test suite, the smoke entry point and the benchmark's CPU-baseline
leg may import this module. The product path (the HIP library and its Python
binding) never touches it, and it shares no code, tables or constants with the
HIP sources: the codebook, the Hadamard matrix and the quaternion algebra are
all written out here independently.

Everything is plain numpy in float64, except where the method itself fixes a
narrower type: the rotated coordinates that are quantized, the per-vector norm
and the quantization thresholds are float32, and the quantization decision is
taken in float32 (the same precision the GPU decides in).

Sources (titles of the pages; section names in brackets):
  [RQ-abs]  arXiv 2608.08081 listing, "RotaryQuant" English abstract.
  [RQ-news] rebasdaily.com news article on RotaryQuant, section on attention
            over packed data ("妙处不只是压缩，而是不再展开").
  [TQ-essay] zhichai.net essay "压缩与速度的博弈——TurboQuant 和 RotorQuant 的真相",
            sections "Beta 分布的魔力", "Lloyd-Max 最优量化", "真正的瓶颈",
            "为什么压缩 KV 缓存这么难？" (the attention formula).
  [RQ-blurb] sd114.wiki RotorQuant page, sections "V 缓存的逆旋转修复" and
            "绕过蝴蝶网络" (the Givens / quaternion variants).
  [TQ-essay] also section "三种变体" (the variant table).

Readings taken where the pages are silent or garbled (each is also listed in
the design notes of the repository):
  * R = B . Hn: the normalised Walsh-Hadamard transform in Sylvester (natural)
    order without random signs comes first, then the block-diagonal SO(4)
    rotation B ([RQ-abs]: "Walsh-Hadamard transform followed by block-diagonal
    SO(4) rotations").
  * Block b acts on dims 4b..4b+3 read as a quaternion (w, x, y, z):
    v -> qL (x) v (x) conj(qR), Hamilton product. Parameters per head:
    32 blocks x (qL, qR) x 4 = 256 ([RQ-abs], [RQ-news]). Stored float32
    quaternions are renormalised in float64 before use.
  * Codebook: 8-level Lloyd-Max quantizer for N(0, 1/d), d = 128
    ([TQ-essay] "Lloyd-Max 最优量化"; the Beta(1/2,(d-1)/2) statement in
    "Beta 分布的魔力" holds for the squared coordinate, the Gaussian limit is
    what the codebook is built for). Centroids and midpoint thresholds are
    computed in float64 and rounded to float32.
  * The norm is that of the float32 rotated vector y (equal to ||x|| up to
    rounding): n = fl32(sqrt(sum_j y_j^2)) with the sum in float64.
  * Quantization: thr_k = fl32(t_k * n) (float32 multiply, round to nearest
    even) and code_j = #{k : y_j > thr_k}; ties go to the lower code, a zero
    vector gives all-zero codes, NaN gives code 0.
  * Code numbering: code c is the c-th centroid in ascending order.
  * Packing of K: code j occupies bits [3j, 3j+3) of a 384-bit little-endian
    bitstream (48 bytes per token row); bytes 3i..3i+2 hold codes 8i..8i+7.
    With 4-bit K (the asymmetric split of [TQ-essay] "K 和 V 的非对称需求":
    K gets more bits than V), K uses the 16-level Lloyd-Max codebook of the
    same N(0, 1/d) and code j occupies bits [4j, 4j+4) (64-byte rows); V
    stays 3-bit.
  * Packing of V: tokens are grouped in tiles of 8 consecutive cache slots
    (slot s in tile s // 8, position s % 8); a tile is a 3072-bit
    little-endian bitstream (384 bytes, the same 48 bytes per token) in which
    the code of dimension j of the token at position r sits at bits
    [24j + 3r, 24j + 3r + 3). The pages only say the codes are packed; this
    dim-major order keeps the eight codes of one dimension together.
  * Rotation variants ([TQ-essay] "三种变体"): the single-quaternion IsoQuant
    is read as the left-isoclinic map v -> q (x) v per 4-dim block (128
    parameters, 512 FMA, no WHT); PlanarQuant as one Givens rotation per dim
    pair (2i, 2i+1) stored as (cos, sin) (128 parameters, 256 FMA, no WHT).
  * Dequantization: x_hat = n . R^-1 c[code], R^-1 = Hn . B^T ([RQ-blurb]:
    the inverse rotation must be applied when reconstructing V).
  * Attention: softmax(scale . q K_hat^T) V_hat per query head
    ([TQ-essay] attention formula), query head g reads KV head g // G.
"""
from __future__ import annotations

import math
import numpy as np

D = 128
N_BLOCKS = D // 4
N_LEVELS = 8
BITS = 3
ROW_BYTES = D * BITS // 8   # 48


# --------------------------------------------------------------------------
# Codebook: Lloyd-Max for a Gaussian ([TQ-essay] "Lloyd-Max 最优量化")
# --------------------------------------------------------------------------
def _pdf(x: float) -> float:
    if math.isinf(x):
        return 0.0
    return math.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)


def _cdf(x: float) -> float:
    return 0.5 * math.erfc(-x / math.sqrt(2.0))


def _cell_mass(a: float, b: float) -> float:
    """P(a < X <= b) for X ~ N(0,1), computed on the side of the smaller tail."""
    if a >= 0:
        return 0.5 * math.erfc(a / math.sqrt(2.0)) - 0.5 * math.erfc(b / math.sqrt(2.0))
    return _cdf(b) - _cdf(a)


def lloyd_max_unit_gaussian(levels: int = N_LEVELS, tol: float = 1e-16, max_iter: int = 100000):
    """Lloyd-Max quantizer of N(0,1): returns (centroids, thresholds) in float64.

    The iteration the essay describes: start from some centroids, assign each
    value to its nearest centroid (the cell boundaries are the midpoints),
    replace every centroid by the mean of its cell, repeat until nothing moves.
    For a Gaussian the cell mean has the closed form
    (pdf(a) - pdf(b)) / (cdf(b) - cdf(a)).
    """
    c = np.linspace(-2.0, 2.0, levels)
    for _ in range(max_iter):
        t = 0.5 * (c[:-1] + c[1:])
        edges = [-math.inf] + list(t) + [math.inf]
        new = np.array([(_pdf(a) - _pdf(b)) / _cell_mass(a, b) for a, b in zip(edges[:-1], edges[1:])])
        done = np.max(np.abs(new - c)) <= tol
        c = new
        if done:
            break
    t = 0.5 * (c[:-1] + c[1:])
    return c, t


def quantizer_mse_unit_gaussian(c: np.ndarray, t: np.ndarray) -> float:
    """E[(X - Q(X))^2] for X ~ N(0,1) and the scalar quantizer (c, t), closed form."""
    edges = [-math.inf] + list(t) + [math.inf]
    total = 0.0
    for k, (a, b) in enumerate(zip(edges[:-1], edges[1:])):
        p = _cell_mass(a, b)
        m1 = _pdf(a) - _pdf(b)                                    # int x pdf
        apdf = 0.0 if math.isinf(a) else a * _pdf(a)
        bpdf = 0.0 if math.isinf(b) else b * _pdf(b)
        m2 = p + apdf - bpdf                                      # int x^2 pdf
        total += m2 - 2.0 * c[k] * m1 + c[k] ** 2 * p
    return total


def codebook(d: int = D, levels: int = N_LEVELS):
    """Codebook for N(0, 1/d): (centroids float32[L], thresholds float32[L-1], centroids float64[L]),
    L = 8 (3-bit, the default) or 16 (4-bit K of the asymmetric K/V split, [TQ-essay] "K 和 V 的非对称需求")."""
    c, t = lloyd_max_unit_gaussian(levels)
    s = 1.0 / math.sqrt(d)
    return (c * s).astype(np.float32), (t * s).astype(np.float32), c * s


def bits_of(table: np.ndarray) -> int:
    """Code width of a codebook's centroids (L entries) or thresholds (L - 1 entries)."""
    n = len(table)
    levels = n if n in (8, 16) else n + 1
    return {8: 3, 16: 4}[levels]


# --------------------------------------------------------------------------
# Rotation: normalised WHT, then block-diagonal SO(4) ([RQ-abs], [RQ-news])
# --------------------------------------------------------------------------
def hadamard(n: int = D) -> np.ndarray:
    """Sylvester Hadamard matrix: H_1 = [1], H_2m = [[H, H], [H, -H]]."""
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def wht(x: np.ndarray) -> np.ndarray:
    """Normalised Walsh-Hadamard transform Hn x = H x / sqrt(d) over the last axis."""
    d = x.shape[-1]
    return np.asarray(x, np.float64) @ (hadamard(d).T / math.sqrt(d))


def quat_mul(p: np.ndarray, q: np.ndarray) -> np.ndarray:
    """Hamilton product p (x) q of quaternions stored (w, x, y, z) on the last axis."""
    pw, px, py, pz = np.moveaxis(p, -1, 0)
    qw, qx, qy, qz = np.moveaxis(q, -1, 0)
    return np.stack([
        pw * qw - px * qx - py * qy - pz * qz,
        pw * qx + px * qw + py * qz - pz * qy,
        pw * qy - px * qz + py * qw + pz * qx,
        pw * qz + px * qy - py * qx + pz * qw,
    ], axis=-1)


def quat_conj(q: np.ndarray) -> np.ndarray:
    return q * np.array([1.0, -1.0, -1.0, -1.0])


def unit_quaternions(rot: np.ndarray):
    """(qL, qR) float64 [..., 32, 4] from stored params [..., 32, 8], renormalised."""
    r = np.asarray(rot, np.float64)
    ql, qr = r[..., 0:4], r[..., 4:8]
    ql = ql / np.linalg.norm(ql, axis=-1, keepdims=True)
    qr = qr / np.linalg.norm(qr, axis=-1, keepdims=True)
    return ql, qr


def so4_apply(y: np.ndarray, rot: np.ndarray, inverse: bool = False) -> np.ndarray:
    """Apply B (or B^T) to [..., 128] vectors; rot is [32, 8] for one head.

    Forward per block: v -> qL (x) v (x) conj(qR). Inverse per block:
    v -> conj(qL) (x) v (x) qR.
    """
    ql, qr = unit_quaternions(rot)
    v = np.asarray(y, np.float64).reshape(y.shape[:-1] + (N_BLOCKS, 4))
    if inverse:
        out = quat_mul(quat_mul(quat_conj(ql), v), qr)
    else:
        out = quat_mul(quat_mul(ql, v), quat_conj(qr))
    return out.reshape(y.shape)


def so4_block_matrices(rot: np.ndarray) -> np.ndarray:
    """The 32 4x4 matrices M_b of the forward block map (columns = images of e_i)."""
    eye = np.eye(4)
    ql, qr = unit_quaternions(rot)
    m = np.empty((N_BLOCKS, 4, 4))
    for i in range(4):
        m[:, :, i] = quat_mul(quat_mul(ql, eye[i]), quat_conj(qr))
    return m


# Rotation variants ([TQ-essay] "三种变体"; [RQ-blurb] section on bypassing the
# butterfly network: independent 2-D Givens rotations per pair or 4-D
# quaternion rotations per group, no WHT, 128 parameters each). The kind of a
# head's parameters follows from their shape:
#   [32, 8]  WHT then SO(4) with (qL, qR) per block  (the IsoQuant of [RQ-abs])
#   [32, 4]  one unit quaternion q per block, v -> q (x) v, no WHT  (a left-
#            isoclinic SO(4) rotation; 32 x 16 = 512 FMA)
#   [64, 2]  one Givens rotation per dim pair (2i, 2i+1), stored (cos, sin),
#            no WHT  (64 x 4 = 256 FMA)
ROT_WHT_SO4, ROT_ISO, ROT_PLANAR = 0, 1, 2


def rotation_kind(rot: np.ndarray) -> int:
    shape = tuple(np.shape(rot)[-2:])
    kinds = {(N_BLOCKS, 8): ROT_WHT_SO4, (N_BLOCKS, 4): ROT_ISO, (D // 2, 2): ROT_PLANAR}
    if shape not in kinds:
        raise ValueError(f"rotation parameters of shape {shape} match no rotation kind")
    return kinds[shape]


def iso_apply(y: np.ndarray, rot: np.ndarray, inverse: bool = False) -> np.ndarray:
    """Per block v -> q (x) v (inverse: conj(q) (x) v); rot [32, 4] renormalised."""
    q = np.asarray(rot, np.float64)
    q = q / np.linalg.norm(q, axis=-1, keepdims=True)
    v = np.asarray(y, np.float64).reshape(y.shape[:-1] + (N_BLOCKS, 4))
    out = quat_mul(quat_conj(q) if inverse else q, v)
    return out.reshape(y.shape)


def givens_apply(y: np.ndarray, rot: np.ndarray, inverse: bool = False) -> np.ndarray:
    """Per pair (x, y) -> (c x - s y, s x + c y) (inverse: the transpose); rot [64, 2] = (c, s) renormalised."""
    cs = np.asarray(rot, np.float64)
    cs = cs / np.linalg.norm(cs, axis=-1, keepdims=True)
    c, s = cs[:, 0], (-cs[:, 1] if inverse else cs[:, 1])
    v = np.asarray(y, np.float64).reshape(y.shape[:-1] + (D // 2, 2))
    out = np.stack([c * v[..., 0] - s * v[..., 1], s * v[..., 0] + c * v[..., 1]], axis=-1)
    return out.reshape(y.shape)


def rotate(x: np.ndarray, rot: np.ndarray) -> np.ndarray:
    """y = R x in float64 for [..., 128] vectors of one head: B . Hn . x for the
    WHT + SO(4) kind, the block map alone for the two others."""
    kind = rotation_kind(rot)
    if kind == ROT_ISO:
        return iso_apply(x, rot)
    if kind == ROT_PLANAR:
        return givens_apply(x, rot)
    return so4_apply(wht(x), rot)


def inverse_rotate(y: np.ndarray, rot: np.ndarray) -> np.ndarray:
    """x = R^-1 y in float64 (Hn . B^T . y for the WHT + SO(4) kind: Hn is symmetric
    and its own inverse)."""
    kind = rotation_kind(rot)
    if kind == ROT_ISO:
        return iso_apply(y, rot, inverse=True)
    if kind == ROT_PLANAR:
        return givens_apply(y, rot, inverse=True)
    return wht(so4_apply(y, rot, inverse=True))


# --------------------------------------------------------------------------
# Norm, quantization, packing ([TQ-essay] "Beta 分布的魔力", "Lloyd-Max 最优量化",
# "真正的瓶颈"; [RQ-abs] "3-bit scalar quantization", "packed 3-bit tensors")
# --------------------------------------------------------------------------
def quantize(y32: np.ndarray, thresholds32: np.ndarray):
    """Codes (uint8 [..., 128]) and norms (float32 [...]) of float32 rotated vectors."""
    y32 = np.asarray(y32, np.float32)
    y64 = y32.astype(np.float64)
    norm = np.sqrt(np.sum(y64 * y64, axis=-1)).astype(np.float32)
    thr = thresholds32.astype(np.float32)[None, :] * norm.reshape(-1, 1)      # float32 products
    thr = thr.reshape(norm.shape + (len(thresholds32),))
    codes = np.sum(y32[..., :, None] > thr[..., None, :], axis=-1).astype(np.uint8)
    return codes, norm


def pack(codes: np.ndarray, bits: int = BITS) -> np.ndarray:
    """[..., 128] codes -> [..., 16 bits] bytes; code j at bits [bits j, bits (j+1)), little-endian
    (48-byte rows for 3-bit codes, 64-byte rows for 4-bit)."""
    codes = np.asarray(codes, np.uint8)
    b = np.stack([(codes >> i) & 1 for i in range(bits)], axis=-1)          # [..., 128, bits]
    b = b.reshape(codes.shape[:-1] + (D * bits,))
    return np.packbits(b, axis=-1, bitorder="little")


def unpack(rows: np.ndarray) -> np.ndarray:
    """[..., 48] or [..., 64] bytes -> [..., 128] codes (inverse of ``pack``; the width follows from
    the row length)."""
    rows = np.asarray(rows, np.uint8)
    bits = rows.shape[-1] * 8 // D
    b = np.unpackbits(rows, axis=-1, bitorder="little")
    b = b.reshape(rows.shape[:-1] + (D, bits)).astype(np.uint8)
    out = np.zeros(b.shape[:-1], np.uint8)
    for i in range(bits):
        out |= b[..., i] << i
    return out


TILE = 8                    # tokens per V tile
TILE_BYTES = TILE * ROW_BYTES   # 384


def pack_tiles(codes: np.ndarray) -> np.ndarray:
    """[..., 8*n, 128] codes of consecutive slots (first slot a multiple of 8) -> [..., n, 384] V tiles."""
    codes = np.asarray(codes, np.uint8)
    n_tok = codes.shape[-2]
    assert n_tok % TILE == 0
    c = codes.reshape(codes.shape[:-2] + (n_tok // TILE, TILE, D))             # [..., tile, r, j]
    bits = np.stack([(c >> b) & 1 for b in range(BITS)], axis=-1)            # [..., tile, r, j, b]
    bits = np.swapaxes(bits, -3, -2)                                          # [..., tile, j, r, b]
    bits = bits.reshape(bits.shape[:-3] + (D * TILE * BITS,))                 # bit 24j + 3r + b
    return np.packbits(bits, axis=-1, bitorder="little")


def unpack_tiles(tiles: np.ndarray) -> np.ndarray:
    """[..., n, 384] V tiles -> [..., 8*n, 128] codes (inverse of ``pack_tiles``)."""
    bits = np.unpackbits(np.asarray(tiles, np.uint8), axis=-1, bitorder="little")
    bits = bits.reshape(tiles.shape[:-1] + (D, TILE, BITS)).astype(np.uint8)  # [..., tile, j, r, b]
    c = bits[..., 0] | (bits[..., 1] << 1) | (bits[..., 2] << 2)              # [..., tile, j, r]
    c = np.swapaxes(c, -1, -2)                                                # [..., tile, r, j]
    return c.reshape(c.shape[:-3] + (c.shape[-3] * TILE, D))


def rotate_quantize(x: np.ndarray, rot: np.ndarray, thresholds32: np.ndarray):
    """Full encode of [..., 128] vectors of one head: (packed rows, norms, float32 y)."""
    y32 = rotate(np.asarray(x, np.float64), rot).astype(np.float32)
    codes, norm = quantize(y32, thresholds32)
    return pack(codes, bits_of(thresholds32)), norm, y32


def dequantize_codes(codes: np.ndarray, norms: np.ndarray, rot: np.ndarray, centroids32: np.ndarray) -> np.ndarray:
    """x_hat = n . Hn . B^T . c[code] in float64 ([RQ-blurb]: V needs the inverse rotation)."""
    c = centroids32.astype(np.float64)[np.asarray(codes)]
    return np.asarray(norms, np.float64)[..., None] * inverse_rotate(c, rot)


def dequantize(rows: np.ndarray, norms: np.ndarray, rot: np.ndarray, centroids32: np.ndarray) -> np.ndarray:
    """Dequantize packed K rows [..., 48]."""
    return dequantize_codes(unpack(rows), norms, rot, centroids32)


# --------------------------------------------------------------------------
# Cache-level encode (the append call) and decode attention
# --------------------------------------------------------------------------
def encode_codes(x: np.ndarray, rot: np.ndarray, thresholds32: np.ndarray):
    """Encode [n_tok][Hkv][128] -> codes [Hkv][n_tok][128] (uint8), norms [Hkv][n_tok]."""
    n_tok, hkv, _ = x.shape
    codes = np.empty((hkv, n_tok, D), np.uint8)
    norms = np.empty((hkv, n_tok), np.float32)
    for h in range(hkv):
        y32 = rotate(np.asarray(x[:, h, :], np.float64), rot[h]).astype(np.float32)
        codes[h], norms[h] = quantize(y32, thresholds32)
    return codes, norms


def encode_tokens(x: np.ndarray, rot: np.ndarray, thresholds32: np.ndarray):
    """Encode [n_tok][Hkv][128] -> K rows [Hkv][n_tok][48] (3-bit thresholds) or [..][64] (4-bit),
    norms [Hkv][n_tok]."""
    codes, norms = encode_codes(x, rot, thresholds32)
    return pack(codes, bits_of(thresholds32)), norms


def encode_tokens_v(x: np.ndarray, rot: np.ndarray, thresholds32: np.ndarray):
    """Encode [n_tok][Hkv][128] (n_tok a multiple of 8, slots 0..n_tok-1) -> V tiles
    [Hkv][n_tok/8][384], norms [Hkv][n_tok]."""
    codes, norms = encode_codes(x, rot, thresholds32)
    return pack_tiles(codes), norms


def softmax(s: np.ndarray) -> np.ndarray:
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def attention(q: np.ndarray, k_hat: np.ndarray, v_hat: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale . q K^T) V for q [m][128], K/V [T][128]; T = 0 gives zeros."""
    if k_hat.shape[0] == 0:
        return np.zeros((q.shape[0], v_hat.shape[-1]))
    p = softmax(scale * (np.asarray(q, np.float64) @ k_hat.T))
    return p @ v_hat


def v_codes_range(v_tiles: np.ndarray, a: int, n: int) -> np.ndarray:
    """Codes [n][128] of slots a..a+n-1 of one head's V tiles [cap/8][384]."""
    t0, t1 = a // TILE, (a + n + TILE - 1) // TILE
    codes = unpack_tiles(v_tiles[t0:t1])
    return codes[a - t0 * TILE:a - t0 * TILE + n]


def decode_attention(q, k_rows, k_norms, v_tiles, v_norms, rot, seq_start, seq_len, scale, centroids32,
                     seqs=None, heads=None, k_centroids32=None):
    """Decode attention straight from the definition, in float64.

    q [n_seqs][Hq][128]; k_rows [Hkv][cap][48]; v_tiles [Hkv][cap/8][384];
    norms [Hkv][cap]; rot [Hkv][32][8]. The packed K and V of each sequence
    are dequantized explicitly and ordinary softmax attention is taken over
    them. ``seqs`` and ``heads`` restrict the computation to a sample; other
    outputs stay NaN. ``k_centroids32``: K's own codebook when K has more bits
    than V (16 levels for 4-bit K rows of 64 bytes).
    """
    kc = centroids32 if k_centroids32 is None else k_centroids32
    n_seqs, hq, _ = q.shape
    hkv = k_rows.shape[0]
    g = hq // hkv
    out = np.full((n_seqs, hq, D), np.nan)
    for s in (range(n_seqs) if seqs is None else seqs):
        a, n = int(seq_start[s]), int(seq_len[s])
        for h in (range(hkv) if heads is None else heads):
            kh = dequantize(k_rows[h, a:a + n], k_norms[h, a:a + n], rot[h], kc)
            vh = dequantize_codes(v_codes_range(v_tiles[h], a, n), v_norms[h, a:a + n], rot[h], centroids32)
            out[s, h * g:(h + 1) * g] = attention(q[s, h * g:(h + 1) * g], kh, vh, scale)
    return out


def decode_attention_deferred(q, k16, v16, prefix_start, prefix_len, k_rows, k_norms, v_tiles, v_norms, rot,
                              seq_start, seq_len, scale, centroids32, k_centroids32=None):
    """Decode attention over a cache whose first tokens stayed fp16 (deferred
    quantization: [RQ-blurb] "延迟量化策略"; [TQ-essay] "延迟量化"), float64.

    Sequence s attends to its fp16 prefix k16/v16 [rows][Hkv][128], rows
    prefix_start[s] .. + prefix_len[s], followed by its packed suffix, cache
    slots seq_start[s] .. + seq_len[s], dequantized explicitly. Plain softmax
    attention over the concatenation.
    """
    kc = centroids32 if k_centroids32 is None else k_centroids32
    n_seqs, hq, _ = q.shape
    hkv = k_rows.shape[0]
    g = hq // hkv
    out = np.zeros((n_seqs, hq, D))
    for s in range(n_seqs):
        pa, pn = int(prefix_start[s]), int(prefix_len[s])
        a, n = int(seq_start[s]), int(seq_len[s])
        for h in range(hkv):
            kh = np.concatenate([np.asarray(k16[pa:pa + pn, h], np.float64),
                                 dequantize(k_rows[h, a:a + n], k_norms[h, a:a + n], rot[h], kc)])
            vh = np.concatenate([np.asarray(v16[pa:pa + pn, h], np.float64),
                                 dequantize_codes(v_codes_range(v_tiles[h], a, n), v_norms[h, a:a + n], rot[h],
                                                  centroids32)])
            out[s, h * g:(h + 1) * g] = attention(q[s, h * g:(h + 1) * g], kh, vh, scale)
    return out


def decode_attention_rotated(q, k_rows, k_norms, v_tiles, v_norms, rot, seq_start, seq_len, scale,
                             centroids32, k_centroids32=None):
    """The packed-domain algorithm, step by step in float64 ([RQ-news], [RQ-abs]).

    Rotate each query once (q' = R q), score every packed key as
    n_t . (q' . c[code_t]), softmax, accumulate n_t . c[vcode_t] with the
    weights, and apply one inverse rotation to the result. By orthogonality
    of R this equals ``decode_attention``.
    """
    n_seqs, hq, _ = q.shape
    hkv = k_rows.shape[0]
    g = hq // hkv
    c = centroids32.astype(np.float64)
    ck = c if k_centroids32 is None else k_centroids32.astype(np.float64)
    out = np.zeros((n_seqs, hq, D))
    for s in range(n_seqs):
        a, n = int(seq_start[s]), int(seq_len[s])
        if n == 0:
            continue
        for h in range(hkv):
            qr = rotate(q[s, h * g:(h + 1) * g].astype(np.float64), rot[h])         # [g][128]
            kc = ck[unpack(k_rows[h, a:a + n])] * k_norms[h, a:a + n, None].astype(np.float64)
            vc = c[v_codes_range(v_tiles[h], a, n)] * v_norms[h, a:a + n, None].astype(np.float64)
            p = softmax(scale * (qr @ kc.T))
            out[s, h * g:(h + 1) * g] = inverse_rotate(p @ vc, rot[h])
    return out
