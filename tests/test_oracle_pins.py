"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each check is written as a function so the mutation tests at the bottom can
re-run it against a deliberately broken copy of the oracle and see it fail.
Nothing here needs a GPU.
"""
import math
import os

import numpy as np
import pytest
import scipy.integrate
import scipy.linalg
import scipy.special
import scipy.stats
from scipy.spatial.transform import Rotation

import iqinputs
from oracle import iqref as R

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rot(seed=7, layer=0, heads=1):
    return iqinputs.rotation_params(seed, layer, heads)


# ---------------------------------------------------------------- WHT ----
def check_wht():
    h = R.hadamard(128)
    assert np.array_equal(h, scipy.linalg.hadamard(128))          # library routine
    hn = R.wht(np.eye(128))                                        # rows = Hn e_i
    assert np.allclose(hn @ hn, np.eye(128), atol=1e-13)           # self-inverse
    assert np.allclose(hn, hn.T, atol=0)                           # symmetric
    assert np.allclose(R.wht(np.eye(128)[0]), np.full(128, 1 / math.sqrt(128)), atol=1e-15)
    x = np.random.default_rng(1).standard_normal((5, 128))
    assert np.allclose(R.wht(x), x @ scipy.linalg.hadamard(128).T / math.sqrt(128), atol=1e-12)


def test_wht_is_normalised_sylvester_hadamard():
    check_wht()


# ------------------------------------------------------- quaternions ----
def check_quaternion_product():
    one, i, j, k = np.eye(4)
    assert np.allclose(R.quat_mul(i, j), k) and np.allclose(R.quat_mul(j, k), i)
    assert np.allclose(R.quat_mul(k, i), j) and np.allclose(R.quat_mul(i, i), -one)
    assert np.allclose(R.quat_mul(j, i), -k)
    g = np.random.default_rng(2)
    p, q = g.standard_normal((2, 50, 4))
    assert np.allclose(np.linalg.norm(R.quat_mul(p, q), axis=-1),
                       np.linalg.norm(p, axis=-1) * np.linalg.norm(q, axis=-1), atol=1e-12)
    # q v q* rotates the vector part like scipy's rotation of the same quaternion
    q = q / np.linalg.norm(q, axis=-1, keepdims=True)
    u = g.standard_normal((50, 3))
    v = np.concatenate([np.zeros((50, 1)), u], axis=1)
    r = R.quat_mul(R.quat_mul(q, v), R.quat_conj(q))
    ref = Rotation.from_quat(np.concatenate([q[:, 1:], q[:, :1]], axis=1)).apply(u)  # scalar-last
    assert np.allclose(r[:, 0], 0, atol=1e-12) and np.allclose(r[:, 1:], ref, atol=1e-12)


def test_quaternion_product_textbook():
    check_quaternion_product()


# --------------------------------------------------------------- SO(4) ----
def check_so4():
    rot = _rot(heads=3)
    for h in range(3):
        m = R.so4_block_matrices(rot[h])
        for b in range(32):
            assert np.allclose(m[b].T @ m[b], np.eye(4), atol=1e-14)
            assert abs(np.linalg.det(m[b]) - 1.0) < 1e-13
        y = np.random.default_rng(h).standard_normal((4, 128))
        blocks = y.reshape(4, 32, 4)
        by_matrix = np.einsum("bij,nbj->nbi", m, blocks).reshape(4, 128)
        assert np.allclose(R.so4_apply(y, rot[h]), by_matrix, atol=1e-13)
        assert np.allclose(R.so4_apply(R.so4_apply(y, rot[h]), rot[h], inverse=True), y, atol=1e-13)


def test_so4_blocks_are_rotations():
    check_so4()


def check_rotation_special_cases():
    # identity quaternions: R reduces to the normalised Hadamard transform
    ident = np.tile(np.array([1, 0, 0, 0, 1, 0, 0, 0], np.float32), (32, 1))
    x = np.random.default_rng(3).standard_normal((6, 128))
    assert np.allclose(R.rotate(x, ident), x @ scipy.linalg.hadamard(128).T / math.sqrt(128), atol=1e-12)
    # qL = qR = q: w is fixed and (x, y, z) is rotated by the SO(3) rotation of q
    g = np.random.default_rng(4)
    q = g.standard_normal((32, 4))
    q /= np.linalg.norm(q, axis=1, keepdims=True)
    rot = np.concatenate([q, q], axis=1)
    y = g.standard_normal(128)
    out = R.so4_apply(y, rot).reshape(32, 4)
    blk = y.reshape(32, 4)
    assert np.allclose(out[:, 0], blk[:, 0], atol=1e-12)
    ref = Rotation.from_quat(np.concatenate([q[:, 1:], q[:, :1]], axis=1)).apply(blk[:, 1:])
    assert np.allclose(out[:, 1:], ref, atol=1e-12)


def test_rotation_special_cases():
    check_rotation_special_cases()


def check_rotation_round_trip():
    rot = _rot(heads=1)[0]
    x = np.random.default_rng(5).standard_normal((10, 128)) * 3
    y = R.rotate(x, rot)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-14)
    assert np.allclose(R.inverse_rotate(y, rot), x, atol=1e-13)
    full = R.rotate(np.eye(128), rot)        # rows: R e_i
    assert np.allclose(full @ full.T, np.eye(128), atol=1e-13)
    assert np.linalg.det(full) > 0


def test_rotation_norm_preserving_and_invertible():
    check_rotation_round_trip()


def test_parameter_and_fma_counts():
    # 256 stored parameters per head and 1,408 FMA per vector (news article on
    # RotaryQuant, paragraph on the structured rotation; abstract: 256 per head)
    rot = _rot(heads=4)
    assert rot.shape == (4, 32, 8) and rot[0].size == 256
    assert np.allclose(np.linalg.norm(rot.reshape(4, 32, 2, 4), axis=-1), 1, atol=1e-6)
    wht_ops = int(math.log2(128)) * 128            # 7 butterfly stages of 128 add/sub
    so4_fma = 32 * 16                              # one 4x4 matrix per block
    assert wht_ops + so4_fma == 1408 and 128 * 128 == 16384


# ------------------------------------------------- rotation variants ----
# The essay's variant table ("三种变体") and the RotorQuant page: PlanarQuant,
# one 2-D Givens rotation per dim pair (128 parameters, 256 FMA); the
# single-quaternion IsoQuant, one 4-D quaternion rotation per 4 dims
# (128 parameters, 512 FMA); neither has a WHT.
def _rot_kind(kind, seed=11, heads=1):
    return iqinputs.rotation_params_kind(seed, 0, heads, kind)


def _is_rotation_without_mixing(m, block):
    """m (columns = images of e_i) orthogonal, det +1, and zero outside its diagonal blocks."""
    assert np.allclose(m @ m.T, np.eye(128), atol=1e-13) and np.linalg.det(m) > 0
    mask = np.kron(np.eye(128 // block), np.ones((block, block))).astype(bool)
    assert np.all(m[~mask] == 0)


def check_planar_rotation():
    rot = _rot_kind("planar")[0]
    assert rot.shape == (64, 2) and rot.size == 128
    m = R.rotate(np.eye(128), rot).T
    _is_rotation_without_mixing(m, 2)
    theta = np.arctan2(rot[:, 1].astype(np.float64), rot[:, 0].astype(np.float64))
    for i in range(64):
        ref = Rotation.from_euler("z", theta[i]).as_matrix()[:2, :2]      # library 2-D rotation
        assert np.allclose(m[2 * i:2 * i + 2, 2 * i:2 * i + 2], ref, atol=1e-12)
    x = np.random.default_rng(2).standard_normal((6, 128))
    assert np.allclose(R.inverse_rotate(R.rotate(x, rot), rot), x, atol=1e-13)
    assert 64 * 4 == 256                          # 2 x 2 matrix per pair: the table's 256 FMA


def test_planar_rotation_is_givens_per_pair():
    check_planar_rotation()


def check_iso_rotation():
    rot = _rot_kind("iso")[0]
    assert rot.shape == (32, 4) and rot.size == 128
    m = R.rotate(np.eye(128), rot).T
    _is_rotation_without_mixing(m, 4)
    # worked example of the convention, by the Hamilton rules (ij = k):
    # (cos a + i sin a) (x) j = j cos a + k sin a
    a = 0.3
    q = np.tile([math.cos(a), math.sin(a), 0.0, 0.0], (32, 1))
    v = np.zeros(128)
    v[2::4] = 1.0
    y = R.rotate(v, q).reshape(32, 4)
    assert np.allclose(y, np.tile([0.0, 0.0, math.cos(a), math.sin(a)], (32, 1)), atol=1e-15)
    # isoclinic: every vector of a block turns by the same angle, cos = q_w
    qn = rot.astype(np.float64) / np.linalg.norm(rot.astype(np.float64), axis=1, keepdims=True)
    x = np.random.default_rng(4).standard_normal((7, 128))
    y = R.rotate(x, rot)
    dots = np.einsum("nbi,nbi->nb", x.reshape(7, 32, 4), y.reshape(7, 32, 4))
    assert np.allclose(dots, qn[None, :, 0] * np.sum(x.reshape(7, 32, 4) ** 2, axis=2), atol=1e-12)
    assert np.allclose(R.rotate(x, np.tile([1.0, 0, 0, 0], (32, 1))), x, atol=0)
    assert np.allclose(R.inverse_rotate(y, rot), x, atol=1e-13)
    assert 32 * 16 == 512                         # 4 x 4 matrix per block: the table's 512 FMA


def test_iso_rotation_is_left_isoclinic_per_block():
    check_iso_rotation()


# ------------------------------------------------------------ codebook ----
def _golden_max():
    th, lv, mse = [], [], None
    with open(os.path.join(GOLDEN, "max1960_gaussian_8level.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            kind, val = line.split()
            if kind == "threshold":
                th.append(float(val))
            elif kind == "level":
                lv.append(float(val))
            else:
                mse = float(val)
    return np.array(th), np.array(lv), mse


def check_codebook():
    c, t = R.lloyd_max_unit_gaussian()
    th, lv, mse = _golden_max()
    assert np.allclose(c[4:], lv, atol=6e-4) and np.allclose(c[:4], -lv[::-1], atol=6e-4)
    assert np.allclose(t[4:], th, atol=6e-4) and np.allclose(t[:3], -th[::-1], atol=6e-4) and t[3] == 0
    d = R.quantizer_mse_unit_gaussian(c, t)
    assert abs(d - mse) < 1e-4
    # optimality conditions by independent numerical integration
    edges = [-np.inf] + list(t) + [np.inf]
    for k in range(8):
        mass = scipy.integrate.quad(scipy.stats.norm.pdf, edges[k], edges[k + 1], epsabs=1e-14)[0]
        mom = scipy.integrate.quad(lambda x: x * scipy.stats.norm.pdf(x), edges[k], edges[k + 1], epsabs=1e-14)[0]
        assert abs(mom / mass - c[k]) < 1e-9
    assert np.allclose(t, 0.5 * (c[:-1] + c[1:]), atol=0)
    quad_mse = sum(scipy.integrate.quad(lambda x, ck=c[k]: (x - ck) ** 2 * scipy.stats.norm.pdf(x),
                                        edges[k], edges[k + 1], epsabs=1e-14)[0] for k in range(8))
    assert abs(quad_mse - d) < 1e-9
    # within ~2.7x of the Shannon lower bound 2^(-2b) (essay, Lloyd-Max section)
    assert 4.0 ** -3 <= d <= 2.7 * 4.0 ** -3
    c32, t32, c64 = R.codebook()
    assert np.array_equal(c32, (c / math.sqrt(128)).astype(np.float32))
    assert np.array_equal(t32, (t / math.sqrt(128)).astype(np.float32))


def test_codebook_is_lloyd_max_gaussian():
    check_codebook()


def test_codebook_matches_kmeans_on_samples():
    # Lloyd's algorithm as run by an independent library on N(0,1) samples
    from sklearn.cluster import KMeans
    x = np.random.default_rng(6).standard_normal(400_000).reshape(-1, 1)
    km = KMeans(n_clusters=8, n_init=1, init=np.linspace(-2, 2, 8).reshape(-1, 1), max_iter=500, tol=1e-10).fit(x)
    c, _ = R.lloyd_max_unit_gaussian()
    assert np.allclose(np.sort(km.cluster_centers_.ravel()), c, atol=0.02)


# ------------------------------------------ 4-bit K (asymmetric K/V) ----
# The essay's "K 和 V 的非对称需求": K needs more bits than V. 4-bit K uses the
# 16-level Lloyd-Max quantizer of the same N(0, 1/d); V stays 3-bit.
def check_codebook16():
    c, t = R.lloyd_max_unit_gaussian(16)
    assert c.shape == (16,) and t.shape == (15,)
    assert np.allclose(c, -c[::-1], atol=1e-12) and abs(t[7]) < 1e-12           # symmetric
    assert np.all(np.diff(c) > 0)
    edges = [-np.inf] + list(t) + [np.inf]
    for k in range(16):                                                         # centroid condition
        mass = scipy.integrate.quad(scipy.stats.norm.pdf, edges[k], edges[k + 1], epsabs=1e-14)[0]
        mom = scipy.integrate.quad(lambda x: x * scipy.stats.norm.pdf(x), edges[k], edges[k + 1], epsabs=1e-14)[0]
        assert abs(mom / mass - c[k]) < 1e-9
    assert np.allclose(t, 0.5 * (c[:-1] + c[1:]), atol=0)                      # midpoint condition
    d = R.quantizer_mse_unit_gaussian(c, t)
    quad_mse = sum(scipy.integrate.quad(lambda x, ck=c[k]: (x - ck) ** 2 * scipy.stats.norm.pdf(x),
                                        edges[k], edges[k + 1], epsabs=1e-14)[0] for k in range(16))
    assert abs(quad_mse - d) < 1e-9
    assert 4.0 ** -4 <= d <= 2.7 * 4.0 ** -4                                  # within ~2.7x of 2^(-2b)
    assert d < R.quantizer_mse_unit_gaussian(*R.lloyd_max_unit_gaussian(8)) / 3   # one more bit: ~4x less
    c32, t32, _ = R.codebook(levels=16)
    assert np.array_equal(c32, (c / math.sqrt(128)).astype(np.float32)) and R.bits_of(c32) == 4


def test_codebook16_is_lloyd_max_gaussian():
    check_codebook16()


def test_codebook16_matches_kmeans_on_samples():
    from sklearn.cluster import KMeans
    x = np.random.default_rng(16).standard_normal(500_000)
    x = np.concatenate([x, -x]).reshape(-1, 1)                 # symmetrised sample: less noise in the tails
    km = KMeans(n_clusters=16, n_init=1, init=np.linspace(-2.5, 2.5, 16).reshape(-1, 1), max_iter=1000,
                tol=1e-12).fit(x)
    c, _ = R.lloyd_max_unit_gaussian(16)
    assert np.allclose(np.sort(km.cluster_centers_.ravel()), c, atol=0.03)


def test_pack4_nibbles_and_round_trip():
    codes = np.tile(np.arange(16, dtype=np.uint8), 8)                          # 0, 1, ..., 15, 0, 1, ...
    row = R.pack(codes, 4)
    assert row.shape == (64,)
    assert list(row[:8]) == [0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE]    # low nibble = even dim
    for pos in range(128):
        for v in (1, 7, 8, 15):
            c = np.zeros(128, np.uint8)
            c[pos] = v
            r = R.pack(c, 4)
            assert r[pos // 2] == (v << (4 * (pos % 2))) and r.sum() == r[pos // 2]
            assert np.array_equal(R.unpack(r), c)
    rnd = np.random.default_rng(17).integers(0, 16, (50, 128)).astype(np.uint8)
    assert np.array_equal(R.unpack(R.pack(rnd, 4)), rnd)


def test_quantize16_is_nearest_centroid():
    c32, t32, _ = R.codebook(levels=16)
    g = np.random.default_rng(18)
    y = (g.standard_normal((2000, 128)) * g.uniform(0.1, 30, (2000, 1))).astype(np.float32)
    codes, n = R.quantize(y, t32)
    u = y.astype(np.float64) / n[:, None].astype(np.float64)
    nearest = np.argmin(np.abs(u[..., None] - c32.astype(np.float64)), axis=-1)
    diff = nearest != codes
    if diff.any():
        gap = np.min(np.abs(u[diff][:, None] - t32.astype(np.float64)), axis=-1)
        assert np.all(gap < 1e-6)
    assert diff.mean() < 1e-5 and codes.max() == 15 and codes.min() == 0


def test_distortion16_isotropic_inputs():
    c32, t32, _ = R.codebook(levels=16)
    c, t = R.lloyd_max_unit_gaussian(16)
    rot = _rot(heads=1)[0]
    x = np.random.default_rng(19).standard_normal((20000, 128))
    x /= np.linalg.norm(x, axis=1, keepdims=True)
    rows, n, _ = R.rotate_quantize(x, rot, t32)
    assert rows.shape == (20000, 64)
    d = np.mean(np.sum((x - R.dequantize(rows, n, rot, c32)) ** 2, axis=1))
    assert abs(d - R.quantizer_mse_unit_gaussian(c, t)) < 0.05 * d


def test_attention_with_4bit_k_packed_domain_equals_brute_force(codebook):
    c32, t32, _ = codebook
    c16, t16, _ = R.codebook(levels=16)
    g = np.random.default_rng(20)
    rot = _rot(seed=20, heads=2)
    k = g.standard_normal((304, 2, 128))
    v = g.standard_normal((304, 2, 128))
    kr, kn = R.encode_tokens(k, rot, t16)
    vr, vn = R.encode_tokens_v(v, rot, t32)
    assert kr.shape == (2, 304, 64)
    q = g.standard_normal((3, 4, 128)).astype(np.float32)
    st, ln = np.array([0, 100, 300], np.int32), np.array([100, 200, 4], np.int32)
    a = R.decode_attention(q, kr, kn, vr, vn, rot, st, ln, 0.09, c32, k_centroids32=c16)
    b = R.decode_attention_rotated(q, kr, kn, vr, vn, rot, st, ln, 0.09, c32, k_centroids32=c16)
    assert np.allclose(a, b, atol=1e-12, rtol=0)
    # the 4-bit keys are closer to the exact ones than the 3-bit keys
    exact = np.concatenate([R.attention(q[0, 2 * h:2 * h + 2].astype(np.float64), k[:100, h], R.dequantize_codes(
        R.unpack_tiles(vr[h])[:100], vn[h, :100], rot[h], c32), 0.09) for h in range(2)])
    kr3, kn3 = R.encode_tokens(k, rot, t32)
    a3 = R.decode_attention(q, kr3, kn3, vr, vn, rot, st, ln, 0.09, c32)
    assert np.linalg.norm(a[0] - exact) < np.linalg.norm(a3[0] - exact)


# --------------------------------------------------------- quantizer ----
def check_quantize(codebook):
    c32, t32, _ = codebook
    g = np.random.default_rng(8)
    y = (g.standard_normal((2000, 128)) * g.uniform(0.1, 30, (2000, 1))).astype(np.float32)
    codes, n = R.quantize(y, t32)
    assert np.array_equal(n, np.sqrt(np.sum(y.astype(np.float64) ** 2, axis=1)).astype(np.float32))
    # brute force: nearest centroid of y/n
    u = y.astype(np.float64) / n[:, None].astype(np.float64)
    nearest = np.argmin(np.abs(u[..., None] - c32.astype(np.float64)), axis=-1)
    diff = nearest != codes
    if diff.any():
        # only where u sits within float32 rounding of a cell boundary
        gap = np.min(np.abs(u[diff][:, None] - t32.astype(np.float64)), axis=-1)
        assert np.all(gap < 1e-6)
    assert diff.mean() < 1e-5
    # special cases
    z, nz = R.quantize(np.zeros((1, 128), np.float32), t32)
    assert nz[0] == 0 and not z.any()
    e = np.zeros((1, 128), np.float32)
    e[0, 5] = 3.0
    ce, ne = R.quantize(e, t32)
    assert ne[0] == 3.0 and ce[0, 5] == 7 and np.all(np.delete(ce[0], 5) == 3)   # 0 > thr_3 = 0 is false
    e[0, 5] = -3.0
    ce, _ = R.quantize(e, t32)
    assert ce[0, 5] == 0
    nan = np.full((1, 128), np.nan, np.float32)
    cn, nn = R.quantize(nan, t32)
    assert np.isnan(nn[0]) and not cn.any()


def test_quantize_nonfinite_norms_follow_the_definition(codebook):
    """code = #{k : y > fl32(t_k n)}: a NaN norm makes every threshold NaN (all codes 0); an infinite
    norm makes the middle threshold 0 * inf = NaN and the others -inf (below) or +inf (above), so a
    code counts the thresholds below the middle (3 of 7; 7 of 15 with 16 levels) when y > -inf."""
    _, t32, _ = codebook
    _, t16, _ = R.codebook(levels=16)
    one_nan = np.ones((1, 128), np.float32)
    one_nan[0, 9] = np.nan
    c, n = R.quantize(one_nan, t32)
    assert np.isnan(n[0]) and not c.any()
    big = np.full((1, 128), 1e38, np.float32)                 # fp64 norm 1.1e39: +inf in fp32
    c, n = R.quantize(big, t32)
    assert n[0] == np.inf and np.all(c == 3)
    c, _ = R.quantize(big, t16)
    assert np.all(c == 7)
    mixed = np.ones((1, 128), np.float32)
    mixed[0, 0], mixed[0, 1] = np.inf, -np.inf
    c, n = R.quantize(mixed, t32)
    assert n[0] == np.inf and c[0, 0] == 3 and c[0, 1] == 0 and np.all(c[0, 2:] == 3)


def test_quantize_is_nearest_centroid(codebook):
    check_quantize(codebook)


def test_quantize_ties_go_to_lower_code(codebook):
    c32, t32, _ = codebook
    # y = (b, a, 0, ...) with n = fl32(sqrt(a^2 + b^2)) == 1 exactly, so the
    # threshold fl32(t_k * n) is t_k itself; put a exactly on it.
    tested = 0
    for k in range(7):
        a = np.float32(t32[k])
        b0 = np.float32(np.sqrt(1.0 - float(a) ** 2))
        for b in [b0, np.nextafter(b0, np.float32(2)), np.nextafter(b0, np.float32(0))]:
            y = np.zeros((1, 128), np.float32)
            y[0, 0], y[0, 1] = b, a
            codes, n = R.quantize(y, t32)
            if n[0] != 1.0:
                continue
            assert codes[0, 1] == k              # y_1 == thr_k is not above threshold k
            y[0, 1] = np.nextafter(a, np.float32(1))
            codes2, n2 = R.quantize(y, t32)
            if n2[0] == 1.0:
                assert codes2[0, 1] == k + 1     # one ulp above moves up one code
            tested += 1
            break
    assert tested >= 5


# ----------------------------------------------------------- packing ----
def test_pack_golden():
    with open(os.path.join(GOLDEN, "pack_pattern.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            lhs, rhs = line.split("|")
            codes = np.zeros(128, np.uint8)
            codes[:8] = [int(v) for v in lhs.split()]
            row = R.pack(codes)
            assert row.shape == (48,)
            assert list(row[:3]) == [int(v, 16) for v in rhs.split()]
            assert not row[3:].any()


def test_pack_unpack_exhaustive():
    for pos in range(128):
        for v in range(8):
            codes = np.zeros(128, np.uint8)
            codes[pos] = v
            row = R.pack(codes)
            bits = np.unpackbits(row, bitorder="little")
            assert bits.sum() == bin(v).count("1")
            assert all(bits[3 * pos + b] == ((v >> b) & 1) for b in range(3))
            assert np.array_equal(R.unpack(row), codes)
    codes = np.random.default_rng(9).integers(0, 8, (100, 128)).astype(np.uint8)
    assert np.array_equal(R.unpack(R.pack(codes)), codes)


def test_tile_pack_golden():
    """V tiles: dim j of slot r (0..7) at bits [24j + 3r, 24j + 3r + 3)."""
    codes = np.zeros((8, 128), np.uint8)
    codes[:, 0] = [1, 2, 3, 4, 5, 6, 7, 0]          # dim 0 holds the same 24-bit pattern as pack_pattern
    codes[3, 1] = 5                                  # dim 1, slot 3 -> bit 24 + 9 = 33 -> byte 4 bits 1, 3
    codes[7, 127] = 7                                # last dim, last slot -> bits 3069..3071
    tile = R.pack_tiles(codes)[0]
    assert tile.shape == (384,)
    assert list(tile[:3]) == [0xD1, 0x58, 0x1F]
    assert tile[4] == 0b1010 and tile[3] == 0 and tile[5] == 0
    assert tile[383] == 0xE0
    assert np.array_equal(R.unpack_tiles(tile[None])[0:8], codes)


def test_tile_pack_round_trip_and_rows_agree():
    codes = np.random.default_rng(12).integers(0, 8, (3, 40, 128)).astype(np.uint8)
    tiles = R.pack_tiles(codes)
    assert tiles.shape == (3, 5, 384)
    assert np.array_equal(R.unpack_tiles(tiles), codes)
    # the same codes are reachable slot by slot through v_codes_range
    for a, n in [(0, 40), (3, 9), (17, 1), (39, 1), (8, 16)]:
        assert np.array_equal(R.v_codes_range(tiles[1], a, n), codes[1, a:a + n])
    # exhaustive single-code placement
    for r in range(8):
        for j in (0, 1, 63, 127):
            for v in range(8):
                c = np.zeros((8, 128), np.uint8)
                c[r, j] = v
                bits = np.unpackbits(R.pack_tiles(c), bitorder="little")
                assert bits.sum() == bin(v).count("1")
                assert all(bits[24 * j + 3 * r + b] == ((v >> b) & 1) for b in range(3))


# ------------------------------------------------------- distortion ----
def test_distortion_isotropic_inputs(codebook):
    c32, t32, _ = codebook
    rot = _rot(heads=1)[0]
    x = np.random.default_rng(10).standard_normal((20000, 128))
    x /= np.linalg.norm(x, axis=1, keepdims=True)
    rows, n, _ = R.rotate_quantize(x, rot, t32)
    d = np.mean(np.sum((x - R.dequantize(rows, n, rot, c32)) ** 2, axis=1))
    assert abs(d - 0.03455) < 0.05 * 0.03455


def test_rotation_isotropizes_outlier_channels():
    rot = _rot(heads=1)[0]
    x = iqinputs.kv(1, 0, "k", 20000, 1, "fixed_x8", "f32")[:, 0, :].astype(np.float64)
    u0 = x / np.linalg.norm(x, axis=1, keepdims=True)
    y = R.rotate(x, rot)
    u = y / np.linalg.norm(y, axis=1, keepdims=True)
    assert scipy.stats.kurtosis(u0.ravel()) > 10
    assert abs(scipy.stats.kurtosis(u.ravel())) < 0.5
    assert abs(u.var() * 128 - 1) < 0.01


# -------------------------------------------------------- attention ----
def _small_cache(codebook, n_tok=304, hkv=2, hq=4, seed=11, lens=(300,), kind="wht_so4"):
    c32, t32, _ = codebook
    g = np.random.default_rng(seed)
    rot = iqinputs.rotation_params_kind(seed, 0, hkv, kind)
    k = g.standard_normal((n_tok, hkv, 128))
    v = g.standard_normal((n_tok, hkv, 128))
    kr, kn = R.encode_tokens(k, rot, t32)
    vr, vn = R.encode_tokens_v(v, rot, t32)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int32)
    q = g.standard_normal((len(lens), hq, 128)).astype(np.float32)
    return q, kr, kn, vr, vn, rot, starts, np.array(lens, np.int32)


@pytest.mark.parametrize("kind", iqinputs.ROTATION_KINDS)
def test_attention_packed_domain_equals_brute_force(codebook, kind):
    c32 = codebook[0]
    args = _small_cache(codebook, n_tok=304, lens=(120, 0, 1, 179), kind=kind)
    scale = 1 / math.sqrt(128)
    a = R.decode_attention(*args, scale, c32)
    b = R.decode_attention_rotated(*args, scale, c32)
    assert np.allclose(a, b, atol=1e-12, rtol=0)
    assert np.all(a[1] == 0)                                          # empty sequence


def test_attention_special_cases(codebook):
    c32 = codebook[0]
    q, kr, kn, vr, vn, rot, st, ln = _small_cache(codebook, n_tok=56, hkv=1, hq=2, lens=(50,))
    v_hat = R.dequantize_codes(R.unpack_tiles(vr[0])[:50], vn[0, :50], rot[0], c32)
    # one token: output is that token's value
    one = R.decode_attention(q, kr, kn, vr, vn, rot, st, np.array([1], np.int32), 0.3, c32)
    assert np.allclose(one[0, 0], v_hat[0], atol=1e-13)
    # scale 0: plain mean of the values
    z = R.decode_attention(q, kr, kn, vr, vn, rot, st, ln, 0.0, c32)
    assert np.allclose(z[0, 1], v_hat.mean(0), atol=1e-13)
    # identical keys: mean of the values
    kr2 = np.repeat(kr[:, :1], 56, axis=1)
    kn2 = np.repeat(kn[:, :1], 56, axis=1)
    same = R.decode_attention(q, kr2, kn2, vr, vn, rot, st, ln, 0.2, c32)
    assert np.allclose(same[0, 0], v_hat.mean(0), atol=1e-13)
    # softmax against the library routine
    s = np.random.default_rng(3).standard_normal((3, 40)) * 20
    assert np.allclose(R.softmax(s), scipy.special.softmax(s, axis=-1), atol=1e-15)


def test_deferred_attention_reduces_to_its_parts(codebook):
    """fp16 prefix + packed suffix: with no prefix it is the packed decode, with no suffix
    plain attention over the fp16 rows, and in general brute force over the concatenation."""
    c32 = codebook[0]
    q, kr, kn, vr, vn, rot, st, ln = _small_cache(codebook, n_tok=304, lens=(120, 0, 1, 179))
    g = np.random.default_rng(21)
    k16 = g.standard_normal((90, 2, 128)).astype(np.float16)
    v16 = g.standard_normal((90, 2, 128)).astype(np.float16)
    scale = 1 / math.sqrt(128)
    pst = np.array([0, 10, 50, 70], np.int32)
    none = np.zeros(4, np.int32)
    assert np.allclose(R.decode_attention_deferred(q, k16, v16, pst, none, kr, kn, vr, vn, rot, st, ln, scale, c32),
                       R.decode_attention(q, kr, kn, vr, vn, rot, st, ln, scale, c32), atol=1e-13)
    pln = np.array([10, 40, 20, 20], np.int32)
    only = R.decode_attention_deferred(q, k16, v16, pst, pln, kr, kn, vr, vn, rot, st, none, scale, c32)
    for s in range(4):
        for h in range(2):
            sl = slice(pst[s], pst[s] + pln[s])
            ref = scipy.special.softmax(scale * q[s, 2 * h:2 * h + 2].astype(np.float64)
                                        @ k16[sl, h].astype(np.float64).T, axis=-1) @ v16[sl, h].astype(np.float64)
            assert np.allclose(only[s, 2 * h:2 * h + 2], ref, atol=1e-13)
    both = R.decode_attention_deferred(q, k16, v16, pst, pln, kr, kn, vr, vn, rot, st, ln, scale, c32)
    s, h = 3, 1
    kh = np.concatenate([k16[70:90, h].astype(np.float64), R.dequantize(kr[h, 121:300], kn[h, 121:300], rot[h], c32)])
    vh = np.concatenate([v16[70:90, h].astype(np.float64),
                         R.dequantize_codes(R.unpack_tiles(vr[h])[121:300], vn[h, 121:300], rot[h], c32)])
    w = scipy.special.softmax(scale * q[s, 2:4].astype(np.float64) @ kh.T, axis=-1)
    assert np.allclose(both[s, 2:4], w @ vh, atol=1e-13)


def test_needle_is_recovered(codebook):
    """A key planted as 4x the query wins the attention (moe30b shape, shortened)."""
    c32, t32, _ = codebook
    w = iqinputs.WORKLOADS["moe30b_gqa_t32768"]
    inp = iqinputs.layer_inputs(w, 0, n_tokens=4096)
    kr, kn = R.encode_tokens(inp["k"], inp["rot"], t32)
    p = int(inp["needle_slot"][0])
    for h in range(w.num_kv_heads):
        kh = R.dequantize(kr[h], kn[h], inp["rot"][h], c32)
        qg = inp["q"][0, h * w.group].astype(np.float64)
        wts = R.softmax(kh @ qg / math.sqrt(128))
        assert int(np.argmax(wts)) == p and wts[p] > 0.99


# ------------------------------------------------------- mutations ----
# A plausible slip anywhere in the oracle must fail one of the pins above.
def _expect_fail(fn, *a):
    with pytest.raises(AssertionError):
        fn(*a)


def test_mutation_wrong_hamilton_sign(monkeypatch):
    good = R.quat_mul

    def bad(p, q):
        out = good(p, q)
        pw, px, py, pz = np.moveaxis(p, -1, 0)
        qw, qx, qy, qz = np.moveaxis(q, -1, 0)
        out = out.copy()
        out[..., 1] = pw * qx + px * qw - py * qz + pz * qy        # cross-product sign flipped
        return out
    monkeypatch.setattr(R, "quat_mul", bad)
    _expect_fail(check_quaternion_product)


def test_mutation_inverse_in_wrong_order(monkeypatch):
    monkeypatch.setattr(R, "inverse_rotate", lambda y, rot: R.so4_apply(R.wht(y), rot, inverse=True))
    _expect_fail(check_rotation_round_trip)


def test_mutation_unnormalised_wht(monkeypatch):
    monkeypatch.setattr(R, "wht", lambda x: np.asarray(x, np.float64) @ R.hadamard(x.shape[-1]).T)
    _expect_fail(check_wht)


def test_mutation_codebook_uniform_init_not_iterated(monkeypatch):
    monkeypatch.setattr(R, "lloyd_max_unit_gaussian",
                        lambda levels=8, **k: (np.linspace(-2, 2, 8), 0.5 * (np.linspace(-2, 2, 8)[:-1] + np.linspace(-2, 2, 8)[1:])))
    _expect_fail(check_codebook)


def test_mutation_quantize_ge_instead_of_gt(monkeypatch, codebook):
    good = R.quantize

    def bad(y32, t32):
        codes, n = good(y32, t32)
        thr = (t32[None, :] * n.reshape(-1, 1)).reshape(n.shape + (7,))
        return np.sum(y32[..., :, None] >= thr[..., None, :], axis=-1).astype(np.uint8), n
    monkeypatch.setattr(R, "quantize", bad)
    _expect_fail(check_quantize, codebook)


def test_mutation_givens_transposed(monkeypatch):
    good = R.givens_apply
    monkeypatch.setattr(R, "givens_apply", lambda y, rot, inverse=False: good(y, rot, not inverse))
    _expect_fail(check_planar_rotation)


def test_mutation_quaternion_multiplied_on_the_right(monkeypatch):
    def bad(y, rot, inverse=False):
        q = np.asarray(rot, np.float64)
        q = q / np.linalg.norm(q, axis=-1, keepdims=True)
        v = np.asarray(y, np.float64).reshape(y.shape[:-1] + (32, 4))
        return R.quat_mul(v, R.quat_conj(q) if inverse else q).reshape(y.shape)
    monkeypatch.setattr(R, "iso_apply", bad)
    _expect_fail(check_iso_rotation)


def test_mutation_codebook16_one_iteration(monkeypatch):
    good = R.lloyd_max_unit_gaussian
    monkeypatch.setattr(R, "lloyd_max_unit_gaussian", lambda levels=8, **k: good(levels, max_iter=1))
    _expect_fail(check_codebook16)
