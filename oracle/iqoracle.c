/*
 * Plain C oracle of the IsoQuant packed KV cache (TEST INFRASTRUCTURE ONLY).
 *
 * Only the test suite and the benchmark's CPU-baseline leg load this library;
 * the product path (the HIP library and its binding) never does, and nothing
 * here is shared with the HIP sources. It restates, in double precision, the
 * same definitions as the numpy oracle beside it (iqref.py), against which
 * the tests pin it:
 *
 *   encode  (arXiv 2608.08081 "RotaryQuant" abstract: normalised
 *            Walsh-Hadamard transform followed by block-diagonal SO(4)
 *            rotations; zhichai.net essay "压缩与速度的博弈——TurboQuant 和
 *            RotorQuant 的真相", sections "Beta 分布的魔力" and
 *            "Lloyd-Max 最优量化"):
 *              y = B . Hn . x, rounded to float;
 *              n = (float) sqrt(sum_j y_j^2), the sum in double;
 *              code_j = #{k : y_j > (float)(t_k * n)}  (float decision);
 *              code j at bits [b j, b j + b) of the row, little-endian.
 *   decode  (rebasdaily.com news article on RotaryQuant, section
 *            "妙处不只是压缩，而是不再展开"; the essay's attention formula
 *            softmax(Q K^T / sqrt(d)) V, section "为什么压缩 KV 缓存这么难？";
 *            sd114.wiki RotorQuant page, section "V 缓存的逆旋转修复"):
 *              K_hat_t = nK_t . Hn . B^T . c[kcode_t], V_hat_t likewise,
 *              o_g = softmax(scale . q_g . K_hat^T) . V_hat for query head g
 *              of KV head g / G.
 *
 * Readings, as in iqref.py: Hn is the Sylvester Hadamard matrix / sqrt(128)
 * without random signs; block b (dims 4b..4b+3, a quaternion w,x,y,z) maps
 * v -> qL (x) v (x) conj(qR) and back by v -> conj(qL) (x) v (x) qR, the
 * stored float quaternions renormalised in double; V is stored in tiles of 8
 * slots, the code of dim j of the slot at tile position r at bits
 * [24 j + 3 r, 24 j + 3 r + 3) of the tile. The WHT is the Sylvester
 * recursion H_2m = [[H, H], [H, -H]] applied as its butterfly stages.
 *
 * Built with gcc -O2 -fopenmp -ffp-contract=off (every product rounded as
 * written); loops over tokens and vectors run in parallel.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define D 128
#define NB 32

/* Threads an OpenMP loop of this library uses. */
int iqo_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Hamilton product r = a (x) b of quaternions (w, x, y, z). */
static void qmul(const double a[4], const double b[4], double r[4]) {
  r[0] = a[0] * b[0] - a[1] * b[1] - a[2] * b[2] - a[3] * b[3];
  r[1] = a[0] * b[1] + a[1] * b[0] + a[2] * b[3] - a[3] * b[2];
  r[2] = a[0] * b[2] - a[1] * b[3] + a[2] * b[0] + a[3] * b[1];
  r[3] = a[0] * b[3] + a[1] * b[2] - a[2] * b[1] + a[3] * b[0];
}

/* The head's unit quaternions (qL, qR) of block b from the stored floats. */
static void unit_pair(const float* rot_head, int b, double ql[4], double qr[4]) {
  const float* p = rot_head + 8 * b;
  double nl = 0.0, nr = 0.0;
  for (int i = 0; i < 4; ++i) {
    ql[i] = p[i];
    qr[i] = p[4 + i];
    nl += ql[i] * ql[i];
    nr += qr[i] * qr[i];
  }
  nl = sqrt(nl);
  nr = sqrt(nr);
  for (int i = 0; i < 4; ++i) {
    ql[i] /= nl;
    qr[i] /= nr;
  }
}

/* In place: x <- H x / sqrt(128), Sylvester order. */
static void wht(double* x) {
  for (int h = 1; h < D; h <<= 1)
    for (int i = 0; i < D; i += 2 * h)
      for (int j = i; j < i + h; ++j) {
        const double a = x[j], b = x[j + h];
        x[j] = a + b;
        x[j + h] = a - b;
      }
  const double s = 1.0 / sqrt((double)D);
  for (int j = 0; j < D; ++j) x[j] *= s;
}

/* In place: x <- B x (forward) or B^T x (inverse), block by block. */
static void blocks(double* x, const float* rot_head, int inverse) {
  for (int b = 0; b < NB; ++b) {
    double ql[4], qr[4], t[4], r[4];
    unit_pair(rot_head, b, ql, qr);
    double* v = x + 4 * b;
    if (!inverse) {
      const double qrc[4] = {qr[0], -qr[1], -qr[2], -qr[3]};
      qmul(ql, v, t);
      qmul(t, qrc, r);
    } else {
      const double qlc[4] = {ql[0], -ql[1], -ql[2], -ql[3]};
      qmul(qlc, v, t);
      qmul(t, qr, r);
    }
    for (int i = 0; i < 4; ++i) v[i] = r[i];
  }
}

/* Code j (width `bits`) of a little-endian bit row. */
static int row_code(const uint8_t* row, int j, int bits) {
  int c = 0;
  for (int b = 0; b < bits; ++b) {
    const int bit = bits * j + b;
    c |= ((row[bit >> 3] >> (bit & 7)) & 1) << b;
  }
  return c;
}

/* Code of dim j of cache slot `slot` in one head's V tiles. */
static int tile_code(const uint8_t* tiles, int64_t slot, int j) {
  const uint8_t* tile = tiles + (slot / 8) * 384;
  const int r = (int)(slot % 8);
  int c = 0;
  for (int b = 0; b < 3; ++b) {
    const int bit = 24 * j + 3 * r + b;
    c |= ((tile[bit >> 3] >> (bit & 7)) & 1) << b;
  }
  return c;
}

/* x_hat = n . Hn . B^T . c */
static void reconstruct(double* x, const double* c, float n, const float* rot_head) {
  for (int j = 0; j < D; ++j) x[j] = c[j];
  blocks(x, rot_head, 1);
  wht(x);
  for (int j = 0; j < D; ++j) x[j] *= (double)n;
}

/*
 * Encode n vectors of one head: x float [n][128] -> rows uint8 [n][16 bits]
 * (bits = 3 with 7 thresholds, 4 with 15), norms float [n]. Returns 0, or -1
 * for an unsupported level count.
 */
int iqo_encode(const float* x, int64_t n, const float* rot_head, const float* thresholds, int levels,
               uint8_t* rows, float* norms) {
  if (levels != 8 && levels != 16) return -1;
  const int bits = levels == 8 ? 3 : 4, row_bytes = 16 * bits;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    double y[D];
    for (int j = 0; j < D; ++j) y[j] = x[i * D + j];
    wht(y);
    blocks(y, rot_head, 0);
    float yf[D];
    double ss = 0.0;
    for (int j = 0; j < D; ++j) {
      yf[j] = (float)y[j];
      ss += (double)yf[j] * (double)yf[j];
    }
    const float nf = (float)sqrt(ss);
    norms[i] = nf;
    uint8_t* row = rows + i * row_bytes;
    memset(row, 0, row_bytes);
    for (int j = 0; j < D; ++j) {
      int c = 0;
      for (int k = 0; k < levels - 1; ++k) {
        const float thr = thresholds[k] * nf;   /* a float product (built without contraction) */
        if (yf[j] > thr) ++c;
      }
      for (int b = 0; b < bits; ++b) {
        const int bit = bits * j + b;
        row[bit >> 3] |= (uint8_t)(((c >> b) & 1) << (bit & 7));
      }
    }
  }
  return 0;
}

/*
 * Decode attention over the packed cache of one layer, straight from the
 * definition (dequantize every row of the sequence, then softmax attention).
 *   q          float [n_seqs][hq][128]
 *   k_rows     uint8 [hkv][capacity][16 k_bits]; k_norms float [hkv][capacity]
 *   v_tiles    uint8 [hkv][capacity / 8][384];   v_norms float [hkv][capacity]
 *   rot        float [hkv][32][8] (WHT + SO(4) parameters)
 *   k_cent     float [2^k_bits] K centroids; v_cent float [8]
 *   seq_start, seq_len  int32 [n_seqs]
 *   heads      int32 [n_heads] KV heads to compute (NULL: all)
 *   out        double [n_seqs][hq][128]; rows of heads not computed are left as they are.
 * Returns 0, or -1 for invalid sizes.
 */
int iqo_decode(const float* q, int n_seqs, int hq, int hkv, int capacity, int k_bits, const uint8_t* k_rows,
               const float* k_norms, const uint8_t* v_tiles, const float* v_norms, const float* rot,
               const float* k_cent, const float* v_cent, const int32_t* seq_start, const int32_t* seq_len,
               const int32_t* heads, int n_heads, double scale, double* out) {
  if (hkv < 1 || hq % hkv != 0 || (k_bits != 3 && k_bits != 4) || capacity % 8 != 0) return -1;
  const int g_per = hq / hkv, k_row_bytes = 16 * k_bits;
  const int nh = heads ? n_heads : hkv;
  for (int s = 0; s < n_seqs; ++s) {
    const int64_t a = seq_start[s], n = seq_len[s];
    for (int hi = 0; hi < nh; ++hi) {
      const int h = heads ? heads[hi] : hi;
      double* o = out + ((int64_t)s * hq + (int64_t)h * g_per) * D;
      if (n <= 0) {
        for (int64_t i = 0; i < (int64_t)g_per * D; ++i) o[i] = 0.0;
        continue;
      }
      const float* rot_head = rot + (int64_t)h * NB * 8;
      double* v_hat = (double*)malloc(sizeof(double) * n * D);
      double* sc = (double*)malloc(sizeof(double) * n * g_per);
      if (!v_hat || !sc) {
        free(v_hat);
        free(sc);
        return -1;
      }
      /* dequantize rows, score them against the group's queries */
#pragma omp parallel for schedule(static)
      for (int64_t t = 0; t < n; ++t) {
        const int64_t slot = a + t;
        double c[D], k_hat[D];
        const uint8_t* kr = k_rows + ((int64_t)h * capacity + slot) * k_row_bytes;
        for (int j = 0; j < D; ++j) c[j] = k_cent[row_code(kr, j, k_bits)];
        reconstruct(k_hat, c, k_norms[(int64_t)h * capacity + slot], rot_head);
        const uint8_t* vt = v_tiles + (int64_t)h * (capacity / 8) * 384;
        for (int j = 0; j < D; ++j) c[j] = v_cent[tile_code(vt, slot, j)];
        reconstruct(v_hat + t * D, c, v_norms[(int64_t)h * capacity + slot], rot_head);
        for (int g = 0; g < g_per; ++g) {
          const float* qg = q + ((int64_t)s * hq + (int64_t)h * g_per + g) * D;
          double dot = 0.0;
          for (int j = 0; j < D; ++j) dot += (double)qg[j] * k_hat[j];
          sc[t * g_per + g] = scale * dot;
        }
      }
      /* softmax over the sequence and the weighted sum of V_hat, per query head */
      for (int g = 0; g < g_per; ++g) {
        double m = -INFINITY;
        for (int64_t t = 0; t < n; ++t) m = sc[t * g_per + g] > m ? sc[t * g_per + g] : m;
        double l = 0.0;
        for (int64_t t = 0; t < n; ++t) {
          sc[t * g_per + g] = exp(sc[t * g_per + g] - m);
          l += sc[t * g_per + g];
        }
#pragma omp parallel for schedule(static)
        for (int j = 0; j < D; ++j) {
          double acc = 0.0;
          for (int64_t t = 0; t < n; ++t) acc += sc[t * g_per + g] * v_hat[t * D + j];
          o[(int64_t)g * D + j] = acc / l;
        }
      }
      free(v_hat);
      free(sc);
    }
  }
  return 0;
}
