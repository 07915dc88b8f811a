// Device-side building blocks shared by the libiq kernels (gfx950, wave64).
//
// Vector layout used by every per-vector kernel: four consecutive lanes own
// one 128-dim vector, lane part p = lane & 3 holding the 32 contiguous dims
// 32p .. 32p+31. The Walsh-Hadamard butterflies over index bits 0..4 then stay
// inside a lane (registers), and the two remaining stages (bits 5 and 6) pair
// lanes p^1 and p^2, which DPP quad permutations reach without LDS. Each SO(4)
// block (4 contiguous dims) lies inside one lane, and the 32 codes of a lane
// are exactly bytes 12p .. 12p+11 of the packed row.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace iq {

constexpr int kDim = 128;
constexpr int kBlocks = 32;          // SO(4) blocks per vector
constexpr int kRowBytes = 48;        // 128 x 3 bits
constexpr int kPerLane = 32;         // dims per lane (4 lanes per vector)

struct Codebook {
  float c[8];        // centroids of N(0, 1/128), ascending
  float t[7];        // cell boundaries (midpoints), ascending; t[3] == 0
  uint16_t h16[4];   // fp16 bit patterns of alpha * c[4..7] (the positive half) ...
  uint16_t l16[4];   // ... and of the remainders alpha * c - h16
  float inv_alpha;   // 1 / alpha: c[k] = (h16 + l16) * inv_alpha to ~2^-22
  // the 16-level codebook of 4-bit K rows, same layout
  float c4[16];
  float t4[15];      // t4[7] == 0
  uint16_t h16k[8];
  uint16_t l16k[8];
  float inv_alpha_k;
};

// K row bytes for 3- or 4-bit codes: 128 dims x bits / 8.
__host__ __device__ constexpr int k_row_bytes(int bits) { return 16 * bits; }

constexpr int kTile = 8;                   // tokens per V tile
constexpr int kTileBytes = kTile * kRowBytes;   // 384

// ---------------------------------------------------------------- DPP ----
// quad_perm selectors: lane i of every quad reads lane sel[i] of that quad.
constexpr int kQuadXor1 = 0xB1;   // [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;   // [2,3,0,1]

// Lane moves with bound_ctrl set: a lane whose source is out of its row or
// disabled reads 0. The patterns used here (quad permutations, rotations and
// mirrors within a row) always have a source in range. A move with an "old"
// operand of 0 instead would give the same values, but costs a v_mov that
// initialises each destination first.
template <int kCtrl>
__device__ __forceinline__ int dpp_i32(int x) {
  return __builtin_amdgcn_mov_dpp(x, kCtrl, 0xF, 0xF, true);
}

template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(float, dpp_i32<kCtrl>(__builtin_bit_cast(int, x)));
}

template <int kCtrl>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return static_cast<uint32_t>(dpp_i32<kCtrl>(static_cast<int>(x)));
}

template <int kCtrl>
__device__ __forceinline__ double dpp_f64(double x) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const int lo = dpp_i32<kCtrl>(static_cast<int>(u & 0xffffffffu));
  const int hi = dpp_i32<kCtrl>(static_cast<int>(u >> 32));
  return __builtin_bit_cast(double, (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) | static_cast<uint32_t>(lo));
}

// ---------------------------------------------------------------- WHT ----
// Unnormalised Sylvester Hadamard transform of the 128-vector held by a quad
// of lanes (x = this lane's 32 dims), without its two innermost stages. The
// transform is the product of seven commuting butterfly stages, one per bit
// of the dim index; the stages of bits 0 and 1 act within each 4-dim block,
// as the 4x4 Hadamard matrix H4, and are folded into the block matrices (M H4
// in place of M, see fold_h4_*), as is the 1/sqrt(128). Every kernel that
// rotates uses folded matrices and skips these two stages, forward and back
// (the inverse applies (M H4)^T = H4 M^T, H4 being symmetric).
__device__ __forceinline__ void wht128_quad(float (&x)[kPerLane], int part) {
#pragma unroll
  for (int h = 4; h < kPerLane; h <<= 1) {
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
      if ((i & h) == 0) {
        const float a = x[i], b = x[i + h];
        x[i] = a + b;
        x[i + h] = a - b;
      }
    }
  }
  // bit 5: partner part ^ 1; the lane with the bit set keeps (partner - self)
  {
    const float s = (part & 1) ? -1.0f : 1.0f;
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) x[i] = __builtin_fmaf(x[i], s, dpp_f32<kQuadXor1>(x[i]));
  }
  {
    const float s = (part & 2) ? -1.0f : 1.0f;
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) x[i] = __builtin_fmaf(x[i], s, dpp_f32<kQuadXor2>(x[i]));
  }
}

// x[i] <- x_partner[i] * s + x[i] for i = i0 .. i0+7, the partner being lane
// part ^ M (M = 1 or 2) of the quad: one v_fmac_f32 per value with its first
// operand moved across lanes by DPP. (The compiler folds a lane move only into
// an add, never into a multiply-add, hence the asm.) A DPP read of a register
// that the instruction before wrote needs two wait states: the s_nop gives
// them, and within the block no instruction reads another's result.
template <int M>
__device__ __forceinline__ void dpp_fmac8(float (&x)[kPerLane], int i0, float s) {
  static_assert(M == 1 || M == 2, "quad partners");
#define IQ_DPP_FMAC(K) "v_fmac_f32_dpp %" #K ", %" #K ", %8 " IQ_QP " row_mask:0xf bank_mask:0xf\n\t"
#define IQ_DPP_BLOCK                                                                                  \
  asm volatile("s_nop 1\n\t" IQ_DPP_FMAC(0) IQ_DPP_FMAC(1) IQ_DPP_FMAC(2) IQ_DPP_FMAC(3) IQ_DPP_FMAC(4) \
                   IQ_DPP_FMAC(5) IQ_DPP_FMAC(6) IQ_DPP_FMAC(7)                                       \
               : "+v"(x[i0]), "+v"(x[i0 + 1]), "+v"(x[i0 + 2]), "+v"(x[i0 + 3]), "+v"(x[i0 + 4]),     \
                 "+v"(x[i0 + 5]), "+v"(x[i0 + 6]), "+v"(x[i0 + 7])                                     \
               : "v"(s))
  if constexpr (M == 1) {
#define IQ_QP "quad_perm:[1,0,3,2]"
    IQ_DPP_BLOCK;
#undef IQ_QP
  } else {
#define IQ_QP "quad_perm:[2,3,0,1]"
    IQ_DPP_BLOCK;
#undef IQ_QP
  }
#undef IQ_DPP_BLOCK
#undef IQ_DPP_FMAC
}

// The same transform up to a sign per lane part: returns eps(part) H x with
// eps(p) = (-1)^popcount(p) (+1 for parts 0 and 3, -1 for parts 1 and 2).
// Each cross-lane stage is then one multiply-add per value whose lane-moved
// operand is the partner's (partner * sigma + self, sigma = -1 on the lane
// with the stage's bit set): the upper lane gets self - partner, the exact
// negation of the butterfly's partner - self. The signs carried through the
// second stage come out as eps(p); a caller folds them into the next linear
// map (negated block matrices), which is exact, so the results are
// bit-identical to wht128_quad's.
// (Without the two innermost stages, as wht128_quad.) kFirstDone: the caller
// has done the first remaining stage (bit 2, h = 4) itself.
template <bool kFirstDone = false>
__device__ __forceinline__ void wht128_quad_signed(float (&x)[kPerLane], int part) {
#pragma unroll
  for (int h = kFirstDone ? 8 : 4; h < kPerLane; h <<= 1) {
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
      if ((i & h) == 0) {
        const float a = x[i], b = x[i + h];
        x[i] = a + b;
        x[i + h] = a - b;
      }
    }
  }
  const float s1 = (part & 1) ? -1.0f : 1.0f, s2 = (part & 2) ? -1.0f : 1.0f;
#pragma unroll
  for (int i = 0; i < kPerLane; i += 8) dpp_fmac8<1>(x, i, s1);
#pragma unroll
  for (int i = 0; i < kPerLane; i += 8) dpp_fmac8<2>(x, i, s2);
}

// ------------------------------------------------------------- SO(4) ----
// The block matrices are built without multiply-add contraction, so that
// every kernel that builds them (each in its own inlining context) gets the
// same bits and the encode is identical wherever it runs.

// Hamilton product of quaternions (w, x, y, z).
__device__ __forceinline__ void qmul(const float a[4], const float b[4], float r[4]) {
#pragma clang fp contract(off)
  r[0] = a[0] * b[0] - a[1] * b[1] - a[2] * b[2] - a[3] * b[3];
  r[1] = a[0] * b[1] + a[1] * b[0] + a[2] * b[3] - a[3] * b[2];
  r[2] = a[0] * b[2] - a[1] * b[3] + a[2] * b[0] + a[3] * b[1];
  r[3] = a[0] * b[3] + a[1] * b[2] - a[2] * b[1] + a[3] * b[0];
}

// Column c of the left-multiplication matrix of q, i.e. q (x) e_c: a signed
// permutation of q's components (the Hamilton product with a unit quaternion
// involves no rounding).
__device__ __forceinline__ void left_column(const float q[4], int c, float t[4]) {
  if (c == 0) {
    t[0] = q[0]; t[1] = q[1]; t[2] = q[2]; t[3] = q[3];
  } else if (c == 1) {
    t[0] = -q[1]; t[1] = q[0]; t[2] = q[3]; t[3] = -q[2];
  } else if (c == 2) {
    t[0] = -q[2]; t[1] = -q[3]; t[2] = q[0]; t[3] = q[1];
  } else {
    t[0] = -q[3]; t[1] = q[2]; t[2] = -q[1]; t[3] = q[0];
  }
}

// Column c of the 4x4 matrix of v -> qL (x) v (x) conj(qR), times `scale`,
// from the 8 stored parameters of one block (quaternions renormalised here).
__device__ __forceinline__ void so4_column(const float* p8, int c, float scale, float col[4]) {
#pragma clang fp contract(off)
  float ql[4], qr[4];
  float nl = 0.f, nr = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ql[i] = p8[i];
    qr[i] = p8[4 + i];
    nl += ql[i] * ql[i];
    nr += qr[i] * qr[i];
  }
  nl = 1.0f / sqrtf(nl);
  nr = 1.0f / sqrtf(nr);
  const float qrc[4] = {qr[0] * nr, -qr[1] * nr, -qr[2] * nr, -qr[3] * nr};
#pragma unroll
  for (int i = 0; i < 4; ++i) ql[i] *= nl;
  float t[4], u[4];
  left_column(ql, c, t);
  qmul(t, qrc, u);
#pragma unroll
  for (int r = 0; r < 4; ++r) col[r] = u[r] * scale;
}

// ------------------------------------------------- rotation kinds ----
// (include/iq.h, iq_rotation) Every kind is applied as 32 block-diagonal 4x4
// matrices, after the WHT for the first kind only:
//   WHT + SO(4): qL (x) v (x) conj(qR) per block, scaled by 1/sqrt(128) (the
//                WHT's normalisation), 8 parameters per block;
//   ISO:         q (x) v per block (left-isoclinic), 4 parameters per block;
//   PLANAR:      Givens (c, s) on dims (4b, 4b+1) and (4b+2, 4b+3), 4
//                parameters per block (the 2x2 blocks of a 4x4 matrix).
constexpr int kRotWhtSo4 = 0, kRotIso = 1, kRotPlanar = 2;

__host__ __device__ constexpr int rot_params_per_block(int kind) { return kind == kRotWhtSo4 ? 8 : 4; }

__device__ __forceinline__ const float* rot_of_head(const float* rot, int kind, int h) {
  return rot + static_cast<size_t>(h) * kBlocks * rot_params_per_block(kind);
}

// Column c of the matrix of v -> q (x) v from 4 stored parameters (q renormalised).
__device__ __forceinline__ void iso_column(const float* p4, int c, float col[4]) {
#pragma clang fp contract(off)
  float q[4];
  float nq = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    q[i] = p4[i];
    nq += q[i] * q[i];
  }
  nq = 1.0f / sqrtf(nq);
#pragma unroll
  for (int i = 0; i < 4; ++i) q[i] *= nq;
  left_column(q, c, col);
}

// Column c of the matrix of two Givens rotations (c0, s0) on dims 0, 1 and
// (c1, s1) on dims 2, 3 (each pair renormalised).
__device__ __forceinline__ void givens_column(const float* p4, int c, float col[4]) {
#pragma clang fp contract(off)
  const int k = c >> 1;   // the pair this column belongs to
  const float a = p4[2 * k], b = p4[2 * k + 1];
  const float n = 1.0f / sqrtf(a * a + b * b);
  const float cs = a * n, sn = b * n;
  const float x = (c & 1) ? -sn : cs, y = (c & 1) ? cs : sn;   // rows 2k, 2k + 1
  col[0] = k == 0 ? x : 0.f;
  col[1] = k == 0 ? y : 0.f;
  col[2] = k == 1 ? x : 0.f;
  col[3] = k == 1 ? y : 0.f;
}

// M H4 for the WHT + SO(4) kind: row r of the block matrix times the 4x4
// Sylvester Hadamard matrix, as two butterfly stages over its four entries in
// a fixed order (u = (m0 + m1, m0 - m1, m2 + m3, m2 - m3), then (u0 + u2, u1 +
// u3, u0 - u2, u1 - u3)). fold_h4_row does it on a row in registers,
// fold_h4_columns on a block whose column c is held by lane c of a quad; both
// perform the same operations on the same operands, so every kernel gets the
// same bits.
__device__ __forceinline__ void fold_h4_row(float* m) {
  const float u0 = m[0] + m[1], u1 = m[0] - m[1], u2 = m[2] + m[3], u3 = m[2] - m[3];
  m[0] = u0 + u2;
  m[1] = u1 + u3;
  m[2] = u0 - u2;
  m[3] = u1 - u3;
}

__device__ __forceinline__ void fold_h4_columns(float (&col)[4], int c) {
  // (the lane with the stage's bit set takes partner - self, as the row form's
  // second operand minus its first)
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float p = dpp_f32<kQuadXor1>(col[r]);
    col[r] = (c & 1) ? p - col[r] : col[r] + p;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float p = dpp_f32<kQuadXor2>(col[r]);
    col[r] = (c & 2) ? p - col[r] : col[r] + p;
  }
}

// Column c of the block matrix of the given kind (every kernel builds the
// matrices through this, so all of them use the same values).
__device__ __forceinline__ void block_column(int kind, const float* p, int c, float col[4]) {
  if (kind == kRotIso) {
    iso_column(p, c, col);
  } else if (kind == kRotPlanar) {
    givens_column(p, c, col);
  } else {
    so4_column(p, c, 0.08838834764831845f, col);   // 1/sqrt(128)
  }
}

// Row-major 4x4 matrix of one block (one branch on the kind, so the four
// columns share their normalisation).
__device__ __forceinline__ void block_matrix(int kind, const float* p, float m[16]) {
  float col[4][4];
  if (kind == kRotIso) {
#pragma unroll
    for (int c = 0; c < 4; ++c) iso_column(p, c, col[c]);
  } else if (kind == kRotPlanar) {
#pragma unroll
    for (int c = 0; c < 4; ++c) givens_column(p, c, col[c]);
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) so4_column(p, c, 0.08838834764831845f, col[c]);
  }
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) m[r * 4 + c] = col[c][r];
  if (kind == kRotWhtSo4) {
#pragma unroll
    for (int r = 0; r < 4; ++r) fold_h4_row(m + 4 * r);
  }
}

// The stored parameters of block b of a head: 8 floats for the WHT + SO(4)
// kind, 4 for the others (p8[4..7] then repeat p8[0..3], unused). Both loads
// are unconditional (a load under a condition makes the compiler wait for it
// where the paths join).
__device__ __forceinline__ void load_block_params(const float* rot_head, int kind, int b, float (&p8)[8]) {
  const int per = rot_params_per_block(kind);
  const float4* r = reinterpret_cast<const float4*>(rot_head + per * b);
  const float4 t0 = r[0], t1 = r[per == 8 ? 1 : 0];
  p8[0] = t0.x; p8[1] = t0.y; p8[2] = t0.z; p8[3] = t0.w;
  p8[4] = t1.x; p8[5] = t1.y; p8[6] = t1.z; p8[7] = t1.w;
}

// The 32 block matrices of one head into LDS (row-major, 16 floats per
// block), one column per thread: threads 0..127 work, with bp from
// load_block_params(rot_head, kind, (threadIdx.x >> 2) & 31, bp).
// kQuadOrder: block 8 p + b (the b-th block of quad-form lane part p) goes to
// slot 4 b + p, so that the four lanes of a vector, reading their b-th blocks
// together, hit different LDS banks (block-major order puts them 512 bytes
// apart, all in one bank); otherwise block-major.
// kSigned (quad order, WHT + SO(4) kind only): the matrices of lane parts 1
// and 2 (blocks 8..23) are negated, to take back wht128_quad_signed's signs.
template <bool kQuadOrder = false, bool kSigned = false>
__device__ __forceinline__ void build_head_matrices(int kind, const float (&bp)[8], float* sm) {
  const int t = threadIdx.x;
  if (t < 4 * kBlocks) {
    const int b = t >> 2, c = t & 3;
    const int slot = kQuadOrder ? (b & 7) * 4 + (b >> 3) : b;
    float col[4];
    block_column(kind, bp, c, col);
    if (kind == kRotWhtSo4) fold_h4_columns(col, c);   // the quad of threads 4b .. 4b + 3 holds the block
    const int p = b >> 3;
    const bool neg = kSigned && kind == kRotWhtSo4 && (p == 1 || p == 2);
#pragma unroll
    for (int r = 0; r < 4; ++r) sm[slot * 16 + r * 4 + c] = neg ? -col[r] : col[r];
  }
}

// Fill LDS with the 32 block matrices of one head (row-major each, in the
// quad-form order that so4_apply_lane reads). Must be called by all threads of
// the block (at least 128): threads 0..127 build one column each.
template <bool kSigned = false>
__device__ __forceinline__ void load_head_matrices(const float* __restrict__ rot_head, int kind, float* sm) {
  float bp[8];
  load_block_params(rot_head, kind, (threadIdx.x >> 2) & (kBlocks - 1), bp);
  build_head_matrices<true, kSigned>(kind, bp, sm);
}

// y_b = M_b y_b for this lane's 8 blocks (transpose = use M_b^T); the
// matrices as load_head_matrices lays them out (block 8 part + b at slot 4 b + part).
template <bool kTranspose>
__device__ __forceinline__ void so4_apply_lane(float (&x)[kPerLane], const float* sm, int part) {
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const float4* mp = reinterpret_cast<const float4*>(sm + (b * 4 + part) * 16);
    const float4 r0 = mp[0], r1 = mp[1], r2 = mp[2], r3 = mp[3];
    const float m[16] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w,
                         r2.x, r2.y, r2.z, r2.w, r3.x, r3.y, r3.z, r3.w};
    const float v0 = x[4 * b], v1 = x[4 * b + 1], v2 = x[4 * b + 2], v3 = x[4 * b + 3];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float a0 = kTranspose ? m[0 * 4 + r] : m[r * 4 + 0];
      const float a1 = kTranspose ? m[1 * 4 + r] : m[r * 4 + 1];
      const float a2 = kTranspose ? m[2 * 4 + r] : m[r * 4 + 2];
      const float a3 = kTranspose ? m[3 * 4 + r] : m[r * 4 + 3];
      x[4 * b + r] = __builtin_fmaf(a3, v3, __builtin_fmaf(a2, v2, __builtin_fmaf(a1, v1, a0 * v0)));
    }
  }
}

// The PLANAR kind's blocks hold two 2x2 Givens blocks (dims 0-1 and 2-3) and
// zeros elsewhere; its products take the four nonzero entries of each row
// pair: 2 multiply-adds per value instead of 4. The skipped terms are exact
// zeros, so the values are so4_apply_*'s (up to the sign of a zero result).
// e[0..7] = m00 m01 m10 m11 m22 m23 m32 m33 of one block.
template <bool kTranspose>
__device__ __forceinline__ void givens_apply4(float* x, const float (&e)[8]) {
  const float v0 = x[0], v1 = x[1], v2 = x[2], v3 = x[3];
  x[0] = __builtin_fmaf(kTranspose ? e[2] : e[1], v1, e[0] * v0);
  x[1] = __builtin_fmaf(e[3], v1, (kTranspose ? e[1] : e[2]) * v0);
  x[2] = __builtin_fmaf(kTranspose ? e[6] : e[5], v3, e[4] * v2);
  x[3] = __builtin_fmaf(e[7], v3, (kTranspose ? e[5] : e[6]) * v2);
}

template <bool kTranspose>
__device__ __forceinline__ void givens_apply_lane(float (&x)[kPerLane], const float* sm, int part) {
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const float* mp = sm + (b * 4 + part) * 16;
    const float2 r0 = *reinterpret_cast<const float2*>(mp), r1 = *reinterpret_cast<const float2*>(mp + 4);
    const float2 r2 = *reinterpret_cast<const float2*>(mp + 10), r3 = *reinterpret_cast<const float2*>(mp + 14);
    const float e[8] = {r0.x, r0.y, r1.x, r1.y, r2.x, r2.y, r3.x, r3.y};
    givens_apply4<kTranspose>(x + 4 * b, e);
  }
}

// The lane's block products for any kind (kind is the same for every lane).
template <bool kTranspose>
__device__ __forceinline__ void blocks_apply_lane(int kind, float (&x)[kPerLane], const float* sm, int part) {
  if (kind == kRotPlanar) givens_apply_lane<kTranspose>(x, sm, part);
  else so4_apply_lane<kTranspose>(x, sm, part);
}

// ------------------------------------------------- 16-lane form ----
// A 128-vector spread over one DPP row (16 consecutive lanes), 8 dims per
// lane: lane p holds dims 8p .. 8p+7, i.e. SO(4) blocks 2p and 2p+1. Four
// times more lanes per vector than the quad form, so a single vector on the
// critical path (a query, an output) takes a quarter of the steps.
constexpr int kRowHalfMirror = 0x141;   // lane i of each 8 reads lane 7 - i
constexpr int kQuadXor3 = 0x1B;         // [3,2,1,0]
constexpr int kRowRor8 = 0x128;         // lane i reads lane (i + 8) mod 16

// Value of lane (p ^ M) of this lane's row.
template <int M>
__device__ __forceinline__ float row_xor(float x) {
  if constexpr (M == 1) return dpp_f32<kQuadXor1>(x);
  if constexpr (M == 2) return dpp_f32<kQuadXor2>(x);
  if constexpr (M == 4) return dpp_f32<kQuadXor3>(dpp_f32<kRowHalfMirror>(x));   // i ^ 7 ^ 3
  if constexpr (M == 8) return dpp_f32<kRowRor8>(x);
  return x;
}

// Value of lane t ^ M of the wave for M = 16 or 32: the gfx950 row swaps hand
// each lane itself and that partner, and the partner is the one whose bits
// differ from the lane's own (either one when they are equal).
template <int M>
__device__ __forceinline__ float lane_xor_far(float x) {
  static_assert(M == 16 || M == 32, "row swap partners");
  const uint32_t b = __builtin_bit_cast(uint32_t, x);
  uint32_t r0, r1;
  if constexpr (M == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(b, b, false, false);
    r0 = r[0];
    r1 = r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(b, b, false, false);
    r0 = r[0];
    r1 = r[1];
  }
  return __builtin_bit_cast(float, r0 == b ? r1 : r0);
}

// A 128-vector held two dims per lane of a full wave: dims t and t + 64 in
// lane t (x0, x1).
//   so4_apply_pair: the block-diagonal SO(4) product (kTranspose: B^T) with
//     the block matrices in mats (row-major 4x4 per block); the four dims of
//     a block are the lanes of one quad, fetched by quad broadcasts.
//   wht128_pair: the unnormalised Sylvester Hadamard transform: bit 6 of the
//     dim in the lane, bits 5 and 4 by row swaps, bits 3 and 2 within a row
//     (bits 1 and 0 folded into the block matrices, as for wht128_quad).
template <bool kTranspose>
__device__ __forceinline__ void so4_apply_pair(float& x0, float& x1, const float* mats, int t) {
  const int i = t & 3;
  const float* m0 = mats + 16 * (t >> 2);
  const float* m1 = m0 + 16 * 16;   // dim t + 64: block t / 4 + 16
  const float u0[4] = {dpp_f32<0x00>(x0), dpp_f32<0x55>(x0), dpp_f32<0xAA>(x0), dpp_f32<0xFF>(x0)};
  const float u1[4] = {dpp_f32<0x00>(x1), dpp_f32<0x55>(x1), dpp_f32<0xAA>(x1), dpp_f32<0xFF>(x1)};
  float a0[4], a1[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    a0[j] = kTranspose ? m0[j * 4 + i] : m0[i * 4 + j];
    a1[j] = kTranspose ? m1[j * 4 + i] : m1[i * 4 + j];
  }
  x0 = __builtin_fmaf(a0[3], u0[3], __builtin_fmaf(a0[2], u0[2], __builtin_fmaf(a0[1], u0[1], a0[0] * u0[0])));
  x1 = __builtin_fmaf(a1[3], u1[3], __builtin_fmaf(a1[2], u1[2], __builtin_fmaf(a1[1], u1[1], a1[0] * u1[0])));
}

__device__ __forceinline__ void wht128_pair(float& x0, float& x1, int t) {
  {
    const float a = x0, b = x1;
    x0 = a + b;
    x1 = a - b;
  }
  // the lane with the bit set keeps (partner - self)
#define IQ_PAIR_STAGE(M, FETCH)                      \
  {                                                  \
    const float sgn = (t & (M)) ? -1.0f : 1.0f;      \
    x0 = __builtin_fmaf(x0, sgn, FETCH(x0));         \
    x1 = __builtin_fmaf(x1, sgn, FETCH(x1));         \
  }
  IQ_PAIR_STAGE(32, lane_xor_far<32>)
  IQ_PAIR_STAGE(16, lane_xor_far<16>)
  IQ_PAIR_STAGE(8, row_xor<8>)
  IQ_PAIR_STAGE(4, row_xor<4>)
  // (dim bits 1 and 0: folded into the block matrices, as for wht128_quad)
#undef IQ_PAIR_STAGE
}

template <int M>
__device__ __forceinline__ void wht_row_stage(float (&x)[8], int p) {
  const float s = (p & M) ? -1.0f : 1.0f;   // the lane with the bit set keeps (partner - self)
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = __builtin_fmaf(x[i], s, row_xor<M>(x[i]));
}

// Unnormalised Sylvester Hadamard transform in the 16-lane form, without
// the stages of dim bits 0 and 1 (folded into the block matrices, as for
// wht128_quad).
__device__ __forceinline__ void wht128_row(float (&x)[8], int p) {
#pragma unroll
  for (int h = 4; h < 8; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if ((i & h) == 0) {
        const float a = x[i], b = x[i + h];
        x[i] = a + b;
        x[i + h] = a - b;
      }
    }
  }
  wht_row_stage<1>(x, p);
  wht_row_stage<2>(x, p);
  wht_row_stage<4>(x, p);
  wht_row_stage<8>(x, p);
}

// ------------------------------------------------- 32-lane form ----
// A 128-vector over 32 consecutive lanes (half a wave), 4 dims per lane: lane
// t holds dims 4t .. 4t+3, i.e. SO(4) block t. Dim bits 0 and 1 are in the
// lane (their WHT stages folded into the block matrices); bits 2 .. 6 are
// lane bits 0 .. 4, exchanged by DPP within a row and by a row swap across
// the two rows.
template <int M>
__device__ __forceinline__ float half_xor(float x) {
  if constexpr (M == 16) return lane_xor_far<16>(x);
  else return row_xor<M>(x);
}

template <int M>
__device__ __forceinline__ void wht_half_stage(float (&x)[4], int t) {
  const float s = (t & M) ? -1.0f : 1.0f;   // the lane with the bit set keeps (partner - self)
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = __builtin_fmaf(x[i], s, half_xor<M>(x[i]));
}

// Unnormalised Sylvester Hadamard transform in the 32-lane form, without the
// stages of dim bits 0 and 1 (folded into the block matrices).
__device__ __forceinline__ void wht128_half(float (&x)[4], int t) {
  wht_half_stage<1>(x, t);
  wht_half_stage<2>(x, t);
  wht_half_stage<4>(x, t);
  wht_half_stage<8>(x, t);
  wht_half_stage<16>(x, t);
}

// The lane's block product in the 32-lane form (m: its row-major matrix).
template <bool kTranspose>
__device__ __forceinline__ void block_apply4(int kind, float (&x)[4], const float (&m)[16]) {
  if (kind == kRotPlanar) {
    const float e[8] = {m[0], m[1], m[4], m[5], m[10], m[11], m[14], m[15]};
    givens_apply4<kTranspose>(x, e);
  } else {
    const float v0 = x[0], v1 = x[1], v2 = x[2], v3 = x[3];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float a0 = kTranspose ? m[0 * 4 + r] : m[r * 4 + 0];
      const float a1 = kTranspose ? m[1 * 4 + r] : m[r * 4 + 1];
      const float a2 = kTranspose ? m[2 * 4 + r] : m[r * 4 + 2];
      const float a3 = kTranspose ? m[3 * 4 + r] : m[r * 4 + 3];
      x[r] = __builtin_fmaf(a3, v3, __builtin_fmaf(a2, v2, __builtin_fmaf(a1, v1, a0 * v0)));
    }
  }
}

// fp64 value of lane (p ^ M) of this lane's row.
template <int M>
__device__ __forceinline__ double row_xor64(double x) {
  if constexpr (M == 1) return dpp_f64<kQuadXor1>(x);
  if constexpr (M == 2) return dpp_f64<kQuadXor2>(x);
  if constexpr (M == 4) return dpp_f64<kQuadXor3>(dpp_f64<kRowHalfMirror>(x));
  if constexpr (M == 8) return dpp_f64<kRowRor8>(x);
  return x;
}

// n = fl32(sqrt(sum y^2)) of the row's vector, the sum in double; the xor
// butterfly gives every lane of the row the identical value.
__device__ __forceinline__ float row_norm(const float (&y)[8]) {
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const double d = static_cast<double>(y[i]);
    s = __builtin_fma(d, d, s);
  }
  s += row_xor64<8>(s);
  s += row_xor64<4>(s);
  s += row_xor64<2>(s);
  s += row_xor64<1>(s);
  return __double2float_rn(sqrt(s));
}

// Row-major matrices of the lane's two blocks from their stored parameters
// (p16 as load_row_params leaves it: the second block's at p16 + 8).
__device__ __forceinline__ void so4_matrices_row(int kind, const float (&p16)[16], float (&m)[32]) {
  block_matrix(kind, p16, m);
  block_matrix(kind, p16 + 8, m + 16);
}

// y_b = M_b y_b (or M_b^T y_b) for the lane's two blocks.
template <bool kTranspose>
__device__ __forceinline__ void so4_apply_row(float (&x)[8], const float (&m)[32]) {
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const float* mb = m + 16 * b;
    const float v0 = x[4 * b], v1 = x[4 * b + 1], v2 = x[4 * b + 2], v3 = x[4 * b + 3];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float a0 = kTranspose ? mb[0 * 4 + r] : mb[r * 4 + 0];
      const float a1 = kTranspose ? mb[1 * 4 + r] : mb[r * 4 + 1];
      const float a2 = kTranspose ? mb[2 * 4 + r] : mb[r * 4 + 2];
      const float a3 = kTranspose ? mb[3 * 4 + r] : mb[r * 4 + 3];
      x[4 * b + r] = __builtin_fmaf(a3, v3, __builtin_fmaf(a2, v2, __builtin_fmaf(a1, v1, a0 * v0)));
    }
  }
}

// so4_apply_row for any kind (the PLANAR kind through its 2x2 blocks).
template <bool kTranspose>
__device__ __forceinline__ void blocks_apply_row(int kind, float (&x)[8], const float (&m)[32]) {
  if (kind == kRotPlanar) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const float* mb = m + 16 * b;
      const float e[8] = {mb[0], mb[1], mb[4], mb[5], mb[10], mb[11], mb[14], mb[15]};
      givens_apply4<kTranspose>(x + 4 * b, e);
    }
  } else {
    so4_apply_row<kTranspose>(x, m);
  }
}

// The stored parameters of the lane's two blocks: the first block's at
// p16[0..], the second's at p16[8..] (8 floats each for the WHT + SO(4) kind,
// 4 for the others, whose p16[4..7] and p16[12..15] repeat a float4 and go
// unused). The second block sits at a constant offset so that no register
// array is indexed at run time (which would put it in scratch memory). All
// four loads are unconditional: a load under a condition makes the compiler
// wait for it where the paths join.
__device__ __forceinline__ void load_row_params(const float* rot_head, int kind, int p, float (&p16)[16]) {
  const int per = 2 * rot_params_per_block(kind);
  const float4* r = reinterpret_cast<const float4*>(rot_head + per * p);
  const bool eight = kind == kRotWhtSo4;
  const float4 t[4] = {r[0], r[eight ? 1 : 0], r[eight ? 2 : 1], r[eight ? 3 : 1]};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    p16[4 * i] = t[i].x; p16[4 * i + 1] = t[i].y; p16[4 * i + 2] = t[i].z; p16[4 * i + 3] = t[i].w;
  }
}

// --------------------------------------------------- norm and codes ----
// n = fl32(sqrt(sum y^2)), sum in double over the quad. Every lane of the quad
// gets the same value.
__device__ __forceinline__ float quad_norm(const float (&y)[kPerLane]) {
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) {
    const double d = static_cast<double>(y[i]);
    s = __builtin_fma(d, d, s);
  }
  s += dpp_f64<kQuadXor1>(s);
  s += dpp_f64<kQuadXor2>(s);
  return __double2float_rn(sqrt(s));
}

// code = #{k : y > thr_k}. The thresholds are symmetric (thr_{6-k} = -thr_k,
// thr_3 = 0), so with a = |y|: y > 0 gives 4 + #{k>=4 : a > thr_k}, and
// y <= 0 gives 3 - #{k>=4 : a >= thr_k}. For a finite norm the thresholds are
// >= 0 and non-negative floats order as their bit patterns, so a >= t is
// bits(a) + 1 > bits(t): one integer comparison per threshold serves both
// signs. Valid for a finite norm (then y is finite too); code_nonfinite
// covers the rest.
__device__ __forceinline__ uint32_t code_of(float y, float t4, float t5, float t6) {
  const uint32_t npos = !(y > 0.0f);   // also for NaN
  const uint32_t u = (__float_as_uint(y) & 0x7fffffffu) + npos;
  const uint32_t m = (u > __float_as_uint(t4)) + (u > __float_as_uint(t5)) + (u > __float_as_uint(t6));
  return m ^ (4u - npos);   // 4 + m or 3 - m, m <= 3
}

// code_of for 8 values, stage by stage across the 8 (each comparison's mask
// is read a few instructions after it is written, not right away).
__device__ __forceinline__ void codes_of8(const float* y, float t4, float t5, float t6, uint32_t* c) {
  uint32_t npos[8], u[8], m[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) npos[i] = !(y[i] > 0.0f);
#pragma unroll
  for (int i = 0; i < 8; ++i) u[i] = (__float_as_uint(y[i]) & 0x7fffffffu) + npos[i];
#pragma unroll
  for (int i = 0; i < 8; ++i) m[i] = u[i] > __float_as_uint(t4);
#pragma unroll
  for (int i = 0; i < 8; ++i) m[i] += u[i] > __float_as_uint(t5);
#pragma unroll
  for (int i = 0; i < 8; ++i) m[i] += u[i] > __float_as_uint(t6);
#pragma unroll
  for (int i = 0; i < 8; ++i) c[i] = m[i] ^ (4u - npos[i]);
}

// 16-level code = #{k : y > thr_k} with the symmetric thresholds of the 4-bit
// codebook (thr_{14-k} = -thr_k, thr_7 = 0); t8..t14 are fl32(t4[8..14] n).
// Same reading as code_of, for a finite norm.
__device__ __forceinline__ uint32_t code16_of(float y, const float (&tp)[7]) {
  const uint32_t npos = !(y > 0.0f);   // also for NaN
  const uint32_t u = (__float_as_uint(y) & 0x7fffffffu) + npos;
  uint32_t m = 0;
#pragma unroll
  for (int k = 0; k < 7; ++k) m += u > __float_as_uint(tp[k]);
  return m ^ (8u - npos);   // 8 + m or 7 - m, m <= 7
}

// The code of y when the vector's norm n is not finite. Then the middle
// threshold fl(0 * n) is NaN and the others are NaN (n NaN) or -inf below it
// and +inf above it (n = +inf), so the definition counts the `below`
// thresholds (3 or 7) when n = +inf and y > -inf, and gives 0 otherwise.
__device__ __forceinline__ uint32_t code_nonfinite(float y, float n, uint32_t below) {
  return (n == __builtin_huge_valf() && y > -__builtin_huge_valf()) ? below : 0u;
}

// True when a norm is NaN or infinite (the codes then come from code_nonfinite).
__device__ __forceinline__ bool norm_nonfinite(float n) { return !(n <= 3.402823466e38f); }

// A wave-uniform codebook entry as a register value. Without it the compiler
// may turn a select between two entries of a by-value kernel argument into a
// select of their addresses and a vector load from the argument segment, one
// round trip to memory per element. (Read every entry unconditionally, then
// select: the read is not speculated into a conditional one.)
__device__ __forceinline__ float cb_value(float x) {
  return __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(x)));
}
__device__ __forceinline__ uint32_t cb_value(uint16_t x) {
  return __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x));
}

// Centroid of a 16-level code by selects: c4[v] = c4[8 + (v - 8)] for v >= 8,
// -c4[8 + (7 - v)] otherwise.
__device__ __forceinline__ float centroid16(uint32_t v, const Codebook& cb) {
  const bool neg = v < 8u;
  const uint32_t m = neg ? 7u - v : v - 8u;
  float e[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) e[i] = cb_value(cb.c4[8 + i]);
  const float a0 = (m & 1u) ? e[1] : e[0], a1 = (m & 1u) ? e[3] : e[2];
  const float a2 = (m & 1u) ? e[5] : e[4], a3 = (m & 1u) ? e[7] : e[6];
  const float b0 = (m & 2u) ? a1 : a0, b1 = (m & 2u) ? a3 : a2;
  const float mag = (m & 4u) ? b1 : b0;
  return neg ? -mag : mag;
}

// fp16 bit pattern of the hi (kLo = false) or lo part of alpha_k * c4[v].
template <bool kLo>
__device__ __forceinline__ uint32_t centroid16_f16(uint32_t v, const Codebook& cb) {
  const uint16_t* t = kLo ? cb.l16k : cb.h16k;
  const bool neg = v < 8u;
  const uint32_t m = neg ? 7u - v : v - 8u;
  uint32_t e[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) e[i] = cb_value(t[i]);
  const uint32_t a0 = (m & 1u) ? e[1] : e[0], a1 = (m & 1u) ? e[3] : e[2];
  const uint32_t a2 = (m & 1u) ? e[5] : e[4], a3 = (m & 1u) ? e[7] : e[6];
  const uint32_t b0 = (m & 2u) ? a1 : a0, b1 = (m & 2u) ? a3 : a2;
  const uint32_t mag = (m & 4u) ? b1 : b0;
  return neg ? (mag ^ 0x8000u) : mag;
}

// Pack 32 codes (3 bits each) into 3 dwords, code i at bits [3i, 3i+3):
// each code is one shift-or into its dword (codes 10 and 21 straddle two).
__device__ __forceinline__ void pack32(const uint32_t (&c)[kPerLane], uint32_t (&w)[3]) {
  w[0] = w[1] = w[2] = 0u;
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) {
    const int bit = 3 * i, word = bit >> 5, off = bit & 31;   // compile-time after unrolling
    w[word] |= c[i] << off;
    if (off > 29) w[word + 1] |= c[i] >> (32 - off);
  }
}

// Code i (0..31) of a 96-bit group held in 3 dwords.
__device__ __forceinline__ uint32_t code_at(const uint32_t (&w)[3], int i) {
  const int bit = 3 * i;
  const int word = bit >> 5, off = bit & 31;
  if (off <= 29) return (w[word] >> off) & 7u;
  return __builtin_amdgcn_alignbit(w[word + 1], w[word], off) & 7u;
}

// Centroid of a code by selects (no dynamically indexed arrays): the codebook
// is symmetric, c[v] = c[4 + (v & 3)] for v >= 4 and -c[7 - v] for v < 4.
__device__ __forceinline__ float centroid(uint32_t v, const Codebook& cb) {
  const uint32_t m = v & 3u;
  const bool neg = v < 4u;
  const uint32_t idx = neg ? (3u - m) : m;
  const float e4 = cb_value(cb.c[4]), e5 = cb_value(cb.c[5]), e6 = cb_value(cb.c[6]), e7 = cb_value(cb.c[7]);
  const float lo = (idx & 1u) ? e5 : e4;
  const float hi = (idx & 1u) ? e7 : e6;
  const float mag = (idx & 2u) ? hi : lo;
  return neg ? -mag : mag;
}

// fp16 bit pattern of the hi (kLo = false) or lo (kLo = true) part of
// alpha * c[v]; negative codes mirror the positive half (a sign flip of both).
template <bool kLo>
__device__ __forceinline__ uint32_t centroid_f16(uint32_t v, const Codebook& cb) {
  const uint16_t* t = kLo ? cb.l16 : cb.h16;
  const uint32_t m = v & 3u;
  const bool neg = v < 4u;
  const uint32_t idx = neg ? (3u - m) : m;
  const uint32_t e0 = cb_value(t[0]), e1 = cb_value(t[1]), e2 = cb_value(t[2]), e3 = cb_value(t[3]);
  const uint32_t a = (idx & 1u) ? e1 : e0;
  const uint32_t b = (idx & 1u) ? e3 : e2;
  const uint32_t mag = (idx & 2u) ? b : a;
  return neg ? (mag ^ 0x8000u) : mag;
}

// 6-bit field starting at compile-time bit OFF of a little-endian dword array.
template <int OFF>
__device__ __forceinline__ uint32_t field6(const uint32_t* w) {
  constexpr int word = OFF >> 5, off = OFF & 31;
  if constexpr (off <= 26) {
    return (w[word] >> off) & 63u;
  } else {
    return __builtin_amdgcn_alignbit(w[word + 1], w[word], off) & 63u;
  }
}

// ------------------------------------------ one token, 16-lane form ----
// K row of a 3-bit token: dim j at bits 3j, so lanes 4k .. 4k+3 (24 bits
// each) own dwords 3k .. 3k+2. Every lane of the quad must call this; lane
// 4k's w holds the quad's three dwords.
__device__ __forceinline__ void k3_row_words(const uint32_t (&c)[8], uint32_t (&w)[3]) {
  uint32_t b24 = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) b24 |= c[i] << (3 * i);
  const uint32_t b1 = dpp_u32<kQuadXor1>(b24), b2 = dpp_u32<kQuadXor2>(b24), b3 = dpp_u32<kQuadXor3>(b24);
  w[0] = b24 | (b1 << 24);
  w[1] = (b1 >> 8) | (b2 << 16);
  w[2] = (b2 >> 16) | (b3 << 8);
}

// V tile of the token's slot: dim j of tile slot r at bit 24 j + 3 r, so
// this lane's dims 8p .. 8p+7 are the tile's dwords 6p .. 6p+5. nb = the
// code bits, mk = the mask of the slot's bits, per dword.
__device__ __forceinline__ void v_tile_fields(const uint32_t (&c)[8], int slot, uint32_t (&nb)[6],
                                              uint32_t (&mk)[6]) {
  const int r3 = 3 * (slot & (kTile - 1));
#pragma unroll
  for (int k = 0; k < 6; ++k) nb[k] = mk[k] = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t f = c[i] << r3, fm = 7u << r3;   // 24-bit fields
    const int pos = 24 * i, wd = pos >> 5, off = pos & 31;   // compile-time after unrolling
    nb[wd] |= f << off;
    mk[wd] |= fm << off;
    if (off > 8) {
      nb[wd + 1] |= f >> (32 - off);
      mk[wd + 1] |= fm >> (32 - off);
    }
  }
}

}  // namespace iq
