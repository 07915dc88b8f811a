// The decode step's new token inside the split launch (iq_append_decode_attention).
//
// One work-group per (KV head, seq), dispatched ahead of the splits and
// running beside them: it encodes the token's K and V exactly as
// iq_rotate_quantize_append does (rotation, fp64 norm, Lloyd-Max codes; the
// encode of IsoQuant, arXiv 2608.08081 "RotaryQuant" abstract), stores them at
// slot seq_start[s] + seq_len[s], and attends to it: for each query head g of
// the group a one-token record
//   m = scale log2(e) nK sum_j q'_{g,j} c[kcode_j],  l = 1,  o' = nV c[vcode]
// (the same quantities as a split's record over one cache slot, in the
// rotated domain) at split index n_splits, which the merge folds in with the
// splits'. The score takes the fp32 centroids directly (no fp16 split).
//
// Waves: 0 encodes K, 1 encodes V (16 lanes each, 8 dims per lane), 2 and 3
// rotate the queries (one per 16-lane row, G = 16 in two passes); after one
// barrier row g forms query g's score and record. The cache stores come last,
// after the records, so no barrier waits on them.
//
// The splits of the same launch never use the slot (its tokens lie before
// it); the last split may read the slot's V tile dwords and norms while they
// change, and masks that slot out by selects.
#pragma once

#include "iq_decode_common.h"

namespace iq {

template <int G>
struct NewTokenSmem {
  float kc[kDim];       // K centroids of the new token (unit scale)
  float vo[kDim];       // its rotated V: centroids times the V norm
  float qr[G][kDim];    // the group's rotated queries
  float knorm;
};

// 8 dims of a new K or V vector (fp16 or fp32 input).
__device__ __forceinline__ void load8_any(const void* base, size_t off, bool f16, float (&x)[8]) {
  if (f16) {
    const half8 v = *reinterpret_cast<const half8*>(static_cast<const _Float16*>(base) + off);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = static_cast<float>(v[i]);
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
    const float4 a = p[0], b = p[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
}

template <int G, int KB>
__device__ __forceinline__ void new_token_block(const DecodeArgs& a, const NewToken& nt, NewTokenSmem<G>& sm) {
  const int h = blockIdx.x, s = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r = lane >> 4, p = lane & 15;
  int start, len;
  const bool sok = seq_ok(a, s, &start, &len);
  const int slot = sok ? start + len : 0;
  const bool valid = sok && slot < a.capacity;
  const size_t row = static_cast<size_t>(h) * a.capacity + slot;
  const bool encoder = wave < 2 && lane < 16;   // wave 0: K, wave 1: V

  // every load first: the vector (K, V or a query), the rotation, the V tile's old dwords
  float x[8], rp[16];
  const float* rot_head = rot_of_head(a.rot, a.rot_kind, h);
  uint32_t old[6] = {0u, 0u, 0u, 0u, 0u, 0u};
  uint32_t* tile = reinterpret_cast<uint32_t*>(nt.v_codes + (row / kTile) * kTileBytes) + 6 * p;
  const int qrow = 4 * (wave - 2) + r;   // waves 2, 3: query rows 0..7
  if (encoder)
    load8_any(wave == 0 ? nt.k_new : nt.v_new, (static_cast<size_t>(s) * a.num_kv_heads + h) * kDim + 8 * p,
              nt.new_f16 != 0, x);
  if (encoder || wave >= 2) load_row_params(rot_head, a.rot_kind, p, rp);
  if (encoder && wave == 1 && valid) {
    const uint2* t2 = reinterpret_cast<const uint2*>(tile);
    const uint2 o0 = t2[0], o1 = t2[1], o2 = t2[2];
    old[0] = o0.x; old[1] = o0.y; old[2] = o1.x; old[3] = o1.y; old[4] = o2.x; old[5] = o2.y;
  }

  float n = 0.f;
  uint32_t kw[3] = {0u, 0u, 0u}, nb[6] = {0u, 0u, 0u, 0u, 0u, 0u}, mk[6] = {0u, 0u, 0u, 0u, 0u, 0u};
  if (encoder) {
    float m[32];
    so4_matrices_row(a.rot_kind, rp, m);
    if (a.rot_kind == kRotWhtSo4) wht128_row(x, p);
    blocks_apply_row<false>(a.rot_kind, x, m);
    n = row_norm(x);
    uint32_t c[8];
    if (wave == 0 && KB == 4) {
      float tp[7];
#pragma unroll
      for (int k = 0; k < 7; ++k) tp[k] = __fmul_rn(a.cb.t4[8 + k], n);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        c[i] = norm_nonfinite(n) ? code_nonfinite(x[i], n, 7u) : code16_of(x[i], tp);
        kw[0] |= c[i] << (4 * i);
        sm.kc[8 * p + i] = centroid16(c[i], a.cb);
      }
    } else {
      const float t4 = __fmul_rn(a.cb.t[4], n), t5 = __fmul_rn(a.cb.t[5], n), t6 = __fmul_rn(a.cb.t[6], n);
      codes_of8(x, t4, t5, t6, c);
      if (norm_nonfinite(n)) {
#pragma unroll
        for (int i = 0; i < 8; ++i) c[i] = code_nonfinite(x[i], n, 3u);
      }
      if (wave == 0) {
        k3_row_words(c, kw);
#pragma unroll
        for (int i = 0; i < 8; ++i) sm.kc[8 * p + i] = centroid(c[i], a.cb);
      } else {
        v_tile_fields(c, slot, nb, mk);
#pragma unroll
        for (int i = 0; i < 8; ++i) sm.vo[8 * p + i] = centroid(c[i], a.cb) * n;
      }
    }
    if (wave == 0 && p == 0) sm.knorm = n;
  } else if (wave >= 2) {
    float m[32];
    so4_matrices_row(a.rot_kind, rp, m);
#pragma unroll
    for (int pass = 0; pass < (G + 7) / 8; ++pass) {
      const int g = qrow + 8 * pass;
      if (g < G) {   // uniform over the row's 16 lanes
        const float4* qp =
            reinterpret_cast<const float4*>(a.q + (static_cast<size_t>(s) * a.num_q_heads + h * G + g) * kDim + 8 * p);
        const float4 q0 = qp[0], q1 = qp[1];
        float y[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
        if (a.rot_kind == kRotWhtSo4) wht128_row(y, p);
        blocks_apply_row<false>(a.rot_kind, y, m);
#pragma unroll
        for (int i = 0; i < 8; ++i) sm.qr[g][8 * p + i] = y[i];
      }
    }
  }
  __syncthreads();

  // row g of the work-group: query g's score and its record
  const int g = tid >> 4;
  if (g < G) {
    float d = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) d = __builtin_fmaf(sm.qr[g][8 * p + i], sm.kc[8 * p + i], d);
    d += row_xor<8>(d);
    d += row_xor<4>(d);
    d += row_xor<2>(d);
    d += row_xor<1>(d);
    const float score = a.qscale * sm.knorm * d;
    float* rec = a.ws + ((static_cast<size_t>(s) * a.num_q_heads + h * G + g) * a.rec_splits + a.rec_offset +
                         a.n_splits) * kRec;
    // a new slot outside the cache: the record (and so the output) is NaN
    // (scalar selects: a select of whole float4 values goes through memory)
    float o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = valid ? sm.vo[8 * p + i] : NAN;
    reinterpret_cast<float4*>(rec + 4)[2 * p] = make_float4(o[0], o[1], o[2], o[3]);
    reinterpret_cast<float4*>(rec + 4)[2 * p + 1] = make_float4(o[4], o[5], o[6], o[7]);
    if (p == 0) *reinterpret_cast<float4*>(rec) = make_float4(valid ? score : 0.f, valid ? 1.f : NAN, 0.f, 0.f);
  }

  // the cache stores
  if (encoder && valid) {
    if (wave == 0) {
      if (KB == 4) {
        reinterpret_cast<uint32_t*>(nt.k_codes + row * k_row_bytes(4))[p] = kw[0];
      } else if ((p & 3) == 0) {
        uint32_t* dst = reinterpret_cast<uint32_t*>(nt.k_codes + row * k_row_bytes(3)) + 3 * (p >> 2);
        dst[0] = kw[0];
        dst[1] = kw[1];
        dst[2] = kw[2];
      }
      if (p == 0) nt.k_norms[row] = n;
    } else {
#pragma unroll
      for (int k = 0; k < 6; ++k) {
        const uint32_t delta = (old[k] & mk[k]) ^ nb[k];
        if (delta != 0u) atomicXor(tile + k, delta);
      }
      if (p == 0) nt.v_norms[row] = n;
    }
  }
}

}  // namespace iq
