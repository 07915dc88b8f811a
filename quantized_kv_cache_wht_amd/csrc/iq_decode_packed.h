// The packed-cache split kernel's body, shared by the packed decode and the
// deferred-quantization decode (see iq_decode.hip for the method).
#pragma once

#include "iq_decode_common.h"

namespace iq {

constexpr int kLutEntries = 64;      // all pairs of 3-bit codes
constexpr int kLutCopies = 16;       // one per lane of a 16-lane group

// Table entry of the code pair at bit BIT of w: {hi|lo of code a, hi|lo of code b}.
template <int BIT, int N>
__device__ __forceinline__ uint2 pair_entry(const uint32_t (&w)[N], const char* lut, uint32_t lane_off) {
  constexpr int word = BIT >> 5, off = BIT & 31;
  const uint32_t src = (off <= 26) ? w[word] : __builtin_amdgcn_alignbit(w[word + 1], w[word], off);
  constexpr int field = (off <= 26) ? off : 0;
  // byte address = field * 128 + lane_off, as one bit-field extract and one
  // shift-add (the compiler's own lowering of this takes three instructions)
  uint32_t addr;
  asm("v_bfe_u32 %0, %1, %2, 6\n\tv_lshl_add_u32 %0, %0, 7, %3" : "=&v"(addr) : "v"(src), "i"(field), "v"(lane_off));
  return *reinterpret_cast<const uint2*>(lut + addr);
}

// Code operand for the 4 codes at bits BIT .. BIT+11 of w (two pairs).
template <int BIT, int N>
__device__ __forceinline__ half8 code_operand(const uint32_t (&w)[N], const char* lut, uint32_t lane_off) {
  H8 r;
  r.u2[0] = pair_entry<BIT>(w, lut, lane_off);
  r.u2[1] = pair_entry<BIT + 6>(w, lut, lane_off);
  return r.h;
}

// Packed codes and norms of one 32-slot block for this lane.
struct BlockData {
  uint32_t kw0[3], kw1[3], vw[6];
  float4 nk0, nk1, nv0, nv1;
};

// K tile T row r <-> token 8 (r/4) + 4T + r%4 of the block; this lane loads
// row n of both tiles (dims 32q .. 32q+31), V tile q (dims 8n .. 8n+7) and
// the norms of tokens 8q .. 8q+7 (its rows in the score output).
__device__ __forceinline__ void load_block(const DecodeArgs& a, size_t slot_base, int slot0, int n, int q,
                                           BlockData& d) {
  const int tok_a0 = 8 * (n >> 2) + (n & 3);
  const uint32_t* k0 = reinterpret_cast<const uint32_t*>(a.k_codes + (slot_base + slot0 + tok_a0) * kRowBytes + 12 * q);
  const uint32_t* k1 = k0 + kRowBytes;   // token + 4: 4 rows of 48 bytes = 48 dwords
  d.kw0[0] = k0[0]; d.kw0[1] = k0[1]; d.kw0[2] = k0[2];
  d.kw1[0] = k1[0]; d.kw1[1] = k1[1]; d.kw1[2] = k1[2];
  const uint2* vp = reinterpret_cast<const uint2*>(a.v_codes + ((slot_base + slot0) / kTile + q) * kTileBytes + 24 * n);
  const uint2 v0 = vp[0], v1 = vp[1], v2 = vp[2];
  d.vw[0] = v0.x; d.vw[1] = v0.y; d.vw[2] = v1.x; d.vw[3] = v1.y; d.vw[4] = v2.x; d.vw[5] = v2.y;
  const float4* nkp = reinterpret_cast<const float4*>(a.k_norms + slot_base + slot0 + 8 * q);
  const float4* nvp = reinterpret_cast<const float4*>(a.v_norms + slot_base + slot0 + 8 * q);
  d.nk0 = nkp[0]; d.nk1 = nkp[1]; d.nv0 = nvp[0]; d.nv1 = nvp[1];
}

template <int G>
struct Consts {
  const uint4* qop;      // this lane's query operand of k-step kk at qop[64 kk] (LDS)
  const uint4* qop_lo;   // G = 16: the lo halves, same layout
  float fscale;
  bool lo_lane;
  uint32_t lane_off;
  int rel_lo, rel_hi;
  const char* lut;
};

template <int G>
__device__ __forceinline__ void process_block(const BlockData& cur, int slot0, int q, const Consts<G>& c,
                                              WaveState& st) {
  constexpr bool kSplitN = (G <= 8);
  // ---- scores: D_T[i] = row 4q + i of tile T = token 8q + 4T + i, column n ----
  floatx4 d0 = {0.f, 0.f, 0.f, 0.f}, d1 = {0.f, 0.f, 0.f, 0.f};
#define IQ_SCORE(KAPPA)                                                        \
  {                                                                            \
    const half8 ka = code_operand<12 * KAPPA>(cur.kw0, c.lut, c.lane_off);     \
    const half8 kb = code_operand<12 * KAPPA>(cur.kw1, c.lut, c.lane_off);     \
    H8 qv;                                                                     \
    qv.u4 = c.qop[64 * KAPPA];                                                 \
    d0 = mfma16(ka, qv.h, d0);                                                 \
    d1 = mfma16(kb, qv.h, d1);                                                 \
    if (!kSplitN) {                                                            \
      qv.u4 = c.qop_lo[64 * KAPPA];                                            \
      d0 = mfma16(ka, qv.h, d0);                                               \
      d1 = mfma16(kb, qv.h, d1);                                               \
    }                                                                          \
  }
  IQ_SCORE(0) IQ_SCORE(1) IQ_SCORE(2) IQ_SCORE(3) IQ_SCORE(4) IQ_SCORE(5) IQ_SCORE(6) IQ_SCORE(7)
#undef IQ_SCORE
  const float nk[8] = {cur.nk0.x, cur.nk0.y, cur.nk0.z, cur.nk0.w, cur.nk1.x, cur.nk1.y, cur.nk1.z, cur.nk1.w};
  const float nv[8] = {cur.nv0.x, cur.nv0.y, cur.nv0.z, cur.nv0.w, cur.nv1.x, cur.nv1.y, cur.nv1.z, cur.nv1.w};
  float t[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    t[i] = d0[i];
    t[4 + i] = d1[i];
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if (kSplitN) t[k] += dpp_row_ror8(t[k]);
    t[k] *= nk[k] * c.fscale;             // the score, log2 units
  }
  float nvmax;
  const bool full = slot0 >= c.rel_lo && slot0 + kBlk <= c.rel_hi;   // wave-uniform
  if (full) {
    nvmax = fmaxf(fmaxf(fmaxf(nv[0], nv[1]), fmaxf(nv[2], nv[3])), fmaxf(fmaxf(nv[4], nv[5]), fmaxf(nv[6], nv[7])));
  } else {
    nvmax = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int rel = slot0 + 8 * q + k;
      const bool valid = rel >= c.rel_lo && rel < c.rel_hi;
      t[k] = valid ? t[k] : -INFINITY;    // 2^-inf = 0 below
      nvmax = fmaxf(nvmax, valid ? nv[k] : 0.f);
    }
  }
  // ---- online softmax with a lazily raised reference ----
  const float tmax = fmaxf(fmaxf(fmaxf(t[0], t[1]), fmaxf(t[2], t[3])), fmaxf(fmaxf(t[4], t[5]), fmaxf(t[6], t[7])));
  const int ex = __builtin_amdgcn_frexp_expf(nvmax);
  float u = tmax + (ex > 0 ? static_cast<float>(ex) : 0.f);
  u = fmaxf(u, __shfl_xor(u, 16, 64));
  u = fmaxf(u, __shfl_xor(u, 32, 64));
  const bool bump = u > st.m + kLazy;   // same for every lane of one head
  if (__any(bump)) {
    const float m_new = bump ? u : st.m;
    const float alpha = bump ? fast_exp2(st.m - m_new) : 1.f;   // m = -inf gives 0
    st.l *= alpha;
    st.m = m_new;
    // accumulator rows 4q + i belong to head (4q + i) mod 8 (or 4q + i when G = 16)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int src = kSplitN ? ((4 * q + i) & 7) : (4 * q + i);
      const float ar = __shfl(alpha, src, 64);
#pragma unroll
      for (int d = 0; d < 8; ++d) st.acc[d][i] *= ar;
    }
  }
  const float mref = (st.m == -INFINITY) ? 0.f : st.m;
  // weights: token group T = tokens 8q + 4T + i; A slots (2i, 2i+1) both hold token i's weight
  H8 pa[2], pa_lo[2];
  float esum = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float e = fast_exp2(t[k] - mref);
    esum += e;
    const float p = e * nv[k];
    // hi = p truncated to 11 significant bits (exact in fp16), lo = the rest
    const float hp = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, p) & 0xffffe000u);
    if (kSplitN) {
      pa[k >> 2].u[k & 3] = dup16(c.lo_lane ? p - hp : hp);
    } else {
      pa[k >> 2].u[k & 3] = dup16(hp);
      pa_lo[k >> 2].u[k & 3] = dup16(p - hp);
    }
  }
  st.l += esum;
  // ---- PV: B = centroids of dim 8n + D for the 4 tokens 4T..4T+3 of V tile q ----
#define IQ_PV(D)                                                                     \
  {                                                                                  \
    const half8 v0 = code_operand<24 * D>(cur.vw, c.lut, c.lane_off);                \
    const half8 v1 = code_operand<24 * D + 12>(cur.vw, c.lut, c.lane_off);           \
    st.acc[D] = mfma16(pa[0].h, v0, st.acc[D]);                                      \
    st.acc[D] = mfma16(pa[1].h, v1, st.acc[D]);                                      \
    if (!kSplitN) {                                                                  \
      st.acc[D] = mfma16(pa_lo[0].h, v0, st.acc[D]);                                 \
      st.acc[D] = mfma16(pa_lo[1].h, v1, st.acc[D]);                                 \
    }                                                                                \
  }
  IQ_PV(0) IQ_PV(1) IQ_PV(2) IQ_PV(3) IQ_PV(4) IQ_PV(5) IQ_PV(6) IQ_PV(7)
#undef IQ_PV
}

// LDS of one packed split work-group.
template <int G>
struct PackedSmem {
  static constexpr bool kSplitN = (G <= 8);        // hi/lo halves share one MFMA (columns / rows g and g+8)
  static constexpr int kRows = kSplitN ? 2 * G : G;   // accumulator rows kept per wave (hi and lo halves)
  uint2 lut[kLutEntries * kLutCopies];
  // query operand of k-step kk for lane 16 q + n: dims 32 q + 4 kk + e (e = 0..3) of
  // head n & 7, each value twice (one fp16 pair); hi halves in columns n < 8, lo
  // halves in n >= 8 (G = 16: hi in qop, lo in qop_lo, column n = head n)
  uint4 qop[8][64];
  uint4 qop_lo[kSplitN ? 1 : 8][64];
  float wo[kWaves][kRows][kDim];
  float qmax[G];
  float wm[kWaves][G], wl[kWaves][G];
};

// One split of the packed decode: work-group (h = KV head, s = sequence,
// split). Records go to split index a.rec_offset + split of a.rec_splits.
template <int G>
__device__ __forceinline__ void packed_split(const DecodeArgs& a, PackedSmem<G>& sm, int split) {
  constexpr bool kSplitN = PackedSmem<G>::kSplitN;
  constexpr int kRows = PackedSmem<G>::kRows;
  uint2* lut = sm.lut;
  auto& qop = sm.qop;
  auto& qop_lo = sm.qop_lo;
  float* qmax = sm.qmax;
  auto& wm = sm.wm;
  auto& wl = sm.wl;
  auto& wo = sm.wo;
  (void)kRows;
  const int h = blockIdx.x, s = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = lane & 15, q = lane >> 4;
  int start, len;
  const bool ok = seq_ok(a, s, &start, &len);
  const int base = start & ~(kBlk - 1);
  const int nblk = ok ? n_blocks(start, len) : 0;
  if (split >= live_splits(nblk, a.blocks_per_split, a.n_splits)) return;   // the merge skips this split
  const int b_begin = split * a.blocks_per_split;
  const int b_end = split == a.n_splits - 1 ? nblk : min(nblk, b_begin + a.blocks_per_split);
  const size_t slot_base = static_cast<size_t>(h) * a.capacity + base;   // cache row of block 0, slot 0

  // This work-group's queries and rotation parameters (16 lanes per query
  // head: 8 dims and 2 SO(4) blocks each) are requested first, then the wave's
  // first two blocks: loads complete in order, so the query rotation below
  // waits only for its own inputs while the blocks are still in flight.
  const int pg = tid >> 4, pl = tid & 15;
  float xq[8], rp[16];
  if (tid < 16 * G) {
    const float4* src = reinterpret_cast<const float4*>(
        a.q + (static_cast<size_t>(s) * a.num_q_heads + h * G + pg) * kDim + 8 * pl);
    const float4 v0 = src[0], v1 = src[1];
    xq[0] = v0.x; xq[1] = v0.y; xq[2] = v0.z; xq[3] = v0.w; xq[4] = v1.x; xq[5] = v1.y; xq[6] = v1.z; xq[7] = v1.w;
    load_row_params(rot_of_head(a.rot, a.rot_kind, h), a.rot_kind, pl, rp);
  }
  // The two block loads are unconditional (a wave with fewer blocks re-reads
  // the split's last one and ignores it): a conditional load would make the
  // compiler's wait for the query inputs also wait for the blocks.
  BlockData buf0, buf1;
  int b = b_begin + wave;
  load_block(a, slot_base, min(b, b_end - 1) * kBlk, n, q, buf0);
  load_block(a, slot_base, min(b + kWaves, b_end - 1) * kBlk, n, q, buf1);

  // ---- prologue: code-pair table, rotated queries ----
  {
    // thread t fills copies 4(t%4) .. 4(t%4)+3 of pair t/4
    const uint32_t p = static_cast<uint32_t>(tid) >> 2, ca = p & 7u, cb = p >> 3;
    const uint2 e = make_uint2(centroid_f16<false>(ca, a.cb) | (centroid_f16<true>(ca, a.cb) << 16),
                               centroid_f16<false>(cb, a.cb) | (centroid_f16<true>(cb, a.cb) << 16));
#pragma unroll
    for (int k = 0; k < 4; ++k) lut[p * kLutCopies + (tid & 3) * 4 + k] = e;
  }
  if (tid < 16 * G) {
    // q' = B Hn q (the 1/sqrt(128) rides in the block matrices)
    float m[32];
    so4_matrices_row(a.rot_kind, rp, m);
    if (a.rot_kind == kRotWhtSo4) wht128_row(xq, pl);
    so4_apply_row<false>(xq, m);
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) mx = fmaxf(mx, fabsf(xq[i]));
    mx = fmaxf(mx, row_xor<8>(mx));
    mx = fmaxf(mx, row_xor<4>(mx));
    mx = fmaxf(mx, row_xor<2>(mx));
    mx = fmaxf(mx, row_xor<1>(mx));
    if (pl == 0) qmax[pg] = mx;
    // operands: q' / max|q'| split into fp16 hi (11 significant bits) and lo
    const float inv = mx > 0.f ? 1.0f / mx : 0.f;
    uint32_t* qd = reinterpret_cast<uint32_t*>(&qop[0][0]);
    uint32_t* qd_lo = reinterpret_cast<uint32_t*>(&qop_lo[0][0]);
    const int qq = pl >> 2;   // this lane's dims 8 pl .. belong to operand lanes 16 qq + ..
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int kk = 2 * (pl & 3) + (i >> 2), e = i & 3;
      const float x = xq[i] * inv;
      const float hx = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, x) & 0xffffe000u);
      if (kSplitN) {
        qd[(kk * 64 + 16 * qq + pg) * 4 + e] = dup16(hx);
        qd[(kk * 64 + 16 * qq + pg + 8) * 4 + e] = dup16(x - hx);
      } else {
        qd[(kk * 64 + 16 * qq + pg) * 4 + e] = dup16(hx);
        qd_lo[(kk * 64 + 16 * qq + pg) * 4 + e] = dup16(x - hx);
      }
    }
  }
  if (kSplitN && G < 8) {
    // columns of heads >= G stay zero
    for (int idx = tid; idx < 8 * 64; idx += kDecThreads) {
      if (((idx & 15) & 7) >= G) qop[idx >> 6][idx & 63] = make_uint4(0u, 0u, 0u, 0u);
    }
  }
  __syncthreads();

  // ---- per-lane constants: query operands, score scale ----
  Consts<G> c;
  const int g = kSplitN ? (n & 7) : n;     // head of this lane's score column / P row
  const float qm = g < G ? qmax[g] : 0.f;
  c.fscale = a.qscale * qm * a.cb.inv_alpha;
  c.qop = &qop[0][lane];
  c.qop_lo = &qop_lo[0][lane];
  c.lo_lane = kSplitN && n >= 8;   // this lane's P row carries the lo half
  c.lane_off = (lane & 15) * 8;
  c.rel_lo = start - base;
  c.rel_hi = start - base + len;
  c.lut = reinterpret_cast<const char*>(lut);

  WaveState st;
#pragma unroll
  for (int d = 0; d < 8; ++d) st.acc[d] = floatx4{0.f, 0.f, 0.f, 0.f};
  st.m = -INFINITY;
  st.l = 0.f;

  // two buffers, alternating: a block is computed while the next one is in
  // flight. The first block is taken outside the loop so that it is computed
  // straight from the registers its loads filled (a loop-carried start would
  // let the compiler copy both buffers first and so wait for both).
  if (b < b_end) {
    process_block<G>(buf0, b * kBlk, q, c, st);
    b += kWaves;
    while (b < b_end) {
      if (b + kWaves < b_end) load_block(a, slot_base, (b + kWaves) * kBlk, n, q, buf0);
      process_block<G>(buf1, b * kBlk, q, c, st);
      b += kWaves;
      if (b >= b_end) break;
      if (b + kWaves < b_end) load_block(a, slot_base, (b + kWaves) * kBlk, n, q, buf1);
      process_block<G>(buf0, b * kBlk, q, c, st);
      b += kWaves;
    }
  }

  // ---- per-wave totals ----
  float l_run = st.l;
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  if (q == 0 && n < G) {
    wm[wave][n] = st.m;
    wl[wave][n] = l_run;
  }
  // accumulator row 4q + i: G <= 8: hi half of head (4q+i) for q < 2, lo half of head (4q+i-8) for q >= 2,
  // kept as rows g and G + g; G = 16: head 4q+i
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = 4 * q + i;
    const int gr = kSplitN ? (m & 7) : m;
    const int row = (kSplitN && m >= 8) ? G + gr : gr;
    if (gr < G) {
#pragma unroll
      for (int d = 0; d < 8; ++d) wo[wave][row][8 * n + d] = st.acc[d][i];
    }
  }
  __syncthreads();
  // ---- merge the waves (and the hi/lo rows) into this split's records ----
  // record of (seq, head hg, split): m, l, pad, pad, o'[128] with o' still in
  // the rotated domain (the merge applies the one inverse rotation)
  float* rec0 = a.ws + ((static_cast<size_t>(s) * a.num_q_heads + h * G) * a.rec_splits + a.rec_offset + split) * kRec;
  const size_t head_stride = static_cast<size_t>(a.rec_splits) * kRec;
  for (int idx = tid; idx < G * kDim; idx += kDecThreads) {
    const int gr = idx >> 7, j = idx & (kDim - 1);
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, wm[w][gr]);
    float o = 0.f;
    if (mx != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float v = kSplitN ? wo[w][gr][j] + wo[w][G + gr][j] : wo[w][gr][j];
        o += fast_exp2(wm[w][gr] - mx) * v;
      }
    }
    rec0[gr * head_stride + 4 + j] = o * a.cb.inv_alpha;   // the PV operand carried alpha * c
  }
  if (tid < G) {
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, wm[w][tid]);
    float l = 0.f;
    if (mx != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) l += exp2f(wm[w][tid] - mx) * wl[w][tid];
    }
    float* r = rec0 + tid * head_stride;
    r[0] = mx;
    r[1] = l;
  }
}

}  // namespace iq
