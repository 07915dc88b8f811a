// The packed-cache split kernel's body, shared by the packed decode and the
// deferred-quantization decode (see iq_decode.hip for the method).
#pragma once

#include "iq_decode_common.h"

namespace iq {

constexpr int kLutEntries = 64;      // all pairs of 3-bit codes
// Copies of the 3-bit table, one per lane of a half-wave: an LDS read of 8
// bytes serves 32 lanes per cycle, so with 16 copies lanes i and i + 16 would
// meet in one bank whenever their entries' parity agrees (measured as ~2
// conflict cycles per LDS instruction in the decode loop).
constexpr int kLutCopies = 32;
constexpr int kKLutCopies = 16;      // the 4-bit K table's (256 entries): one per lane of a row

// Table entry of the code pair at bit BIT of w: {hi|lo of code a, hi|lo of code b}.
template <int BIT, int N>
__device__ __forceinline__ uint2 pair_entry(const uint32_t (&w)[N], const char* lut, uint32_t lane_off) {
  constexpr int word = BIT >> 5, off = BIT & 31;
  const uint32_t src = (off <= 26) ? w[word] : __builtin_amdgcn_alignbit(w[word + 1], w[word], off);
  constexpr int field = (off <= 26) ? off : 0;
  // byte address = field * 256 + lane_off, as one bit-field extract and one
  // shift-add (the compiler's own lowering of this takes three instructions)
  uint32_t addr;
  asm("v_bfe_u32 %0, %1, %2, 6\n\tv_lshl_add_u32 %0, %0, 8, %3" : "=&v"(addr) : "v"(src), "i"(field), "v"(lane_off));
  return *reinterpret_cast<const uint2*>(lut + addr);
}

// 4-bit K: table entry of the code pair in byte BIT / 8 of w (256 entries of
// 16 copies, 128 bytes apart); the byte never straddles a dword.
template <int BIT, int N>
__device__ __forceinline__ uint2 pair_entry4(const uint32_t (&w)[N], const char* lut, uint32_t lane_off) {
  constexpr int word = BIT >> 5, field = BIT & 31;
  uint32_t addr;
  asm("v_bfe_u32 %0, %1, %2, 8\n\tv_lshl_add_u32 %0, %0, 7, %3" : "=&v"(addr) : "v"(w[word]), "i"(field), "v"(lane_off));
  return *reinterpret_cast<const uint2*>(lut + addr);
}

template <int BIT, int N>
__device__ __forceinline__ half8 code_operand4(const uint32_t (&w)[N], const char* lut, uint32_t lane_off) {
  H8 r;
  r.u2[0] = pair_entry4<BIT>(w, lut, lane_off);
  r.u2[1] = pair_entry4<BIT + 8>(w, lut, lane_off);
  return r.h;
}

// Code operand for the 4 codes at bits BIT .. BIT+11 of w (two pairs).
template <int BIT, int N>
__device__ __forceinline__ half8 code_operand(const uint32_t (&w)[N], const char* lut, uint32_t lane_off) {
  H8 r;
  r.u2[0] = pair_entry<BIT>(w, lut, lane_off);
  r.u2[1] = pair_entry<BIT + 6>(w, lut, lane_off);
  return r.h;
}

// Packed codes and norms of one 32-slot block for this lane (KB = K bits).
template <int KB>
struct BlockData {
  uint32_t kw0[KB], kw1[KB], vw[6];
  float4 nk0, nk1, nv0, nv1;
};

// K tile T row r <-> token 8 (r/4) + 4T + r%4 of the block; this lane loads
// row n of both tiles (dims 32q .. 32q+31), V tile q (dims 8n .. 8n+7) and
// the norms of tokens 8q .. 8q+7 (its rows in the score output).
template <int KB>
__device__ __forceinline__ void load_block(const DecodeArgs& a, size_t slot_base, int slot0, int n, int q,
                                           BlockData<KB>& d) {
  constexpr int kRow = k_row_bytes(KB);   // 48 or 64
  const int tok_a0 = 8 * (n >> 2) + (n & 3);
  const uint32_t* k0 = reinterpret_cast<const uint32_t*>(a.k_codes + (slot_base + slot0 + tok_a0) * kRow + 4 * KB * q);
  const uint32_t* k1 = k0 + kRow;   // token + 4: 4 rows = kRow dwords
  if constexpr (KB == 4) {
    const uint4 x0 = *reinterpret_cast<const uint4*>(k0), x1 = *reinterpret_cast<const uint4*>(k1);
    d.kw0[0] = x0.x; d.kw0[1] = x0.y; d.kw0[2] = x0.z; d.kw0[3] = x0.w;
    d.kw1[0] = x1.x; d.kw1[1] = x1.y; d.kw1[2] = x1.z; d.kw1[3] = x1.w;
  } else {
    d.kw0[0] = k0[0]; d.kw0[1] = k0[1]; d.kw0[2] = k0[2];
    d.kw1[0] = k1[0]; d.kw1[1] = k1[1]; d.kw1[2] = k1[2];
  }
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
  uint32_t lane_off;    // this lane's copy of the 3-bit table: (lane & 31) * 8
  uint32_t klane_off;   // and of the 4-bit K table: (lane & 15) * 8
  int rel_lo, rel_hi;
  const char* lut;    // 3-bit code pairs (V, and K when 3-bit)
  const char* klut;   // 4-bit K code pairs
};

template <int G, int KB>
__device__ __forceinline__ void process_block(const BlockData<KB>& cur, int slot0, int q, const Consts<G>& c,
                                              WaveState& st) {
  constexpr bool kSplitN = (G <= 8);
  // ---- scores: D_T[i] = row 4q + i of tile T = token 8q + 4T + i, column n ----
  floatx4 d0 = {0.f, 0.f, 0.f, 0.f}, d1 = {0.f, 0.f, 0.f, 0.f};
#define IQ_SCORE(KAPPA)                                                        \
  {                                                                            \
    const half8 ka = KB == 4 ? code_operand4<16 * KAPPA>(cur.kw0, c.klut, c.klane_off) \
                             : code_operand<12 * KAPPA>(cur.kw0, c.lut, c.lane_off);  \
    const half8 kb = KB == 4 ? code_operand4<16 * KAPPA>(cur.kw1, c.klut, c.klane_off) \
                             : code_operand<12 * KAPPA>(cur.kw1, c.lut, c.lane_off);  \
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
  float nv[8] = {cur.nv0.x, cur.nv0.y, cur.nv0.z, cur.nv0.w, cur.nv1.x, cur.nv1.y, cur.nv1.z, cur.nv1.w};
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
      nv[k] = valid ? nv[k] : 0.f;        // a slot outside the range may hold anything
      nvmax = fmaxf(nvmax, nv[k]);
    }
  }
  // ---- online softmax with a lazily raised reference ----
  const float tmax = fmaxf(fmaxf(fmaxf(t[0], t[1]), fmaxf(t[2], t[3])), fmaxf(fmaxf(t[4], t[5]), fmaxf(t[6], t[7])));
  const int ex = __builtin_amdgcn_frexp_expf(nvmax);
  float u = tmax + (ex > 0 ? static_cast<float>(ex) : 0.f);
  u = rows_reduce<true>(u);
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
template <int G, int KB>
struct PackedSmem {
  static constexpr bool kSplitN = (G <= 8);        // hi/lo halves share one MFMA (columns / rows g and g+8)
  static constexpr int kRows = kSplitN ? 2 * G : G;   // accumulator rows kept per wave (hi and lo halves)
  uint2 lut[kLutEntries * kLutCopies];
  // the wave accumulators after the loop; during it (4-bit K) the K code-pair table
  union {
    float wo[kWaves][kRows][kDim];
    uint2 klut[KB == 4 ? 256 * kKLutCopies : 2];
  } big;
  // query operand of k-step kk for lane 16 q + n: dims 32 q + 4 kk + e (e = 0..3) of
  // head n & 7, each value twice (one fp16 pair); hi halves in columns n < 8, lo
  // halves in n >= 8 (G = 16: hi in qop, lo in qop_lo, column n = head n)
  uint4 qop[8][64];
  uint4 qop_lo[kSplitN ? 1 : 8][64];
  float mats[kBlocks * 16];   // the head's 32 block matrices, row-major
  float qmax[G];
  float wm[kWaves][G], wl[kWaves][G];
};

// One split of the packed decode: work-group (h = KV head, s = sequence,
// split). Records go to split index a.rec_offset + split of a.rec_splits.
template <int G, int KB>
__device__ __forceinline__ void packed_split(const DecodeArgs& a, PackedSmem<G, KB>& sm, int split) {
#include "iq_decode_packed_body.inc"

}

}  // namespace iq
