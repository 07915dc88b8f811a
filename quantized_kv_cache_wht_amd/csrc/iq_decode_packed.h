// The packed-cache split kernel's body, shared by the packed decode and the
// deferred-quantization decode (see iq_decode.hip for the method).
#pragma once

#include "iq_decode_common.h"

namespace iq {

constexpr int kLutEntries = 64;      // all pairs of 3-bit codes
// Copies of the 3-bit table, one per lane of a 16-lane group. (An LDS read of
// 8 bytes serves 32 lanes per cycle, so lanes i and i + 16 meet in one bank
// when their entries' parity agrees; 32 copies remove those conflicts but
// measured no faster, and their extra 8 KB would cost a third work-group per
// CU.)
constexpr int kLutCopies = 16;
// the 4-bit K table's (256 entries): one per lane of half a row, so that with
// the staged blocks two work-groups still fit in a CU's LDS
constexpr int kKLutCopies = 8;
// bit pattern of 2^-80: the V norm floor of the softmax reference
constexpr uint32_t kNormFloorBits = (127u - 80u) << 23;

// Table entry of the code pair (a, b) at bit BIT of w: {hi(a) | hi(b) << 16,
// lo(a) | lo(b) << 16}, the fp16 halves of alpha c. The score operand takes
// the whole entry (against a query operand laid out (x_a, x_b, x_a, x_b)); the
// PV operand only its first dword, the hi halves (pair_hi).
template <int BIT, int N>
__device__ __forceinline__ uint2 pair_entry(const uint32_t (&w)[N], const char* lut, uint32_t lane_off) {
  constexpr int word = BIT >> 5, off = BIT & 31;
  const uint32_t src = (off <= 26) ? w[word] : __builtin_amdgcn_alignbit(w[word + 1], w[word], off);
  constexpr int field = (off <= 26) ? off : 0;
  // byte address = field * 8 kLutCopies + lane_off, as one bit-field extract
  // and one shift-add (the compiler's own lowering of this takes three)
  constexpr int shift = kLutCopies == 16 ? 7 : 8;
  static_assert(kLutCopies == 16 || kLutCopies == 32, "entry stride is a shift");
  uint32_t addr;
  asm("v_bfe_u32 %0, %1, %2, 6\n\tv_lshl_add_u32 %0, %0, %4, %3"
      : "=&v"(addr)
      : "v"(src), "i"(field), "v"(lane_off), "i"(shift));
  return *reinterpret_cast<const uint2*>(lut + addr);
}

// 4-bit K: table entry of the code pair in byte BIT / 8 of w (256 entries of
// kKLutCopies copies, 8 kKLutCopies bytes apart); the byte never straddles a dword.
template <int BIT, int N>
__device__ __forceinline__ uint2 pair_entry4(const uint32_t (&w)[N], const char* lut, uint32_t lane_off) {
  constexpr int word = BIT >> 5, field = BIT & 31;
  constexpr int shift = kKLutCopies == 8 ? 6 : 7;
  static_assert(kKLutCopies == 8 || kKLutCopies == 16, "entry stride is a shift");
  uint32_t addr;
  asm("v_bfe_u32 %0, %1, %2, 8\n\tv_lshl_add_u32 %0, %0, %4, %3"
      : "=&v"(addr)
      : "v"(w[word]), "i"(field), "v"(lane_off), "i"(shift));
  return *reinterpret_cast<const uint2*>(lut + addr);
}

template <int BIT, int N>
__device__ __forceinline__ half8 code_operand4(const uint32_t (&w)[N], const char* lut, uint32_t lane_off) {
  H8 r;
  r.u2[0] = pair_entry4<BIT>(w, lut, lane_off);
  r.u2[1] = pair_entry4<BIT + 8>(w, lut, lane_off);
  return r.h;
}

// Score operand for the 4 codes at bits BIT .. BIT+11 of w (two pairs):
// (hi a, hi b, lo a, lo b, hi c, hi d, lo c, lo d).
template <int BIT, int N>
__device__ __forceinline__ half8 code_operand(const uint32_t (&w)[N], const char* lut, uint32_t lane_off) {
  H8 r;
  r.u2[0] = pair_entry<BIT>(w, lut, lane_off);
  r.u2[1] = pair_entry<BIT + 6>(w, lut, lane_off);
  return r.h;
}

// The hi halves of the table entry of the code pair at bit BIT of w (its first dword).
template <int BIT, int N>
__device__ __forceinline__ uint32_t pair_hi(const uint32_t (&w)[N], const char* lut, uint32_t lane_off) {
  constexpr int word = BIT >> 5, off = BIT & 31;
  const uint32_t src = (off <= 26) ? w[word] : __builtin_amdgcn_alignbit(w[word + 1], w[word], off);
  constexpr int field = (off <= 26) ? off : 0;
  constexpr int shift = kLutCopies == 16 ? 7 : 8;
  uint32_t addr;
  asm("v_bfe_u32 %0, %1, %2, 6\n\tv_lshl_add_u32 %0, %0, %4, %3"
      : "=&v"(addr)
      : "v"(src), "i"(field), "v"(lane_off), "i"(shift));
  return *reinterpret_cast<const uint32_t*>(lut + addr);
}

// PV operand: hi(alpha c) of the 8 codes at bits BIT .. BIT+23 of w (the 8
// tokens of one dim of a V tile), two per table read. The hi half alone is
// within 2e-5 of alpha c (alpha is chosen for that), and an error of the V
// centroids enters the output linearly, never through the softmax.
template <int BIT, int N>
__device__ __forceinline__ half8 code_operand_hi(const uint32_t (&w)[N], const char* lut, uint32_t lane_off) {
  H8 r;
  r.u[0] = pair_hi<BIT>(w, lut, lane_off);
  r.u[1] = pair_hi<BIT + 6>(w, lut, lane_off);
  r.u[2] = pair_hi<BIT + 12>(w, lut, lane_off);
  r.u[3] = pair_hi<BIT + 18>(w, lut, lane_off);
  return r.h;
}

// The codebook's fp16 words (kernel arguments) into scalar registers at
// this point: a use in asm makes the compiler load them here, with the
// kernel's first argument loads. A scalar wait covers every scalar load in
// flight, so these must not be loaded after the sequence bounds, or the code
// table's fill would wait for the bounds.
template <int KB>
__device__ __forceinline__ void touch_codebook_words(const Codebook& cb) {
  static_assert(__builtin_offsetof(Codebook, l16) == __builtin_offsetof(Codebook, h16) + 8 &&
                    __builtin_offsetof(Codebook, l16k) == __builtin_offsetof(Codebook, h16k) + 16,
                "each lo table follows its hi table");
  uint32_t cw[4];
  __builtin_memcpy(cw, cb.h16, sizeof(cw));   // h16[4], l16[4]
  asm volatile("" ::"s"(cw[0]), "s"(cw[1]), "s"(cw[2]), "s"(cw[3]));
  if constexpr (KB == 4) {
    uint32_t kw[8];
    __builtin_memcpy(kw, cb.h16k, sizeof(kw));   // h16k[8], l16k[8]
    asm volatile("" ::"s"(kw[0]), "s"(kw[1]), "s"(kw[2]), "s"(kw[3]), "s"(kw[4]), "s"(kw[5]), "s"(kw[6]),
                 "s"(kw[7]));
  }
}

// Packed codes and norms of one 32-slot block for this lane (KB = K bits).
template <int KB>
struct BlockData {
  uint32_t kw0[KB], kw1[KB], vw[6];
  float4 nk0, nk1, nv0, nv1;
};

// One wave's copy of a 32-slot block in LDS: the K rows, the V tiles, then
// the K and V norms, each as contiguous in the cache (a block starts at a
// multiple of 32 slots, so every part is 16-byte aligned there and here).
template <int KB>
struct Stage {
  static constexpr int kK = 0;
  static constexpr int kV = kBlk * k_row_bytes(KB);                // 1536 or 2048
  static constexpr int kNK = kV + kBlk / kTile * kTileBytes;       // + 1536
  static constexpr int kNV = kNK + kBlk * 4;
  static constexpr int kBytes = kNV + kBlk * 4;
  static constexpr int kLoads = 6;   // global->LDS load instructions per block
};

// LDS of a split work-group that its waves fill and read on their own: two
// stages per wave during the loop, the wave's accumulators after it (a wave
// writes only its own area, so no barrier separates the two uses).
template <int G, int KB>
struct StageMem {
  static constexpr int kRows = (G <= 8) ? 2 * G : G;   // accumulator rows (hi and lo halves when G <= 8)
  static constexpr int kStageBytes = Stage<KB>::kBytes;
  static constexpr int kAreaBytes = 2 * kStageBytes > kRows * kDim * 4 ? 2 * kStageBytes : kRows * kDim * 4;
  union Area {
    uint4 stage[2][kStageBytes / 16];
    float wo[kRows][kDim];
    uint4 raw[kAreaBytes / 16];
  };
  Area w[kWaves];
};

// One global->LDS load: 16 bytes per lane from base + voff (base wave-uniform)
// to LDS address lds + 16 * lane. Written as inline asm: the compiler's own
// form of it is not kept inside divergent branches (it merged the two halves
// of a conditional pair of these into one load with the wrong LDS base). M0,
// which holds the LDS address, is saved and restored around the load (the
// compiler does not let inline asm clobber it).
__device__ __forceinline__ void load_lds16(uintptr_t base, uint32_t voff, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(base), "s"(lds)
      : "memory");
}

// Copies block `slot` (absolute slot of the head's cache row, a multiple of
// 32; wave-uniform) into the stage at LDS address `lds` (wave-uniform): K and
// V take two loads each, the K and V norms one each (lanes 0-7, 8-15);
// voff = 16 * lane. Every load counts once on vmcnt.
template <int KB>
__device__ __forceinline__ void issue_block_loads(const DecodeArgs& a, size_t slot, uint32_t lds, uint32_t voff,
                                                  int lane) {
  using S = Stage<KB>;
  const uintptr_t kp = reinterpret_cast<uintptr_t>(a.k_codes) + slot * k_row_bytes(KB);
  const uintptr_t vp = reinterpret_cast<uintptr_t>(a.v_codes) + slot / kTile * kTileBytes;
  load_lds16(kp, voff, lds + S::kK);
  if (KB == 4 || lane < 32) load_lds16(kp + 1024, voff, lds + S::kK + 1024);
  load_lds16(vp, voff, lds + S::kV);
  if (lane < 32) load_lds16(vp + 1024, voff, lds + S::kV + 1024);
  if (lane < 8) load_lds16(reinterpret_cast<uintptr_t>(a.k_norms + slot), voff, lds + S::kNK);
  else if (lane < 16) load_lds16(reinterpret_cast<uintptr_t>(a.v_norms + slot) - 128, voff, lds + S::kNK);
}

// This lane's part of a staged block (K tile rows n of both tiles, dims
// 32q..; V tile q, dims 8n..; the norms of tokens 8q..8q+7), read once the
// block's loads have landed: kPending is how many global->LDS loads issued
// after them may still be in flight (vmcnt counts in issue order). The reads
// are inline asm with their own waits, so the compiler neither delays them
// behind the younger loads nor reuses their registers early. kOff = the
// stage's byte offset from stage 0; ka, va, na = this lane's K, V and norm
// addresses in stage 0.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
template <int KB, int kOff, int kPending>
__device__ __forceinline__ void read_stage(uint32_t ka, uint32_t va, uint32_t na, BlockData<KB>& d) {
  f32x4 nk0, nk1, nv0, nv1;   // (float outputs: a bit cast of a vector element reads element 0)
  u32x2 v0, v1, v2;
  if constexpr (KB == 3) {
    // K: 12 bytes at a 4-byte-aligned offset per tile row -> three dword reads
    uint32_t k[6];
    asm volatile(
        "s_waitcnt vmcnt(%[n])\n\t"
        "ds_read_b32 %[k0], %[ka] offset:%[o0]\n\t"
        "ds_read_b32 %[k1], %[ka] offset:%[o1]\n\t"
        "ds_read_b32 %[k2], %[ka] offset:%[o2]\n\t"
        "ds_read_b32 %[k3], %[ka] offset:%[o3]\n\t"
        "ds_read_b32 %[k4], %[ka] offset:%[o4]\n\t"
        "ds_read_b32 %[k5], %[ka] offset:%[o5]\n\t"
        "ds_read_b64 %[v0], %[va] offset:%[v0o]\n\t"
        "ds_read_b64 %[v1], %[va] offset:%[v1o]\n\t"
        "ds_read_b64 %[v2], %[va] offset:%[v2o]\n\t"
        "ds_read_b128 %[nk0], %[na] offset:%[n0]\n\t"
        "ds_read_b128 %[nk1], %[na] offset:%[n1]\n\t"
        "ds_read_b128 %[nv0], %[na] offset:%[n2]\n\t"
        "ds_read_b128 %[nv1], %[na] offset:%[n3]\n\t"
        "s_waitcnt lgkmcnt(0)"
        : [k0] "=&v"(k[0]), [k1] "=&v"(k[1]), [k2] "=&v"(k[2]), [k3] "=&v"(k[3]), [k4] "=&v"(k[4]),
          [k5] "=&v"(k[5]), [v0] "=&v"(v0), [v1] "=&v"(v1), [v2] "=&v"(v2), [nk0] "=&v"(nk0), [nk1] "=&v"(nk1),
          [nv0] "=&v"(nv0), [nv1] "=&v"(nv1)
        : [ka] "v"(ka), [va] "v"(va), [na] "v"(na), [n] "n"(kPending), [o0] "n"(kOff), [o1] "n"(kOff + 4),
          [o2] "n"(kOff + 8), [o3] "n"(kOff + 4 * 48), [o4] "n"(kOff + 4 * 48 + 4), [o5] "n"(kOff + 4 * 48 + 8),
          [v0o] "n"(kOff), [v1o] "n"(kOff + 8), [v2o] "n"(kOff + 16), [n0] "n"(kOff),
          [n1] "n"(kOff + 16), [n2] "n"(kOff + 128), [n3] "n"(kOff + 144)
        : "memory");
    d.kw0[0] = k[0]; d.kw0[1] = k[1]; d.kw0[2] = k[2];
    d.kw1[0] = k[3]; d.kw1[1] = k[4]; d.kw1[2] = k[5];
  } else {
    u32x4 k0, k1;
    asm volatile(
        "s_waitcnt vmcnt(%[n])\n\t"
        "ds_read_b128 %[k0], %[ka] offset:%[o0]\n\t"
        "ds_read_b128 %[k1], %[ka] offset:%[o1]\n\t"
        "ds_read_b64 %[v0], %[va] offset:%[v0o]\n\t"
        "ds_read_b64 %[v1], %[va] offset:%[v1o]\n\t"
        "ds_read_b64 %[v2], %[va] offset:%[v2o]\n\t"
        "ds_read_b128 %[nk0], %[na] offset:%[n0]\n\t"
        "ds_read_b128 %[nk1], %[na] offset:%[n1]\n\t"
        "ds_read_b128 %[nv0], %[na] offset:%[n2]\n\t"
        "ds_read_b128 %[nv1], %[na] offset:%[n3]\n\t"
        "s_waitcnt lgkmcnt(0)"
        : [k0] "=&v"(k0), [k1] "=&v"(k1), [v0] "=&v"(v0), [v1] "=&v"(v1), [v2] "=&v"(v2), [nk0] "=&v"(nk0), [nk1] "=&v"(nk1),
          [nv0] "=&v"(nv0), [nv1] "=&v"(nv1)
        : [ka] "v"(ka), [va] "v"(va), [na] "v"(na), [n] "n"(kPending), [o0] "n"(kOff), [o1] "n"(kOff + 4 * 64),
          [v0o] "n"(kOff), [v1o] "n"(kOff + 8), [v2o] "n"(kOff + 16), [n0] "n"(kOff),
          [n1] "n"(kOff + 16), [n2] "n"(kOff + 128), [n3] "n"(kOff + 144)
        : "memory");
    d.kw0[0] = k0[0]; d.kw0[1] = k0[1]; d.kw0[2] = k0[2]; d.kw0[3] = k0[3];
    d.kw1[0] = k1[0]; d.kw1[1] = k1[1]; d.kw1[2] = k1[2]; d.kw1[3] = k1[3];
  }
  d.vw[0] = v0[0]; d.vw[1] = v0[1]; d.vw[2] = v1[0]; d.vw[3] = v1[1]; d.vw[4] = v2[0]; d.vw[5] = v2[1];
  d.nk0 = make_float4(nk0[0], nk0[1], nk0[2], nk0[3]);
  d.nk1 = make_float4(nk1[0], nk1[1], nk1[2], nk1[3]);
  d.nv0 = make_float4(nv0[0], nv0[1], nv0[2], nv0[3]);
  d.nv1 = make_float4(nv1[0], nv1[1], nv1[2], nv1[3]);
}

template <int G>
struct Consts {
  uint4 q[8];            // this lane's query operand of k-step kk (registers: read every block)
  const uint4* qop_lo;   // G = 16: the lo halves, at qop_lo[64 kk] (LDS)
  float fscale;
  uint32_t lo_mask;     // G <= 8: 0xffffe000 where the lane's P row carries the lo halves, else 0
  uint32_t lane_off;    // this lane's copy of the 3-bit table: (lane % kLutCopies) * 8
  uint32_t klane_off;   // and of the 4-bit K table: (lane % kKLutCopies) * 8
  int rel_lo, rel_hi;
  const char* lut;    // 3-bit code pairs (V, and K when 3-bit)
  const char* klut;   // 4-bit K code pairs
};

// One 32-slot block of the loop, in three parts (running the next block's
// scores beside this block's PV product was built and measured slower: 167
// VGPRs, no gain from the interleaving):
//   block_scores:  D_T[i] = row 4q + i of tile T = token 8q + 4T + i, column n
//   block_softmax: the scores in log2 units, the running reference, the
//                  weights p = 2^(s - m) nV as fp16 operands
//   block_pv:      acc[D] += P x (V centroids of dims 8n + D), all 32 tokens
//                  in one MFMA (K = the tokens: lane group q holds 8q .. 8q+7)
template <int G, int KB>
__device__ __forceinline__ void block_scores(const BlockData<KB>& cur, const Consts<G>& c, floatx4& d0,
                                             floatx4& d1) {
  constexpr bool kSplitN = (G <= 8);
  d0 = floatx4{0.f, 0.f, 0.f, 0.f};
  d1 = floatx4{0.f, 0.f, 0.f, 0.f};
#define IQ_SCORE(KAPPA)                                                        \
  {                                                                            \
    const half8 ka = KB == 4 ? code_operand4<16 * KAPPA>(cur.kw0, c.klut, c.klane_off) \
                             : code_operand<12 * KAPPA>(cur.kw0, c.lut, c.lane_off);  \
    const half8 kb = KB == 4 ? code_operand4<16 * KAPPA>(cur.kw1, c.klut, c.klane_off) \
                             : code_operand<12 * KAPPA>(cur.kw1, c.lut, c.lane_off);  \
    H8 qv;                                                                     \
    qv.u4 = c.q[KAPPA];                                                        \
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
}

// P operand of one block: lane (n, q) holds row n, tokens 8q .. 8q+7 (G <= 8:
// rows g the hi halves of head g's weights, rows g + 8 the lo halves; G = 16:
// hi halves in pa, lo halves in pa_lo, row = head)
struct BlockWeights {
  H8 pa, pa_lo;
};

// kFull: every slot of the block lies in the sequence (the caller's
// wave-uniform test), so no slot is masked. A separate instantiation rather
// than a branch inside: a branch that may rewrite the scores and norms costs
// the common case a copy of each at the join.
template <int G, int KB, bool kFull>
__device__ __forceinline__ void block_softmax(const floatx4& d0, const floatx4& d1, const BlockData<KB>& cur,
                                              int slot0, int q, const Consts<G>& c, WaveState& st,
                                              BlockWeights& w) {
  constexpr bool kSplitN = (G <= 8);
  const float nk[8] = {cur.nk0.x, cur.nk0.y, cur.nk0.z, cur.nk0.w, cur.nk1.x, cur.nk1.y, cur.nk1.z, cur.nk1.w};
  float nv[8] = {cur.nv0.x, cur.nv0.y, cur.nv0.z, cur.nv0.w, cur.nv1.x, cur.nv1.y, cur.nv1.z, cur.nv1.w};
  // ts = the score before the scale fscale (log2 units after it)
  float ts[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ts[i] = d0[i];
    ts[4 + i] = d1[i];
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if (kSplitN) ts[k] += dpp_row_ror8(ts[k]);
    ts[k] *= nk[k];
  }
  bool valid[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int rel = slot0 + 8 * q + k;
    valid[k] = kFull || (rel >= c.rel_lo && rel < c.rel_hi);
    if (!kFull) nv[k] = valid[k] ? nv[k] : 0.f;   // a slot outside the range may hold anything
  }
  // ---- online softmax with a lazily raised reference m ----
  // The weights against the current m go straight into the P operand: e =
  // 2^(s - m), p = e nV, split into fp16 halves. The hi half of p is p rounded
  // toward zero to fp16 (its 11 leading bits: what the conversion does with p
  // itself), the lo half p minus those bits; a lane of a lo row subtracts
  // them (its mask keeps them), a lane of a hi row subtracts 0 and converts p.
  // m must be raised (rarely) when some weight would pass 2^15 (fp16's range)
  // or some e would pass 2^96 (the sum's range); m starts at kRefStart, so the
  // first token of the wave raises it. Then the weights are formed again.
  float esum, emax, pmax;
  auto weights = [&]() {
    esum = 0.f;
    emax = 0.f;
    pmax = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float x[2], xl[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int k = 2 * i + j;
        const float arg = __builtin_fmaf(ts[k], c.fscale, -st.m);
        const float e = fast_exp2(kFull || valid[k] ? arg : -INFINITY);   // 2^-inf = 0
        const float p = e * nv[k];
        esum += e;
        emax = max_hw(emax, e);
        pmax = max_hw(pmax, p);
        const uint32_t pb = __builtin_bit_cast(uint32_t, p);
        if (kSplitN) {
          x[j] = p - __builtin_bit_cast(float, pb & c.lo_mask);
        } else {
          x[j] = p;
          xl[j] = p - __builtin_bit_cast(float, pb & 0xffffe000u);
        }
      }
      w.pa.u[i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(x[0], x[1]));
      if (!kSplitN) w.pa_lo.u[i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(xl[0], xl[1]));
    }
  };
  weights();
  if (__any(pmax > 0x1p15f || emax > 0x1p96f)) {
    // The new reference follows the largest log2 of a weight, i.e. of
    // s + log2 nV, token by token, so that the fp16 halves of the weights
    // keep their precision whatever the scale of the V norms. lg(x) =
    // bits(x) / 2^23 - 127 is a lower bound of log2 x within 0.09 (the bit
    // pattern read as a number); a norm below 2^-80 counts as 2^-80 here,
    // which keeps e below 2^96. (Norms are >= 0.) The largest weight becomes
    // 2^kWeightRefLog2; m is raised only when a weight would pass
    // 2^kWeightMaxLog2, and the same for every lane of one head.
    float u8[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float sk = kFull || valid[k] ? ts[k] * c.fscale : -INFINITY;
      const uint32_t nb = max(__builtin_bit_cast(uint32_t, nv[k]), kNormFloorBits);
      u8[k] = __builtin_fmaf(static_cast<float>(nb), 0x1p-23f, sk);   // s + lg(nV) + 127
    }
    float u = max_hw(max3_hw(u8[0], u8[1], u8[2]), max3_hw(max3_hw(u8[3], u8[4], u8[5]), u8[6], u8[7]));
    u = rows_reduce<true>(u);
    const bool bump = u > st.m + (kWeightMaxLog2 + 127.0f);
    const float m_new = bump ? u - (kWeightRefLog2 + 127.0f) : st.m;
    const float alpha = bump ? fast_exp2(st.m - m_new) : 1.f;   // from the start value: 0
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
    weights();
  }
  st.l += esum;
}

// PV operands: B = hi(alpha c) of dim 8n + D for the tokens 8q .. 8q+7 (V
// tile q). (Requesting them before the softmax, so that their table reads
// overlap it, needs the query operands back in LDS for the registers: measured
// slower, MoE step 15.6 -> 15.8 us, 131K decode 39.3 -> 41.2 us.)
struct BlockVOps {
  H8 v[8];
};

template <int G>
__device__ __forceinline__ void block_v_ops(const uint32_t (&vw)[6], const Consts<G>& c, BlockVOps& o) {
#define IQ_VOP(D) o.v[D].h = code_operand_hi<24 * D>(vw, c.lut, c.lane_off);
  IQ_VOP(0) IQ_VOP(1) IQ_VOP(2) IQ_VOP(3) IQ_VOP(4) IQ_VOP(5) IQ_VOP(6) IQ_VOP(7)
#undef IQ_VOP
}

template <int G>
__device__ __forceinline__ void block_pv(const BlockVOps& o, const BlockWeights& w, WaveState& st) {
  constexpr bool kSplitN = (G <= 8);
#pragma unroll
  for (int D = 0; D < 8; ++D) {
    st.acc[D] = mfma16(w.pa.h, o.v[D].h, st.acc[D]);
    if (!kSplitN) st.acc[D] = mfma16(w.pa_lo.h, o.v[D].h, st.acc[D]);
  }
}

template <int G, int KB>
__device__ __forceinline__ void process_block(const BlockData<KB>& cur, int slot0, int q, const Consts<G>& c,
                                              WaveState& st) {
  floatx4 d0, d1;
  BlockWeights w;
  BlockVOps vo;
  block_scores<G, KB>(cur, c, d0, d1);
  if (slot0 >= c.rel_lo && slot0 + kBlk <= c.rel_hi)   // wave-uniform
    block_softmax<G, KB, true>(d0, d1, cur, slot0, q, c, st, w);
  else
    block_softmax<G, KB, false>(d0, d1, cur, slot0, q, c, st, w);
  block_v_ops<G>(cur.vw, c, vo);
  block_pv<G>(vo, w, st);
}

// LDS of one packed split work-group.
// (the staged blocks and, after the loop, the wave accumulators are in a
// StageMem beside it)
template <int G, int KB>
struct PackedSmem {
  static constexpr bool kSplitN = (G <= 8);        // hi/lo halves share one MFMA (columns / rows g and g+8)
  uint2 lut[kLutEntries * kLutCopies];
  uint2 klut[KB == 4 ? 256 * kKLutCopies : 2];
  // query operand of k-step kk for lane 16 q + n: dims 32 q + 4 kk + e (e = 0..3) of
  // head n & 7, each value twice (one fp16 pair); hi halves in columns n < 8, lo
  // halves in n >= 8 (G = 16: hi in qop, lo in qop_lo, column n = head n)
  uint4 qop[8][64];
  uint4 qop_lo[kSplitN ? 1 : 8][kSplitN ? 1 : 64];   // (unused when kSplitN)
  float mats[kBlocks * 16];   // the head's 32 block matrices, row-major
  float qmax[G];
  float wm[kWaves][G], wl[kWaves][G];
};

// One split of the packed decode: work-group (h = KV head, s = sequence,
// split). Records go to split index a.rec_offset + split of a.rec_splits.
template <int G, int KB>
__device__ __forceinline__ void packed_split(const DecodeArgs& a, PackedSmem<G, KB>& sm, StageMem<G, KB>& stg,
                                             int split) {
#include "iq_decode_packed_body.inc"

}

}  // namespace iq
