// Encode-side kernels of libiq: rotate (WHT then SO(4)), quantize to 3-bit
// Lloyd-Max codes with a per-vector norm, pack; plus the inverse direction.
//
// The method is the encode of IsoQuant (arXiv 2608.08081 "RotaryQuant"
// abstract: Walsh-Hadamard transform followed by block-diagonal SO(4)
// rotations, then 3-bit scalar quantization; zhichai.net TurboQuant/RotorQuant
// essay, sections "Beta 分布的魔力" and "Lloyd-Max 最优量化" for the unit-norm
// Gaussian codebook; section "真正的瓶颈" for reading packed codes in whole
// words rather than byte by byte).
//
// Launch shape: 256 threads = 64 vectors per pass (4 lanes per vector, see
// iq_device.h); every block works on one KV head (its 32 SO(4) matrices sit in
// LDS) and strides over tokens. All kernels keep every lane alive through the
// DPP butterflies and only mask loads and stores.
#include "iq_device.h"
#include "iq_launch.h"

namespace iq {

constexpr int kEncThreads = 256;
constexpr int kVecPerBlock = kEncThreads / 4;
constexpr int kRowAppendMax = 64;   // appends of up to this many tokens use the 16-lane kernel

template <typename T>
__device__ __forceinline__ void load_vec(const T* __restrict__ src, bool ok, float (&x)[kPerLane]);

template <>
__device__ __forceinline__ void load_vec<float>(const float* __restrict__ src, bool ok, float (&x)[kPerLane]) {
#pragma unroll
  for (int i = 0; i < kPerLane / 4; ++i) {
    float4 v = ok ? reinterpret_cast<const float4*>(src)[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    x[4 * i] = v.x;
    x[4 * i + 1] = v.y;
    x[4 * i + 2] = v.z;
    x[4 * i + 3] = v.w;
  }
}

template <>
__device__ __forceinline__ void load_vec<_Float16>(const _Float16* __restrict__ src, bool ok, float (&x)[kPerLane]) {
  typedef _Float16 half8 __attribute__((ext_vector_type(8)));
#pragma unroll
  for (int i = 0; i < kPerLane / 8; ++i) {
    half8 v;
    if (ok) {
      v = reinterpret_cast<const half8*>(src)[i];
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = 0;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) x[8 * i + j] = static_cast<float>(v[j]);
  }
}

// This lane's inputs of one vector as raw words (32 values: 4 uint4 for fp16,
// 8 for fp32), loaded unconditionally from a valid address, so that the load
// can be issued a window ahead and waited for only where raw_to_x uses it.
template <typename T>
struct RawVec {
  static constexpr int kWords = kPerLane * sizeof(T) / 16;
  uint4 w[kWords];
};

template <typename T>
__device__ __forceinline__ void load_raw(const T* __restrict__ src, RawVec<T>& r) {
#pragma unroll
  for (int i = 0; i < RawVec<T>::kWords; ++i) r.w[i] = reinterpret_cast<const uint4*>(src)[i];
}

// (A vector past the call's tokens converts its stand-in row as well: nothing
// of it is stored.)
template <typename T>
__device__ __forceinline__ void raw_to_x(const RawVec<T>& r, float (&x)[kPerLane]) {
  if constexpr (sizeof(T) == 2) {
    typedef _Float16 half8 __attribute__((ext_vector_type(8)));
#pragma unroll
    for (int i = 0; i < RawVec<T>::kWords; ++i) {
      const half8 v = __builtin_bit_cast(half8, r.w[i]);
#pragma unroll
      for (int k = 0; k < 8; ++k) x[8 * i + k] = static_cast<float>(v[k]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < RawVec<T>::kWords; ++i) {
      const uint32_t u[4] = {r.w[i].x, r.w[i].y, r.w[i].z, r.w[i].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) x[4 * i + k] = __builtin_bit_cast(float, u[k]);
    }
  }
}

// The WHT's first stage (dim bit 2: dims i and i + 4 of the lane, which are
// the same fp16 half of input words i / 2 and i / 2 + 2) straight from the
// fp16 input, in place of the conversion: v_fma_mix_f32 converts each half
// exactly and rounds the sum once, the same bits as converting first and
// adding after.
template <int kHalf>
__device__ __forceinline__ void mix_butterfly(uint32_t a, uint32_t b, float one, float& sum, float& dif) {
  if constexpr (kHalf == 0) {
    asm("v_fma_mix_f32 %0, %2, %4, %3 op_sel:[0,0,0] op_sel_hi:[1,0,1]\n\t"
        "v_fma_mix_f32 %1, %2, %4, -%3 op_sel:[0,0,0] op_sel_hi:[1,0,1]"
        : "=&v"(sum), "=v"(dif)
        : "v"(a), "v"(b), "s"(one));
  } else {
    asm("v_fma_mix_f32 %0, %2, %4, %3 op_sel:[1,0,1] op_sel_hi:[1,0,1]\n\t"
        "v_fma_mix_f32 %1, %2, %4, -%3 op_sel:[1,0,1] op_sel_hi:[1,0,1]"
        : "=&v"(sum), "=v"(dif)
        : "v"(a), "v"(b), "s"(one));
  }
}

__device__ __forceinline__ void wht_first_stage_f16(const RawVec<_Float16>& r, float (&x)[kPerLane]) {
  const float one = 1.0f;
  uint32_t u[16];
#pragma unroll
  for (int i = 0; i < RawVec<_Float16>::kWords; ++i) {
    u[4 * i] = r.w[i].x;
    u[4 * i + 1] = r.w[i].y;
    u[4 * i + 2] = r.w[i].z;
    u[4 * i + 3] = r.w[i].w;
  }
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    if ((k & 2) == 0) {   // words k and k + 2: dims 2k, 2k + 1 and 2k + 4, 2k + 5
      mix_butterfly<0>(u[k], u[k + 2], one, x[2 * k], x[2 * k + 4]);
      mix_butterfly<1>(u[k], u[k + 2], one, x[2 * k + 1], x[2 * k + 5]);
    }
  }
}

template <typename T>
__device__ __forceinline__ void store_vec(T* __restrict__ dst, const float (&x)[kPerLane]);

template <>
__device__ __forceinline__ void store_vec<float>(float* __restrict__ dst, const float (&x)[kPerLane]) {
#pragma unroll
  for (int i = 0; i < kPerLane / 4; ++i)
    reinterpret_cast<float4*>(dst)[i] = make_float4(x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]);
}

template <>
__device__ __forceinline__ void store_vec<_Float16>(_Float16* __restrict__ dst, const float (&x)[kPerLane]) {
  typedef _Float16 half8 __attribute__((ext_vector_type(8)));
#pragma unroll
  for (int i = 0; i < kPerLane / 8; ++i) {
    half8 v;
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = static_cast<_Float16>(x[8 * i + j]);
    reinterpret_cast<half8*>(dst)[i] = v;
  }
}

// Codes of 32 values straight into their 3 packed dwords (code i at bits
// [3i, 3i+3)), for a finite norm: the count of code_of in two comparisons per
// value, and one add with carry per code bit.
//  - With a = |y| and neg = !(y > 0), u = 2 bits(a) + neg compares with
//    T = 2 bits(t) as bits(a) + neg does with bits(t); bits(y) + bits(y) drops
//    the sign, so u is one add with neg as the carry.
//  - m = #{k >= 4 : u > T_k} by bisection (T4 <= T5 <= T6): c1 = u > T5, then
//    c0 = u > (c1 ? T6 : T4), m = 2 c1 + c0.
//  - The code, 4 + m (y > 0) or 3 - m, has bits (1, c1, c0) or (0, !c1, !c0):
//    (!neg, c1 ^ neg, c0 ^ neg). Each dword is built from its top bit down as
//    w = w + w + bit, the bit being a lane mask used as the carry; neg is
//    pushed in place of !neg and the caller flips those bits afterwards.
// One asm block handles dims 2g+1 and 2g, top dim first, so its masks are
// made and used inside it: a lane mask that a VALU instruction writes is read
// by another VALU instruction only after two wait states, which the s_nops
// and the order of the block give; SALU reads of such masks wait in hardware.
// The adds' carry-out goes to VCC, which the block clobbers. kSplit: how many
// of the pair's 6 bits (the top ones) go to the higher dword wh before the
// rest go to wl.
#define IQ_PUSH(W, M) "v_addc_co_u32_e64 %[" #W "], vcc, %[" #W "], %[" #W "], %[" #M "]\n\t"
#define IQ_CODES_HEAD                                         \
  "v_cmp_ngt_f32_e64 %[n1], %[y1], 0\n\t"                     \
  "v_cmp_ngt_f32_e64 %[n0], %[y0], 0\n\t"                     \
  "s_nop 0\n\t"                                               \
  "v_addc_co_u32_e64 %[u1], vcc, %[y1], %[y1], %[n1]\n\t"     \
  "v_addc_co_u32_e64 %[u0], vcc, %[y0], %[y0], %[n0]\n\t"     \
  "v_cmp_gt_u32_e64 %[p1], %[u1], %[t5]\n\t"                  \
  "v_cmp_gt_u32_e64 %[p0], %[u0], %[t5]\n\t"                  \
  "s_nop 0\n\t"                                               \
  "v_cndmask_b32_e64 %[x], %[t4], %[t6], %[p1]\n\t"           \
  "v_cmp_gt_u32_e64 %[q1], %[u1], %[x]\n\t"                   \
  "v_cndmask_b32_e64 %[x], %[t4], %[t6], %[p0]\n\t"           \
  "v_cmp_gt_u32_e64 %[q0], %[u0], %[x]\n\t"                   \
  "s_xor_b64 %[p1], %[p1], %[n1]\n\t"                         \
  "s_xor_b64 %[q1], %[q1], %[n1]\n\t"                         \
  "s_xor_b64 %[p0], %[p0], %[n0]\n\t"                         \
  "s_xor_b64 %[q0], %[q0], %[n0]\n\t"
#define IQ_CODES_OPERANDS                                                                                     \
  [u1] "=&v"(u[1]), [u0] "=&v"(u[0]), [x] "=&v"(xs), [n1] "=&s"(n[1]), [n0] "=&s"(n[0]), [p1] "=&s"(p[1]), \
      [p0] "=&s"(p[0]), [q1] "=&s"(q[1]), [q0] "=&s"(q[0])
#define IQ_CODES_INPUTS \
  [y1] "v"(y[2 * g + 1]), [y0] "v"(y[2 * g]), [t4] "v"(T4), [t5] "v"(T5), [t6] "v"(T6)
template <int g>
__device__ __forceinline__ void codes_pair(const float (&y)[kPerLane], uint32_t T4, uint32_t T5, uint32_t T6,
                                           uint32_t (&w)[3]) {
  constexpr int top = 6 * g + 5, wh = top >> 5, wl = (6 * g) >> 5;
  constexpr int kSplit = wh == wl ? 6 : top - 32 * wh + 1;
  static_assert(kSplit == 6 || kSplit == 4 || kSplit == 2, "pair layout");
  uint32_t u[2], xs;
  uint64_t n[2], p[2], q[2];
  if constexpr (kSplit == 6) {
    asm(IQ_CODES_HEAD IQ_PUSH(wh, n1) IQ_PUSH(wh, p1) IQ_PUSH(wh, q1) IQ_PUSH(wh, n0) IQ_PUSH(wh, p0)
            IQ_PUSH(wh, q0)
        : [wh] "+v"(w[wh]), IQ_CODES_OPERANDS
        : IQ_CODES_INPUTS
        : "vcc");
  } else if constexpr (kSplit == 4) {
    asm(IQ_CODES_HEAD IQ_PUSH(wh, n1) IQ_PUSH(wh, p1) IQ_PUSH(wh, q1) IQ_PUSH(wh, n0) IQ_PUSH(wl, p0)
            IQ_PUSH(wl, q0)
        : [wh] "+v"(w[wh]), [wl] "+v"(w[wl]), IQ_CODES_OPERANDS
        : IQ_CODES_INPUTS
        : "vcc");
  } else {
    asm(IQ_CODES_HEAD IQ_PUSH(wh, n1) IQ_PUSH(wh, p1) IQ_PUSH(wl, q1) IQ_PUSH(wl, n0) IQ_PUSH(wl, p0)
            IQ_PUSH(wl, q0)
        : [wh] "+v"(w[wh]), [wl] "+v"(w[wl]), IQ_CODES_OPERANDS
        : IQ_CODES_INPUTS
        : "vcc");
  }
}
#undef IQ_CODES_INPUTS
#undef IQ_CODES_OPERANDS
#undef IQ_CODES_HEAD
#undef IQ_PUSH

// Pairs g, g - 1, .. 0 in that order (the dwords fill from their top bit down).
template <int g>
__device__ __forceinline__ void codes_pairs_down(const float (&y)[kPerLane], uint32_t T4, uint32_t T5, uint32_t T6,
                                                 uint32_t (&w)[3]) {
  codes_pair<g>(y, T4, T5, T6, w);
  if constexpr (g > 0) codes_pairs_down<g - 1>(y, T4, T5, T6, w);
}

__device__ __forceinline__ void codes_pack32(const float (&y)[kPerLane], float t4, float t5, float t6,
                                             uint32_t (&w)[3]) {
  const uint32_t T4 = __float_as_uint(t4) << 1, T5 = __float_as_uint(t5) << 1, T6 = __float_as_uint(t6) << 1;
  w[0] = w[1] = w[2] = 0u;
  codes_pairs_down<15>(y, T4, T5, T6, w);
  // bit 3i + 2 holds neg of value i: flip it to !neg
  w[0] ^= 0x24924924u;
  w[1] ^= 0x49249249u;
  w[2] ^= 0x92492492u;
}

// v = 0 where y > -inf, else y (-inf or NaN): the values that give a
// non-finite norm's codes through the packing above. One value at a time:
// v_cmp_class with classes 7 (signalling NaN, quiet NaN, -inf); the s_nop
// gives the mask's two wait states.
__device__ __forceinline__ void zero_above_neg_inf(const float (&y)[kPerLane], float (&v)[kPerLane]) {
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) {
    uint64_t m;
    asm("v_cmp_class_f32_e64 %[m], %[y], 7\n\t"
        "s_nop 1\n\t"
        "v_cndmask_b32_e64 %[v], 0, %[y], %[m]"
        : [v] "=v"(v[i]), [m] "=&s"(m)
        : [y] "v"(y[i]));
  }
}

// Norm, codes and the lane's 3 packed dwords of a rotated vector.
__device__ __forceinline__ float quantize_pack_lane(const float (&y)[kPerLane], const Codebook& cb,
                                                    uint32_t (&w)[3]) {
  const float n = quad_norm(y);
  float t4 = __fmul_rn(cb.t[4], n), t5 = __fmul_rn(cb.t[5], n), t6 = __fmul_rn(cb.t[6], n);
  float v[kPerLane];
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) v[i] = y[i];
  if (norm_nonfinite(n)) {
    // code_nonfinite's codes through the same packing: 3 where n = +inf and
    // y > -inf, else 0. A value of 0 against thresholds of 2 (the bits of the
    // least subnormal, doubled) gives code 3; -inf, NaN, or any value against
    // thresholds of 0, gives code 0.
    zero_above_neg_inf(y, v);
    t4 = t5 = t6 = n == __builtin_huge_valf() ? __uint_as_float(1u) : 0.0f;
  }
  codes_pack32(v, t4, t5, t6, w);
  return n;
}

// The 16-level codes of 4-bit K rows the same way (code i at bits [4i, 4i+4)
// of dword i / 8): with the positive thresholds T_0 .. T_6 (doubled bits of
// fl(thr_{8+k} n)), m = #{k : u > T_k} by three bisection steps, c2 = u > T3,
// c1 = u > (c2 ? T5 : T1), c0 = u > T_{4 c2 + 2 c1}; the code 8 + m or 7 - m
// has bits (!neg, c2 ^ neg, c1 ^ neg, c0 ^ neg). Dims 2g+1 and 2g per block,
// dword g / 4 filled from its top; the last comparison's threshold is picked
// by c2 between (T4, T0) and (T6, T2), then by c1.
#define IQ_PUSH16(M) "v_addc_co_u32_e64 %[w], vcc, %[w], %[w], %[" #M "]\n\t"
template <int g>
__device__ __forceinline__ void codes16_pair(const float (&y)[kPerLane], const uint32_t (&T)[7], uint32_t& w) {
  uint32_t u1, u0, x1, x0, ya1, yb1, ya0, yb0;
  uint64_t n1, n0, a1, a0, b1, b0, c1, c0;
  asm("v_cmp_ngt_f32_e64 %[n1], %[y1], 0\n\t"
      "v_cmp_ngt_f32_e64 %[n0], %[y0], 0\n\t"
      "s_nop 0\n\t"
      "v_addc_co_u32_e64 %[u1], vcc, %[y1], %[y1], %[n1]\n\t"
      "v_addc_co_u32_e64 %[u0], vcc, %[y0], %[y0], %[n0]\n\t"
      "v_cmp_gt_u32_e64 %[a1], %[u1], %[t3]\n\t"
      "v_cmp_gt_u32_e64 %[a0], %[u0], %[t3]\n\t"
      "s_nop 0\n\t"
      "v_cndmask_b32_e64 %[x1], %[t1], %[t5], %[a1]\n\t"
      "v_cndmask_b32_e64 %[x0], %[t1], %[t5], %[a0]\n\t"
      "v_cndmask_b32_e64 %[ya1], %[t0], %[t4], %[a1]\n\t"
      "v_cndmask_b32_e64 %[yb1], %[t2], %[t6], %[a1]\n\t"
      "v_cndmask_b32_e64 %[ya0], %[t0], %[t4], %[a0]\n\t"
      "v_cndmask_b32_e64 %[yb0], %[t2], %[t6], %[a0]\n\t"
      "v_cmp_gt_u32_e64 %[b1], %[u1], %[x1]\n\t"
      "v_cmp_gt_u32_e64 %[b0], %[u0], %[x0]\n\t"
      "s_nop 0\n\t"
      "v_cndmask_b32_e64 %[x1], %[ya1], %[yb1], %[b1]\n\t"
      "v_cndmask_b32_e64 %[x0], %[ya0], %[yb0], %[b0]\n\t"
      "v_cmp_gt_u32_e64 %[c1], %[u1], %[x1]\n\t"
      "v_cmp_gt_u32_e64 %[c0], %[u0], %[x0]\n\t"
      "s_xor_b64 %[a1], %[a1], %[n1]\n\t"
      "s_xor_b64 %[b1], %[b1], %[n1]\n\t"
      "s_xor_b64 %[c1], %[c1], %[n1]\n\t"
      "s_xor_b64 %[a0], %[a0], %[n0]\n\t"
      "s_xor_b64 %[b0], %[b0], %[n0]\n\t"
      "s_xor_b64 %[c0], %[c0], %[n0]\n\t"
      IQ_PUSH16(n1) IQ_PUSH16(a1) IQ_PUSH16(b1) IQ_PUSH16(c1) IQ_PUSH16(n0) IQ_PUSH16(a0) IQ_PUSH16(b0)
      IQ_PUSH16(c0)
      : [w] "+v"(w), [u1] "=&v"(u1), [u0] "=&v"(u0), [x1] "=&v"(x1), [x0] "=&v"(x0), [ya1] "=&v"(ya1),
        [yb1] "=&v"(yb1), [ya0] "=&v"(ya0), [yb0] "=&v"(yb0), [n1] "=&s"(n1), [n0] "=&s"(n0), [a1] "=&s"(a1),
        [a0] "=&s"(a0), [b1] "=&s"(b1), [b0] "=&s"(b0), [c1] "=&s"(c1), [c0] "=&s"(c0)
      : [y1] "v"(y[2 * g + 1]), [y0] "v"(y[2 * g]), [t0] "v"(T[0]), [t1] "v"(T[1]), [t2] "v"(T[2]),
        [t3] "v"(T[3]), [t4] "v"(T[4]), [t5] "v"(T[5]), [t6] "v"(T[6])
      : "vcc");
}
#undef IQ_PUSH16

template <int g>
__device__ __forceinline__ void codes16_pairs_down(const float (&y)[kPerLane], const uint32_t (&T)[7],
                                                   uint32_t (&w)[4]) {
  codes16_pair<g>(y, T, w[g >> 2]);
  if constexpr (g > 0) codes16_pairs_down<g - 1>(y, T, w);
}

// Norm, 16-level codes and the lane's 4 packed dwords (code i at bits 4i) of a
// rotated vector: the 4-bit K rows. A non-finite norm goes through the same
// packing as in quantize_pack_lane (code 7 or 0).
__device__ __forceinline__ float quantize_pack_lane16(const float (&y)[kPerLane], const Codebook& cb,
                                                      uint32_t (&w)[4]) {
  const float n = quad_norm(y);
  float tp[7];
#pragma unroll
  for (int k = 0; k < 7; ++k) tp[k] = __fmul_rn(cb.t4[8 + k], n);
  float v[kPerLane];
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) v[i] = y[i];
  if (norm_nonfinite(n)) {
    zero_above_neg_inf(y, v);
#pragma unroll
    for (int k = 0; k < 7; ++k) tp[k] = n == __builtin_huge_valf() ? __uint_as_float(1u) : 0.0f;
  }
  uint32_t T[7];
#pragma unroll
  for (int k = 0; k < 7; ++k) T[k] = __float_as_uint(tp[k]) << 1;
  w[0] = w[1] = w[2] = w[3] = 0u;
  codes16_pairs_down<15>(v, T, w);
#pragma unroll
  for (int d = 0; d < 4; ++d) w[d] ^= 0x88888888u;   // bit 3 of each code held neg: flip it to !neg
  return n;
}

// ---------------------------------------------------------------------------
// Append: x (K or V of new tokens) -> codes + norms in the cache.
// grid = (windows, num_kv_heads, 2 [K, V]). Without a slot list a window is
// 64 consecutive slots starting at a multiple of 8 (so every V tile belongs
// to exactly one window); with a slot list it is 64 consecutive tokens.

// Assemble the 96 bits of dims 4jq .. 4jq+3 of one V tile from the packed
// rows of its 8 slots (rows in LDS, 12 dwords each): bit 24 d + 3 r holds
// the code of dim 4 jq + d of the slot at position r.
__device__ __forceinline__ void tile_quad_bits(const uint32_t (*rows)[12], int r0, int jq, uint32_t (&out)[3]) {
  out[0] = out[1] = out[2] = 0u;
  const int bit = 12 * jq;                  // dims 4jq.. start at bit 12 jq of a row
  const int word = bit >> 5, off = bit & 31;
  // the next word's bits are used only when the 12 bits cross into it (off >
  // 20, and then word + 1 <= 11); otherwise any word of the row will do, and
  // an unconditional read keeps the lanes together
  const int word_hi = min(word + 1, 11);
#pragma unroll
  for (int r = 0; r < kTile; ++r) {
    const uint32_t lo = rows[r0 + r][word];
    const uint32_t hi = rows[r0 + r][word_hi];
    const uint32_t c12 = __builtin_amdgcn_alignbit(hi, lo, off);   // 4 codes in bits 0..11
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t c = __builtin_amdgcn_ubfe(c12, 3 * d, 3);
      const int pos = 24 * d + 3 * r;       // compile-time after unrolling
      out[pos >> 5] |= c << (pos & 31);
      if ((pos & 31) > 29) out[(pos >> 5) + 1] |= c >> (32 - (pos & 31));
    }
  }
}

// Bits of a V tile's dim-quad that belong to the slots NOT set in `mask`.
__device__ __forceinline__ void tile_keep_bits(uint32_t mask, uint32_t (&keep)[3]) {
  keep[0] = keep[1] = keep[2] = 0u;
#pragma unroll
  for (int r = 0; r < kTile; ++r) {
    if (!(mask & (1u << r))) {
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const int pos = 24 * d + 3 * r;
        keep[pos >> 5] |= 7u << (pos & 31);
        if ((pos & 31) > 29) keep[(pos >> 5) + 1] |= 7u >> (32 - (pos & 31));
      }
    }
  }
}

// kK4: the cache's K rows are 4-bit; kGivens: the PLANAR kind (2x2 blocks,
// no WHT), an instance of its own so that the other kinds' loop keeps its
// register budget.
template <typename T, bool kK4, bool kGivens>
__global__ __launch_bounds__(kEncThreads) void append_kernel(AppendArgs a) {
  __shared__ __align__(16) float sm[kBlocks * 16];
  __shared__ __align__(16) uint32_t rows[kVecPerBlock][12];
  const int h = blockIdx.y;
  const bool is_v = blockIdx.z != 0;
  const T* __restrict__ src = static_cast<const T*>(is_v ? a.v : a.k);
  uint8_t* __restrict__ codes = is_v ? a.v_codes : a.k_codes;
  float* __restrict__ norms = is_v ? a.v_norms : a.k_norms;
  const int part = threadIdx.x & 3;
  const int vec = threadIdx.x >> 2;
  const bool scatter = a.slots != nullptr;
  const int w0 = scatter ? 0 : (a.first_slot & ~(kTile - 1));   // first window start (slot or token)
  const int span = scatter ? a.n_tokens : (a.first_slot - w0 + a.n_tokens);
  const int n_windows = (span + kVecPerBlock - 1) / kVecPerBlock;
  // V tile (tt) and dim quad (jq) this thread writes in the contiguous case
  const int tt = threadIdx.x >> 5, jq = threadIdx.x & 31;

  // The first window's inputs (and, for V, the tile words a partial tile
  // keeps) are requested before the rotation matrices are built, so the
  // three memory round trips of a short append overlap.
  int win = blockIdx.x;
  auto token_of = [&](int w) { return scatter ? w * kVecPerBlock + vec : w0 + w * kVecPerBlock + vec - a.first_slot; };
  // slots of tile tt that this call writes (contiguous slots only, where the
  // host has checked 0 <= first_slot and first_slot + n_tokens <= capacity):
  // positions [lo, hi) of the tile's 8
  auto tile_mask = [&](int w) {
    const int s0 = w0 + w * kVecPerBlock + tt * kTile;
    const int lo = max(a.first_slot - s0, 0);
    const int hi = min(a.first_slot + a.n_tokens - s0, kTile);
    return hi > lo ? ((1u << hi) - 1u) & ~((1u << lo) - 1u) : 0u;
  };
  auto tile_dst = [&](int w) {
    return reinterpret_cast<uint32_t*>(
        codes + ((static_cast<size_t>(h) * a.capacity + w0 + w * kVecPerBlock + tt * kTile) / kTile) * kTileBytes +
        12 * jq);
  };
  float x[kPerLane];
  uint32_t old[3] = {0u, 0u, 0u};
  // raw inputs of the window being processed; the next window's are requested
  // before this one is rotated and quantized (not for 4-bit K, where the
  // extra registers cost a work-group per CU: measured slower)
  constexpr bool kPrefetch = !kK4;
  RawVec<T> raw;
  auto src_of = [&](int w) {
    const int tk = token_of(w);
    const bool in = tk >= 0 && tk < a.n_tokens;
    return src + (static_cast<size_t>(in ? tk : 0) * a.num_kv_heads + h) * kDim + part * kPerLane;
  };
  if (win < n_windows) {
    if (kPrefetch) {
      load_raw<T>(src_of(win), raw);
    } else {
      const int tok = token_of(win);
      load_vec<T>(src_of(win), tok >= 0 && tok < a.n_tokens, x);
    }
    if (is_v && !scatter) {
      const uint32_t m = tile_mask(win);
      if (m != 0u && m != 0xffu) {
        const uint32_t* d = tile_dst(win);
        old[0] = d[0]; old[1] = d[1]; old[2] = d[2];
      }
    }
  }
  // matrices with the signs of wht128_quad_signed folded in
  load_head_matrices<true>(rot_of_head(a.rot, a.rot_kind, h), a.rot_kind, sm);
  __syncthreads();

  for (; win < n_windows; win += gridDim.x) {
    const int tok = token_of(win);
    const bool ok = tok >= 0 && tok < a.n_tokens;
    // fp16 input with the WHT: its first stage reads the raw halves (no conversion)
    constexpr bool kMixFirst = kPrefetch && sizeof(T) == 2;
    const bool wht = !kGivens && a.rot_kind == kRotWhtSo4;
    if (kPrefetch) {
      if constexpr (kMixFirst) {
        if (wht) wht_first_stage_f16(raw, x);
        else raw_to_x<T>(raw, x);
      } else {
        raw_to_x<T>(raw, x);
      }
      if (win + static_cast<int>(gridDim.x) < n_windows) load_raw<T>(src_of(win + gridDim.x), raw);
    } else if (win != static_cast<int>(blockIdx.x)) {
      load_vec<T>(src_of(win), ok, x);
    }
    if (wht) {
      if constexpr (kMixFirst) wht128_quad_signed<true>(x, part);
      else wht128_quad_signed<false>(x, part);
    }
    if constexpr (kGivens) givens_apply_lane<false>(x, sm, part);
    else so4_apply_lane<false>(x, sm, part);
    if (kK4 && !is_v) {
      uint32_t w4[4];
      const float n4 = quantize_pack_lane16(x, a.cb, w4);
      const int slot = ok ? (scatter ? a.slots[tok] : a.first_slot + tok) : -1;
      if (slot >= 0 && slot < a.capacity) {
        const size_t row = static_cast<size_t>(h) * a.capacity + slot;
        if (part == 0) norms[row] = n4;
        *reinterpret_cast<uint4*>(codes + row * k_row_bytes(4) + part * 16) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
      }
      continue;
    }
    uint32_t w[3];
    const float n = quantize_pack_lane(x, a.cb, w);
    const int slot = ok ? (scatter ? a.slots[tok] : a.first_slot + tok) : -1;
    const bool in_cap = slot >= 0 && slot < a.capacity;
    const size_t row = static_cast<size_t>(h) * a.capacity + (in_cap ? slot : 0);
    if (in_cap && part == 0) norms[row] = n;
    if (!is_v) {
      if (in_cap) {
        uint32_t* dst = reinterpret_cast<uint32_t*>(codes + row * kRowBytes + part * 12);
        dst[0] = w[0];
        dst[1] = w[1];
        dst[2] = w[2];
      }
      continue;
    }
    if (scatter) {
      // V, arbitrary slots: merge this token's codes into its tile with atomics
      if (in_cap) {
        uint32_t* tile = reinterpret_cast<uint32_t*>(codes + (row / kTile) * kTileBytes);
        const int r = slot & (kTile - 1);
#pragma unroll
        for (int i = 0; i < kPerLane; ++i) {
          const uint32_t c = code_at(w, i);
          const int pos = 24 * (part * kPerLane + i) + 3 * r;
          const int wd = pos >> 5, off = pos & 31;
          atomicAnd(tile + wd, ~(7u << off));
          atomicOr(tile + wd, c << off);
          if (off > 29) {
            atomicAnd(tile + wd + 1, ~(7u >> (32 - off)));
            atomicOr(tile + wd + 1, c >> (32 - off));
          }
        }
      }
      continue;
    }
    // V, contiguous slots: stage rows in LDS, then write whole tile groups.
    // A wave's 16 vectors are exactly the two tiles its threads assemble
    // (tt = 2 wave, 2 wave + 1), so the exchange stays inside the wave: its
    // LDS operations execute in issue order, and a wave barrier (no
    // instruction) only keeps the compiler from moving them across.
    rows[vec][3 * part] = w[0];
    rows[vec][3 * part + 1] = w[1];
    rows[vec][3 * part + 2] = w[2];
    __builtin_amdgcn_wave_barrier();
    const uint32_t mask = tile_mask(win);
    if (mask != 0u) {
      uint32_t bits[3];
      tile_quad_bits(rows, tt * kTile, jq, bits);
      uint32_t* dst = tile_dst(win);
      if (mask != 0xffu) {
        if (win != static_cast<int>(blockIdx.x)) {
          old[0] = dst[0]; old[1] = dst[1]; old[2] = dst[2];
        }
        uint32_t keep[3];
        tile_keep_bits(mask, keep);
#pragma unroll
        for (int k = 0; k < 3; ++k) bits[k] = (old[k] & keep[k]) | (bits[k] & ~keep[k]);
      }
      dst[0] = bits[0];
      dst[1] = bits[1];
      dst[2] = bits[2];
    }
    __builtin_amdgcn_wave_barrier();   // (the next window's rows go where these were read)
  }
}

// ---------------------------------------------------------------------------
// Short appends: one vector per DPP row (16 lanes x 8 dims), so encoding a
// single token is a short dependent chain rather than the bulk kernel's
// window pipeline. grid = (ceil(n_tokens / 4), num_kv_heads, 2 [K, V]),
// 64 threads = 4 vectors. A V code lands in its tile through one atomic XOR
// per dword that flips only this slot's bits, so tokens sharing a tile (in
// this work-group or another) never overwrite each other.

template <typename T>
__device__ __forceinline__ void load8(const T* __restrict__ src, bool ok, float (&x)[8]);

template <>
__device__ __forceinline__ void load8<float>(const float* __restrict__ src, bool ok, float (&x)[8]) {
  const float4 a = ok ? reinterpret_cast<const float4*>(src)[0] : make_float4(0.f, 0.f, 0.f, 0.f);
  const float4 b = ok ? reinterpret_cast<const float4*>(src)[1] : make_float4(0.f, 0.f, 0.f, 0.f);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

template <>
__device__ __forceinline__ void load8<_Float16>(const _Float16* __restrict__ src, bool ok, float (&x)[8]) {
  typedef _Float16 half8 __attribute__((ext_vector_type(8)));
  half8 v;
  if (ok) {
    v = reinterpret_cast<const half8*>(src)[0];
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = 0;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = static_cast<float>(v[j]);
}


template <typename T>
__global__ __launch_bounds__(64) void append_row_kernel(AppendArgs a) {
  const int h = blockIdx.y;
  const bool is_v = blockIdx.z != 0;
  const int p = threadIdx.x & 15;
  const int tok = blockIdx.x * 4 + (threadIdx.x >> 4);
  const bool ok = tok < a.n_tokens;
  const int slot = ok ? (a.slots != nullptr ? a.slots[tok] : a.first_slot + tok) : -1;
  const bool in_cap = slot >= 0 && slot < a.capacity;
  const size_t row = static_cast<size_t>(h) * a.capacity + (in_cap ? slot : 0);

  // every load is issued before any arithmetic
  float x[8];
  load8<T>(static_cast<const T*>(is_v ? a.v : a.k) + (static_cast<size_t>(ok ? tok : 0) * a.num_kv_heads + h) * kDim +
               8 * p,
           ok, x);
  float rp[16];
  load_row_params(rot_of_head(a.rot, a.rot_kind, h), a.rot_kind, p, rp);
  // V: this lane's dims 8p .. 8p+7 are the tile's dwords 6p .. 6p+5
  uint32_t* tile = reinterpret_cast<uint32_t*>(a.v_codes + (row / kTile) * kTileBytes) + 6 * p;
  uint32_t old[6] = {0u, 0u, 0u, 0u, 0u, 0u};
  if (is_v && in_cap) {
    const uint2* t2 = reinterpret_cast<const uint2*>(tile);
    const uint2 o0 = t2[0], o1 = t2[1], o2 = t2[2];
    old[0] = o0.x; old[1] = o0.y; old[2] = o1.x; old[3] = o1.y; old[4] = o2.x; old[5] = o2.y;
  }

  float m[32];
  so4_matrices_row(a.rot_kind, rp, m);
  if (a.rot_kind == kRotWhtSo4) wht128_row(x, p);
  blocks_apply_row<false>(a.rot_kind, x, m);
  const float n = row_norm(x);
  if (!is_v && a.k_bits == 4) {
    // 4-bit K: this lane's 8 codes are the row's dword p
    float tp[7];
#pragma unroll
    for (int k = 0; k < 7; ++k) tp[k] = __fmul_rn(a.cb.t4[8 + k], n);
    const bool nf = norm_nonfinite(n);
    uint32_t w = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) w |= (nf ? code_nonfinite(x[i], n, 7u) : code16_of(x[i], tp)) << (4 * i);
    if (!in_cap) return;
    if (p == 0) a.k_norms[row] = n;
    reinterpret_cast<uint32_t*>(a.k_codes + row * k_row_bytes(4))[p] = w;
    return;
  }
  const float t4 = __fmul_rn(a.cb.t[4], n), t5 = __fmul_rn(a.cb.t[5], n), t6 = __fmul_rn(a.cb.t[6], n);
  uint32_t c[8];
  codes_of8(x, t4, t5, t6, c);
  if (norm_nonfinite(n)) {
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = code_nonfinite(x[i], n, 3u);
  }
  if (!in_cap) return;
  if (p == 0) (is_v ? a.v_norms : a.k_norms)[row] = n;

  if (!is_v) {
    uint32_t w[3];
    k3_row_words(c, w);
    if ((p & 3) == 0) {
      uint32_t* dst = reinterpret_cast<uint32_t*>(a.k_codes + row * kRowBytes) + 3 * (p >> 2);
      dst[0] = w[0];
      dst[1] = w[1];
      dst[2] = w[2];
    }
    return;
  }
  uint32_t nb[6], mk[6];
  v_tile_fields(c, slot, nb, mk);
#pragma unroll
  for (int k = 0; k < 6; ++k) {
    const uint32_t delta = (old[k] & mk[k]) ^ nb[k];
    if (delta != 0u) atomicXor(tile + k, delta);
  }
}

// ---------------------------------------------------------------------------
// Rotate fp32 vectors: y = R x (forward) or x = R^-1 y (inverse); for the
// WHT + SO(4) kind R = B Hn and R^-1 = Hn B^T.
// grid = (token blocks, num_heads)
template <bool kInverse>
__global__ __launch_bounds__(kEncThreads) void rotate_kernel(RotateArgs a) {
  __shared__ __align__(16) float sm[kBlocks * 16];
  const int h = blockIdx.y;
  load_head_matrices(rot_of_head(a.rot, a.rot_kind, h), a.rot_kind, sm);
  __syncthreads();
  const bool wht = a.rot_kind == kRotWhtSo4;
  const int part = threadIdx.x & 3;
  const int vec = threadIdx.x >> 2;
  for (int tok0 = blockIdx.x * kVecPerBlock; tok0 < a.n_tokens; tok0 += gridDim.x * kVecPerBlock) {
    const int tok = tok0 + vec;
    const bool ok = tok < a.n_tokens;
    const size_t off = (static_cast<size_t>(ok ? tok : 0) * a.num_heads + h) * kDim + part * kPerLane;
    float x[kPerLane];
    load_vec<float>(a.x + off, ok, x);
    if (kInverse) {
      blocks_apply_lane<true>(a.rot_kind, x, sm, part);
      if (wht) wht128_quad(x, part);
    } else {
      if (wht) wht128_quad(x, part);
      blocks_apply_lane<false>(a.rot_kind, x, sm, part);
    }
    if (ok) store_vec<float>(a.y + off, x);
  }
}

// ---------------------------------------------------------------------------
// Quantize + pack already-rotated fp32 vectors (flat [n][128] -> [n][48], [n]).
__global__ __launch_bounds__(kEncThreads) void quantize_pack_kernel(QuantArgs a) {
  const int part = threadIdx.x & 3;
  for (int64_t v0 = static_cast<int64_t>(blockIdx.x) * kVecPerBlock; v0 < a.n_vectors;
       v0 += static_cast<int64_t>(gridDim.x) * kVecPerBlock) {
    const int64_t v = v0 + (threadIdx.x >> 2);
    const bool ok = v < a.n_vectors;
    float y[kPerLane];
    load_vec<float>(a.y + (ok ? v : 0) * kDim + part * kPerLane, ok, y);
    uint32_t w[3];
    const float n = quantize_pack_lane(y, a.cb, w);
    if (ok) {
      uint32_t* dst = reinterpret_cast<uint32_t*>(a.codes + v * kRowBytes + part * 12);
      dst[0] = w[0];
      dst[1] = w[1];
      dst[2] = w[2];
      if (part == 0) a.norms[v] = n;
    }
  }
}

// ---------------------------------------------------------------------------
// Dequantize cache rows: x_hat = n Hn B^T c[code].
// grid = (token blocks, num_kv_heads, 2 [K, V])
template <typename T>
__global__ __launch_bounds__(kEncThreads) void dequant_kernel(DequantArgs a) {
  __shared__ __align__(16) float sm[kBlocks * 16];
  const int h = blockIdx.y;
  const bool is_v = blockIdx.z != 0;
  T* __restrict__ out = static_cast<T*>(is_v ? a.v_out : a.k_out);
  if (out == nullptr) return;   // uniform across the block
  load_head_matrices(rot_of_head(a.rot, a.rot_kind, h), a.rot_kind, sm);
  __syncthreads();
  const uint8_t* __restrict__ codes = is_v ? a.v_codes : a.k_codes;
  const float* __restrict__ norms = is_v ? a.v_norms : a.k_norms;
  const int part = threadIdx.x & 3;
  const int vec = threadIdx.x >> 2;
  for (int tok0 = blockIdx.x * kVecPerBlock; tok0 < a.n_tokens; tok0 += gridDim.x * kVecPerBlock) {
    const int tok = tok0 + vec;
    const bool ok = tok < a.n_tokens;
    const size_t row = static_cast<size_t>(h) * a.capacity + a.first_slot + (ok ? tok : 0);
    uint32_t w[3] = {0u, 0u, 0u};
    uint4 w4 = make_uint4(0u, 0u, 0u, 0u);
    const bool k4 = !is_v && a.k_bits == 4;
    float n = 0.f;
    if (ok) {
      n = norms[row];
      if (k4) {
        w4 = *reinterpret_cast<const uint4*>(codes + row * k_row_bytes(4) + part * 16);
      } else if (!is_v) {
        const uint32_t* src = reinterpret_cast<const uint32_t*>(codes + row * kRowBytes + part * 12);
        w[0] = src[0];
        w[1] = src[1];
        w[2] = src[2];
      } else {
        // dims 32p .. 32p+31 of this slot: 3 bits at 24 j + 3 r of its tile
        const uint32_t* tile = reinterpret_cast<const uint32_t*>(codes + (row / kTile) * kTileBytes);
        const int r = static_cast<int>(row & (kTile - 1));
        uint32_t c[kPerLane];
#pragma unroll
        for (int i = 0; i < kPerLane; ++i) {
          const int pos = 24 * (part * kPerLane + i) + 3 * r;
          const int wd = pos >> 5, off = pos & 31;
          const uint32_t lo = tile[wd];
          const uint32_t hi = off > 29 ? tile[wd + 1] : 0u;
          c[i] = __builtin_amdgcn_alignbit(hi, lo, off) & 7u;
        }
        pack32(c, w);
      }
    }
    float x[kPerLane];
    if (k4) {
      const uint32_t wd[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
      for (int i = 0; i < kPerLane; ++i) x[i] = centroid16((wd[i >> 3] >> (4 * (i & 7))) & 15u, a.cb);
    } else {
#pragma unroll
      for (int i = 0; i < kPerLane; ++i) x[i] = centroid(code_at(w, i), a.cb);
    }
    blocks_apply_lane<true>(a.rot_kind, x, sm, part);
    if (a.rot_kind == kRotWhtSo4) wht128_quad(x, part);
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) x[i] *= n;
    if (ok) store_vec<T>(out + (static_cast<size_t>(tok) * a.num_kv_heads + h) * kDim + part * kPerLane, x);
  }
}

// ------------------------------------------------------------- launchers ----
static int enc_grid_x(int64_t n_vectors_per_y, int64_t y_blocks) {
  // enough blocks to fill the chip several times over, each looping a few passes
  const int64_t need = (n_vectors_per_y + kVecPerBlock - 1) / kVecPerBlock;
  const int64_t target = (2048 + y_blocks - 1) / y_blocks;
  int64_t g = need < target ? need : target;
  if (g < 1) g = 1;
  return static_cast<int>(g);
}

hipError_t launch_append(const AppendArgs& a, bool f16, hipStream_t s) {
  if (a.n_tokens <= kRowAppendMax) {
    dim3 grid((a.n_tokens + 3) / 4, a.num_kv_heads, 2);
    if (f16)
      hipLaunchKernelGGL(append_row_kernel<_Float16>, grid, dim3(64), 0, s, a);
    else
      hipLaunchKernelGGL(append_row_kernel<float>, grid, dim3(64), 0, s, a);
    return hipGetLastError();
  }
  dim3 grid(enc_grid_x(a.n_tokens, 2LL * a.num_kv_heads), a.num_kv_heads, 2);
  const bool k4 = a.k_bits == 4, givens = a.rot_kind == kRotPlanar;
#define IQ_APPEND(T, K4, GV) hipLaunchKernelGGL((append_kernel<T, K4, GV>), grid, dim3(kEncThreads), 0, s, a)
  if (f16) {
    if (givens) {
      if (k4) IQ_APPEND(_Float16, true, true); else IQ_APPEND(_Float16, false, true);
    } else {
      if (k4) IQ_APPEND(_Float16, true, false); else IQ_APPEND(_Float16, false, false);
    }
  } else {
    if (givens) {
      if (k4) IQ_APPEND(float, true, true); else IQ_APPEND(float, false, true);
    } else {
      if (k4) IQ_APPEND(float, true, false); else IQ_APPEND(float, false, false);
    }
  }
#undef IQ_APPEND
  return hipGetLastError();
}

hipError_t launch_rotate(const RotateArgs& a, bool inverse, hipStream_t s) {
  dim3 grid(enc_grid_x(a.n_tokens, a.num_heads), a.num_heads, 1);
  if (inverse)
    hipLaunchKernelGGL(rotate_kernel<true>, grid, dim3(kEncThreads), 0, s, a);
  else
    hipLaunchKernelGGL(rotate_kernel<false>, grid, dim3(kEncThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_quantize_pack(const QuantArgs& a, hipStream_t s) {
  dim3 grid(enc_grid_x(a.n_vectors, 1), 1, 1);
  hipLaunchKernelGGL(quantize_pack_kernel, grid, dim3(kEncThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_dequant(const DequantArgs& a, bool f16, hipStream_t s) {
  dim3 grid(enc_grid_x(a.n_tokens, 2LL * a.num_kv_heads), a.num_kv_heads, 2);
  if (f16)
    hipLaunchKernelGGL(dequant_kernel<_Float16>, grid, dim3(kEncThreads), 0, s, a);
  else
    hipLaunchKernelGGL(dequant_kernel<float>, grid, dim3(kEncThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace iq
