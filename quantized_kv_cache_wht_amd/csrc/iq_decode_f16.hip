// Decode attention over a plain fp16 K/V cache: the baseline the packed
// cache is compared with, and the second half of the unfused path
// (iq_dequantize, then this). News article on RotaryQuant, section on memory
// savings versus speed: the fused packed kernels against the unfused version,
// and FP16 KV against IsoQuant.
//
//   s_{g,t} = scale log2(e) q_g . K_t,  o_g = sum_t 2^(s - m) V_t / sum_t 2^(s - m)
//
// Same split-K geometry, online softmax and merge as the packed decode
// (records in the model's basis, merged without a rotation). Per wave and
// per block of 32 tokens, on v_mfma_f32_16x16x32_f16:
//   * scores: two 16-token tiles x 4 k-steps of 32 dims; A = K rows straight
//     from memory (16 bytes per lane), B = the query split into fp16 hi
//     (columns g) and lo (columns g + 8), so the query keeps ~22 bits;
//   * PV: 8 tiles of 16 dims, K = the 32 tokens; A = weights (hi rows g, lo
//     rows g + 8), B = V. The MFMA wants one dim's 8 consecutive tokens per
//     lane, so each wave writes its V block to LDS transposed (dim-major,
//     rows padded to 72 bytes against bank conflicts) and reads it back.
#include "iq_decode_common.h"
#include "iq_decode_packed.h"

namespace iq {

namespace {

constexpr int kVtRow = 36;                  // halfwords per transposed V row (32 tokens + pad)
constexpr int kVtWave = kDim * kVtRow;      // halfwords per wave

struct F16Block {
  uint4 k[2][4];   // [tile][k-step]: 8 dims of one token
  uint4 v[8];      // [combo][token]: 8 dims of 4 tokens (see load_f16_block)
};

// K: tile T row n <-> token 8 (n / 4) + 4 T + n % 4, dims 32 kk + 8 q .. +7,
// so that score row 4 q + i of tile T is token 8 q + 4 T + i.
// V: combo c = lane + 64 j (j = 0, 1) covers tokens 4 (c % 8) .. +3, dims
// 8 (c / 8) .. +7; v[4 j + u] is token 4 (c % 8) + u.
__device__ __forceinline__ void load_f16_block(const F16DecodeArgs& a, const _Float16* kh, const _Float16* vh,
                                               int slot0, int lane, F16Block& d) {
  const int n = lane & 15, q = lane >> 4;
#pragma unroll
  for (int T = 0; T < 2; ++T) {
    const int tok = slot0 + 8 * (n >> 2) + 4 * T + (n & 3);
    const uint4* src = reinterpret_cast<const uint4*>(kh + static_cast<int64_t>(tok) * a.token_stride + 8 * q);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) d.k[T][kk] = src[4 * kk];
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = lane + 64 * j;
    const int tok = slot0 + 4 * (c & 7);
    const _Float16* base = vh + static_cast<int64_t>(tok) * a.token_stride + 8 * (c >> 3);
#pragma unroll
    for (int u = 0; u < 4; ++u) d.v[4 * j + u] = *reinterpret_cast<const uint4*>(base + u * a.token_stride);
  }
}

// Transposed store: Vt[dim][token], four tokens (8 bytes) per write.
__device__ __forceinline__ void store_vt(const F16Block& d, int lane, _Float16* vt) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = lane + 64 * j;
    const int t0 = 4 * (c & 7), d0 = 8 * (c >> 3);
    const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&d.v[4 * j + 0]);
    const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&d.v[4 * j + 1]);
    const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&d.v[4 * j + 2]);
    const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&d.v[4 * j + 3]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // halfword e of each token's 16 bytes: dword e / 2, high half when e is odd
      const int wd = e >> 1;
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;   // v_perm: pick the e-th halves
      const uint32_t lo = __builtin_amdgcn_perm(w1[wd], w0[wd], sel);   // tokens t0, t0 + 1
      const uint32_t hi = __builtin_amdgcn_perm(w3[wd], w2[wd], sel);   // tokens t0 + 2, t0 + 3
      *reinterpret_cast<uint2*>(vt + (d0 + e) * kVtRow + t0) = make_uint2(lo, hi);
    }
  }
}

template <int G>
struct F16Consts {
  const uint4* qop;      // this lane's query operand of k-step kk at qop[64 kk] (LDS)
  const uint4* qop_lo;   // G = 16: the lo halves
  float fscale;
  bool lo_lane;
  int rel_lo, rel_hi;
};

// Scores of the block's 32 tokens against the G queries: t[4 T + i] is token
// 8 q + 4 T + i (raw dot products of the normalised query, hi + lo columns).
template <int G>
__device__ __forceinline__ void f16_scores(const F16Block& cur, const F16Consts<G>& c, floatx4& d0, floatx4& d1) {
  constexpr bool kSplitN = (G <= 8);
  d0 = floatx4{0.f, 0.f, 0.f, 0.f};
  d1 = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    H8 ka, kb, qv;
    ka.u4 = cur.k[0][kk];
    kb.u4 = cur.k[1][kk];
    qv.u4 = c.qop[64 * kk];
    d0 = mfma16(ka.h, qv.h, d0);
    d1 = mfma16(kb.h, qv.h, d1);
    if (!kSplitN) {
      qv.u4 = c.qop_lo[64 * kk];
      d0 = mfma16(ka.h, qv.h, d0);
      d1 = mfma16(kb.h, qv.h, d1);
    }
  }
}

template <int G>
__device__ __forceinline__ void f16_softmax_pv(floatx4 d0, floatx4 d1, const _Float16* vt, int slot0, int lane,
                                               const F16Consts<G>& c, WaveState& st) {
  constexpr bool kSplitN = (G <= 8);
  const int n = lane & 15, q = lane >> 4;
  float t[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    t[i] = d0[i];
    t[4 + i] = d1[i];
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if (kSplitN) t[k] += dpp_row_ror8(t[k]);
    t[k] *= c.fscale;   // the score, log2 units
  }
  const bool full = slot0 >= c.rel_lo && slot0 + kBlk <= c.rel_hi;   // wave-uniform
  if (!full) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int rel = slot0 + 8 * q + k;
      t[k] = (rel >= c.rel_lo && rel < c.rel_hi) ? t[k] : -INFINITY;
    }
  }
  // ---- online softmax, reference raised lazily (weights stay <= 2^15: fp16-safe) ----
  float u = fmaxf(fmaxf(fmaxf(t[0], t[1]), fmaxf(t[2], t[3])), fmaxf(fmaxf(t[4], t[5]), fmaxf(t[6], t[7])));
  u = rows_reduce<true>(u);
  const bool bump = u > st.m + kWeightMaxLog2;
  if (__any(bump)) {
    const float m_new = bump ? u - kWeightRefLog2 : st.m;
    const float alpha = bump ? fast_exp2(st.m - m_new) : 1.f;
    st.l *= alpha;
    st.m = m_new;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int src = kSplitN ? ((4 * q + i) & 7) : (4 * q + i);
      const float ar = __shfl(alpha, src, 64);
#pragma unroll
      for (int d = 0; d < 8; ++d) st.acc[d][i] *= ar;
    }
  }
  const float mref = (st.m == -INFINITY) ? 0.f : st.m;
  // weights of tokens 8 q .. 8 q + 7 (this lane's A slots)
  H8 pa, pa_lo;
  float esum = 0.f;
#pragma unroll
  for (int k = 0; k < 8; k += 2) {
    const float e0 = fast_exp2(t[k] - mref), e1 = fast_exp2(t[k + 1] - mref);
    esum += e0 + e1;
    const float h0 = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, e0) & 0xffffe000u);
    const float h1 = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, e1) & 0xffffe000u);
    if (kSplitN) {
      pa.u[k >> 1] = __builtin_bit_cast(uint32_t, c.lo_lane ? __builtin_amdgcn_cvt_pkrtz(e0 - h0, e1 - h1)
                                                            : __builtin_amdgcn_cvt_pkrtz(h0, h1));
    } else {
      pa.u[k >> 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(h0, h1));
      pa_lo.u[k >> 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(e0 - h0, e1 - h1));
    }
  }
  st.l += esum;
  // ---- PV: B = V[tokens 8 q .. 8 q + 7][dim 16 dt + n] from the transposed block ----
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    const uint2* src = reinterpret_cast<const uint2*>(vt + (16 * dt + n) * kVtRow + 8 * q);
    H8 vb;
    vb.u2[0] = src[0];
    vb.u2[1] = src[1];
    st.acc[dt] = mfma16(pa.h, vb.h, st.acc[dt]);
    if (!kSplitN) st.acc[dt] = mfma16(pa_lo.h, vb.h, st.acc[dt]);
  }
}

// LDS of one fp16 split work-group.
template <int G>
struct F16Smem {
  static constexpr bool kSplitN = (G <= 8);
  static constexpr int kRows = kSplitN ? 2 * G : G;
  // per wave: the transposed V block during the loop, then the wave's accumulator rows
  _Float16 vts[kWaves][kVtWave];
  // query operand of k-step kk for lane 16 q + n: dims 32 kk + 8 q .. +7 of head
  // n & 7, hi halves in columns n < 8 and lo halves in n >= 8 (G = 16: hi in qop,
  // lo in qop_lo, column n = head n)
  uint4 qop[4][64];
  uint4 qop_lo[kSplitN ? 1 : 4][64];
  float orec[G][kDim];   // merged output before the forward rotation (deferred decode)
  float qmax[G];
  float wm[kWaves][G], wl[kWaves][G];
  static_assert(kRows * kDim * sizeof(float) <= kVtWave * sizeof(_Float16), "accumulators fit the V block");
};

// One split of the fp16 decode: work-group (h = KV head, s = sequence, split).
// Records go to split index a.rec_offset + split of a.rec_splits; with a.rot
// they are rotated forward (o' = R o) so that they merge with packed records.
template <int G>
__device__ __forceinline__ void f16_split(const F16DecodeArgs& a, F16Smem<G>& sm, int split) {
  constexpr bool kSplitN = F16Smem<G>::kSplitN;
  auto& qop = sm.qop;
  auto& qop_lo = sm.qop_lo;
  float* qmax = sm.qmax;
  auto& wm = sm.wm;
  auto& wl = sm.wl;
  auto& vts = sm.vts;
  const int h = blockIdx.x, s = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = lane & 15, q = lane >> 4;
  int start, len;
  const bool ok = seq_ok(a, s, &start, &len);
  const int base = start & ~(kBlk - 1);
  const int nblk = ok ? n_blocks(start, len) : 0;
  if (split >= live_splits(nblk, a.blocks_per_split, a.n_splits)) return;
  const int b_begin = split * a.blocks_per_split;
  const int b_end = split == a.n_splits - 1 ? nblk : min(nblk, b_begin + a.blocks_per_split);
  const _Float16* kh = a.k + static_cast<int64_t>(h) * a.head_stride + static_cast<int64_t>(base) * a.token_stride;
  const _Float16* vh = a.v + static_cast<int64_t>(h) * a.head_stride + static_cast<int64_t>(base) * a.token_stride;

  // query loads (16 lanes per head, 8 dims each) first, then the wave's first block
  const int pg = tid >> 4, pl = tid & 15;
  float xq[8], rp[16];
  if (tid < 16 * G) {
    const float4* src = reinterpret_cast<const float4*>(
        a.q + (static_cast<size_t>(s) * a.num_q_heads + h * G + pg) * kDim + 8 * pl);
    const float4 v0 = src[0], v1 = src[1];
    xq[0] = v0.x; xq[1] = v0.y; xq[2] = v0.z; xq[3] = v0.w; xq[4] = v1.x; xq[5] = v1.y; xq[6] = v1.z; xq[7] = v1.w;
    if (a.rot != nullptr) load_row_params(rot_of_head(a.rot, a.rot_kind, h), a.rot_kind, pl, rp);
  }
  int b = b_begin + wave;
  F16Block cur;
  load_f16_block(a, kh, vh, min(b, b_end - 1) * kBlk, lane, cur);   // unconditional: see the packed decode

  if (tid < 16 * G) {
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) mx = fmaxf(mx, fabsf(xq[i]));
    mx = fmaxf(mx, row_xor<8>(mx));
    mx = fmaxf(mx, row_xor<4>(mx));
    mx = fmaxf(mx, row_xor<2>(mx));
    mx = fmaxf(mx, row_xor<1>(mx));
    if (pl == 0) qmax[pg] = mx;
    const float inv = mx > 0.f ? 1.0f / mx : 0.f;
    H8 hi, lo;
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      const float x0 = (xq[i] * inv) * 128.0f, x1 = (xq[i + 1] * inv) * 128.0f;   // 2^7 q / max|q|
      const float h0 = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, x0) & 0xffffe000u);
      const float h1 = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, x1) & 0xffffe000u);
      hi.u[i >> 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(h0, h1));
      lo.u[i >> 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(x0 - h0, x1 - h1));
    }
    const int kk = pl >> 2, qq = pl & 3;   // dims 8 pl .. = k-step kk, lane group qq
    if (kSplitN) {
      qop[kk][16 * qq + pg] = hi.u4;
      qop[kk][16 * qq + pg + 8] = lo.u4;
    } else {
      qop[kk][16 * qq + pg] = hi.u4;
      qop_lo[kk][16 * qq + pg] = lo.u4;
    }
  }
  if (kSplitN && G < 8) {
    for (int idx = tid; idx < 4 * 64; idx += kDecThreads) {
      if (((idx & 15) & 7) >= G) qop[idx >> 6][idx & 63] = make_uint4(0u, 0u, 0u, 0u);
    }
  }
  __syncthreads();

  F16Consts<G> c;
  const int g = kSplitN ? (n & 7) : n;
  c.fscale = a.qscale * ((g < G ? qmax[g] : 0.f) * 0x1p-7f);
  c.qop = &qop[0][lane];
  c.qop_lo = &qop_lo[0][lane];
  c.lo_lane = kSplitN && n >= 8;
  c.rel_lo = start - base;
  c.rel_hi = start - base + len;
  _Float16* vt = vts[wave];

  WaveState st;
#pragma unroll
  for (int d = 0; d < 8; ++d) st.acc[d] = floatx4{0.f, 0.f, 0.f, 0.f};
  st.m = -INFINITY;
  st.l = 0.f;

  // per block: V to LDS and the scores from the K registers, then the next
  // block's loads go out into the same registers while softmax and PV run
  while (b < b_end) {
    store_vt(cur, lane, vt);
    floatx4 d0, d1;
    f16_scores<G>(cur, c, d0, d1);
    if (b + kWaves < b_end) load_f16_block(a, kh, vh, (b + kWaves) * kBlk, lane, cur);
    f16_softmax_pv<G>(d0, d1, vt, b * kBlk, lane, c, st);
    b += kWaves;
  }
  // Every accumulator element is read once (see the packed kernel's body:
  // with G < 4 some are never stored, and their registers must not be reused
  // while the MFMA writing them is in flight).
  {
    float sink = 0.f;
#pragma unroll
    for (int d = 0; d < 8; ++d) sink += (st.acc[d][0] + st.acc[d][1]) + (st.acc[d][2] + st.acc[d][3]);
    asm volatile("" ::"v"(sink));
  }

  // ---- per-wave totals ----
  float l_run = st.l;
  l_run = rows_reduce<false>(l_run);
  if (q == 0 && n < G) {
    wm[wave][n] = st.m;
    wl[wave][n] = l_run;
  }
  float* wo = reinterpret_cast<float*>(vt);   // [kRows][kDim], this wave's region
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = 4 * q + i;
    const int gr = kSplitN ? (m & 7) : m;
    const int row = (kSplitN && m >= 8) ? G + gr : gr;
    if (gr < G) {
#pragma unroll
      for (int d = 0; d < 8; ++d) wo[row * kDim + 16 * d + n] = st.acc[d][i];
    }
  }
  __syncthreads();
  // ---- merge the waves (and the hi/lo rows) into this split's records ----
  float* rec0 = a.ws + ((static_cast<size_t>(s) * a.num_q_heads + h * G) * a.rec_splits + a.rec_offset + split) * kRec;
  const size_t head_stride = static_cast<size_t>(a.rec_splits) * kRec;
  const bool rotate = a.rot != nullptr;
  for (int idx = tid; idx < G * kDim; idx += kDecThreads) {
    const int gr = idx >> 7, j = idx & (kDim - 1);
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, wm[w][gr]);
    float o = 0.f;
    if (mx != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float* wow = reinterpret_cast<const float*>(vts[w]);
        const float v = kSplitN ? wow[gr * kDim + j] + wow[(G + gr) * kDim + j] : wow[gr * kDim + j];
        o += fast_exp2(wm[w][gr] - mx) * v;
      }
    }
    if (rotate) {
      sm.orec[gr][j] = o;
    } else {
      rec0[gr * head_stride + 4 + j] = o;
    }
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
  if (rotate) {
    // o' = R o per query head, 16 lanes per head (R linear: the unnormalised sum rotates)
    __syncthreads();
    if (tid < 16 * G) {
      float x[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = sm.orec[pg][8 * pl + i];
      float m[32];
      so4_matrices_row(a.rot_kind, rp, m);
      if (a.rot_kind == kRotWhtSo4) wht128_row(x, pl);
      blocks_apply_row<false>(a.rot_kind, x, m);
      float4* dst = reinterpret_cast<float4*>(rec0 + pg * head_stride + 4 + 8 * pl);
      dst[0] = make_float4(x[0], x[1], x[2], x[3]);
      dst[1] = make_float4(x[4], x[5], x[6], x[7]);
    }
  }
}

template <int G>
__global__ __launch_bounds__(kDecThreads, 2) void decode_f16_split_kernel(F16DecodeArgs a) {
  __shared__ F16Smem<G> sm;
  f16_split<G>(a, sm, blockIdx.z);
}

// Deferred quantization (RotorQuant page, deferred-quantization strategy;
// essay section "延迟量化"): the prompt's K/V stay fp16, generated tokens are
// packed. One launch holds both parts' splits, the prefix's first (grid z <
// pre.n_splits); their records meet in one merge.
template <int G, int KB>
__global__ __launch_bounds__(kDecThreads, 2) void decode_deferred_split_kernel(F16DecodeArgs pre, DecodeArgs suf) {
  __shared__ union {
    F16Smem<G> f;
    struct {
      PackedSmem<G, KB> p;
      StageMem<G, KB> stg;
    } k;
  } sm;
  const int z = blockIdx.z;
  if (z < pre.n_splits) {
    f16_split<G>(pre, sm.f, z);
  } else {
    touch_codebook_words<KB>(suf.cb);
    packed_split<G, KB>(suf, sm.k.p, sm.k.stg, z - pre.n_splits);
  }
}

}  // namespace

template <int KB>
static hipError_t launch_deferred_split(const F16DecodeArgs& pre, const DecodeArgs& suf, hipStream_t st) {
  dim3 grid(suf.num_kv_heads, suf.n_seqs, pre.n_splits + suf.n_splits);
  switch (suf.group) {
    case 1: hipLaunchKernelGGL((decode_deferred_split_kernel<1, KB>), grid, dim3(kDecThreads), 0, st, pre, suf); break;
    case 2: hipLaunchKernelGGL((decode_deferred_split_kernel<2, KB>), grid, dim3(kDecThreads), 0, st, pre, suf); break;
    case 4: hipLaunchKernelGGL((decode_deferred_split_kernel<4, KB>), grid, dim3(kDecThreads), 0, st, pre, suf); break;
    case 8: hipLaunchKernelGGL((decode_deferred_split_kernel<8, KB>), grid, dim3(kDecThreads), 0, st, pre, suf); break;
    case 16:
      hipLaunchKernelGGL((decode_deferred_split_kernel<16, KB>), grid, dim3(kDecThreads), 0, st, pre, suf);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode_deferred(const F16DecodeArgs& pre, const DecodeArgs& suf, hipStream_t st) {
  const hipError_t le = suf.k_bits == 4 ? launch_deferred_split<4>(pre, suf, st) : launch_deferred_split<3>(pre, suf, st);
  if (le != hipSuccess) return le;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  MergeArgs m{suf.rot_kind, suf.rot, suf.out, suf.ws, suf.n_seqs, suf.num_q_heads, suf.group, suf.rec_splits, 2, -1, {}};
  m.seg[0] = MergeSegment{pre.seq_start, pre.seq_len, pre.capacity, pre.max_seq_len, pre.blocks_per_split,
                          pre.n_splits, 0};
  m.seg[1] = MergeSegment{suf.seq_start, suf.seq_len, suf.capacity, suf.max_seq_len, suf.blocks_per_split,
                          suf.n_splits, pre.n_splits};
  return launch_merge(m, st);
}

hipError_t launch_decode_f16(const F16DecodeArgs& a, hipStream_t st) {
  dim3 grid(a.num_kv_heads, a.n_seqs, a.n_splits);
  switch (a.group) {
    case 1: hipLaunchKernelGGL(decode_f16_split_kernel<1>, grid, dim3(kDecThreads), 0, st, a); break;
    case 2: hipLaunchKernelGGL(decode_f16_split_kernel<2>, grid, dim3(kDecThreads), 0, st, a); break;
    case 4: hipLaunchKernelGGL(decode_f16_split_kernel<4>, grid, dim3(kDecThreads), 0, st, a); break;
    case 8: hipLaunchKernelGGL(decode_f16_split_kernel<8>, grid, dim3(kDecThreads), 0, st, a); break;
    case 16: hipLaunchKernelGGL(decode_f16_split_kernel<16>, grid, dim3(kDecThreads), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  MergeArgs m{kRotWhtSo4, nullptr, a.out, a.ws, a.n_seqs, a.num_q_heads, a.group, a.rec_splits, 1, -1, {}};
  m.seg[0] = MergeSegment{a.seq_start, a.seq_len, a.capacity, a.max_seq_len, a.blocks_per_split, a.n_splits, 0};
  return launch_merge(m, st);
}

}  // namespace iq
