// Decode attention straight from the packed 3-bit cache on the matrix cores
// (split-K over the context, cross-workgroup softmax merge).
//
// What is computed (news article on RotaryQuant, section on attention over
// packed data; arXiv 2608.08081 abstract; zhichai.net essay's attention
// formula softmax(Q K^T / sqrt(d)) V):
//   q'_g    = R q_g                                          (query rotated once)
//   s_{g,t} = scale log2(e) nK_t sum_j q'_{g,j} c[kcode_{t,j}] (score in the rotated domain)
//   o'_g    = sum_t 2^(s_{g,t} - m) nV_t c[vcode_t] / sum_t 2^(s_{g,t} - m)
//   out_g   = R^-1 o'_g = Hn B^T o'_g                          (one inverse rotation)
// Full-precision K and V are never formed in memory.
//
// Contractions on MFMA (v_mfma_f32_16x16x32_f16, fp32 accumulate). Per wave
// and per block of 32 cache slots:
//   * scores: two 16-token tiles x 4 k-steps; A = centroids of the packed K
//     codes, B = the rotated queries. For G <= 8 the 16 B columns hold the
//     query split into fp16 hi (columns g) and lo (columns g + 8) parts and
//     one DPP row rotation adds the two halves, so the query keeps ~22 bits.
//   * PV: A = softmax weights times V norms, again split hi (rows g) / lo
//     (rows g + 8); B = centroids of the packed V codes; 8 column tiles of 16
//     dims, K = the 32 tokens.
// Centroids enter the MFMA as fp16(alpha c) with a scale alpha chosen so that
// all eight are within 2e-5 relative of the float32 codebook; 1/alpha is
// applied to the fp32 results.
//
// Code -> fp16 pair conversion: a 64-entry table (all pairs of codes) in LDS,
// replicated 32 times so each lane of a half-wave reads its own bank.
//
// Layout of the cache (see include/iq.h): K rows of 48 bytes per token; V in
// tiles of 8 slots, dim-major, so the 8 codes one PV operand needs (one dim,
// 8 consecutive tokens) are 24 adjacent bits.
//
// Softmax reference: m tracks max_t(s_t + max(0, log2 nV_t)) (an exponent
// bound), so p_t nV_t <= 1 and the fp16 operand never overflows.
#include <math.h>

#include "iq_device.h"
#include "iq_launch.h"

namespace iq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

union H8 {
  half8 h;
  uint32_t u[4];
};

constexpr int kDecThreads = 256;
constexpr int kWaves = kDecThreads / 64;
constexpr int kBlk = 32;             // cache slots per wave iteration
constexpr int kRec = 132;            // floats per partial record: m, l, 2 pad, o[128]
constexpr int kTargetBlocks = 512;   // split-K occupancy target (work-groups)
constexpr int kMinBlocksPerSplit = 8;
constexpr int kMaxSplits = 2048;
constexpr int kLutEntries = 64;      // all pairs of 3-bit codes
constexpr int kLutCopies = 16;       // one per lane of a 16-lane group (8-byte entries)

// The pair table: entry p holds {hi(c[p&7]) | hi(c[p>>3]) << 16, lo(...) | lo(...) << 16}.
struct Operand {
  half8 hi, lo;
};

__device__ __forceinline__ bool seq_ok(const DecodeArgs& a, int s, int* start, int* len) {
  const int st = a.seq_start[s];
  const int ln = a.seq_len[s];
  *start = st;
  *len = ln;
  return st >= 0 && ln >= 0 && ln <= a.max_seq_len && static_cast<int64_t>(st) + ln <= a.capacity;
}

// 32-slot blocks covering [start, start + len) from the 32-aligned base.
__device__ __forceinline__ int n_blocks(int start, int len) {
  return len > 0 ? ((start - (start & ~(kBlk - 1)) + len + kBlk - 1) / kBlk) : 0;
}

__device__ __forceinline__ floatx4 mfma16(const half8& a, const half8& b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float dpp_row_ror8(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xF, 0xF, false));
}

// Operand (hi and lo halves) for the 8 codes at bits BIT .. BIT+23 of w:
// four code pairs, each one 8-byte table read.
template <int BIT, int N>
__device__ __forceinline__ Operand pair_operand(const uint32_t (&w)[N], const uint2* __restrict__ lut, uint32_t l15) {
  H8 hi, lo;
  const uint2 e0 = lut[(field6<BIT + 0>(w) << 4) | l15];
  const uint2 e1 = lut[(field6<BIT + 6>(w) << 4) | l15];
  const uint2 e2 = lut[(field6<BIT + 12>(w) << 4) | l15];
  const uint2 e3 = lut[(field6<BIT + 18>(w) << 4) | l15];
  hi.u[0] = e0.x; hi.u[1] = e1.x; hi.u[2] = e2.x; hi.u[3] = e3.x;
  lo.u[0] = e0.y; lo.u[1] = e1.y; lo.u[2] = e2.y; lo.u[3] = e3.y;
  return Operand{hi.h, lo.h};
}

// A operand of the score MFMA for k-step KAPPA: codes of dims 32q + 8 KAPPA .. +7,
// bits 24 KAPPA .. +23 of the lane's 96 K bits.
template <int KAPPA>
__device__ __forceinline__ Operand k_operand(const uint32_t (&kw)[3], const uint2* __restrict__ lut, uint32_t l15) {
  return pair_operand<24 * KAPPA>(kw, lut, l15);
}

// B operand of the PV MFMA for column tile D: the 8 tokens of dim 8n + D,
// bits 24 D .. +23 of the lane's 192 V bits.
template <int D>
__device__ __forceinline__ Operand v_operand(const uint32_t (&vw)[6], const uint2* __restrict__ lut, uint32_t l15) {
  return pair_operand<24 * D>(vw, lut, l15);
}

template <int G>
__global__ __launch_bounds__(kDecThreads) void decode_split_kernel(DecodeArgs a) {
  constexpr bool kSplitN = (G <= 8);   // hi/lo halves share one MFMA (columns / rows g and g+8)
  __shared__ uint2 lut[kLutEntries * kLutCopies];
  __shared__ __align__(16) float qs[G][kDim];
  __shared__ float qmax[G];
  __shared__ __align__(16) float sm[kBlocks * 16];
  __shared__ float wm[kWaves][G], wl[kWaves][G], mfin[G], lfin[G];
  __shared__ __align__(16) float wo[kWaves][G][kDim];

  const int split = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = lane & 15, q = lane >> 4;
  const uint32_t l15 = lane & 15;
  int start, len;
  const bool ok = seq_ok(a, s, &start, &len);
  const int base = start & ~(kBlk - 1);
  const int nblk = ok ? n_blocks(start, len) : 0;
  const int b_begin = split * a.blocks_per_split;
  const int b_end = min(nblk, b_begin + a.blocks_per_split);

  // ---- prologue: code-pair table, SO(4) matrices, rotated queries ----
  for (int i = tid; i < kLutEntries * kLutCopies; i += kDecThreads) {
    const uint32_t p = static_cast<uint32_t>(i) >> 4;
    lut[i] = make_uint2(centroid_f16<false>(p & 7u, a.cb) | (centroid_f16<false>(p >> 3, a.cb) << 16),
                        centroid_f16<true>(p & 7u, a.cb) | (centroid_f16<true>(p >> 3, a.cb) << 16));
  }
  load_head_matrices(a.rot + static_cast<size_t>(h) * kBlocks * 8, sm);
  __syncthreads();
  if (tid < 4 * G) {
    const int g = tid >> 2, part = tid & 3;
    float x[kPerLane];
    const float* src = a.q + (static_cast<size_t>(s) * a.num_q_heads + h * G + g) * kDim + part * kPerLane;
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) x[i] = src[i];
    wht128_quad(x, part);
    so4_apply_lane<false>(x, sm, part);
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
      qs[g][part * kPerLane + i] = x[i];
      mx = fmaxf(mx, fabsf(x[i]));
    }
    mx = fmaxf(mx, dpp_f32<kQuadXor1>(mx));
    mx = fmaxf(mx, dpp_f32<kQuadXor2>(mx));
    if (part == 0) qmax[g] = mx;
  }
  __syncthreads();

  // ---- per-lane constants: query operands, score scale ----
  const int g = kSplitN ? (n & 7) : n;     // head of this lane's score column / P row
  const bool gvalid = g < G;
  const float qm = gvalid ? qmax[g] : 0.f;
  const float inv_qm = qm > 0.f ? 1.0f / qm : 0.f;
  const float fscale = a.qscale * qm * a.cb.inv_alpha;
  H8 qb[4], qb_lo[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float x = gvalid ? qs[g][32 * q + 8 * kk + i] * inv_qm : 0.f;
      const _Float16 hh = static_cast<_Float16>(x);
      const _Float16 ll = static_cast<_Float16>(x - static_cast<float>(hh));
      if (kSplitN) {
        qb[kk].h[i] = (n < 8) ? hh : ll;
      } else {
        qb[kk].h[i] = hh;
        qb_lo[kk].h[i] = ll;
      }
    }
  }

  floatx4 acc[8];
#pragma unroll
  for (int d = 0; d < 8; ++d) acc[d] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const size_t slot_base = static_cast<size_t>(h) * a.capacity + base;   // cache row of block 0, slot 0
  const int rel_lo = start - base, rel_hi = start - base + len;          // valid slots relative to base
  // A-operand rows of the two score tiles: tile T row r <-> token 8 (r/4) + 4 T + r % 4
  const int tok_a0 = 8 * (n >> 2) + (n & 3);

  for (int b = b_begin + wave; b < b_end; b += kWaves) {
    const int slot0 = b * kBlk;
    // ---- loads ----
    uint32_t kw0[3], kw1[3], vw[6];
    {
      const uint32_t* k0 = reinterpret_cast<const uint32_t*>(a.k_codes + (slot_base + slot0 + tok_a0) * kRowBytes + 12 * q);
      const uint32_t* k1 = reinterpret_cast<const uint32_t*>(a.k_codes + (slot_base + slot0 + tok_a0 + 4) * kRowBytes + 12 * q);
      kw0[0] = k0[0]; kw0[1] = k0[1]; kw0[2] = k0[2];
      kw1[0] = k1[0]; kw1[1] = k1[1]; kw1[2] = k1[2];
      const uint2* vp = reinterpret_cast<const uint2*>(a.v_codes + ((slot_base + slot0) / kTile + q) * kTileBytes + 24 * n);
      const uint2 v0 = vp[0], v1 = vp[1], v2 = vp[2];
      vw[0] = v0.x; vw[1] = v0.y; vw[2] = v1.x; vw[3] = v1.y; vw[4] = v2.x; vw[5] = v2.y;
    }
    const float4* nkp = reinterpret_cast<const float4*>(a.k_norms + slot_base + slot0 + 8 * q);
    const float4* nvp = reinterpret_cast<const float4*>(a.v_norms + slot_base + slot0 + 8 * q);
    const float4 nk0 = nkp[0], nk1 = nkp[1], nv0 = nvp[0], nv1 = nvp[1];
    const float nk[8] = {nk0.x, nk0.y, nk0.z, nk0.w, nk1.x, nk1.y, nk1.z, nk1.w};
    const float nv[8] = {nv0.x, nv0.y, nv0.z, nv0.w, nv1.x, nv1.y, nv1.z, nv1.w};

    // ---- scores: D_T[i] = row 4q + i of tile T = token 8q + 4T + i, column n ----
    floatx4 d0 = {0.f, 0.f, 0.f, 0.f}, d1 = {0.f, 0.f, 0.f, 0.f};
    // (c_hi + c_lo)(q_hi + q_lo) without the c_lo q_lo term (~2^-22)
#define IQ_SCORE(KAPPA)                                                      \
    {                                                                        \
      const Operand ka = k_operand<KAPPA>(kw0, lut, l15);                    \
      const Operand kb = k_operand<KAPPA>(kw1, lut, l15);                    \
      d0 = mfma16(ka.hi, qb[KAPPA].h, d0);                                   \
      d1 = mfma16(kb.hi, qb[KAPPA].h, d1);                                   \
      d0 = mfma16(ka.lo, qb[KAPPA].h, d0);                                   \
      d1 = mfma16(kb.lo, qb[KAPPA].h, d1);                                   \
      if (!kSplitN) {                                                        \
        d0 = mfma16(ka.hi, qb_lo[KAPPA].h, d0);                              \
        d1 = mfma16(kb.hi, qb_lo[KAPPA].h, d1);                              \
      }                                                                      \
    }
    IQ_SCORE(0) IQ_SCORE(1) IQ_SCORE(2) IQ_SCORE(3)
#undef IQ_SCORE
    float sv[8];
    bool valid[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[i] = d0[i];
      sv[4 + i] = d1[i];
    }
    float mloc = -INFINITY, nvmax = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (kSplitN) sv[k] += dpp_row_ror8(sv[k]);
      const int rel = slot0 + 8 * q + k;
      valid[k] = rel >= rel_lo && rel < rel_hi;
      sv[k] = valid[k] ? sv[k] * fscale * nk[k] : -INFINITY;
      mloc = fmaxf(mloc, sv[k]);
      nvmax = fmaxf(nvmax, valid[k] ? nv[k] : 0.f);
    }
    // ---- online softmax (reference m bounds s + log2 nV) ----
    const int ex = __builtin_amdgcn_frexp_expf(nvmax);
    float u = mloc + (ex > 0 ? static_cast<float>(ex) : 0.f);
    u = fmaxf(u, __shfl_xor(u, 16, 64));
    u = fmaxf(u, __shfl_xor(u, 32, 64));
    const float m_new = fmaxf(m_run, u);
    const float mref = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2f(m_run - mref);
    float esum = 0.f, pv[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float e = exp2f(sv[k] - mref);
      esum += e;
      pv[k] = (valid[k] && gvalid) ? e * nv[k] : 0.f;
    }
    l_run = l_run * alpha + esum;
    m_run = m_new;
    if (__any(alpha != 1.0f)) {
      // accumulator rows 4q + i belong to head (4q + i) mod 8 (or 4q + i when G = 16)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int src = kSplitN ? ((4 * q + i) & 7) : (4 * q + i);
        const float ar = __shfl(alpha, src, 64);
#pragma unroll
        for (int d = 0; d < 8; ++d) acc[d][i] *= ar;
      }
    }
    // ---- PV: A row n holds weights of head g for tokens 8q .. 8q+7 ----
    H8 pa, pa_lo;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const _Float16 hh = static_cast<_Float16>(pv[k]);
      const _Float16 ll = static_cast<_Float16>(pv[k] - static_cast<float>(hh));
      if (kSplitN) {
        pa.h[k] = (n < 8) ? hh : ll;
      } else {
        pa.h[k] = hh;
        pa_lo.h[k] = ll;
      }
    }
#define IQ_PV(D)                                              \
    {                                                         \
      const Operand vb = v_operand<D>(vw, lut, l15);          \
      acc[D] = mfma16(pa.h, vb.hi, acc[D]);                   \
      acc[D] = mfma16(pa.h, vb.lo, acc[D]);                   \
      if (!kSplitN) acc[D] = mfma16(pa_lo.h, vb.hi, acc[D]);  \
    }
    IQ_PV(0) IQ_PV(1) IQ_PV(2) IQ_PV(3) IQ_PV(4) IQ_PV(5) IQ_PV(6) IQ_PV(7)
#undef IQ_PV
  }

  // ---- per-wave totals ----
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  if (kSplitN) {
#pragma unroll
    for (int d = 0; d < 8; ++d)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[d][i] += __shfl_xor(acc[d][i], 32, 64);   // hi rows + lo rows
  }
  if (q == 0 && n < G) {
    wm[wave][n] = m_run;
    wl[wave][n] = l_run;
  }
  if (!kSplitN || q < 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int gr = 4 * q + i;
      if (gr < G) {
#pragma unroll
        for (int d = 0; d < 8; ++d) wo[wave][gr][8 * n + d] = acc[d][i];
      }
    }
  }
  __syncthreads();
  // ---- merge the waves ----
  for (int idx = tid; idx < G * kDim; idx += kDecThreads) {
    const int gr = idx >> 7, j = idx & (kDim - 1);
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, wm[w][gr]);
    float o = 0.f;
    if (mx != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) o += exp2f(wm[w][gr] - mx) * wo[w][gr][j];
    }
    wo[0][gr][j] = o * a.cb.inv_alpha;   // the PV operand carried alpha * c
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
    mfin[tid] = mx;
    lfin[tid] = l;
  }
  __syncthreads();
  // ---- rotate back (linear, so the unnormalised sum can be rotated) and store ----
  if (tid < 4 * G) {
    const int gr = tid >> 2, part = tid & 3;
    float x[kPerLane];
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) x[i] = wo[0][gr][part * kPerLane + i];
    so4_apply_lane<true>(x, sm, part);
    wht128_quad(x, part);
    float* rec = a.ws + ((static_cast<size_t>(s) * a.num_q_heads + h * G + gr) * a.n_splits + split) * kRec;
#pragma unroll
    for (int i = 0; i < kPerLane; i += 4)
      *reinterpret_cast<float4*>(rec + 4 + part * kPerLane + i) = make_float4(x[i], x[i + 1], x[i + 2], x[i + 3]);
    if (part == 0) *reinterpret_cast<float4*>(rec) = make_float4(mfin[gr], lfin[gr], 0.f, 0.f);
  }
}

// Merge the splits of one (sequence, query head, 32-dim chunk):
// out_j = sum_s 2^(m_s - M) o_{s,j} / sum_s 2^(m_s - M) l_s.
constexpr int kMergeThreads = 256;
constexpr int kMergeChunk = 32;

__global__ __launch_bounds__(kMergeThreads) void decode_merge_kernel(DecodeArgs a) {
  __shared__ float wts[kMaxSplits];
  __shared__ float red[kMergeThreads / kMergeChunk][kMergeChunk];
  __shared__ float rmax[kMergeThreads / 64], rsum[kMergeThreads / 64];
  const int chunk = blockIdx.x, qh = blockIdx.y, s = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int start, len;
  const bool ok = seq_ok(a, s, &start, &len);
  float* out = a.out + (static_cast<size_t>(s) * a.num_q_heads + qh) * kDim + chunk * kMergeChunk;
  if (!ok || len == 0) {
    if (tid < kMergeChunk) out[tid] = ok ? 0.f : NAN;
    return;   // uniform
  }
  const int used = (n_blocks(start, len) + a.blocks_per_split - 1) / a.blocks_per_split;
  const float* rec = a.ws + (static_cast<size_t>(s) * a.num_q_heads + qh) * a.n_splits * kRec;
  float mx = -INFINITY;
  for (int k = tid; k < used; k += kMergeThreads) mx = fmaxf(mx, rec[static_cast<size_t>(k) * kRec]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  if (lane == 0) rmax[wave] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(rmax[0], rmax[1]), fmaxf(rmax[2], rmax[3]));
  float l = 0.f;
  for (int k = tid; k < used; k += kMergeThreads) {
    const float* r = rec + static_cast<size_t>(k) * kRec;
    const float w = exp2f(r[0] - mx);
    wts[k] = w;
    l += w * r[1];
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) l += __shfl_xor(l, o, 64);
  if (lane == 0) rsum[wave] = l;
  __syncthreads();
  l = rsum[0] + rsum[1] + rsum[2] + rsum[3];
  const int j = tid & (kMergeChunk - 1), part = tid / kMergeChunk;
  float acc = 0.f;
  for (int k = part; k < used; k += kMergeThreads / kMergeChunk)
    acc += wts[k] * rec[static_cast<size_t>(k) * kRec + 4 + chunk * kMergeChunk + j];
  red[part][j] = acc;
  __syncthreads();
  if (tid < kMergeChunk) {
    float t = 0.f;
#pragma unroll
    for (int p = 0; p < kMergeThreads / kMergeChunk; ++p) t += red[p][tid];
    out[tid] = t / l;
  }
}

void decode_plan(int32_t n_seqs, int32_t num_kv_heads, int32_t max_seq_len, int32_t* blocks_per_split,
                 int32_t* n_splits) {
  const int64_t blocks = (static_cast<int64_t>(max_seq_len) + 2 * kBlk - 2) / kBlk;   // worst-case alignment
  const int64_t pairs = static_cast<int64_t>(n_seqs > 0 ? n_seqs : 1) * (num_kv_heads > 0 ? num_kv_heads : 1);
  const int64_t want_splits = (kTargetBlocks + pairs - 1) / pairs;
  int64_t bps = (blocks + want_splits - 1) / want_splits;
  if (bps < kMinBlocksPerSplit) bps = kMinBlocksPerSplit;
  int64_t ns = (blocks + bps - 1) / bps;
  if (ns > kMaxSplits) {
    bps = (blocks + kMaxSplits - 1) / kMaxSplits;
    ns = (blocks + bps - 1) / bps;
  }
  if (ns < 1) ns = 1;
  *blocks_per_split = static_cast<int32_t>(bps);
  *n_splits = static_cast<int32_t>(ns);
}

size_t decode_workspace_floats(int32_t n_seqs, int32_t num_q_heads, int32_t n_splits) {
  return static_cast<size_t>(n_seqs) * num_q_heads * n_splits * kRec;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) {
  dim3 grid(a.n_splits, a.num_kv_heads, a.n_seqs);
  switch (a.group) {
    case 1: hipLaunchKernelGGL(decode_split_kernel<1>, grid, dim3(kDecThreads), 0, st, a); break;
    case 2: hipLaunchKernelGGL(decode_split_kernel<2>, grid, dim3(kDecThreads), 0, st, a); break;
    case 4: hipLaunchKernelGGL(decode_split_kernel<4>, grid, dim3(kDecThreads), 0, st, a); break;
    case 8: hipLaunchKernelGGL(decode_split_kernel<8>, grid, dim3(kDecThreads), 0, st, a); break;
    case 16: hipLaunchKernelGGL(decode_split_kernel<16>, grid, dim3(kDecThreads), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_merge_kernel, dim3(kDim / kMergeChunk, a.num_q_heads, a.n_seqs), dim3(kMergeThreads), 0,
                     st, a);
  return hipGetLastError();
}

}  // namespace iq
