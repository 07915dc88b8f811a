// Decode attention straight from the packed 3-bit cache (split-K over the
// context, cross-workgroup softmax merge, one inverse rotation at the end).
//
// What is computed (news article on RotaryQuant, section on attention over
// packed data; arXiv 2608.08081 abstract; zhichai.net essay's attention
// formula softmax(Q K^T / sqrt(d)) V):
//   q'_g   = R q_g * scale * log2(e)                        (query rotated once)
//   s_{g,t} = nK_t * sum_j q'_{g,j} c[kcode_{t,j}]          (score in the rotated domain)
//   o'_g   = sum_t 2^(s_{g,t} - m) nV_t c[vcode_t] / sum_t 2^(s_{g,t} - m)
//   out_g  = R^-1 o'_g = Hn B^T o'_g                         (one inverse rotation)
// K and V are never expanded to full precision in memory.
//
// Kernel A (split): grid (split, kv head, seq), 256 threads. One block owns
// one KV head of one sequence over a token range and serves all G query heads
// of that KV head, so every packed row is read once per (token, KV head).
// Kernel B (merge): grid (q head, seq); combines the per-split (m, l, o')
// partials and applies the inverse rotation.
#include <math.h>

#include "iq_device.h"
#include "iq_launch.h"

namespace iq {

constexpr int kDecThreads = 256;
constexpr int kChunk = 256;          // tokens per pass (one per thread in the score phase)
constexpr int kRec = 132;            // floats per partial record: m, l, 2 pad, o'[128]
constexpr int kTargetBlocks = 1024;  // split-K occupancy target

__device__ __forceinline__ bool seq_ok(const DecodeArgs& a, int s, int* start, int* len) {
  const int st = a.seq_start[s];
  const int ln = a.seq_len[s];
  *start = st;
  *len = ln;
  return st >= 0 && ln >= 0 && ln <= a.max_seq_len && static_cast<int64_t>(st) + ln <= a.capacity;
}

template <int G>
__global__ __launch_bounds__(kDecThreads) void decode_split_kernel(DecodeArgs a) {
  constexpr int NG = (G + 1) / 2;      // query heads per thread in the PV phase
  __shared__ __align__(16) float qs[G][kDim];
  __shared__ __align__(16) float sc[G][kChunk];
  __shared__ __align__(16) uint32_t vbuf[kChunk][12];
  __shared__ float vn[kChunk];
  __shared__ float sm[kBlocks * 16];
  __shared__ float ctab[8];
  __shared__ float m_run[G], l_run[G], alpha[G];

  const int split = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
  const int tid = threadIdx.x;
  int start, len;
  const bool ok = seq_ok(a, s, &start, &len);
  const int t_begin = split * a.split_len;
  const int t_end = ok ? min(len, t_begin + a.split_len) : 0;

  // ---- prologue: rotate the G queries of this KV head ----
  load_head_matrices(a.rot + static_cast<size_t>(h) * kBlocks * 8, sm);
  if (tid < 8) ctab[tid] = centroid(static_cast<uint32_t>(tid), a.cb);
  if (tid < G) {
    m_run[tid] = -INFINITY;
    l_run[tid] = 0.f;
  }
  __syncthreads();
  if (tid < 4 * G) {
    const int g = tid >> 2, part = tid & 3;
    float x[kPerLane];
    const float* src = a.q + (static_cast<size_t>(s) * a.num_q_heads + h * G + g) * kDim + part * kPerLane;
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) x[i] = src[i];
    wht128_quad(x, part);
    so4_apply_lane<false>(x, sm, part);
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) qs[g][part * kPerLane + i] = x[i] * a.qscale;
  }

  // PV-phase ownership: dim j, query heads g = gh + 2i
  const int j = tid & (kDim - 1);
  const int gh = tid >> 7;
  float acc[NG];
#pragma unroll
  for (int i = 0; i < NG; ++i) acc[i] = 0.f;

  const size_t row0 = static_cast<size_t>(h) * a.capacity + start;
  for (int c0 = t_begin; c0 < t_end; c0 += kChunk) {
    const int n_valid = min(kChunk, t_end - c0);
    __syncthreads();   // previous chunk fully consumed (and prologue done)
    // ---- score phase: one token per thread ----
    {
      const bool valid = tid < n_valid;
      float sg[G];
#pragma unroll
      for (int g = 0; g < G; ++g) sg[g] = 0.f;
      if (valid) {
        const size_t row = row0 + c0 + tid;
        const uint4* kp = reinterpret_cast<const uint4*>(a.k_codes + row * kRowBytes);
        const uint4* vp = reinterpret_cast<const uint4*>(a.v_codes + row * kRowBytes);
        const uint4 k0 = kp[0], k1 = kp[1], k2 = kp[2];
        const uint4 v0 = vp[0], v1 = vp[1], v2 = vp[2];
        const float kn = a.k_norms[row];
        vn[tid] = a.v_norms[row];
        const uint32_t kw[12] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w, k2.x, k2.y, k2.z, k2.w};
        const uint32_t vw[12] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w, v2.x, v2.y, v2.z, v2.w};
#pragma unroll
        for (int i = 0; i < 12; ++i) vbuf[tid][i] = vw[i];
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) {
          const uint32_t w[3] = {kw[3 * grp], kw[3 * grp + 1], kw[3 * grp + 2]};
#pragma unroll
          for (int i4 = 0; i4 < 8; ++i4) {
            float cv[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) cv[u] = ctab[code_at(w, i4 * 4 + u)];
#pragma unroll
            for (int g = 0; g < G; ++g) {
              const float4 qv = *reinterpret_cast<const float4*>(&qs[g][grp * 32 + i4 * 4]);
              sg[g] = __builtin_fmaf(qv.x, cv[0], sg[g]);
              sg[g] = __builtin_fmaf(qv.y, cv[1], sg[g]);
              sg[g] = __builtin_fmaf(qv.z, cv[2], sg[g]);
              sg[g] = __builtin_fmaf(qv.w, cv[3], sg[g]);
            }
          }
        }
#pragma unroll
        for (int g = 0; g < G; ++g) sg[g] *= kn;
      }
#pragma unroll
      for (int g = 0; g < G; ++g) sc[g][tid] = valid ? sg[g] : -INFINITY;
    }
    __syncthreads();
    // ---- online softmax: wave w handles heads w, w+4, ... ----
    {
      const int wave = tid >> 6, lane = tid & 63;
      for (int g = wave; g < G; g += kDecThreads / 64) {
        float v4[4];
        float mx = -INFINITY;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          v4[k] = sc[g][lane + 64 * k];
          mx = fmaxf(mx, v4[k]);
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
        const float m_old = m_run[g];
        const float m_new = fmaxf(m_old, mx);
        float psum = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int t = lane + 64 * k;
          const float p = (t < n_valid) ? exp2f(v4[k] - m_new) : 0.f;
          psum += p;
          sc[g][t] = (t < n_valid) ? p * vn[t] : 0.f;
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) psum += __shfl_xor(psum, o, 64);
        if (lane == 0) {
          const float al = (m_old == -INFINITY) ? 0.f : exp2f(m_old - m_new);
          alpha[g] = al;
          l_run[g] = l_run[g] * al + psum;
          m_run[g] = m_new;
        }
      }
    }
    __syncthreads();
    // ---- PV phase: thread owns dim j for heads gh, gh+2, ... ----
    {
      const int word = (3 * j) >> 5, off = (3 * j) & 31;
#pragma unroll
      for (int i = 0; i < NG; ++i) {
        const int g = gh + 2 * i;
        if (g < G) acc[i] *= alpha[g];
      }
      for (int t = 0; t < n_valid; ++t) {
        uint32_t code;
        if (off <= 29) {
          code = (vbuf[t][word] >> off) & 7u;
        } else {
          code = __builtin_amdgcn_alignbit(vbuf[t][word + 1], vbuf[t][word], off) & 7u;
        }
        const float cv = ctab[code];
#pragma unroll
        for (int i = 0; i < NG; ++i) {
          const int g = gh + 2 * i;
          if (g < G) acc[i] = __builtin_fmaf(sc[g][t], cv, acc[i]);
        }
      }
    }
  }
  __syncthreads();
  // ---- write partials ----
  float* rec0 = a.ws + ((static_cast<size_t>(s) * a.num_q_heads + h * G) * a.n_splits + split) * kRec;
#pragma unroll
  for (int i = 0; i < NG; ++i) {
    const int g = gh + 2 * i;
    if (g < G) {
      float* rec = rec0 + static_cast<size_t>(g) * a.n_splits * kRec;
      rec[4 + j] = acc[i];
      if (j == 0) {
        rec[0] = m_run[g];
        rec[1] = l_run[g];
      }
    }
  }
}

// Merge the splits of one (sequence, query head) and rotate back.
// 64 threads: lanes own dims {j, j+64}; the first quad does the rotation.
constexpr int kMergeThreads = 64;

__global__ __launch_bounds__(kMergeThreads) void decode_merge_kernel(DecodeArgs a) {
  __shared__ __align__(16) float o_s[kDim];
  __shared__ __align__(16) float sm[kBlocks * 16];
  const int qh = blockIdx.x, s = blockIdx.y;
  const int tid = threadIdx.x;
  const int h = qh / a.group;
  int start, len;
  const bool ok = seq_ok(a, s, &start, &len);
  float* out = a.out + (static_cast<size_t>(s) * a.num_q_heads + qh) * kDim;
  if (!ok || len == 0) {
    const float fill = ok ? 0.f : NAN;
    for (int j = tid; j < kDim; j += kMergeThreads) out[j] = fill;
    return;   // uniform: the whole block takes this path
  }
  load_head_matrices(a.rot + static_cast<size_t>(h) * kBlocks * 8, sm);
  const int used = (len + a.split_len - 1) / a.split_len;
  const float* rec = a.ws + (static_cast<size_t>(s) * a.num_q_heads + qh) * a.n_splits * kRec;
  float m = -INFINITY;
  for (int k = 0; k < used; ++k) m = fmaxf(m, rec[k * kRec]);
  float l = 0.f, o0 = 0.f, o1 = 0.f;
  for (int k = 0; k < used; ++k) {
    const float* r = rec + k * kRec;
    const float w = exp2f(r[0] - m);
    l = __builtin_fmaf(w, r[1], l);
    o0 = __builtin_fmaf(w, r[4 + tid], o0);
    o1 = __builtin_fmaf(w, r[4 + 64 + tid], o1);
  }
  const float inv = 1.0f / l;
  o_s[tid] = o0 * inv;
  o_s[tid + 64] = o1 * inv;
  __syncthreads();
  if (tid < 4) {
    const int part = tid;
    float x[kPerLane];
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) x[i] = o_s[part * kPerLane + i];
    so4_apply_lane<true>(x, sm, part);
    wht128_quad(x, part);
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) out[part * kPerLane + i] = x[i];
  }
}

void decode_plan(int32_t n_seqs, int32_t num_kv_heads, int32_t max_seq_len, int32_t* split_len,
                 int32_t* n_splits) {
  const int64_t per_head = n_seqs > 0 && num_kv_heads > 0
                               ? (kTargetBlocks + static_cast<int64_t>(n_seqs) * num_kv_heads - 1) /
                                     (static_cast<int64_t>(n_seqs) * num_kv_heads)
                               : 1;
  int64_t sl = (max_seq_len + per_head - 1) / per_head;
  sl = (sl + kChunk - 1) / kChunk * kChunk;
  if (sl < kChunk) sl = kChunk;
  *split_len = static_cast<int32_t>(sl);
  const int64_t ns = (static_cast<int64_t>(max_seq_len) + sl - 1) / sl;
  *n_splits = static_cast<int32_t>(ns < 1 ? 1 : ns);
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
  hipLaunchKernelGGL(decode_merge_kernel, dim3(a.num_q_heads, a.n_seqs), dim3(kMergeThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace iq
