// C ABI of libiq (declared in include/iq.h): host-side validation, the
// codebook, and kernel launches. No allocation, no retained device state.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/iq.h"
#include "iq_launch.h"

namespace iq {

// Lloyd-Max quantizer of N(0,1) with 8 levels, solved on the positive half
// (the optimum is symmetric): cells (0, b1], (b1, b2], (b2, b3], (b3, inf)
// with b_k the midpoints of neighbouring levels, each level the Gaussian mean
// of its cell, iterated to a fixed point (zhichai.net essay, section
// "Lloyd-Max 最优量化": assign to the nearest level, move each level to the
// mean of what it received, repeat).
template <int N>
static void lloyd_max_positive_half(double (&level)[N], double (&bound)[N - 1]) {
  const double inv_sqrt_2pi = 0.39894228040143267794;
  auto pdf = [&](double x) { return isinf(x) ? 0.0 : inv_sqrt_2pi * exp(-0.5 * x * x); };
  auto upper_tail = [](double x) { return isinf(x) ? 0.0 : 0.5 * erfc(x * 0.70710678118654752440); };
  double y[N];
  for (int k = 0; k < N; ++k) y[k] = (k + 0.5) * 2.5 / N;   // spread over (0, 2.5)
  for (int it = 0; it < 1000000; ++it) {
    double e[N + 1];
    e[0] = 0.0;
    e[N] = INFINITY;
    for (int k = 1; k < N; ++k) e[k] = 0.5 * (y[k - 1] + y[k]);
    double ny[N];
    for (int k = 0; k < N; ++k) ny[k] = (pdf(e[k]) - pdf(e[k + 1])) / (upper_tail(e[k]) - upper_tail(e[k + 1]));
    bool same = true;
    for (int k = 0; k < N; ++k) {
      if (ny[k] != y[k]) same = false;
      y[k] = ny[k];
    }
    if (same) break;
  }
  for (int k = 0; k < N; ++k) level[k] = y[k];
  for (int k = 0; k < N - 1; ++k) bound[k] = 0.5 * (y[k] + y[k + 1]);
}

// fp16 form of the centroids for the matrix-core contractions: alpha * c is
// split into an fp16 hi part and an fp16 remainder, together good to ~2^-22.
// alpha in [8, 16) is searched (2^-20 grid) so that the hi part alone is as
// close as possible (worst ~2e-5 relative for 8 levels), which keeps the
// remainders small. pos = the N positive centroids.
template <int N>
static float centroid_fp16(const float* pos, uint16_t* h16, uint16_t* l16) {
  double best = 1e30, best_a = 8.0;
  const int steps = 1 << 20;
  for (int i = 0; i < steps; ++i) {
    const double al = 8.0 + 8.0 * i / steps;
    double worst = 0.0;
    for (int k = 0; k < N; ++k) {
      const double x = al * static_cast<double>(pos[k]);
      const double r = static_cast<double>(static_cast<_Float16>(static_cast<float>(x)));
      const double e = fabs(r - x) / x;
      worst = e > worst ? e : worst;
    }
    if (worst < best) {
      best = worst;
      best_a = al;
    }
  }
  for (int k = 0; k < N; ++k) {
    const double x = best_a * static_cast<double>(pos[k]);
    const _Float16 hv = static_cast<_Float16>(static_cast<float>(x));
    const _Float16 lv = static_cast<_Float16>(static_cast<float>(x - static_cast<double>(hv)));
    h16[k] = __builtin_bit_cast(uint16_t, hv);
    l16[k] = __builtin_bit_cast(uint16_t, lv);
  }
  return static_cast<float>(1.0 / best_a);
}

// Symmetric float32 codebook of 2N levels for N(0, 1/128) from the positive half.
template <int N>
static void fill_codebook(float* c, float* t) {
  double lv[N], bd[N - 1];
  lloyd_max_positive_half<N>(lv, bd);
  const double s = 1.0 / sqrt(128.0);       // N(0, 1/d), d = 128
  for (int k = 0; k < N; ++k) {
    c[N + k] = static_cast<float>(lv[k] * s);
    c[N - 1 - k] = -c[N + k];
  }
  t[N - 1] = 0.0f;
  for (int k = 0; k < N - 1; ++k) {
    t[N + k] = static_cast<float>(bd[k] * s);
    t[N - 2 - k] = -t[N + k];
  }
}

static const Codebook& codebook() {
  static Codebook cb;
  static std::once_flag once;
  std::call_once(once, [] {
    fill_codebook<4>(cb.c, cb.t);
    cb.inv_alpha = centroid_fp16<4>(cb.c + 4, cb.h16, cb.l16);
    fill_codebook<8>(cb.c4, cb.t4);
    cb.inv_alpha_k = centroid_fp16<8>(cb.c4 + 8, cb.h16k, cb.l16k);
  });
  return cb;
}

static iq_status hip_status(hipError_t e) { return e == hipSuccess ? IQ_OK : IQ_ERR_HIP; }

static iq_status check_view(const iq_cache_view* v) {
  if (v == nullptr) return IQ_ERR_INVALID_ARG;
  if (v->head_dim != kDim) return IQ_ERR_UNSUPPORTED;
  if (v->num_kv_heads < 1 || v->capacity < 0 || v->capacity % 32 != 0) return IQ_ERR_INVALID_ARG;
  if (!v->k_codes || !v->v_codes || !v->k_norms || !v->v_norms || !v->rot) return IQ_ERR_INVALID_ARG;
  if (v->rotation != IQ_ROT_WHT_SO4 && v->rotation != IQ_ROT_ISO && v->rotation != IQ_ROT_PLANAR)
    return IQ_ERR_INVALID_ARG;
  if (v->k_bits != 3 && v->k_bits != 4) return IQ_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(v->k_codes) | reinterpret_cast<uintptr_t>(v->v_codes) |
       reinterpret_cast<uintptr_t>(v->k_norms) | reinterpret_cast<uintptr_t>(v->v_norms)) & 15u)
    return IQ_ERR_INVALID_ARG;
  return IQ_OK;
}

// Device of the stream the work goes to (the current device for the null stream).
static hipError_t stream_device(hipStream_t s, int* dev) {
  if (s == nullptr) return hipGetDevice(dev);
  hipDevice_t d = 0;
  const hipError_t e = hipStreamGetDevice(s, &d);
  if (e == hipSuccess) *dev = static_cast<int>(d);
  return e;
}

// Scratch of iq_append_decode_attention_noalloc: the split-K records, in a
// file-scope device array of IQ_NOALLOC_SCRATCH_BYTES. Every GPU the library
// runs on holds its own copy, at its own address, until the process ends; in
// host code `scratch` names a host-side stand-in, so kernels and copies take
// the address that hipGetSymbolAddress returns with that GPU current, asked
// once per device and kept here.
static __device__ __align__(256) float scratch[IQ_NOALLOC_SCRATCH_BYTES / sizeof(float)];

static void* scratch_address(int dev) {
  constexpr int kDevices = 64;
  static void* addr[kDevices] = {};
  static std::mutex mu;
  if (dev < 0 || dev >= kDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] != nullptr) return addr[dev];
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return nullptr;
  if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
  void* p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (cur != dev) (void)hipSetDevice(cur);
  if (e != hipSuccess) return nullptr;
  addr[dev] = p;
  return p;
}

}  // namespace iq

using namespace iq;

extern "C" {

const char* iq_status_string(iq_status s) {
  switch (s) {
    case IQ_OK: return "ok";
    case IQ_ERR_INVALID_ARG: return "invalid argument";
    case IQ_ERR_UNSUPPORTED: return "unsupported shape";
    case IQ_ERR_CAPACITY: return "slot range outside the cache capacity";
    case IQ_ERR_WORKSPACE: return "workspace too small";
    case IQ_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

iq_status iq_codebook(float centroids[8], float thresholds[7]) {
  if (!centroids || !thresholds) return IQ_ERR_INVALID_ARG;
  const Codebook& cb = codebook();
  for (int k = 0; k < 8; ++k) centroids[k] = cb.c[k];
  for (int k = 0; k < 7; ++k) thresholds[k] = cb.t[k];
  return IQ_OK;
}

iq_status iq_codebook_levels(int32_t levels, float* centroids, float* thresholds) {
  if (!centroids || !thresholds || (levels != 8 && levels != 16)) return IQ_ERR_INVALID_ARG;
  const Codebook& cb = codebook();
  for (int k = 0; k < levels; ++k) centroids[k] = levels == 8 ? cb.c[k] : cb.c4[k];
  for (int k = 0; k < levels - 1; ++k) thresholds[k] = levels == 8 ? cb.t[k] : cb.t4[k];
  return IQ_OK;
}

iq_status iq_rotate(const float* rot, int32_t rotation, int32_t num_heads, const float* x, float* y,
                    int32_t n_tokens, int32_t inverse, void* stream) {
  if (!rot || !x || !y || num_heads < 1 || n_tokens < 0 || (inverse != 0 && inverse != 1))
    return IQ_ERR_INVALID_ARG;
  if (rotation != IQ_ROT_WHT_SO4 && rotation != IQ_ROT_ISO && rotation != IQ_ROT_PLANAR) return IQ_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(y)) & 15u) return IQ_ERR_INVALID_ARG;
  if (n_tokens == 0) return IQ_OK;
  RotateArgs a{rotation, x, y, rot, n_tokens, num_heads};
  return hip_status(launch_rotate(a, inverse != 0, static_cast<hipStream_t>(stream)));
}

iq_status iq_quantize_pack(const float* y, int64_t n_vectors, uint8_t* codes, float* norms, void* stream) {
  if (!y || !codes || !norms || n_vectors < 0) return IQ_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(y) & 15u) || (reinterpret_cast<uintptr_t>(codes) & 3u))
    return IQ_ERR_INVALID_ARG;
  if (n_vectors == 0) return IQ_OK;
  QuantArgs a{y, codes, norms, n_vectors, codebook()};
  return hip_status(launch_quantize_pack(a, static_cast<hipStream_t>(stream)));
}

iq_status iq_rotate_quantize_append(const iq_cache_view* view, const void* k, const void* v,
                                    iq_dtype in_dtype, int32_t n_tokens, int32_t first_slot,
                                    const int32_t* slots, void* stream) {
  iq_status st = check_view(view);
  if (st != IQ_OK) return st;
  if (in_dtype != IQ_F32 && in_dtype != IQ_F16) return IQ_ERR_INVALID_ARG;
  if (n_tokens < 0) return IQ_ERR_INVALID_ARG;
  if (n_tokens == 0) return IQ_OK;
  if (!k || !v) return IQ_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v)) & 15u) return IQ_ERR_INVALID_ARG;
  if (!slots && (first_slot < 0 || static_cast<int64_t>(first_slot) + n_tokens > view->capacity))
    return IQ_ERR_CAPACITY;
  AppendArgs a{view->rotation, view->k_bits, k, v, slots, view->rot, view->k_codes, view->v_codes, view->k_norms, view->v_norms,
               n_tokens, first_slot, view->num_kv_heads, view->capacity, codebook()};
  return hip_status(launch_append(a, in_dtype == IQ_F16, static_cast<hipStream_t>(stream)));
}

iq_status iq_dequantize(const iq_cache_view* view, int32_t first_slot, int32_t n_tokens, iq_dtype out_dtype,
                        void* k_out, void* v_out, void* stream) {
  iq_status st = check_view(view);
  if (st != IQ_OK) return st;
  if (out_dtype != IQ_F32 && out_dtype != IQ_F16) return IQ_ERR_INVALID_ARG;
  if (n_tokens < 0) return IQ_ERR_INVALID_ARG;
  if (first_slot < 0 || static_cast<int64_t>(first_slot) + n_tokens > view->capacity) return IQ_ERR_CAPACITY;
  if ((reinterpret_cast<uintptr_t>(k_out) | reinterpret_cast<uintptr_t>(v_out)) & 15u) return IQ_ERR_INVALID_ARG;
  if (n_tokens == 0 || (!k_out && !v_out)) return IQ_OK;
  DequantArgs a{view->rotation, view->k_bits, view->k_codes, view->v_codes, view->k_norms, view->v_norms, view->rot, k_out, v_out,
                first_slot, n_tokens, view->num_kv_heads, view->capacity, codebook()};
  return hip_status(launch_dequant(a, out_dtype == IQ_F16, static_cast<hipStream_t>(stream)));
}

static bool group_supported(int32_t g) { return g == 1 || g == 2 || g == 4 || g == 8 || g == 16; }

size_t iq_decode_workspace_bytes(int32_t n_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t max_seq_len) {
  if (n_seqs < 0 || num_q_heads < 1 || num_kv_heads < 1 || max_seq_len < 0) return 0;
  return decode_workspace_bytes(n_seqs, num_q_heads, decode_plan(n_seqs, num_kv_heads, max_seq_len));
}

iq_status iq_decode_attention(const iq_cache_view* view, const float* q, int32_t num_q_heads,
                              const int32_t* seq_start, const int32_t* seq_len, int32_t n_seqs,
                              int32_t max_seq_len, float scale, float* out, void* workspace,
                              size_t workspace_bytes, void* stream) {
  iq_status st = check_view(view);
  if (st != IQ_OK) return st;
  if (n_seqs < 0 || max_seq_len < 0 || num_q_heads < 1) return IQ_ERR_INVALID_ARG;
  if (num_q_heads % view->num_kv_heads != 0) return IQ_ERR_INVALID_ARG;
  const int32_t group = num_q_heads / view->num_kv_heads;
  if (!group_supported(group)) return IQ_ERR_UNSUPPORTED;
  if (n_seqs == 0) return IQ_OK;
  if (!q || !seq_start || !seq_len || !out || !workspace) return IQ_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(workspace) & 15u) return IQ_ERR_INVALID_ARG;
  if (n_seqs > 65535 || view->num_kv_heads > 65535) return IQ_ERR_UNSUPPORTED;   // grid y / z limits
  const DecodePlan plan = decode_plan(n_seqs, view->num_kv_heads, max_seq_len);
  if (workspace_bytes < decode_workspace_bytes(n_seqs, num_q_heads, plan)) return IQ_ERR_WORKSPACE;
  DecodeArgs a{};
  a.k_codes = view->k_codes;
  a.v_codes = view->v_codes;
  a.k_norms = view->k_norms;
  a.v_norms = view->v_norms;
  a.rot = view->rot;
  a.rot_kind = view->rotation;
  a.k_bits = view->k_bits;
  a.q = q;
  a.seq_start = seq_start;
  a.seq_len = seq_len;
  a.out = out;
  a.ws = static_cast<float*>(workspace);
  a.n_seqs = n_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = view->num_kv_heads;
  a.group = group;
  a.capacity = view->capacity;
  a.max_seq_len = max_seq_len;
  a.blocks_per_split = plan.blocks_per_split;
  a.n_splits = plan.n_splits;
  a.rec_offset = 0;
  a.rec_splits = plan.n_splits;
  a.qscale = scale * 1.4426950408889634f;   // log2(e): scores kept in base 2
  a.cb = codebook();
  return hip_status(launch_decode(a, static_cast<hipStream_t>(stream)));
}

iq_status iq_decode_attention_f16(const void* k, const void* v, int64_t token_stride, int64_t head_stride,
                                  int32_t num_kv_heads, int32_t capacity, const float* q, int32_t num_q_heads,
                                  const int32_t* seq_start, const int32_t* seq_len, int32_t n_seqs,
                                  int32_t max_seq_len, float scale, float* out, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  if (num_kv_heads < 1 || capacity < 0 || (capacity % 32) != 0) return IQ_ERR_INVALID_ARG;
  if (token_stride <= 0 || head_stride < 0 || (token_stride % 8) != 0 || (head_stride % 8) != 0)
    return IQ_ERR_INVALID_ARG;
  if (n_seqs < 0 || max_seq_len < 0 || num_q_heads < 1) return IQ_ERR_INVALID_ARG;
  if (num_q_heads % num_kv_heads != 0) return IQ_ERR_INVALID_ARG;
  const int32_t group = num_q_heads / num_kv_heads;
  if (!group_supported(group)) return IQ_ERR_UNSUPPORTED;
  if (n_seqs == 0) return IQ_OK;
  if (!k || !v || !q || !seq_start || !seq_len || !out || !workspace) return IQ_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(workspace)) & 15u)
    return IQ_ERR_INVALID_ARG;
  if (n_seqs > 65535 || num_kv_heads > 65535) return IQ_ERR_UNSUPPORTED;
  const DecodePlan plan = decode_plan(n_seqs, num_kv_heads, max_seq_len);
  if (workspace_bytes < decode_workspace_bytes(n_seqs, num_q_heads, plan)) return IQ_ERR_WORKSPACE;
  F16DecodeArgs a{};
  a.k = static_cast<const _Float16*>(k);
  a.v = static_cast<const _Float16*>(v);
  a.token_stride = token_stride;
  a.head_stride = head_stride;
  a.q = q;
  a.seq_start = seq_start;
  a.seq_len = seq_len;
  a.out = out;
  a.ws = static_cast<float*>(workspace);
  a.n_seqs = n_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = group;
  a.capacity = capacity;
  a.max_seq_len = max_seq_len;
  a.blocks_per_split = plan.blocks_per_split;
  a.n_splits = plan.n_splits;
  a.rec_offset = 0;
  a.rec_splits = plan.n_splits;
  a.qscale = scale * 1.4426950408889634f;
  return hip_status(launch_decode_f16(a, static_cast<hipStream_t>(stream)));
}

// The fused decode step into a workspace of `workspace_bytes` bytes: the
// caller's, or (use_scratch) the library's scratch array of this GPU, whose
// address is asked for only after every host-side check has passed.
static iq_status append_decode(const iq_cache_view* view, const void* k_new, const void* v_new, iq_dtype in_dtype,
                               const float* q, int32_t num_q_heads, const int32_t* seq_start, const int32_t* seq_len,
                               int32_t n_seqs, int32_t max_seq_len, float scale, float* out, void* workspace,
                               size_t workspace_bytes, bool use_scratch, void* stream) {
  iq_status st = check_view(view);
  if (st != IQ_OK) return st;
  if (in_dtype != IQ_F32 && in_dtype != IQ_F16) return IQ_ERR_INVALID_ARG;
  if (n_seqs < 0 || max_seq_len < 0 || num_q_heads < 1) return IQ_ERR_INVALID_ARG;
  if (num_q_heads % view->num_kv_heads != 0) return IQ_ERR_INVALID_ARG;
  const int32_t group = num_q_heads / view->num_kv_heads;
  if (!group_supported(group)) return IQ_ERR_UNSUPPORTED;
  if (n_seqs == 0) return IQ_OK;
  if (!k_new || !v_new || !q || !seq_start || !seq_len || !out || (!use_scratch && !workspace))
    return IQ_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new) |
       reinterpret_cast<uintptr_t>(workspace)) & 15u)
    return IQ_ERR_INVALID_ARG;
  if (n_seqs > 65535 || view->num_kv_heads > 65535) return IQ_ERR_UNSUPPORTED;
  const DecodePlan plain = decode_plan(n_seqs, view->num_kv_heads, max_seq_len);
  if (workspace_bytes < decode_workspace_bytes(n_seqs, num_q_heads, plain)) return IQ_ERR_WORKSPACE;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  int dev = 0;
  if (stream_device(hs, &dev) != hipSuccess) return IQ_ERR_HIP;
  if (use_scratch && (workspace = scratch_address(dev)) == nullptr) return IQ_ERR_HIP;
  // The new token's work-groups join the split launch: if they and the plain
  // plan's splits do not all fit on the GPU at once, the plan leaves them room
  // (a second round of work-groups would cost a whole split's time).
  const int64_t wgs = static_cast<int64_t>(plain.n_splits + 1) * n_seqs * view->num_kv_heads;
  const DecodePlan plan = wgs <= split_new_resident_wgs(dev, group, view->k_bits)
                              ? plain
                              : decode_plan(n_seqs, view->num_kv_heads, max_seq_len, 1);
  DecodeArgs a{};
  a.k_codes = view->k_codes;
  a.v_codes = view->v_codes;
  a.k_norms = view->k_norms;
  a.v_norms = view->v_norms;
  a.rot = view->rot;
  a.rot_kind = view->rotation;
  a.k_bits = view->k_bits;
  a.q = q;
  a.seq_start = seq_start;
  a.seq_len = seq_len;
  a.out = out;
  a.ws = static_cast<float*>(workspace);
  a.n_seqs = n_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = view->num_kv_heads;
  a.group = group;
  a.capacity = view->capacity;
  a.max_seq_len = max_seq_len;
  a.blocks_per_split = plan.blocks_per_split;
  a.n_splits = plan.n_splits;
  a.rec_offset = 0;
  a.rec_splits = plan.n_splits + 1;   // the splits' records, then the new token's
  a.qscale = scale * 1.4426950408889634f;
  a.cb = codebook();
  NewToken nt{};
  nt.k_new = k_new;
  nt.v_new = v_new;
  nt.new_f16 = in_dtype == IQ_F16 ? 1 : 0;
  nt.k_codes = view->k_codes;
  nt.v_codes = view->v_codes;
  nt.k_norms = view->k_norms;
  nt.v_norms = view->v_norms;
  hipError_t e = launch_decode_splits_new(a, nt, hs);
  if (e != hipSuccess) return IQ_ERR_HIP;
  MergeArgs m{a.rot_kind, a.rot, a.out, a.ws, a.n_seqs, a.num_q_heads, a.group, a.rec_splits, 1, plan.n_splits, {}};
  m.seg[0] = MergeSegment{a.seq_start, a.seq_len, a.capacity, a.max_seq_len, a.blocks_per_split, a.n_splits, 0};
  return hip_status(launch_merge(m, hs));
}

iq_status iq_append_decode_attention(const iq_cache_view* view, const void* k_new, const void* v_new,
                                     iq_dtype in_dtype, const float* q, int32_t num_q_heads, const int32_t* seq_start,
                                     const int32_t* seq_len, int32_t n_seqs, int32_t max_seq_len, float scale,
                                     float* out, void* workspace, size_t workspace_bytes, void* stream) {
  return append_decode(view, k_new, v_new, in_dtype, q, num_q_heads, seq_start, seq_len, n_seqs, max_seq_len, scale,
                       out, workspace, workspace_bytes, false, stream);
}

iq_status iq_append_decode_attention_noalloc(const iq_cache_view* view, const void* k_new, const void* v_new,
                                             iq_dtype in_dtype, const float* q, int32_t num_q_heads,
                                             const int32_t* seq_start, const int32_t* seq_len, int32_t n_seqs,
                                             int32_t max_seq_len, float scale, float* out, void* stream) {
  return append_decode(view, k_new, v_new, in_dtype, q, num_q_heads, seq_start, seq_len, n_seqs, max_seq_len, scale,
                       out, nullptr, IQ_NOALLOC_SCRATCH_BYTES, true, stream);
}

size_t iq_decode_deferred_workspace_bytes(int32_t n_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                          int32_t max_prefix_len, int32_t max_seq_len) {
  if (n_seqs < 0 || num_q_heads < 1 || num_kv_heads < 1 || max_prefix_len < 0 || max_seq_len < 0) return 0;
  const DecodePlan pre = decode_plan(n_seqs, num_kv_heads, max_prefix_len);
  const DecodePlan suf = decode_plan(n_seqs, num_kv_heads, max_seq_len);
  return static_cast<size_t>(n_seqs) * num_q_heads * (pre.n_splits + suf.n_splits) * 132 * sizeof(float);
}

iq_status iq_decode_attention_deferred(const iq_cache_view* view, const int32_t* seq_start, const int32_t* seq_len,
                                       int32_t max_seq_len, const void* k16, const void* v16, int64_t token_stride,
                                       int64_t head_stride, int32_t capacity16, const int32_t* prefix_start,
                                       const int32_t* prefix_len, int32_t max_prefix_len, const float* q,
                                       int32_t num_q_heads, int32_t n_seqs, float scale, float* out,
                                       void* workspace, size_t workspace_bytes, void* stream) {
  iq_status st = check_view(view);
  if (st != IQ_OK) return st;
  const int32_t hkv = view->num_kv_heads;
  if (capacity16 < 0 || (capacity16 % 32) != 0) return IQ_ERR_INVALID_ARG;
  if (token_stride <= 0 || head_stride < 0 || (token_stride % 8) != 0 || (head_stride % 8) != 0)
    return IQ_ERR_INVALID_ARG;
  if (n_seqs < 0 || max_seq_len < 0 || max_prefix_len < 0 || num_q_heads < 1) return IQ_ERR_INVALID_ARG;
  if (num_q_heads % hkv != 0) return IQ_ERR_INVALID_ARG;
  const int32_t group = num_q_heads / hkv;
  if (!group_supported(group)) return IQ_ERR_UNSUPPORTED;
  if (n_seqs == 0) return IQ_OK;
  if (!k16 || !v16 || !prefix_start || !prefix_len || !q || !seq_start || !seq_len || !out || !workspace)
    return IQ_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(k16) | reinterpret_cast<uintptr_t>(v16) | reinterpret_cast<uintptr_t>(workspace)) &
      15u)
    return IQ_ERR_INVALID_ARG;
  if (n_seqs > 65535 || hkv > 65535) return IQ_ERR_UNSUPPORTED;
  const DecodePlan pp = decode_plan(n_seqs, hkv, max_prefix_len);
  const DecodePlan sp = decode_plan(n_seqs, hkv, max_seq_len);
  if (workspace_bytes < iq_decode_deferred_workspace_bytes(n_seqs, num_q_heads, hkv, max_prefix_len, max_seq_len))
    return IQ_ERR_WORKSPACE;
  const int32_t total = pp.n_splits + sp.n_splits;
  const float qscale = scale * 1.4426950408889634f;
  F16DecodeArgs pre{};
  pre.rot_kind = view->rotation;
  pre.rot = view->rot;
  pre.k = static_cast<const _Float16*>(k16);
  pre.v = static_cast<const _Float16*>(v16);
  pre.token_stride = token_stride;
  pre.head_stride = head_stride;
  pre.q = q;
  pre.seq_start = prefix_start;
  pre.seq_len = prefix_len;
  pre.out = out;
  pre.ws = static_cast<float*>(workspace);
  pre.n_seqs = n_seqs;
  pre.num_q_heads = num_q_heads;
  pre.num_kv_heads = hkv;
  pre.group = group;
  pre.capacity = capacity16;
  pre.max_seq_len = max_prefix_len;
  pre.blocks_per_split = pp.blocks_per_split;
  pre.n_splits = pp.n_splits;
  pre.rec_offset = 0;
  pre.rec_splits = total;
  pre.qscale = qscale;
  DecodeArgs suf{};
  suf.k_codes = view->k_codes;
  suf.v_codes = view->v_codes;
  suf.k_norms = view->k_norms;
  suf.v_norms = view->v_norms;
  suf.rot = view->rot;
  suf.rot_kind = view->rotation;
  suf.k_bits = view->k_bits;
  suf.q = q;
  suf.seq_start = seq_start;
  suf.seq_len = seq_len;
  suf.out = out;
  suf.ws = static_cast<float*>(workspace);
  suf.n_seqs = n_seqs;
  suf.num_q_heads = num_q_heads;
  suf.num_kv_heads = hkv;
  suf.group = group;
  suf.capacity = view->capacity;
  suf.max_seq_len = max_seq_len;
  suf.blocks_per_split = sp.blocks_per_split;
  suf.n_splits = sp.n_splits;
  suf.rec_offset = pp.n_splits;
  suf.rec_splits = total;
  suf.qscale = qscale;
  suf.cb = codebook();
  return hip_status(launch_decode_deferred(pre, suf, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
