// Decode attention straight from the packed 3-bit cache on the matrix cores
// (split-K over the context, cross-workgroup softmax merge).
//
// What is computed (news article on RotaryQuant, section on attention over
// packed data; arXiv 2608.08081 abstract; zhichai.net essay's attention
// formula softmax(Q K^T / sqrt(d)) V):
//   q'_g    = R q_g                                            (query rotated once)
//   s_{g,t} = scale log2(e) nK_t sum_j q'_{g,j} c[kcode_{t,j}]   (score in the rotated domain)
//   o'_g    = sum_t 2^(s_{g,t} - m) nV_t c[vcode_t] / sum_t 2^(s_{g,t} - m)
//   out_g   = R^-1 o'_g = Hn B^T o'_g                            (one inverse rotation)
// Full-precision K and V are never formed in memory.
//
// Contractions on MFMA (v_mfma_f32_16x16x32_f16, fp32 accumulate). Each
// centroid enters as alpha * c = hi + lo (two fp16 numbers, ~22 bits
// together); the two halves sit in adjacent K slots of the code operand and
// the other operand repeats its value in both slots, so one MFMA forms
// (hi + lo) * x. Per wave and per block of 32 cache slots:
//   * scores: two 16-token tiles x 8 k-steps of 4 dims; A = code centroids,
//     B = the rotated query. For G <= 8 the 16 B columns hold the query split
//     into fp16 hi (columns g) and lo (columns g + 8) and one DPP row rotation
//     adds the halves, so the query keeps ~22 bits as well.
//   * PV: 8 column tiles of 16 dims x 2 groups of 16 tokens; A = softmax
//     weights times V norms (hi rows g, lo rows g + 8), B = code centroids.
// Code pairs become operand dwords through a 64-entry table in LDS (entry p =
// {hi(c_a) | lo(c_a) << 16, hi(c_b) | lo(c_b) << 16} for the codes a, b of
// pair p), replicated 16 times (one copy per lane of a 16-lane group); one
// 8-byte read fills two operand registers. Each wave streams its blocks
// through two LDS stages of its own with global->LDS loads (iq_decode_packed.h).
//
// Layout of the cache (see include/iq.h): K rows of 48 bytes per token; V in
// tiles of 8 slots, dim-major, so the codes one PV operand needs (one dim,
// consecutive tokens) are adjacent bits.
//
// Softmax reference m: tracks max_t (s_t + log2 nV_t), token by token, and is
// raised lazily (only when a weight would exceed 2^15, and then to where the
// largest weight is 2^7), so 2^(s_t - m) nV_t stays within fp16's range with
// normal halves over ~21 binary orders below the largest, whatever the scale
// of the V norms, while accumulator rescaling is rare.
#include <atomic>

#include "iq_decode_packed.h"
#include "iq_decode_new_token.h"

namespace iq {

// work-groups go round-robin to the XCDs in launch order; with the split
// index slowest (grid z), the live splits (short sequences have few) spread evenly
//
// kNew: grid z has one more slice, dispatched first: z = 0 encodes the decode
// step's new token (new_token_block) while the splits z - 1 run beside it.
template <int G, int KB, bool kNew>
__global__ __launch_bounds__(kDecThreads, 2) void decode_split_kernel(DecodeArgs a, NewToken nt) {
  __shared__ PackedSmem<G, KB> sm;
  __shared__ StageMem<G, KB> stg;
  static_assert(sizeof(PackedSmem<G, KB>) >= sizeof(NewTokenSmem<G>), "new-token LDS must fit");
  touch_codebook_words<KB>(a.cb);
  if constexpr (kNew) {
    if (blockIdx.z == 0) {
      new_token_block<G, KB>(a, nt, *reinterpret_cast<NewTokenSmem<G>*>(&sm));
      return;
    }
  }
  const int split = kNew ? blockIdx.z - 1 : blockIdx.z;
#include "iq_decode_packed_body.inc"
}

// One work-group per (seq, query head): merges the live splits' records
//   M = max m_k, l = sum 2^(m_k - M) l_k, o' = sum 2^(m_k - M) o'_k,
// then out = Hn B^T (o' / l), the single inverse rotation (kRotate; the fp16
// decode's records are already in the model's basis). Lane t first reads
// dims 4 (t % 32) .. +3 of records t / 32, t / 32 + kRows, ... (coalesced),
// keeps a running merge of them, and parks the result in LDS; wave 0 then
// combines the kRows rows and rotates, two dims per lane. An empty sequence
// gives 0, an invalid one NaN.
//
// kRows rows of 32 lanes (kRows <= 32): 8 when the records fit one round of
// loads (a batch with few splits per sequence: 256 threads, so that many
// work-groups start fast), 32 otherwise.
template <bool kRotate, int kRows>
__global__ __launch_bounds__(kRows * kMergeLanes) void decode_merge_kernel(MergeArgs a) {
  constexpr int kMergeRows = kRows;
  static_assert(kRows <= 32 && kRows * kMergeLanes >= 4 * kBlocks, "one row per lane of wave 0; 128 builders");
  __shared__ float rm[kMergeRows], rl[kMergeRows];
  __shared__ __align__(16) float ro[kMergeRows][kDim];
  __shared__ __align__(16) float mats[kBlocks * 16];   // the head's block matrices (kRotate)
  const int hq = blockIdx.x, s = blockIdx.y;
  const int tid = threadIdx.x, row = tid / kMergeLanes, d4 = tid % kMergeLanes;
  const int h = hq / a.group;
  // threads 0..127 build the head's block matrices (one column each) for the
  // inverse rotation; every thread loads parameters (a load under a
  // condition would hold up the record loads behind it)
  float bp[8];
  if (kRotate) load_block_params(rot_of_head(a.rot, a.rot_kind, h), a.rot_kind, (tid >> 2) & (kBlocks - 1), bp);
  // Record positions: segment 0 at [0, n_splits0), segment 1 (if any) from
  // split_offset on, the new token's (if any) at extra_rec. The first round
  // of record loads goes out before the sequence bounds are read (two round
  // trips would otherwise follow each other); records past a segment's live
  // splits are stale and masked out.
  const float* recs = a.ws + (static_cast<size_t>(s) * a.num_q_heads + hq) * a.rec_splits * kRec;
  float mv[kMergeChunk], lv[kMergeChunk];
  float4 ov[kMergeChunk];
#pragma unroll
  for (int i = 0; i < kMergeChunk; ++i) {
    const int p = row + i * kMergeRows;
    const float* r = recs + static_cast<size_t>(p < a.rec_splits ? p : 0) * kRec;
    const float2 ml = *reinterpret_cast<const float2*>(r);
    mv[i] = ml.x;
    lv[i] = ml.y;
    ov[i] = reinterpret_cast<const float4*>(r + 4)[d4];
  }
  float* const dst = a.out + (static_cast<size_t>(s) * a.num_q_heads + hq) * kDim;
  bool ok = true;
  int live0 = 0, live1 = 0;
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    if (g >= a.n_segments) break;
    const MergeSegment& sg = a.seg[g];
    int start, len;
    const bool okg = seq_ok(sg, s, &start, &len);
    ok = ok && okg;
    const int live = live_splits(okg ? n_blocks(start, len) : 0, sg.blocks_per_split, sg.n_splits);
    if (g == 0) live0 = live; else live1 = live;
  }
  const int off1 = a.n_segments > 1 ? a.seg[1].split_offset : a.rec_splits;
  auto live_at = [&](int p) { return p < live0 || (p >= off1 && p - off1 < live1) || p == a.extra_rec; };
  // the block matrices while the records are in flight (their parameters were requested first)
  if (kRotate) build_head_matrices(a.rot_kind, bp, mats);
  float mx = -INFINITY, l = 0.f;
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int p0 = row;; p0 += kMergeRows * kMergeChunk) {
    if (p0 != row) {
      if (p0 >= a.rec_splits) break;
#pragma unroll
      for (int i = 0; i < kMergeChunk; ++i) {
        const int p = p0 + i * kMergeRows;
        const float* r = recs + static_cast<size_t>(p < a.rec_splits ? p : 0) * kRec;
        const float2 ml = *reinterpret_cast<const float2*>(r);
        mv[i] = ml.x;
        lv[i] = ml.y;
        ov[i] = reinterpret_cast<const float4*>(r + 4)[d4];
      }
    }
    // selects, not products, so stale non-finite values cannot leak in
#pragma unroll
    for (int i = 0; i < kMergeChunk; ++i) {
      const bool in = live_at(p0 + i * kMergeRows);
      mv[i] = in ? mv[i] : -INFINITY;
      lv[i] = in ? lv[i] : 0.f;
      ov[i] = in ? ov[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float cm = mx;
#pragma unroll
    for (int i = 0; i < kMergeChunk; ++i) cm = fmaxf(cm, mv[i]);
    if (cm == -INFINITY) continue;   // only records without tokens so far
    const float f = fast_exp2(mx - cm);   // mx = -inf gives 0
    l *= f;
    o.x *= f; o.y *= f; o.z *= f; o.w *= f;
#pragma unroll
    for (int i = 0; i < kMergeChunk; ++i) {
      const float w = fast_exp2(mv[i] - cm);   // -inf gives 0
      l += w * lv[i];
      o.x += w * ov[i].x; o.y += w * ov[i].y; o.z += w * ov[i].z; o.w += w * ov[i].w;
    }
    mx = cm;
  }
  if (d4 == 0) {
    rm[row] = mx;
    rl[row] = l;
  }
  reinterpret_cast<float4*>(ro[row])[d4] = o;
  __syncthreads();
  // The rows' weights w_r = 2^(m_r - M) and 1 / L (L = sum_r w_r l_r), by
  // the first kRows lanes, into LDS; then the weighted sum over the rows in
  // two levels: every thread sums four rows of one dim (kRows / 4 groups x
  // 128 dims: all the threads), and wave 0 adds the group sums of two dims
  // per lane (t and t + 64) and applies the inverse rotation in registers.
  __shared__ __align__(16) float rw[kMergeRows];
  __shared__ float rinv;
  constexpr int kGroups = kMergeRows / 4;
  static_assert(kGroups * kDim == kMergeRows * kMergeLanes, "one thread per (row group, dim)");
  __shared__ float part[kGroups][kDim];
  if (tid < 64) {
    const int r = tid & 31;
    const float m_r = r < kMergeRows ? rm[r & (kMergeRows - 1)] : -INFINITY;
    const float M = half_wave_reduce<true>(m_r);
    const float w = M == -INFINITY ? 0.f : fast_exp2(m_r - M);   // rows past kMergeRows: 0
    const float L = half_wave_reduce<false>(w * (r < kMergeRows ? rl[r & (kMergeRows - 1)] : 0.f));
    if (tid < kMergeRows) rw[tid] = w;
    if (tid == 0) rinv = L > 0.f ? __builtin_amdgcn_rcpf(L) : 0.f;
  }
  __syncthreads();
  {
    const int d = tid & (kDim - 1), g = tid / kDim;
    const float4 w4 = *reinterpret_cast<const float4*>(&rw[4 * g]);
    const float x = __builtin_fmaf(w4.w, ro[4 * g + 3][d],
                                   __builtin_fmaf(w4.z, ro[4 * g + 2][d],
                                                  __builtin_fmaf(w4.y, ro[4 * g + 1][d], w4.x * ro[4 * g][d])));
    part[g][d] = x;
  }
  __syncthreads();
  if (tid < 64) {
    const int t = tid;
    float x0[kGroups], x1[kGroups];
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
      x0[g] = part[g][t];
      x1[g] = part[g][t + 64];
    }
#pragma unroll
    for (int w = 1; w < kGroups; w *= 2) {   // pairwise sums
#pragma unroll
      for (int g = 0; g + w < kGroups; g += 2 * w) {
        x0[g] += x0[g + w];
        x1[g] += x1[g + w];
      }
    }
    const float inv = rinv;
    float y0 = x0[0] * inv;
    float y1 = x1[0] * inv;
    if (kRotate) {
      so4_apply_pair<true>(y0, y1, mats, t);
      if (a.rot_kind == kRotWhtSo4) wht128_pair(y0, y1, t);
    }
    dst[t] = ok ? y0 : NAN;
    dst[t + 64] = ok ? y1 : NAN;
  }
}

DecodePlan decode_plan(int32_t n_seqs, int32_t num_kv_heads, int32_t max_seq_len, int32_t extra_per_pair) {
  DecodePlan p{};
  // blocks of a 32-aligned start; a misaligned one adds a block, which the last split takes
  const int64_t blocks = (static_cast<int64_t>(max_seq_len > 0 ? max_seq_len : 1) + kBlk - 1) / kBlk;
  const int64_t pairs = static_cast<int64_t>(n_seqs > 0 ? n_seqs : 1) * (num_kv_heads > 0 ? num_kv_heads : 1);
  // the launch's other work-groups (the new token's) take resident slots too
  int64_t want_splits = (kTargetBlocks + pairs - 1) / pairs - extra_per_pair;
  if (want_splits < 1) want_splits = 1;
  int64_t bps = (blocks + want_splits - 1) / want_splits;
  if (bps < kMinBlocksPerSplit) bps = kMinBlocksPerSplit;
  if (bps > kMaxBlocksPerSplit) bps = kMaxBlocksPerSplit;
  int64_t ns = (blocks + bps - 1) / bps;
  if (ns > kMaxSplits) {
    bps = (blocks + kMaxSplits - 1) / kMaxSplits;
    ns = (blocks + bps - 1) / bps;
  }
  if (ns < 1) ns = 1;
  p.blocks_per_split = static_cast<int32_t>(bps);
  p.n_splits = static_cast<int32_t>(ns);
  return p;
}

size_t decode_workspace_bytes(int32_t n_seqs, int32_t num_q_heads, const DecodePlan& p) {
  return static_cast<size_t>(n_seqs) * num_q_heads * (p.n_splits + 1) * kRec * sizeof(float);
}

template <int KB, bool kNew>
static hipError_t launch_split(const DecodeArgs& a, const NewToken& nt, hipStream_t st) {
  dim3 grid(a.num_kv_heads, a.n_seqs, a.n_splits + (kNew ? 1 : 0));
  switch (a.group) {
    case 1: hipLaunchKernelGGL((decode_split_kernel<1, KB, kNew>), grid, dim3(kDecThreads), 0, st, a, nt); break;
    case 2: hipLaunchKernelGGL((decode_split_kernel<2, KB, kNew>), grid, dim3(kDecThreads), 0, st, a, nt); break;
    case 4: hipLaunchKernelGGL((decode_split_kernel<4, KB, kNew>), grid, dim3(kDecThreads), 0, st, a, nt); break;
    case 8: hipLaunchKernelGGL((decode_split_kernel<8, KB, kNew>), grid, dim3(kDecThreads), 0, st, a, nt); break;
    case 16: hipLaunchKernelGGL((decode_split_kernel<16, KB, kNew>), grid, dim3(kDecThreads), 0, st, a, nt); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int KB>
static const void* split_new_kernel(int group) {
  switch (group) {
    case 1: return reinterpret_cast<const void*>(&decode_split_kernel<1, KB, true>);
    case 2: return reinterpret_cast<const void*>(&decode_split_kernel<2, KB, true>);
    case 4: return reinterpret_cast<const void*>(&decode_split_kernel<4, KB, true>);
    case 8: return reinterpret_cast<const void*>(&decode_split_kernel<8, KB, true>);
    case 16: return reinterpret_cast<const void*>(&decode_split_kernel<16, KB, true>);
    default: return nullptr;
  }
}

int64_t split_new_resident_wgs(int dev, int group, int k_bits) {
  // per device (up to 64), group (1, 2, 4, 8, 16) and K width; 0 = not yet asked
  constexpr int kDevices = 64;
  static std::atomic<int64_t> cache[kDevices][5][2];
  if (dev < 0 || dev >= kDevices) return 0;
  const int gi = group == 1 ? 0 : group == 2 ? 1 : group == 4 ? 2 : group == 8 ? 3 : group == 16 ? 4 : -1;
  if (gi < 0) return 0;
  std::atomic<int64_t>& slot = cache[dev][gi][k_bits == 4 ? 1 : 0];
  int64_t v = slot.load(std::memory_order_relaxed);
  if (v > 0) return v;
  const void* f = k_bits == 4 ? split_new_kernel<4>(group) : split_new_kernel<3>(group);
  if (f == nullptr) return 0;
  // the occupancy query answers for the current device: make it `dev` for the call
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return 0;
  if (cur != dev && hipSetDevice(dev) != hipSuccess) return 0;
  int per_cu = 0, cus = 0;
  const bool ok = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, f, kDecThreads, 0) == hipSuccess &&
                  hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess;
  if (cur != dev) (void)hipSetDevice(cur);
  if (!ok) return 0;
  v = static_cast<int64_t>(per_cu) * cus;
  if (v > 0) slot.store(v, std::memory_order_relaxed);
  return v;
}

hipError_t launch_decode_splits(const DecodeArgs& a, hipStream_t st) {
  const NewToken none{};
  return a.k_bits == 4 ? launch_split<4, false>(a, none, st) : launch_split<3, false>(a, none, st);
}

hipError_t launch_decode_splits_new(const DecodeArgs& a, const NewToken& nt, hipStream_t st) {
  return a.k_bits == 4 ? launch_split<4, true>(a, nt, st) : launch_split<3, true>(a, nt, st);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) {
  const hipError_t le = launch_decode_splits(a, st);
  if (le != hipSuccess) return le;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  MergeArgs m{a.rot_kind, a.rot, a.out, a.ws, a.n_seqs, a.num_q_heads, a.group, a.rec_splits, 1, -1, {}};
  m.seg[0] = MergeSegment{a.seq_start, a.seq_len, a.capacity, a.max_seq_len, a.blocks_per_split, a.n_splits, 0};
  return launch_merge(m, st);
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t st) {
  const dim3 grid(a.num_q_heads, a.n_seqs);
  const bool small = a.rec_splits <= 8 * kMergeChunk;   // one round of loads with 8 rows
  if (a.rot != nullptr) {
    if (small) hipLaunchKernelGGL((decode_merge_kernel<true, 8>), grid, dim3(8 * kMergeLanes), 0, st, a);
    else hipLaunchKernelGGL((decode_merge_kernel<true, 32>), grid, dim3(32 * kMergeLanes), 0, st, a);
  } else {
    if (small) hipLaunchKernelGGL((decode_merge_kernel<false, 8>), grid, dim3(8 * kMergeLanes), 0, st, a);
    else hipLaunchKernelGGL((decode_merge_kernel<false, 32>), grid, dim3(32 * kMergeLanes), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace iq
