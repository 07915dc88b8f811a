// Host-side launch interface between the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "iq_device.h"

namespace iq {

struct AppendArgs {
  int32_t rot_kind;      // iq_rotation
  int32_t k_bits;        // 3 or 4
  const void* k;
  const void* v;
  const int32_t* slots;
  const float* rot;
  uint8_t* k_codes;
  uint8_t* v_codes;
  float* k_norms;
  float* v_norms;
  int32_t n_tokens;
  int32_t first_slot;
  int32_t num_kv_heads;
  int32_t capacity;
  Codebook cb;
};

struct RotateArgs {
  int32_t rot_kind;      // iq_rotation
  const float* x;
  float* y;
  const float* rot;
  int32_t n_tokens;
  int32_t num_heads;
};

struct QuantArgs {
  const float* y;
  uint8_t* codes;
  float* norms;
  int64_t n_vectors;
  Codebook cb;
};

struct DequantArgs {
  int32_t rot_kind;      // iq_rotation
  int32_t k_bits;        // 3 or 4
  const uint8_t* k_codes;
  const uint8_t* v_codes;
  const float* k_norms;
  const float* v_norms;
  const float* rot;
  void* k_out;
  void* v_out;
  int32_t first_slot;
  int32_t n_tokens;
  int32_t num_kv_heads;
  int32_t capacity;
  Codebook cb;
};

// The 32-bit fields come first: one wide scalar load at the kernel's start
// then covers every size a work-group's first addresses need.
struct DecodeArgs {
  int32_t rot_kind;      // iq_rotation
  int32_t n_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;
  int32_t capacity;
  int32_t max_seq_len;
  int32_t blocks_per_split;   // 32-slot blocks per split
  int32_t n_splits;           // splits per (seq, kv head) at max_seq_len
  int32_t rec_offset;         // record index of split 0 ...
  int32_t rec_splits;         // ... among this many records per (seq, query head)
  int32_t k_bits;             // 3 or 4
  float qscale;               // softmax scale * log2(e)
  const uint8_t* k_codes;
  const uint8_t* v_codes;
  const float* k_norms;
  const float* v_norms;
  const float* rot;
  const float* q;
  const int32_t* seq_start;
  const int32_t* seq_len;
  float* out;
  float* ws;             // split partials [n_seqs][Hq][n_splits][132]
  Codebook cb;
};

// Decode over a plain fp16 K/V cache (the baseline and the unfused path):
// element (token t, KV head h, dim j) at k[t * token_stride + h * head_stride + j].
struct F16DecodeArgs {
  int32_t rot_kind;          // with rot: records are rotated forward (deferred decode)
  const float* rot;          // nullptr: records stay in the model's basis
  const _Float16* k;
  const _Float16* v;
  int64_t token_stride;
  int64_t head_stride;
  const float* q;
  const int32_t* seq_start;
  const int32_t* seq_len;
  float* out;
  float* ws;
  int32_t n_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;
  int32_t capacity;
  int32_t max_seq_len;
  int32_t blocks_per_split;
  int32_t n_splits;
  int32_t rec_offset;
  int32_t rec_splits;
  float qscale;
};

// One group of split records: the splits of a token range planned with its
// own block count (records split_offset .. split_offset + n_splits - 1).
struct MergeSegment {
  const int32_t* seq_start;
  const int32_t* seq_len;
  int32_t capacity;
  int32_t max_seq_len;
  int32_t blocks_per_split;
  int32_t n_splits;
  int32_t split_offset;
};

// Split-K merge: rot = nullptr for records already in the model's basis (fp16
// cache), else the rotation whose inverse is applied once. Records of
// (seq, query head) are rec_splits apart; 1 or 2 segments (deferred decode:
// the fp16 prefix's splits, then the packed suffix's), plus, if extra_rec >= 0,
// the record at that index (the decode step's new token), always live.
struct MergeArgs {
  int32_t rot_kind;      // iq_rotation
  const float* rot;
  float* out;
  const float* ws;
  int32_t n_seqs;
  int32_t num_q_heads;
  int32_t group;
  int32_t rec_splits;
  int32_t n_segments;
  int32_t extra_rec;
  MergeSegment seg[2];
};

// The decode step's new token (iq_append_decode_attention): extra work-groups
// of the split launch encode token s into cache slot seq_start[s] +
// seq_len[s] and write its record (score, 1, rotated V) for each query head
// of the group at split index n_splits.
struct NewToken {
  const void* k_new;     // [n_seqs][Hkv][128], fp16 or fp32
  const void* v_new;
  int32_t new_f16;
  uint8_t* k_codes;      // the cache the splits read, writable
  uint8_t* v_codes;
  float* k_norms;
  float* v_norms;
};

hipError_t launch_append(const AppendArgs& a, bool f16, hipStream_t s);
hipError_t launch_rotate(const RotateArgs& a, bool inverse, hipStream_t s);
hipError_t launch_quantize_pack(const QuantArgs& a, hipStream_t s);
hipError_t launch_dequant(const DequantArgs& a, bool f16, hipStream_t s);

// split-K plan for decode (shared by the workspace query and the launch);
// extra_per_pair: work-groups per (seq, KV head) the launch runs beside the
// splits. Fewer splits never need more workspace, so the plan without extras
// sizes it.
struct DecodePlan {
  int32_t blocks_per_split, n_splits;
};
DecodePlan decode_plan(int32_t n_seqs, int32_t num_kv_heads, int32_t max_seq_len, int32_t extra_per_pair = 0);
// Workspace: one partial record (m, l, 2 pad, o[128] fp32) per (seq, query head, split).
size_t decode_workspace_bytes(int32_t n_seqs, int32_t num_q_heads, const DecodePlan& p);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);
hipError_t launch_decode_f16(const F16DecodeArgs& a, hipStream_t s);
// fp16 prefix and packed suffix in one split launch, then the merge
hipError_t launch_decode_deferred(const F16DecodeArgs& pre, const DecodeArgs& suf, hipStream_t s);
hipError_t launch_merge(const MergeArgs& a, hipStream_t s);
// split kernels only (the packed decode's first launch); with nt, one more
// work-group per (KV head, seq) encodes the new token and writes its records
hipError_t launch_decode_splits(const DecodeArgs& a, hipStream_t s);
hipError_t launch_decode_splits_new(const DecodeArgs& a, const NewToken& nt, hipStream_t s);
// Work-groups of the append-decode split kernel for (group, K bits) that
// device `dev` holds at once (occupancy x CUs, asked once per device); 0 if
// the runtime cannot say.
int64_t split_new_resident_wgs(int dev, int group, int k_bits);

}  // namespace iq
