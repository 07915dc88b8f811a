/*
 * iq.h -- C ABI of libiq: IsoQuant packed 3-bit KV cache on AMD MI355X (gfx950).
 *
 * The method (arXiv 2608.08081 "RotaryQuant" abstract; rebasdaily.com news
 * article on RotaryQuant, section on attention over packed data):
 *   encode   y = B . Hn . x   (normalised Walsh-Hadamard transform Hn, then
 *                              block-diagonal SO(4) rotation B, 32 blocks of 4
 *                              dims, each from two unit quaternions: 256
 *                              parameters per head), n = ||y||, 3-bit
 *                              Lloyd-Max code per coordinate for N(0, 1/128)
 *                              (zhichai.net TurboQuant/RotorQuant essay,
 *                              sections "Beta 分布的魔力" and
 *                              "Lloyd-Max 最优量化"), packed 48 bytes per row.
 *   decode   attention computed directly on the packed K/V in the rotated
 *            domain, followed by one inverse rotation of the output.
 *
 * Conventions shared by every entry point:
 *   - d = head_dim = 128 only (anything else: IQ_ERR_UNSUPPORTED).
 *   - Pointers marked "device" are device memory owned by the caller; the
 *     library never allocates, frees or retains them. Its only state: a
 *     lazily computed host copy of the codebook, the number of decode-step
 *     work-groups each device holds at once (asked once per device and
 *     kept), and the scratch array of iq_append_decode_attention_noalloc in
 *     each GPU's memory (with its device address, asked once per device).
 *   - All GPU work is enqueued asynchronously on `stream` (a hipStream_t;
 *     NULL = the legacy default stream). A return of IQ_OK means the work was
 *     launched, not that it has finished.
 *   - Errors: every argument that can be checked on the host is checked
 *     before anything is launched; a failed check returns a negative
 *     iq_status and launches nothing. IQ_ERR_HIP reports a failed launch.
 *     NaN/Inf inputs are not checked; they propagate.
 *   - Codes: code c is the c-th centroid in ascending order, 3 bits each.
 *   - K layout: one 48-byte row per cache slot; code j of the row occupies
 *     bits [3j, 3j+3) of a 384-bit little-endian bitstream (bytes 3i..3i+2
 *     hold codes 8i..8i+7).
 *   - V layout: tiles of 8 consecutive slots (slot s in tile s/8 at position
 *     r = s%8), 384 bytes each; the code of dim j of the slot at position r
 *     occupies bits [24j + 3r, 24j + 3r + 3) of the tile's little-endian
 *     bitstream. (The same 48 bytes per slot, ordered so that the 8 codes of
 *     one dim are adjacent.)
 *   - Capacity must be a multiple of 32 slots; code arrays and norm arrays
 *     must be 16-byte aligned.
 *   - Rotation parameters: float rot[num_kv_heads][32][8]; block b of head h
 *     is rot[h][b] = {qL.w, qL.x, qL.y, qL.z, qR.w, qR.x, qR.y, qR.z} and maps
 *     dims 4b..4b+3, read as a quaternion v = (w,x,y,z), to qL (x) v (x) conj(qR).
 *     Quaternions are renormalised before use. K and V of a head share it.
 */
#ifndef IQ_H_
#define IQ_H_

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define IQ_API __attribute__((visibility("default")))
#else
#define IQ_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  IQ_OK = 0,
  IQ_ERR_INVALID_ARG = -1,   /* null pointer, negative size, bad enum, Hq % Hkv != 0 ... */
  IQ_ERR_UNSUPPORTED = -2,   /* head_dim != 128, group size > 16 */
  IQ_ERR_CAPACITY = -3,      /* contiguous slot range outside [0, capacity) */
  IQ_ERR_WORKSPACE = -4,     /* workspace smaller than iq_decode_workspace_bytes() */
  IQ_ERR_HIP = -5            /* a HIP launch failed */
} iq_status;

typedef enum { IQ_F32 = 0, IQ_F16 = 1 } iq_dtype;

/* The rotation applied before quantization (arXiv 2608.08081 abstract for the
 * first; zhichai.net essay, section "三种变体", and the sd114.wiki RotorQuant
 * page, section on bypassing the butterfly network, for the two variants).
 * Parameters per KV head, float32, stored quaternions / pairs renormalised on
 * use:
 *   IQ_ROT_WHT_SO4  normalised Walsh-Hadamard transform, then per 4-dim block
 *                   b: v -> qL (x) v (x) conj(qR); rot [Hkv][32][8] = (qL, qR)
 *                   as (w, x, y, z) each: 256 per head.
 *   IQ_ROT_ISO      no WHT; per 4-dim block v -> q (x) v (left-isoclinic);
 *                   rot [Hkv][32][4]: 128 per head.
 *   IQ_ROT_PLANAR   no WHT; per dim pair (2i, 2i+1) the Givens rotation
 *                   (x, y) -> (c x - s y, s x + c y); rot [Hkv][64][2] = (c, s):
 *                   128 per head. */
typedef enum { IQ_ROT_WHT_SO4 = 0, IQ_ROT_ISO = 1, IQ_ROT_PLANAR = 2 } iq_rotation;

/* One layer of the packed cache. All pointers are device memory. */
typedef struct {
  int32_t head_dim;       /* must be 128 */
  int32_t num_kv_heads;   /* Hkv >= 1 */
  int32_t capacity;       /* slots per KV head (one flat token axis shared by all
                             sequences); a multiple of 32 */
  uint8_t* k_codes;       /* [num_kv_heads][capacity][16 * k_bits] K rows, 16-byte aligned */
  uint8_t* v_codes;       /* [num_kv_heads][capacity/8][384] V tiles, 16-byte aligned */
  float* k_norms;         /* [num_kv_heads][capacity] */
  float* v_norms;         /* [num_kv_heads][capacity] */
  const float* rot;       /* rotation parameters, layout per `rotation` */
  int32_t rotation;       /* iq_rotation; K and V of a head share it */
  int32_t k_bits;         /* 3, or 4 for 4-bit K (16-level codebook, code j at
                             bits [4j, 4j+4) of a 64-byte row); V is 3-bit */
} iq_cache_view;

/* Human-readable name of a status code (static string). */
IQ_API const char* iq_status_string(iq_status s);

/* Host only. The codebook: 8 Lloyd-Max centroids of N(0, 1/128) in ascending
 * order and the 7 cell boundaries (midpoints), computed in double and rounded
 * to float (zhichai.net essay, section "Lloyd-Max 最优量化"). Both arrays are
 * host memory written by the call. */
IQ_API iq_status iq_codebook(float centroids[8], float thresholds[7]);

/* Host only. The codebook of `levels` = 8 (3-bit) or 16 (4-bit K, zhichai.net
 * essay, section "K 和 V 的非对称需求": K needs more bits than V) Lloyd-Max
 * levels of N(0, 1/128), ascending, and its levels - 1 midpoints. */
IQ_API iq_status iq_codebook_levels(int32_t levels, float* centroids, float* thresholds);

/* Rotate fp32 vectors with the per-head rotation (the first half of the
 * encode; the same transform is applied to queries before scoring).
 *   x, y      device float [n_tokens][num_heads][128]; y may equal x.
 *   rot       device float, layout of `rotation` (see iq_rotation).
 *   inverse = 0: y = R x (B . Hn . x for IQ_ROT_WHT_SO4); inverse = 1: y = R^-1 x. */
IQ_API iq_status iq_rotate(const float* rot, int32_t rotation, int32_t num_heads, const float* x, float* y,
                    int32_t n_tokens, int32_t inverse, void* stream);

/* Quantize and pack vectors that are already rotated (the second half of the
 * encode: norm, 3-bit codes, packing).
 *   y      device float [n_vectors][128] (rotated coordinates).
 *   codes  device uint8 [n_vectors][48]; norms device float [n_vectors].
 * n = fl32(sqrt(sum y_j^2)) with a double-precision sum; code_j =
 * #{k : y_j > fl32(t_k * n)}. A zero vector gives n = 0 and all-zero codes. */
IQ_API iq_status iq_quantize_pack(const float* y, int64_t n_vectors, uint8_t* codes, float* norms,
                           void* stream);

/* Rotate, quantize and pack new K and V tokens into the cache (the pages'
 * quantize-on-insert; RotorQuant page, deferred quantization section).
 *   k, v        device [n_tokens][num_kv_heads][128] of in_dtype (f32 or f16).
 *   slots       device int32 [n_tokens] destination rows, or NULL for the
 *               contiguous rows first_slot .. first_slot + n_tokens - 1
 *               (checked against capacity on the host). With `slots`, a slot
 *               outside [0, capacity) is skipped on the device (nothing written).
 * Writes view->k_codes rows, the slots' bits of view->v_codes tiles (other
 * slots of a partly written tile keep their codes) and view->k_norms/v_norms
 * entries. Calls that write the same V tile must not run concurrently.
 * Slots in a slot list must be distinct. n_tokens = 0 is a no-op. */
IQ_API iq_status iq_rotate_quantize_append(const iq_cache_view* view, const void* k, const void* v,
                                    iq_dtype in_dtype, int32_t n_tokens, int32_t first_slot,
                                    const int32_t* slots, void* stream);

/* Reconstruct K and V rows explicitly: x_hat = n . Hn . B^T . c[code]
 * (the unfused path; RotorQuant page, inverse-rotation fix for V).
 *   rows first_slot .. first_slot + n_tokens - 1 of every KV head
 *   k_out, v_out  device [n_tokens][num_kv_heads][128] of out_dtype; either
 *                 may be NULL to skip it. */
IQ_API iq_status iq_dequantize(const iq_cache_view* view, int32_t first_slot, int32_t n_tokens,
                        iq_dtype out_dtype, void* k_out, void* v_out, void* stream);

/* Bytes of workspace iq_decode_attention, iq_decode_attention_f16 and
 * iq_append_decode_attention need for these sizes (0 if the sizes are
 * invalid). */
IQ_API size_t iq_decode_workspace_bytes(int32_t n_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t max_seq_len);

/* Decode attention on the packed cache (news article on RotaryQuant:
 * scores on packed K, softmax, accumulation from packed V, inverse rotation;
 * zhichai.net essay: softmax(Q K^T / sqrt(d)) V).
 *   q          device float [n_seqs][num_q_heads][128], one query per sequence.
 *   seq_start  device int32 [n_seqs], first cache row of each sequence.
 *   seq_len    device int32 [n_seqs], rows of each sequence; each must be
 *              <= max_seq_len (a host-side bound that sizes the launch).
 *   scale      softmax scale (1/sqrt(128) for plain attention).
 *   out        device float [n_seqs][num_q_heads][128].
 *   workspace  device memory of at least iq_decode_workspace_bytes() bytes,
 *              16-byte aligned, owned by the caller. It holds the split-K
 *              partial results (no initialisation needed); calls that share a
 *              workspace must not run concurrently.
 *   n_seqs     0 .. 65535.
 * Query head g reads KV head g / (num_q_heads / num_kv_heads); the group size
 * must be 1, 2, 4, 8 or 16. A sequence with seq_len = 0 gets a zero output. A sequence
 * whose rows fall outside [0, capacity), or whose length exceeds max_seq_len,
 * gets NaN outputs (no out-of-bounds read happens). */
IQ_API iq_status iq_decode_attention(const iq_cache_view* view, const float* q, int32_t num_q_heads,
                              const int32_t* seq_start, const int32_t* seq_len, int32_t n_seqs,
                              int32_t max_seq_len, float scale, float* out, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Decode attention over a plain fp16 K/V cache: the FP16-KV baseline, and
 * with iq_dequantize in front of it the unfused path (news article on
 * RotaryQuant, section on memory savings versus speed: fused against unfused
 * kernels, FP16 KV against IsoQuant). Same semantics as iq_decode_attention
 * with K and V given explicitly:
 *   k, v          device fp16; element (row t, KV head h, dim j) at
 *                 k[t * token_stride + h * head_stride + j]. Both strides are
 *                 in elements and multiples of 8; k and v 16-byte aligned.
 *                 [capacity][Hkv][128] (iq_dequantize's output): token_stride
 *                 = 128 Hkv, head_stride = 128. [Hkv][capacity][128]:
 *                 token_stride = 128, head_stride = 128 capacity.
 *   capacity      rows per KV head, a multiple of 32; rows [0, capacity) of
 *                 every head must be readable.
 *   q, seq_start, seq_len, n_seqs, max_seq_len, scale, out: as for
 *                 iq_decode_attention, rows indexed like the cache's slots.
 *   workspace     at least iq_decode_workspace_bytes(n_seqs, num_q_heads,
 *                 num_kv_heads, max_seq_len) bytes, 16-byte aligned.
 * Query head g reads KV head g / (num_q_heads / num_kv_heads); group sizes 1,
 * 2, 4, 8, 16. Empty sequences give 0, invalid ones NaN. */
IQ_API iq_status iq_decode_attention_f16(const void* k, const void* v, int64_t token_stride, int64_t head_stride,
                                  int32_t num_kv_heads, int32_t capacity, const float* q, int32_t num_q_heads,
                                  const int32_t* seq_start, const int32_t* seq_len, int32_t n_seqs,
                                  int32_t max_seq_len, float scale, float* out, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* One decode step: append one new token per sequence and attend to the cache
 * including it, in the two launches of iq_decode_attention (extra
 * work-groups of the first launch encode and score the new token beside the
 * splits). Equivalent to
 * iq_rotate_quantize_append of token s at slot seq_start[s] + seq_len[s]
 * followed by iq_decode_attention over seq_len[s] + 1 slots (the codes and
 * norms written are the same):
 *   k_new, v_new  device [n_seqs][num_kv_heads][128] of in_dtype, 16-byte aligned.
 *   seq_len       device int32 [n_seqs]: tokens already in the cache (<=
 *                 max_seq_len); the new token's slot must be < capacity.
 *   other arguments as for iq_decode_attention (same workspace size).
 * Sequences must not share the new token's slot. A sequence whose rows or new
 * slot fall outside the cache gets NaN outputs and nothing is written for it. */
IQ_API iq_status iq_append_decode_attention(const iq_cache_view* view, const void* k_new, const void* v_new,
                                     iq_dtype in_dtype, const float* q, int32_t num_q_heads,
                                     const int32_t* seq_start, const int32_t* seq_len, int32_t n_seqs,
                                     int32_t max_seq_len, float scale, float* out, void* workspace,
                                     size_t workspace_bytes, void* stream);

/* Size of the library's scratch array on each GPU, the most that
 * iq_append_decode_attention_noalloc can use (16 MiB). */
#define IQ_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * iq_append_decode_attention without a workspace argument. The split-K
 * records go to a scratch array of IQ_NOALLOC_SCRATCH_BYTES that the library
 * holds in device memory, one per GPU, from the library's loading until the
 * process ends; the call allocates nothing. Arguments and results are those
 * of iq_append_decode_attention (same kernels, same plan, same outputs).
 *   Errors: IQ_ERR_WORKSPACE when iq_decode_workspace_bytes() for these
 *   sizes exceeds IQ_NOALLOC_SCRATCH_BYTES (nothing is launched); IQ_ERR_HIP
 *   when the scratch array's address on the stream's GPU cannot be obtained.
 *   The array keeps the last call's contents; no call depends on them.
 *   Calls that overlap on one GPU (other streams, other host threads) share
 *   the array and race: they must be serialised by the caller. */
IQ_API iq_status iq_append_decode_attention_noalloc(const iq_cache_view* view, const void* k_new, const void* v_new,
                                             iq_dtype in_dtype, const float* q, int32_t num_q_heads,
                                             const int32_t* seq_start, const int32_t* seq_len, int32_t n_seqs,
                                             int32_t max_seq_len, float scale, float* out, void* stream);

/* Bytes of workspace iq_decode_attention_deferred needs (0 if invalid). */
IQ_API size_t iq_decode_deferred_workspace_bytes(int32_t n_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                          int32_t max_prefix_len, int32_t max_seq_len);

/* Decode attention over a deferred-quantization cache (sd114.wiki RotorQuant
 * page, deferred-quantization strategy; zhichai.net essay, section
 * "延迟量化"): the prompt's K/V stay fp16, tokens added later are packed.
 * Sequence s attends to its fp16 prefix followed by its packed suffix:
 *   view, seq_start, seq_len, max_seq_len: the packed suffix, as for
 *                 iq_decode_attention (seq_len may be 0).
 *   k16, v16, token_stride, head_stride, capacity16: the fp16 prefix cache,
 *                 as for iq_decode_attention_f16; it shares the view's KV
 *                 heads (and its rotation, which the prefix's partial results
 *                 are rotated by so that both merge in one basis).
 *   prefix_start, prefix_len (device int32 [n_seqs]), max_prefix_len: the
 *                 prefix rows of each sequence (prefix_len may be 0).
 *   q, num_q_heads, n_seqs, scale, out: as for iq_decode_attention.
 *   workspace     at least iq_decode_deferred_workspace_bytes() bytes,
 *                 16-byte aligned.
 * A sequence with no tokens gets 0; one whose prefix or suffix rows are
 * invalid gets NaN. */
IQ_API iq_status iq_decode_attention_deferred(const iq_cache_view* view, const int32_t* seq_start,
                                       const int32_t* seq_len, int32_t max_seq_len, const void* k16,
                                       const void* v16, int64_t token_stride, int64_t head_stride,
                                       int32_t capacity16, const int32_t* prefix_start, const int32_t* prefix_len,
                                       int32_t max_prefix_len, const float* q, int32_t num_q_heads, int32_t n_seqs,
                                       float scale, float* out, void* workspace, size_t workspace_bytes,
                                       void* stream);

#ifdef __cplusplus
}
#endif

#endif /* IQ_H_ */
