// Pieces shared by the decode kernels (packed 3-bit cache and fp16 cache):
// split-K geometry, the per-wave online-softmax state, the wave-level
// reductions and the MFMA wrapper.
#pragma once

#include <math.h>

#include "iq_device.h"
#include "iq_launch.h"

namespace iq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

union H8 {
  half8 h;
  uint32_t u[4];
  uint2 u2[2];
  uint4 u4;
};

constexpr int kDecThreads = 256;
constexpr int kWaves = kDecThreads / 64;
constexpr int kBlk = 32;             // cache slots per wave iteration
constexpr int kRec = 132;            // floats per partial record: m, l, 2 pad, o[128]
constexpr int kTargetBlocks = 512;   // split-K occupancy target (work-groups): 2 per CU
constexpr int kMinBlocksPerSplit = 4;
// Split length cap (blocks of 32 slots, 16 per wave): long enough that a
// split's fixed prologue and epilogue are small beside its loop, short enough
// that the splits of a ragged batch balance over the CUs (measured on 32
// sequences of 1K..32K tokens: 32 blocks 217 us, 48 204 us, 64 200 us, 128
// 205 us per layer).
constexpr int kMaxBlocksPerSplit = 64;
constexpr int kMaxSplits = 2048;
constexpr int kMergeLanes = kDim / 4;                    // lanes per record, 4 dims each
// records per lane per round of loads (a fifth, so that 129 records take one
// round, measured no faster: a merge work-group is bound by how fast its CU
// pulls the ~68 KB of records, not by the rounds)
constexpr int kMergeChunk = 4;
// Online-softmax reference m (log2 units). A weight w = 2^(s - m) (times the
// V norm in the packed decode) enters the PV MFMA as fp16 hi/lo halves. m is
// raised only when some weight would exceed 2^kWeightMaxLog2, and then to
// where the largest weight is 2^kWeightRefLog2: the weights stay below the
// fp16 maximum (65504 > 2^15.09), and those down to 2^-21 of the largest keep
// normal fp16 halves, so that accumulator rescaling is rare and small weights
// keep their precision.
constexpr float kWeightMaxLog2 = 15.0f;
constexpr float kWeightRefLog2 = 7.0f;
// Start value of the packed decode's reference: finite, so that 2^(s - m)
// overflows for the first token that is not masked, which raises m; a wave
// that saw no token keeps it, and its weight in the merge of the waves is 0.
constexpr float kRefStart = -0x1p126f;

// Max (or sum) of x over lanes i and i ^ 16, then i ^ 32, of a full wave: the
// gfx950 row swaps hand each lane itself and its partner, in some order, in
// the two halves of the result, so a commutative op on the halves is the
// reduction (one instruction per step, no lane-index arithmetic). The halves
// are copied to scalars before the bit casts: a bit cast of a vector element
// is compiled as a read of the vector's first element.
// Max of floats as the hardware computes it (a quiet NaN operand yields the
// other one, as fmaxf does). fmaxf itself is compiled with a canonicalising
// max of each operand not known to be canonical (loads, inline-asm outputs,
// lane exchanges) in front: two or three instructions per max. No signalling
// NaN reaches these.
__device__ __forceinline__ float max_hw(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float max3_hw(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

template <bool kMax>
__device__ __forceinline__ float rows_reduce(float x) {
  auto op = [](float u, float v) { return kMax ? max_hw(u, v) : u + v; };
  const uint32_t b = __builtin_bit_cast(uint32_t, x);
  const auto r16 = __builtin_amdgcn_permlane16_swap(b, b, false, false);
  const uint32_t a0 = r16[0], a1 = r16[1];
  x = op(__builtin_bit_cast(float, a0), __builtin_bit_cast(float, a1));
  const uint32_t c = __builtin_bit_cast(uint32_t, x);
  const auto r32 = __builtin_amdgcn_permlane32_swap(c, c, false, false);
  const uint32_t c0 = r32[0], c1 = r32[1];
  return op(__builtin_bit_cast(float, c0), __builtin_bit_cast(float, c1));
}

// A value no kernel writes while the reading kernel runs, read through the
// constant address space: at a wave-uniform address this is a scalar load,
// which neither waits behind nor holds up the wave's vector loads.
template <typename T>
__device__ __forceinline__ T load_invariant(const T* p) {
  return *(const __attribute__((address_space(4))) T*)(p);
}

// Sequence bounds that are valid for the launch: rows inside the cache and a
// length within max_seq_len.
template <typename Args>
__device__ __forceinline__ bool seq_check(const Args& a, int st, int ln) {
  return st >= 0 && ln >= 0 && ln <= a.max_seq_len && static_cast<int64_t>(st) + ln <= a.capacity;
}

template <typename Args>
__device__ __forceinline__ bool seq_ok(const Args& a, int s, int* start, int* len) {
  const int st = load_invariant(a.seq_start + s);
  const int ln = load_invariant(a.seq_len + s);
  *start = st;
  *len = ln;
  return seq_check(a, st, ln);
}

// 32-slot blocks covering [start, start + len) from the 32-aligned base.
__device__ __forceinline__ int n_blocks(int start, int len) {
  return len > 0 ? ((start - (start & ~(kBlk - 1)) + len + kBlk - 1) / kBlk) : 0;
}

// Work-group barrier for LDS traffic only: waits for this wave's LDS
// operations, not for its global loads. (__syncthreads' fence also waits for
// every global->LDS load in flight, which would drain the block prefetch.)
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// LDS byte address of a __shared__ object (for inline asm operands).
template <typename T>
__device__ __forceinline__ uint32_t lds_address(const T* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) T*)(p)));
}

__device__ __forceinline__ floatx4 mfma16(const half8& a, const half8& b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float dpp_row_ror8(float x) {
  return dpp_f32<0x128>(x);   // row_ror:8
}

// 2^x on the transcendental unit (results below 2^-126 flush to 0, which the
// softmax weights tolerate).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// fp16 pair (x, x) of one value.
__device__ __forceinline__ uint32_t dup16(float x) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(x, x));
}

// Per-wave running state of the online softmax and the PV accumulators.
struct WaveState {
  floatx4 acc[8];      // [dim tile d]: rows 4q + i, column n (dim 8n + d)
  float m, l;
};

// Splits of (seq, kv head) that hold at least one block: split k covers
// blocks [k bps, (k+1) bps), the last one also the block that a start not
// aligned to 32 adds beyond the plan.
__device__ __forceinline__ int live_splits(int nblk, int bps, int n_splits) {
  return nblk > 0 ? min(n_splits, (nblk + bps - 1) / bps) : 0;
}

// Sum (or max) over the 32 lanes of a half-wave: four DPP rotations within
// each row of 16, then one row swap (lane ^ 16) across the two rows.
template <bool kMax>
__device__ __forceinline__ float half_wave_reduce(float x) {
  auto op = [](float u, float v) { return kMax ? fmaxf(u, v) : u + v; };
  x = op(x, dpp_f32<0x128>(x));   // row_ror:8
  x = op(x, dpp_f32<0x124>(x));   // row_ror:4
  x = op(x, dpp_f32<0x122>(x));   // row_ror:2
  x = op(x, dpp_f32<0x121>(x));   // row_ror:1
  const uint32_t b = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane16_swap(b, b, false, false);
  const uint32_t r0 = r[0], r1 = r[1];   // this lane and lane ^ 16, in some order
  return op(__builtin_bit_cast(float, r0), __builtin_bit_cast(float, r1));
}

}  // namespace iq
