// Device helpers for gfx950 (CDNA4, wave64): element traits, bf16 packing,
// cross-lane reductions on DPP, and the launch interface of the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pagedkv.h"

namespace pa {

constexpr int kWave = 64;

// Storage traits. One lane moves 16 bytes per load: VEC elements.
template <int DTYPE> struct Elt;
template <> struct Elt<PA_F32> { static constexpr int bytes = 4; };
template <> struct Elt<PA_BF16> { static constexpr int bytes = 2; };
template <> struct Elt<PA_FP8_E4M3> { static constexpr int bytes = 1; };

template <int DTYPE, int D>
struct RowShape {
  static constexpr int VEC = 16 / Elt<DTYPE>::bytes;  // elements per 16-byte load
  static constexpr int LPR = D / VEC;                 // lanes covering one token row
  static constexpr int NR = kWave / LPR;              // token rows per wave-wide load
  static_assert(LPR >= 1 && LPR <= kWave && kWave % LPR == 0, "unsupported head_dim");
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming load: K/V rows are read once per step, so they are marked
// non-temporal to keep them from displacing reused data in the caches.
__device__ __forceinline__ uint4 load_stream16(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> packed bfloat16 pair (low half = lo), round to nearest even,
// NaN kept quiet: one v_cvt_pk_bf16_f32 on gfx950.
typedef __bf16 bf16x2_native __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const bf16x2_native v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint32_t f32_to_bf16(float f) { return pack_bf16(f, 0.f) & 0xffffu; }

// DPP move inside rows of 16 lanes (all rows and banks enabled).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, true));
}
constexpr int kQuadSwap1 = 0xb1;      // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4e;      // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141; // lane i <-> 7-i inside each half row
constexpr int kRowMirror = 0x140;     // lane i <-> 15-i inside each row

// Sum over aligned groups of N consecutive lanes; every lane gets its group's sum.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp<kQuadSwap1>(x);
  if constexpr (N >= 4) x += dpp<kQuadSwap2>(x);
  if constexpr (N >= 8) x += dpp<kRowHalfMirror>(x);
  if constexpr (N >= 16) x += dpp<kRowMirror>(x);
  if constexpr (N >= 32) x += __shfl_xor(x, 16);
  if constexpr (N >= 64) x += __shfl_xor(x, 32);
  return x;
}

// MFMA operand types.
typedef short bf16x8_t __attribute__((ext_vector_type(8)));
typedef short bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

// 16 E4M3 codes -> 16 bf16 values (exact) in two 16-byte chunks.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3_pair(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(int(w), 1.f, HI));
}
__device__ __forceinline__ void widen_e4m3(const uint4& c, uint4& lo, uint4& hi) {
  lo = make_uint4(e4m3_pair<false>(c.x), e4m3_pair<true>(c.x), e4m3_pair<false>(c.y),
                  e4m3_pair<true>(c.y));
  hi = make_uint4(e4m3_pair<false>(c.z), e4m3_pair<true>(c.z), e4m3_pair<false>(c.w),
                  e4m3_pair<true>(c.w));
}

// ---------------------------------------------------------------- launches --
struct DecodeArgs {
  void* out;
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  float* ws_acc;   // [2 * workers][heads per unit][D] unnormalised partial sums
  float2* ws_ml;   // [2 * workers][kMLStride] (running max in log2 units, denominator) per head
  int4* ws_seg;    // [workers] split segment each wave started: (seq, unit, last wave, head)
  int32_t max_blocks_per_seq;
  int32_t num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, dtype;
  int32_t workers;
  int32_t num_cus;  // compute units of the device (sizes the workgroups)
  float scale;
  float k_scale, v_scale;  // FP8 pools: a code c stands for e4m3(c) * scale (1 otherwise)
  float* lse;  // optional [num_seqs][num_q_heads]: log2 of each row's softmax denominator
               // in log2-scaled score units (-inf for an empty sequence)
  int32_t len_offset;  // attend to tokens len_offset .. seq_lens[s]-1; block_tables then
                       // points at the row entry of block len_offset / block_size
  // Grouped decode (set prefix_lens): the sequences form num_groups consecutive
  // groups of group_size; the first prefix_lens[s] tokens of every member of a
  // group (a multiple of block_size, equal within the group) are the same
  // physical blocks. Each (group, KV head) is one unit of group_size * G <= 16
  // columns: the shared blocks are read once for all of them, then each
  // member's own tokens for its columns only.
  const int32_t* prefix_lens;
  int32_t group_size, num_groups;
  // Several query rows per sequence (set q_start_loc, int32 [num_seqs + 1]):
  // sequence s has rows q_start_loc[s] .. q_start_loc[s+1]-1 of q and out,
  // row r at position seq_lens[s] - rows + r, attending causally to keys
  // 0 .. that position. Each (sequence, KV head) is one unit whose columns
  // are (row r, query head h) = r * G + h, at most kMultiRowCols of them.
  const int32_t* q_start_loc;
  // Multi-row units of more than 16 columns (mr_pair = 1) run on a workgroup
  // of two waves, each holding 16 of the columns and loading half of every
  // K/V tile into LDS that both read; `workers` then counts the pairs.
  int32_t mr_pair;
};
constexpr int kMultiRowCols = 32;
constexpr int kMultiRowWaves = 8;  // multi-row decode: waves per CU (two per SIMD)

hipError_t launch_cache_write(const pa_pool& pool, const void* k_new, const void* v_new,
                              const int64_t* slots, int32_t T, hipStream_t stream);
hipError_t launch_stream_read(const void* buf, size_t bytes, int grid, uint32_t* sink,
                              hipStream_t stream);
constexpr int kSwapBatch = 256;  // block pairs per swap launch (kernel argument size)
struct SwapBatch {
  int32_t pairs[2 * kSwapBatch];  // (src, dst) block ids, checked on the host
};
// Copies n <= kSwapBatch whole blocks (block_bytes per block, K and V) from
// the src pool to the dst pool; either side may be pinned host memory given
// by its device-accessible address.
hipError_t launch_swap_blocks(const SwapBatch& b, int32_t n, const void* src_k, const void* src_v,
                              void* dst_k, void* dst_v, int64_t block_bytes, hipStream_t stream);
hipError_t launch_copy_blocks(const pa_pool& pool, const int32_t* src_dst, int32_t n,
                              hipStream_t stream);
// Returns hipErrorInvalidValue for shapes without a compiled kernel.
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
// Columns (query heads of all members) of one unit of the grouped decode.
constexpr int kGroupedCols = 16;
// (max, denominator) records per partial slot of the decode workspace: one
// 128-byte line per slot, whatever the unit's head count, so that a slot's
// records never share a line with another slot's.
constexpr int kMLStride = 16;
bool decode_supported(int dtype, int head_dim, int group);
// Query heads handled together with their KV head by one wave (divides the group size).
int decode_heads_per_unit(int group);

// Shared-prefix decode: the regular decode runs over the suffixes (table rows
// offset by the shared blocks, len_offset = their tokens, lse on), then
// launch_prefix computes the shared part once and merges it into `out`.
struct PrefixArgs {
  void* out;                    // [S][Hq][D] bf16: suffix output in, final output out
  const void* q;                // [S][Hq][D] bf16
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_tables;  // row 0's first num_prefix_blocks entries: the shared blocks
  const float* lse;             // [S][Hq] suffix log-sum-exp (log2 units, -inf if empty)
  uint16_t* p_acc;              // [n_split][S][Hq][D] unnormalised prefix partials, bf16
  float2* p_ml;                 // [n_split][S][Hq] (max in log2 units, denominator)
  int32_t num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, dtype;
  int32_t num_prefix_blocks, n_split;
  float scale, k_scale, v_scale;
};
struct PrefixPlan {
  int32_t groups_per_wave;  // 16-column groups one wave computes (1 or 2)
  int32_t n_cblk;           // column blocks (one per wave) per KV head (S * G columns)
  int32_t n_tiles;          // 16-key tiles of the shared part
  int32_t tiles_per_split;  // tiles per key range
  int32_t n_split;          // key ranges (partials per row)
};
PrefixPlan prefix_plan(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t block_size, int32_t num_prefix_blocks, int32_t num_cus);
hipError_t launch_prefix(const PrefixArgs& a, const PrefixPlan& p, hipStream_t stream);

struct PrefillArgs {
  void* out;
  const void* q;
  const int32_t* q_start_loc;
  const int32_t* seq_lens;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_tables;
  int32_t max_blocks_per_seq;
  int32_t num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_q_len;
  float scale;
};
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);
bool prefill_supported(int dtype, int head_dim, int block_size, int group);

}  // namespace pa
