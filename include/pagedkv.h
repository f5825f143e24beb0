/*
 * pagedkv.h — C ABI of a paged KV-cache attention library for AMD MI355X (gfx950).
 *
 * The KV cache of every sequence lives in fixed-size physical blocks taken
 * from one shared pool; a per-sequence block table maps logical block j to a
 * physical block ("Why PagedAttention multiplies LLM serving throughput",
 * section "Block Table: the GPU page table"; "vLLM PagedAttention explained",
 * sections 3.1-3.4). This library provides the device operations on that
 * pool — writing new tokens' K/V into their slots, block copies for
 * copy-on-write, decode attention and chunked-prefill attention read through
 * the block tables — and a host block allocator that produces the tables.
 *
 * Conventions shared by every device entry point
 *  - Memory: every device pointer is caller-owned device memory; the library
 *    never allocates or frees device memory. Host pointers are marked "host".
 *  - Streams: `stream` is a hipStream_t passed as void* (NULL = null stream).
 *    Device calls are asynchronous on that stream; they return after the
 *    launch is queued.
 *  - Layout: all arrays are dense, row-major, without padding.
 *      k_pool, v_pool : [num_blocks][num_kv_heads][block_size][head_dim]
 *    i.e. head-major inside a block, so one (block, head) tile is contiguous.
 *    Token t of a sequence with table `bt` is at physical block bt[t / B],
 *    offset t % B. A slot is the flat index block * B + offset
 *    ("LLM inference engine internals", section 2.3, append_slot).
 *  - Grouped heads: query head h reads KV head h / (num_q_heads / num_kv_heads).
 *  - Errors: entry points return a pa_status and never abort. Every argument
 *    that can be checked on the host is checked before any launch; when such a
 *    check fails no work is queued. A call that launches several kernels and
 *    gets PA_ERR_HIP from a later launch may leave its earlier launches queued.
 *    Contents of device arrays (block ids, slots, lengths, copy pairs) are
 *    preconditions: they must index inside the pool and the tables. The
 *    pa_check_* functions below verify them on host copies of those arrays
 *    (a debug aid; the device calls do not read them back).
 *    pa_last_error() gives a message for the most recent failure on the calling
 *    thread.
 *  - Softmax scale: every attention call takes `scale` (typically
 *    1/sqrt(head_dim)); it must be finite and > 0, else PA_ERR_INVALID.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_INVALID = -1,      /* bad argument (null pointer, size, shape mismatch)      */
  PA_ERR_UNSUPPORTED = -2,  /* valid but not built (dtype, head_dim, group size, ...) */
  PA_ERR_OOM = -3,          /* allocator: not enough free blocks; state unchanged     */
  PA_ERR_STATE = -4,        /* allocator: unknown / duplicate sequence id             */
  PA_ERR_WORKSPACE = -5,    /* decode: workspace smaller than required                */
  PA_ERR_HIP = -6           /* a HIP runtime call or kernel launch failed             */
} pa_status;

typedef enum pa_dtype {
  PA_F32 = 0,      /* IEEE float32                                               */
  PA_BF16 = 1,     /* bfloat16 (upper 16 bits of float32)                        */
  PA_FP8_E4M3 = 2  /* KV pools only: 8-bit codes of the OCP E4M3 format (1 sign,
                      4 exponent bits with bias 7, 3 mantissa bits, largest
                      finite value 448, no infinities), one scale per pool.
                      This is the FP8 KV cache of "vLLM PagedAttention
                      explained", section 7 (the pages fix neither format nor
                      scale; both are this library's reading).              */
} pa_dtype;

/* One layer's KV pool: two device arrays of identical shape and dtype. */
typedef struct pa_pool {
  void* k_pool;            /* device, [num_blocks][num_kv_heads][block_size][head_dim] */
  void* v_pool;            /* device, same shape                                       */
  int32_t num_blocks;      /* > 0                                                      */
  int32_t num_kv_heads;    /* > 0                                                      */
  int32_t block_size;      /* B: power of two, 1..256                                  */
  int32_t head_dim;        /* D: 64 or 128                                             */
  int32_t dtype;           /* pa_dtype                                                 */
  float k_scale;           /* PA_FP8_E4M3: K code c stands for e4m3(c) * k_scale; finite, > 0 */
  float v_scale;           /* PA_FP8_E4M3: the same for V. Both ignored for other dtypes.      */
} pa_pool;

const char* pa_status_string(pa_status s);
/* Message for the last failing call on this thread ("" if none). */
const char* pa_last_error(void);
/* Library version: major * 10000 + minor * 100 + patch. */
int32_t pa_version(void);

/* ---------------------------------------------------------------- device --- */

/*
 * pa_cache_write — store the K/V of new tokens into their slots.
 * ("vLLM PagedAttention explained", section 3.3: the KV of the prompt and of
 * each generated token is written into the physical blocks the block table
 * maps; slot rule of "LLM inference engine internals", section 2.3.)
 *   k_new, v_new : device, [num_tokens][num_kv_heads][head_dim], pool dtype
 *                  (bfloat16 for a PA_FP8_E4M3 pool)
 *   slot_mapping : device, int64 [num_tokens]; token i goes to block
 *                  slot / B, offset slot % B, for every KV head. A negative
 *                  slot means "skip this token" (padding).
 * For F32 and BF16 pools the result is a byte copy: bit-exact. For an FP8
 * pool each value x is stored as the E4M3 code nearest to
 * min(max(x / scale, -448), 448), x / scale an IEEE single-precision
 * division, ties to the even mantissa (a deterministic function of x and the
 * pool's k_scale / v_scale). Quotients beyond +-448, +-infinity included,
 * saturate to the code of +-448 (0x7E / 0xFE); a NaN value of either sign is
 * stored as the NaN code 0x7F. Slots must be distinct and < num_blocks * B;
 * nothing else in the pool is touched. num_tokens == 0 is a no-op.
 */
pa_status pa_cache_write(const pa_pool* pool, const void* k_new, const void* v_new,
                         const int64_t* slot_mapping, int32_t num_tokens, void* stream);

/*
 * pa_copy_blocks — copy whole physical blocks (all KV heads, K and V):
 * pool[dst] = pool[src] for each pair, the device side of copy-on-write
 * ("vLLM PagedAttention explained", section 4.1; the scheduler's
 * blocks_to_copy output, "LLM inference engine internals", section 3.1).
 *   src_dst : device, int32 [num_pairs][2] = {src, dst}. No block may appear
 *             both as a source and as a destination in one call.
 * Bit-exact. num_pairs == 0 is a no-op.
 */
pa_status pa_copy_blocks(const pa_pool* pool, const int32_t* src_dst, int32_t num_pairs,
                         void* stream);

/* Direction of pa_swap_blocks. */
enum { PA_SWAP_OUT = 0, PA_SWAP_IN = 1 };

/*
 * pa_swap_blocks — move whole blocks between the device pool and a CPU swap
 * space, the device side of preemption by swapping ("LLM inference engine
 * internals", sections 3.1 and 3.2: the scheduler's blocks_to_swap_out /
 * blocks_to_swap_in; "Why PagedAttention multiplies LLM serving throughput",
 * section "Scheduling and preemption"). One kernel per 256 pairs reads and
 * writes the host pool across the host link directly (no staging copy).
 *   device_pool : the pool in device memory
 *   host_pool   : a pool of the same num_kv_heads, block_size, head_dim, dtype
 *                 (and FP8 scales) whose k_pool / v_pool are pinned host memory
 *                 the device can address (hipHostMalloc, or a pinned torch
 *                 tensor); num_blocks is its own
 *   src_dst     : HOST, int32 [num_pairs][2] = {src, dst}, read during the
 *                 call. PA_SWAP_OUT: host[dst] = device[src]; PA_SWAP_IN:
 *                 device[dst] = host[src]. Every id must lie in its pool and no
 *                 destination may appear twice (PA_ERR_INVALID otherwise,
 *                 checked before anything is launched)
 *   direction   : PA_SWAP_OUT or PA_SWAP_IN
 * Bit-exact. Asynchronous on `stream`: synchronize it before the host reads a
 * swapped-out block, and keep the host pool allocated and unchanged until the
 * stream has passed the call. Memory that HIP does not know as pinned host
 * memory (e.g. plain malloc) is rejected with PA_ERR_INVALID.
 */
pa_status pa_swap_blocks(const pa_pool* device_pool, const pa_pool* host_pool,
                         const int32_t* src_dst, int32_t num_pairs, int32_t direction,
                         void* stream);

/*
 * pa_probe_stream_read — measurement aid, not part of the attention path:
 * reads `bytes` of device memory once, with 16-byte non-temporal loads from
 * `grid` workgroups of 256 threads (grid <= 0: 16 per compute unit), each
 * wavefront reading contiguous 8 KB runs (8 loads in flight per lane). Timing
 * it gives this device's streaming-read rate, the ceiling that the decode
 * kernels' HBM rate is compared against.
 *   buf  : device, 16-byte aligned; bytes a multiple of 16 (0: no-op)
 *   sink : device uint32; written only if the XOR of all loaded words equals
 *          a fixed constant (it keeps the loads from being optimized away)
 */
pa_status pa_probe_stream_read(const void* buf, size_t bytes, int32_t grid, uint32_t* sink,
                               void* stream);

/*
 * Workspace needed by pa_decode, in bytes, for these sizes and worker count
 * (0 = the library's default: sized for 8 wavefronts per compute unit of the
 * current device, which covers every default launch). Returns 0 for invalid
 * sizes.
 */
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t num_workers);

/*
 * pa_decode — decode-step attention through the block tables.
 * For every sequence s and query head h: out[s][h] = softmax(scale * K_s q) V_s
 * over the seq_lens[s] cached tokens of s, the newest token included
 * ("vLLM PagedAttention explained", section 3.3 step 2; kernel outline of
 * "LLM inference engine internals", section 2.4, whose softmax and V step are
 * completed here). The work — every (sequence, KV head) cut into 16-token
 * tiles — is split evenly over `num_workers` wavefronts; a sequence split
 * between wavefronts is recombined exactly with the log-sum-exp rule.
 *   out          : device, [num_seqs][num_q_heads][head_dim], dtype of the pool
 *                  (bfloat16 for a PA_FP8_E4M3 pool)
 *   q            : device, [num_seqs][num_q_heads][head_dim], same dtype as out
 *   block_tables : device, int32 [num_seqs][max_blocks_per_seq]; only the first
 *                  ceil(seq_lens[s] / B) entries of a row are read
 *   seq_lens     : device, int32 [num_seqs], each in [0, max_blocks_per_seq * B];
 *                  a sequence of length 0 gets an all-zero output
 *   num_q_heads  : multiple of pool->num_kv_heads
 *   scale        : softmax scale, finite and > 0 (typically 1/sqrt(head_dim))
 *   num_workers  : 0 = default (8 wavefronts per compute unit; 4 for bf16
 *                  pools whose query groups run on the matrix cores, 4 or
 *                  more query heads per unit); any positive count gives the
 *                  same result up to fp32 rounding order
 *   workspace    : device, >= pa_decode_workspace_bytes(...) bytes, 16-byte
 *                  aligned; scratch (no contents are needed before or kept
 *                  after a call). Calls that share a workspace must not overlap.
 * Two kernels run on the stream: the split decode, then the combine of the
 * partials of sequences that were split between wavefronts.
 * Accumulation is fp32 for every dtype; bf16 output is rounded to nearest
 * even. An FP8 pool is read as e4m3(code) * scale: the codes widen exactly
 * to bfloat16 and the two scales are applied to the scores and the output.
 */
pa_status pa_decode(void* out, const void* q, const pa_pool* pool,
                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                    float scale, int32_t num_workers,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_noalloc — pa_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc). Same arguments, kernels and results as pa_decode with
 * the same num_workers, but no workspace argument: the scratch lives in a
 * static device array of the library, pa_decode_noalloc_scratch_bytes()
 * (32 MiB) per device, held by every device the library runs on until the
 * process ends. The caller still passes inputs and outputs. The call
 * allocates nothing; its first call on a device looks up that device's copy
 * of the array. A call whose workspace (pa_decode_workspace_bytes) exceeds
 * the array returns PA_ERR_WORKSPACE with nothing queued; the default worker
 * count needs at most 16.6 MiB on 256 compute units. All calls on one device
 * share its array: calls that overlap on one device (other streams, other
 * host threads) race and must be serialized by the caller.
 */
pa_status pa_decode_noalloc(void* out, const void* q, const pa_pool* pool,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                            float scale, int32_t num_workers, void* stream);
/* Bytes of the static scratch array behind pa_decode_noalloc. */
size_t pa_decode_noalloc_scratch_bytes(void);

/*
 * Workspace needed by pa_decode_shared_prefix, in bytes (0 for invalid sizes).
 * block_size and num_prefix_blocks size the partials of the shared part.
 */
size_t pa_decode_shared_prefix_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                               int32_t num_kv_heads, int32_t head_dim,
                                               int32_t block_size, int32_t num_prefix_blocks,
                                               int32_t num_workers);

/*
 * pa_decode_shared_prefix — pa_decode for a batch whose block tables all begin
 * with the same num_prefix_blocks physical blocks, the case prefix caching
 * produces when requests share a prompt start ("Why PagedAttention multiplies
 * LLM serving throughput", section "Automatic prefix caching"; "LLM inference
 * engine internals", section 2.3). The result is the same attention as
 * pa_decode gives (every sequence attends over all seq_lens[s] tokens), but
 * the shared blocks are read once per KV head for the whole batch instead of
 * once per sequence:
 *   1. the tail of each sequence (tokens P*B .. seq_lens[s]-1) runs through the
 *      pa_decode kernels, which also record each row's log-sum-exp;
 *   2. one pass on the matrix cores attends all num_seqs * G query rows of a KV
 *      head to the P*B shared tokens, keys cut into ranges, and writes
 *      unnormalised partials (sums as bf16, maxima and denominators fp32);
 *   3. a merge combines the partials and the tail result by the log-sum-exp
 *      rule into `out`.
 * Arguments are those of pa_decode, plus:
 *   num_prefix_blocks : host, P in [0, max_blocks_per_seq]. Precondition: for
 *                  every s, block_tables[s][0..P-1] == block_tables[0][0..P-1]
 *                  and seq_lens[s] >= P * B (the shared blocks are full). The
 *                  library reads the shared blocks through row 0 only; a batch
 *                  that breaks the precondition gets wrong results (tails
 *                  shorter than 0 count as 0). P = 0 is the plain pa_decode.
 *   workspace    : device, >= pa_decode_shared_prefix_workspace_bytes(...)
 *                  bytes, 16-byte aligned, scratch; calls sharing one must
 *                  not overlap.
 * bf16 and PA_FP8_E4M3 pools, head_dim 64 or 128 (PA_ERR_UNSUPPORTED
 * otherwise); output bf16. The tail result is rounded to bf16 once before the
 * merge, which adds at most one bf16 rounding of the tail's share of each
 * output element.
 */
pa_status pa_decode_shared_prefix(void* out, const void* q, const pa_pool* pool,
                                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                                  const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                                  float scale, int32_t num_prefix_blocks, int32_t num_workers,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* Workspace needed by pa_decode_grouped, in bytes (0 for invalid sizes). */
size_t pa_decode_grouped_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                         int32_t num_kv_heads, int32_t head_dim,
                                         int32_t num_workers);

/*
 * pa_decode_grouped — pa_decode for a batch of groups of sequences that share
 * the blocks of a common start: the parallel samples of one prompt, or the
 * beams of one beam search ("vLLM PagedAttention explained", sections 4.1 and
 * 4.2: forked sequences share their blocks through reference counts until
 * they diverge). The result is the same attention as pa_decode gives (every
 * sequence attends over its own seq_lens[s] tokens), but a group's shared
 * blocks are read once per KV head for the whole group instead of once per
 * member: the members' query heads are the columns of one unit on the matrix
 * cores, which scores the shared blocks for all of them and then each
 * member's own later blocks for that member's columns only.
 * Arguments are those of pa_decode, plus:
 *   prefix_lens  : device, int32 [num_seqs]: the first prefix_lens[s] tokens
 *                  of sequence s are the same physical blocks for every
 *                  member of its group. Precondition: a multiple of B, equal
 *                  within each group, <= seq_lens[s], and block_tables rows of
 *                  a group equal in their first prefix_lens / B entries
 *                  (pa_group_prefix_lens computes it from host tables,
 *                  pa_check_grouped checks it). Shared blocks are read through
 *                  the group's first row; a batch that breaks the
 *                  precondition gets wrong results. 0 everywhere is valid
 *                  (nothing read once).
 *   group_size   : sequences 0..group_size-1 form group 0, and so on;
 *                  num_seqs must be a multiple of it. Groups whose query heads
 *                  (group_size * num_q_heads / num_kv_heads) exceed 16 are
 *                  handled as sub-groups of the largest divisor that fits (the
 *                  shared blocks are then read once per sub-group);
 *                  PA_ERR_UNSUPPORTED when even one sequence's query heads
 *                  per KV head exceed 16.
 *   num_workers  : 0 = default (4 wavefronts per compute unit for bf16
 *                  pools, 8 for FP8 pools)
 *   workspace    : device, >= pa_decode_grouped_workspace_bytes(...) bytes,
 *                  16-byte aligned, scratch; calls sharing one must not overlap.
 * bf16 and PA_FP8_E4M3 pools, head_dim 64 or 128 (PA_ERR_UNSUPPORTED
 * otherwise); output in bf16, fp32 accumulation. Two kernels: the grouped
 * decode, then the log-sum-exp combine of units split between wavefronts.
 */
pa_status pa_decode_grouped(void* out, const void* q, const pa_pool* pool,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* seq_lens, const int32_t* prefix_lens,
                            int32_t num_seqs, int32_t group_size, int32_t num_q_heads,
                            float scale, int32_t num_workers, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * pa_prefill_chunk — causal attention of a chunk of prompt rows per sequence
 * over that sequence's paged K/V ("vLLM PagedAttention explained", section
 * 7.2: a long prompt is processed in chunks that join the block table).
 * The chunk's own K/V must already be in the pool (pa_cache_write).
 *   out, q       : device, bf16 [total_rows][num_q_heads][head_dim];
 *                  rows q_start_loc[s] .. q_start_loc[s+1]-1 belong to sequence s
 *   q_start_loc  : device, int32 [num_seqs + 1], non-decreasing, q_start_loc[0] = 0
 *   seq_lens     : device, int32 [num_seqs]: tokens in the pool for s, chunk
 *                  included; chunk row i sits at absolute position
 *                  seq_lens[s] - q_len_s + i and sees keys 0 .. that position
 *   max_q_len    : host, >= every q_len_s (sizes the launch)
 * bf16 only (PA_ERR_UNSUPPORTED otherwise); fp32 accumulation.
 */
pa_status pa_prefill_chunk(void* out, const void* q, const int32_t* q_start_loc,
                           const int32_t* seq_lens, const pa_pool* pool,
                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                           int32_t num_seqs, int32_t num_q_heads, int32_t max_q_len,
                           float scale, void* stream);

/*
 * pa_attention_mixed — one call for a batch that mixes decode sequences and
 * chunked-prefill sequences, as a scheduler with chunked prefill forms it
 * ("vLLM PagedAttention explained", section 7.2: a prompt chunk joins the
 * decode requests of the same step). Every query row attends causally over its
 * own sequence's paged K/V; the row's position is seq_lens[s] - q_len_s + i.
 * Sequences 0 .. num_decode-1 are decode sequences with one row each (rows
 * 0 .. num_decode-1, the pa_decode kernels); sequences num_decode ..
 * num_decode+num_prefill-1 are prefill chunks (the pa_prefill_chunk kernel).
 *   out, q       : device, [total_rows][num_q_heads][head_dim], the pool's dtype
 *                  (bf16 for a PA_FP8_E4M3 pool)
 *   q_start_loc  : device, int32 [num_decode + num_prefill + 1]; q_start_loc[i]
 *                  = i for i <= num_decode (read only when num_prefill > 0)
 *   seq_lens     : device, int32 [num_decode + num_prefill], tokens in the pool
 *                  for each sequence, its rows of this call included
 *   block_tables : device, int32 [num_decode + num_prefill][max_blocks_per_seq]
 *   max_q_len    : host, >= every prefill chunk's row count
 *   num_workers  : decode work slices, one wavefront each (on the multi-row
 *                  path below with more than 16 columns per unit, a
 *                  workgroup of two wavefronts); 0 = default (2 wavefronts per
 *                  compute unit when the batch also has chunks, 8 on the
 *                  multi-row path, else pa_decode's default)
 *   workspace    : device, pa_attention_mixed_workspace_bytes(num_decode,
 *                  num_prefill, num_q_heads, num_kv_heads, head_dim, max_q_len,
 *                  num_workers) bytes, 16-byte aligned (unused when the batch
 *                  has no decode rows and no short chunks)
 * Short chunks (a bf16 or PA_FP8_E4M3 pool and max_q_len * num_q_heads /
 * num_kv_heads <= 32, or <= 16 for FP8 pools of head_dim 64: small prompt
 * pieces, and the target model checking a draft model's k tokens in one pass,
 * "vLLM PagedAttention explained" section 7.5 and "vLLM inference engine deep
 * dive" section 5.2) take the multi-row decode: every sequence, decode rows
 * included, is one unit per KV head whose MFMA columns are its (row, query
 * head) pairs, each masked at its own row's position, so each K/V row is read
 * once for all of a sequence's rows (units of more than 16 columns: two
 * wavefronts of one workgroup, 16 columns each, that share every K/V tile
 * through LDS).
 * Otherwise, with both kinds of rows, the chunks run on a second stream of the
 * library's (one per host thread and device, default priority) that forks
 * from and joins back into `stream`, so that the two kernels share the chip.
 * Chunks the multi-row decode does not take need a bf16 pool
 * (PA_ERR_UNSUPPORTED otherwise); decode rows take every pa_decode dtype.
 * Each row's result is that of pa_decode or pa_prefill_chunk for it alone
 * (up to the decode's worker count), or, on the multi-row path, the same
 * causal attention up to rounding.
 */
/* Workspace bytes of pa_attention_mixed for a batch of this shape (0 for
 * invalid sizes). */
size_t pa_attention_mixed_workspace_bytes(int32_t num_decode, int32_t num_prefill,
                                          int32_t num_q_heads, int32_t num_kv_heads,
                                          int32_t head_dim, int32_t max_q_len,
                                          int32_t num_workers);
pa_status pa_attention_mixed(void* out, const void* q, const int32_t* q_start_loc,
                             const int32_t* seq_lens, const pa_pool* pool,
                             const int32_t* block_tables, int32_t max_blocks_per_seq,
                             int32_t num_decode, int32_t num_prefill, int32_t num_q_heads,
                             int32_t max_q_len, float scale, int32_t num_workers, void* workspace,
                             size_t workspace_bytes, void* stream);

/* ------------------------------------------- host checks of preconditions --- */

/*
 * The device calls take block tables, lengths, slots, copy pairs and chunk
 * offsets in device memory and do not read them back on the host, so their
 * contents are preconditions (a table entry outside the pool makes a kernel
 * read outside it). These functions check host copies of those arrays before
 * a launch: a debug aid for callers and bindings. Each returns PA_OK, or
 * PA_ERR_INVALID with pa_last_error() naming the first violation. All array
 * arguments are HOST memory, read during the call; pools are used only for
 * num_blocks and block_size (their data pointers are not touched).
 */

/* Tables and lengths of pa_decode (and of the decode rows of the other calls):
 * 0 <= seq_lens[s] <= max_blocks_per_seq * B, and the first
 * ceil(seq_lens[s] / B) entries of row s lie in [0, num_blocks)
 * ("Why PagedAttention multiplies LLM serving throughput", section "Block
 * Table: the GPU page table"). */
pa_status pa_check_batch(const pa_pool* pool, const int32_t* block_tables,
                         int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t num_seqs);
/* Slots of pa_cache_write: each negative (skipped) or < num_blocks * B, and no
 * slot named twice ("LLM inference engine internals", section 2.3). */
pa_status pa_check_slots(const pa_pool* pool, const int64_t* slot_mapping, int32_t num_tokens);
/* Pairs of pa_copy_blocks: ids in [0, num_blocks), no block both a source and a
 * destination, no destination twice ("vLLM PagedAttention explained", 4.1). */
pa_status pa_check_copies(const pa_pool* pool, const int32_t* src_dst, int32_t num_pairs);
/* Row offsets of pa_prefill_chunk / pa_attention_mixed: q_start_loc[0] = 0;
 * the first num_decode sequences have one row each; every other sequence has
 * 0 <= q_len <= max_q_len rows and q_len <= seq_lens[s] (its rows are in the
 * pool); q_start_loc[num_seqs] <= total_rows (the rows of q and out);
 * seq_lens >= 0 ("vLLM PagedAttention explained", section 7.2). */
pa_status pa_check_chunks(const int32_t* q_start_loc, const int32_t* seq_lens, int32_t num_seqs,
                          int32_t num_decode, int32_t max_q_len, int64_t total_rows);
/* pa_check_batch, plus the precondition of pa_decode_shared_prefix: every row
 * begins with row 0's first num_prefix_blocks entries and every sequence is at
 * least num_prefix_blocks * B tokens long. */
pa_status pa_check_shared_prefix(const pa_pool* pool, const int32_t* block_tables,
                                 int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                 int32_t num_seqs, int32_t num_prefix_blocks);

/* Shared prefix of each group of group_size consecutive rows (host arrays):
 * the leading table entries identical in every member's row, counting only
 * blocks full in every member (j < min over members of seq_lens / B), times B;
 * written to prefix_lens[s] for every member (host int32 [num_seqs]). What a
 * pa_alloc_fork family of sequences shares ("vLLM PagedAttention explained",
 * sections 4.1-4.2). */
pa_status pa_group_prefix_lens(const int32_t* block_tables, int32_t max_blocks_per_seq,
                               const int32_t* seq_lens, int32_t num_seqs, int32_t group_size,
                               int32_t block_size, int32_t* prefix_lens);
/* pa_check_batch plus the precondition of pa_decode_grouped on host copies of
 * its arrays (see there). */
pa_status pa_check_grouped(const pa_pool* pool, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, const int32_t* seq_lens,
                           const int32_t* prefix_lens, int32_t num_seqs, int32_t group_size);

/* ------------------------------------------------------------------ host --- */

/*
 * Host block allocator ("LLM inference engine internals", section 2.3; "vLLM
 * PagedAttention explained", sections 4.1, 4.2, 7.1; "Why PagedAttention
 * multiplies LLM serving throughput", section "Automatic prefix caching").
 * FIFO free list, per-block reference counts, fork with copy-on-write of a
 * shared partial last block, and hash-based sharing of full prompt blocks.
 * It touches no device memory; it produces block tables, slots and the list
 * of block copies for pa_copy_blocks. Not thread-safe: one owner at a time.
 * Every call that fails leaves the allocator state unchanged.
 */
typedef struct pa_alloc pa_alloc;

/* free_order: host, int32 [num_blocks] permutation giving the initial free-list
 * order, or NULL for 0, 1, 2, ... */
pa_status pa_alloc_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                          pa_alloc** out);
void pa_alloc_destroy(pa_alloc* a);

/* New sequence with an n-token prompt (host tokens[n]). Leading full blocks
 * found in the prefix cache are shared; *cached_out (nullable) receives the
 * number of leading tokens whose K/V is already in the pool. slots_out
 * (host, nullable, int64 [n]) receives the slot of every position. */
pa_status pa_alloc_allocate(pa_alloc* a, int64_t seq_id, const int32_t* tokens, int32_t n,
                            int32_t* cached_out, int64_t* slots_out);
/* Append one token; *slot_out receives its slot. May queue one block copy. */
pa_status pa_alloc_append_slot(pa_alloc* a, int64_t seq_id, int32_t token, int64_t* slot_out);
/* Append an n-token chunk (all or nothing); slots_out host int64 [n] (nullable). */
pa_status pa_alloc_extend(pa_alloc* a, int64_t seq_id, const int32_t* tokens, int32_t n,
                          int64_t* slots_out);
/* child shares all of parent's blocks (reference counts + 1). */
pa_status pa_alloc_fork(pa_alloc* a, int64_t parent, int64_t child);
/* Release a sequence's blocks in table order; count 0 returns a block to the free list. */
pa_status pa_alloc_free(pa_alloc* a, int64_t seq_id);
/* Move the queued (src, dst) copies into host src_dst[cap][2], oldest first.
 * *n_out = number queued; if cap < that, PA_ERR_INVALID and nothing is moved. */
pa_status pa_alloc_take_copies(pa_alloc* a, int32_t* src_dst, int32_t cap, int32_t* n_out);
/* Copy a sequence's block table into host out[cap]; *n_out = its length. */
pa_status pa_alloc_block_table(const pa_alloc* a, int64_t seq_id, int32_t* out, int32_t cap,
                               int32_t* n_out);
pa_status pa_alloc_seq_len(const pa_alloc* a, int64_t seq_id, int32_t* len_out);
/* Build a padded batch: host tables[n][max_blocks] (unused entries 0) and
 * host seq_lens[n] for seq_ids[n]. PA_ERR_INVALID if a table is longer than max_blocks. */
pa_status pa_alloc_batch_tables(const pa_alloc* a, const int64_t* seq_ids, int32_t n,
                                int32_t* tables, int32_t max_blocks, int32_t* seq_lens);
int32_t pa_alloc_num_free(const pa_alloc* a);
/* Reference count of a physical block (0 = free). */
pa_status pa_alloc_ref_count(const pa_alloc* a, int32_t block, int32_t* out);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
