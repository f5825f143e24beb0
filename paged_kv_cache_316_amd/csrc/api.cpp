// C ABI entry points of the device calls: host-side argument checks,
// workspace sizing and dispatch to the HIP launchers.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <vector>

#include "api_internal.h"
#include "device.h"
#include "pagedkv.h"
#include "status.h"

namespace pa {

namespace {
constexpr int32_t kWavesPerCU = 8;  // default decode workers per compute unit
constexpr int32_t kMatrixWavesPerCU = 4;  // the same for the bf16 matrix-core decodes

int32_t device_cus() {
  static int32_t cached = 0;
  if (cached == 0) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0) {
      (void)hipGetLastError();
      cus = 256;  // MI355X
    }
    cached = cus;
  }
  return cached;
}

int32_t default_workers() { return device_cus() * kWavesPerCU; }

struct DecodeLayout {
  int32_t workers, heads_per_unit, units;
  size_t acc_bytes, ml_bytes, seg_bytes;
  size_t total() const { return acc_bytes + ml_bytes + seg_bytes; }
};

DecodeLayout decode_layout(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                           int32_t head_dim, int32_t workers) {
  DecodeLayout d{};
  d.workers = workers > 0 ? workers : default_workers();
  // partial slots are sized for the largest unit a launch may use: FP8 MHA
  // pools pair KV heads (2 heads per unit), which dtype-free sizing covers
  const int32_t G = num_q_heads / num_kv_heads;
  d.heads_per_unit = G == 1 ? 2 : decode_heads_per_unit(G);
  d.units = num_q_heads / d.heads_per_unit;
  const size_t slots = size_t(2) * d.workers * d.heads_per_unit;
  d.acc_bytes = slots * head_dim * 4;
  d.ml_bytes = size_t(2) * d.workers * kMLStride * 8;
  d.seg_bytes = size_t(d.workers) * 16;
  (void)num_seqs;
  return d;
}

size_t align16(size_t n) { return (n + 15) & ~size_t(15); }

// Grouped decode: the same partial slots with 16 columns per unit.
DecodeLayout grouped_layout(int32_t head_dim, int32_t workers) {
  DecodeLayout d{};
  d.workers = workers > 0 ? workers : default_workers();
  d.heads_per_unit = kGroupedCols;
  const size_t slots = size_t(2) * d.workers * d.heads_per_unit;
  d.acc_bytes = slots * head_dim * 4;
  d.ml_bytes = size_t(2) * d.workers * kMLStride * 8;
  d.seg_bytes = size_t(d.workers) * 16;
  return d;
}

// Multi-row decode: per work slice, slots of kMultiRowCols bf16 partial rows
// and records of as many (max, denominator) pairs. A slice is one wave, or a
// pair of waves when units have more than 16 columns; 8 waves per compute
// unit by default.
DecodeLayout multirow_layout(int32_t head_dim, int32_t workers, bool pair) {
  DecodeLayout d{};
  d.workers = workers > 0 ? workers : device_cus() * kMultiRowWaves / (pair ? 2 : 1);
  d.heads_per_unit = kMultiRowCols;
  const size_t slots = size_t(2) * d.workers * d.heads_per_unit;
  d.acc_bytes = slots * head_dim * 2;
  d.ml_bytes = slots * 8;
  d.seg_bytes = size_t(d.workers) * 16;
  return d;
}

// Units of more than 16 columns run on a pair of waves (16 columns each).
bool multirow_pair(int32_t G, int32_t max_q_len) { return int64_t(max_q_len) * G > 16; }

// A mixed batch runs as one multi-row decode when its chunks are short: a
// bf16 or FP8 pool and every sequence's rows x query heads per KV head within
// the columns of one unit. FP8 rows of 64 dims fill a tile with one wave-wide
// load, which a pair of waves cannot split: there, at most 16 columns.
bool multirow_fits(int32_t dtype, int32_t head_dim, int32_t G, int32_t num_prefill,
                   int32_t max_q_len) {
  const int64_t cols = int64_t(max_q_len) * G;
  const int64_t max_cols = dtype == PA_FP8_E4M3 && head_dim == 64 ? 16 : kMultiRowCols;
  return (dtype == PA_BF16 || dtype == PA_FP8_E4M3) && (head_dim == 64 || head_dim == 128) &&
         num_prefill > 0 && max_q_len >= 1 && cols <= max_cols;
}

// Members per unit of the grouped decode: the largest divisor of group_size
// whose members' query heads fit the 16 columns of one unit (0 if none).
int32_t grouped_members(int32_t group_size, int32_t G) {
  for (int32_t m = group_size; m >= 1; --m)
    if (group_size % m == 0 && m * G <= kGroupedCols) return m;
  return 0;
}

// Shared-prefix decode workspace: the decode's, then the tail log-sum-exp and
// the prefix partials.
struct PrefixLayout {
  DecodeLayout dec;
  PrefixPlan plan;
  size_t lse_off, ml_off, acc_off, end;
  size_t total() const { return end; }
};

PrefixLayout prefix_layout(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                           int32_t head_dim, int32_t block_size, int32_t num_prefix_blocks,
                           int32_t workers) {
  PrefixLayout p{};
  p.dec = decode_layout(num_seqs, num_q_heads, num_kv_heads, head_dim, workers);
  p.plan = prefix_plan(num_seqs, num_q_heads, num_kv_heads, block_size, num_prefix_blocks,
                       device_cus());
  const size_t rows = size_t(num_seqs) * num_q_heads;
  p.lse_off = align16(p.dec.total());
  p.ml_off = p.lse_off + align16(rows * 4);
  p.acc_off = p.ml_off + align16(size_t(p.plan.n_split) * rows * 8);
  p.end = p.acc_off + size_t(p.plan.n_split) * rows * head_dim * 2;
  return p;
}

bool pow2(int32_t x) { return x > 0 && (x & (x - 1)) == 0; }

// Second stream for work that may overlap the caller's (default priority),
// with the two events of a fork / join; one set per host thread and device,
// created on first use and kept until the process ends.
constexpr int32_t kMixedDecodeWavesPerCU = 2;  // default decode workers beside prefill chunks
constexpr bool kMixedDecodeFirst = false;      // launch order of the two kernels
struct SideStream {
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
hipError_t side_stream(SideStream** out) {
  constexpr int kMaxDevices = 64;
  thread_local SideStream per_device[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  SideStream& s = per_device[dev];
  if (!s.stream) {
    if ((e = hipEventCreateWithFlags(&s.fork, hipEventDisableTiming)) != hipSuccess) return e;
    if ((e = hipEventCreateWithFlags(&s.join, hipEventDisableTiming)) != hipSuccess) return e;
    if ((e = hipStreamCreateWithFlags(&s.stream, hipStreamNonBlocking)) != hipSuccess) return e;
  }
  *out = &s;
  return hipSuccess;
}

int32_t elt_bytes(int32_t dtype) { return dtype == PA_F32 ? 4 : dtype == PA_BF16 ? 2 : 1; }

pa_status check_pool(const pa_pool* p, const char* who) {
  if (!p) return fail(PA_ERR_INVALID, "%s: pool is NULL", who);
  if (!p->k_pool || !p->v_pool) return fail(PA_ERR_INVALID, "%s: k_pool/v_pool is NULL", who);
  if (p->num_blocks <= 0 || p->num_kv_heads <= 0)
    return fail(PA_ERR_INVALID, "%s: num_blocks=%d num_kv_heads=%d must be > 0", who,
                p->num_blocks, p->num_kv_heads);
  if (!pow2(p->block_size) || p->block_size > 256)
    return fail(PA_ERR_INVALID, "%s: block_size=%d must be a power of two in 1..256", who,
                p->block_size);
  if (p->dtype != PA_F32 && p->dtype != PA_BF16 && p->dtype != PA_FP8_E4M3)
    return fail(PA_ERR_UNSUPPORTED, "%s: dtype %d not supported", who, p->dtype);
  if (p->dtype == PA_FP8_E4M3 &&
      !(p->k_scale > 0.f && p->k_scale <= 3.4e38f && p->v_scale > 0.f && p->v_scale <= 3.4e38f))
    return fail(PA_ERR_INVALID, "%s: FP8 pool needs finite scales > 0 (k_scale=%g v_scale=%g)",
                who, double(p->k_scale), double(p->v_scale));
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "%s: head_dim=%d not supported (64, 128)", who, p->head_dim);
  return PA_OK;
}

// Softmax scale: finite and > 0. A negative scale would turn the running max
// into the smallest logit and the weights could overflow; zero or non-finite
// scales have no meaningful attention.
pa_status check_scale(float scale, const char* who) {
  if (!(scale > 0.f && scale <= 3.402823466e38f))
    return fail(PA_ERR_INVALID, "%s: scale=%g must be finite and > 0", who, double(scale));
  return PA_OK;
}

pa_status hip_status(hipError_t e, const char* who) {
  if (e == hipSuccess) return PA_OK;
  return fail(PA_ERR_HIP, "%s: %s", who, hipGetErrorString(e));
}

DecodeArgs decode_args(void* out, const void* q, const pa_pool* pool, const int32_t* block_tables,
                       int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t num_seqs,
                       int32_t num_q_heads, float scale, const DecodeLayout& lay, void* workspace) {
  DecodeArgs a{};
  a.out = out;
  a.q = q;
  a.k_pool = pool->k_pool;
  a.v_pool = pool->v_pool;
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  char* ws = static_cast<char*>(workspace);
  a.ws_acc = reinterpret_cast<float*>(ws);
  a.ws_ml = reinterpret_cast<float2*>(ws + lay.acc_bytes);
  a.ws_seg = reinterpret_cast<int4*>(ws + lay.acc_bytes + lay.ml_bytes);
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = pool->num_kv_heads;
  a.head_dim = pool->head_dim;
  a.block_size = pool->block_size;
  a.dtype = pool->dtype;
  a.workers = lay.workers;
  a.num_cus = device_cus();
  a.scale = scale;
  const bool fp8 = pool->dtype == PA_FP8_E4M3;
  a.k_scale = fp8 ? pool->k_scale : 1.f;
  a.v_scale = fp8 ? pool->v_scale : 1.f;
  a.lse = nullptr;
  a.len_offset = 0;
  a.prefix_lens = nullptr;
  a.group_size = 1;
  a.num_groups = num_seqs;
  a.q_start_loc = nullptr;
  a.mr_pair = 0;
  return a;
}

}  // namespace

pa_status decode_check(const DecodeCall& c, const char* who, size_t* need) {
  *need = 0;
  const pa_pool* pool = c.pool;
  if (pa_status s = check_pool(pool, who)) return s;
  if (c.num_seqs < 0 || c.max_blocks_per_seq <= 0 || c.num_q_heads <= 0)
    return fail(PA_ERR_INVALID, "%s: num_seqs=%d max_blocks_per_seq=%d num_q_heads=%d", who,
                c.num_seqs, c.max_blocks_per_seq, c.num_q_heads);
  if (c.num_seqs == 0) return PA_OK;
  if (!c.out || !c.q || !c.block_tables || !c.seq_lens)
    return fail(PA_ERR_INVALID, "%s: out/q/block_tables/seq_lens is NULL", who);
  if (c.num_q_heads % pool->num_kv_heads)
    return fail(PA_ERR_INVALID, "%s: num_q_heads=%d not a multiple of num_kv_heads=%d", who,
                c.num_q_heads, pool->num_kv_heads);
  if (pa_status s = check_scale(c.scale, who)) return s;
  if (c.num_workers < 0 || c.num_workers > (1 << 24))
    return fail(PA_ERR_INVALID, "%s: num_workers=%d out of range", who, c.num_workers);
  if ((reinterpret_cast<uintptr_t>(c.out) | reinterpret_cast<uintptr_t>(c.q) |
       reinterpret_cast<uintptr_t>(pool->k_pool) | reinterpret_cast<uintptr_t>(pool->v_pool)) & 15)
    return fail(PA_ERR_INVALID, "%s: out/q/pools must be 16-byte aligned", who);
  const int32_t G = c.num_q_heads / pool->num_kv_heads;
  if (!decode_supported(pool->dtype, pool->head_dim, G))
    return fail(PA_ERR_UNSUPPORTED, "%s: dtype=%d head_dim=%d group=%d not built", who,
                pool->dtype, pool->head_dim, G);
  *need = decode_layout(c.num_seqs, c.num_q_heads, pool->num_kv_heads, pool->head_dim,
                        c.num_workers).total();
  return PA_OK;
}

// Default work slices of the bf16 matrix-core decodes (query groups of 4 or
// more heads per unit, and the grouped decode): they stream as fast with 4
// waves per CU as with 8, and fewer slices split fewer units (Llama-2-70B
// layer +0.8 %, one tensor-parallel shard of it +5 %, parallel samples /
// beams +3 %). MHA and FP8 pools keep 8 per CU. Workspaces stay sized for
// the larger default, so the size queries need no dtype.
int32_t matrix_default_workers(int32_t layout_workers) {
  const int32_t w = device_cus() * kMatrixWavesPerCU;
  return w < layout_workers ? w : layout_workers;
}

pa_status decode_launch(const DecodeCall& c, void* workspace, void* stream, const char* who) {
  const DecodeLayout lay = decode_layout(c.num_seqs, c.num_q_heads, c.pool->num_kv_heads,
                                         c.pool->head_dim, c.num_workers);
  DecodeArgs a = decode_args(c.out, c.q, c.pool, c.block_tables, c.max_blocks_per_seq,
                             c.seq_lens, c.num_seqs, c.num_q_heads, c.scale, lay, workspace);
  const int32_t G = c.num_q_heads / c.pool->num_kv_heads;
  if (c.num_workers == 0 && c.pool->dtype == PA_BF16 && decode_heads_per_unit(G) >= 4)
    a.workers = matrix_default_workers(lay.workers);
  return hip_status(launch_decode(a, static_cast<hipStream_t>(stream)), who);
}

}  // namespace pa

using pa::fail;

extern "C" {

pa_status pa_cache_write(const pa_pool* pool, const void* k_new, const void* v_new,
                         const int64_t* slot_mapping, int32_t num_tokens, void* stream) {
  pa::clear_error();
  if (pa_status s = pa::check_pool(pool, "pa_cache_write")) return s;
  if (num_tokens < 0) return fail(PA_ERR_INVALID, "pa_cache_write: num_tokens=%d < 0", num_tokens);
  if (num_tokens == 0) return PA_OK;
  if (!k_new || !v_new || !slot_mapping)
    return fail(PA_ERR_INVALID, "pa_cache_write: k_new/v_new/slot_mapping is NULL");
  if ((reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new) |
       reinterpret_cast<uintptr_t>(pool->k_pool) | reinterpret_cast<uintptr_t>(pool->v_pool)) & 15)
    return fail(PA_ERR_INVALID, "pa_cache_write: K/V arrays must be 16-byte aligned");
  return pa::hip_status(pa::launch_cache_write(*pool, k_new, v_new, slot_mapping, num_tokens,
                                               static_cast<hipStream_t>(stream)),
                        "pa_cache_write");
}

pa_status pa_copy_blocks(const pa_pool* pool, const int32_t* src_dst, int32_t num_pairs,
                         void* stream) {
  pa::clear_error();
  if (pa_status s = pa::check_pool(pool, "pa_copy_blocks")) return s;
  if (num_pairs < 0) return fail(PA_ERR_INVALID, "pa_copy_blocks: num_pairs=%d < 0", num_pairs);
  if (num_pairs == 0) return PA_OK;
  if (!src_dst) return fail(PA_ERR_INVALID, "pa_copy_blocks: src_dst is NULL");
  if ((reinterpret_cast<uintptr_t>(pool->k_pool) | reinterpret_cast<uintptr_t>(pool->v_pool)) & 15)
    return fail(PA_ERR_INVALID, "pa_copy_blocks: pools must be 16-byte aligned");
  const int32_t kMaxPairsPerLaunch = 65535;
  for (int32_t off = 0; off < num_pairs; off += kMaxPairsPerLaunch) {
    const int32_t n = num_pairs - off < kMaxPairsPerLaunch ? num_pairs - off : kMaxPairsPerLaunch;
    hipError_t e = pa::launch_copy_blocks(*pool, src_dst + 2 * int64_t(off), n,
                                          static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return pa::hip_status(e, "pa_copy_blocks");
  }
  return PA_OK;
}

pa_status pa_swap_blocks(const pa_pool* device_pool, const pa_pool* host_pool,
                         const int32_t* src_dst, int32_t num_pairs, int32_t direction,
                         void* stream) {
  pa::clear_error();
  const char* who = "pa_swap_blocks";
  if (pa_status s = pa::check_pool(device_pool, who)) return s;
  if (pa_status s = pa::check_pool(host_pool, who)) return s;
  if (direction != PA_SWAP_OUT && direction != PA_SWAP_IN)
    return fail(PA_ERR_INVALID, "%s: direction=%d (PA_SWAP_OUT or PA_SWAP_IN)", who, direction);
  if (host_pool->num_kv_heads != device_pool->num_kv_heads ||
      host_pool->block_size != device_pool->block_size ||
      host_pool->head_dim != device_pool->head_dim || host_pool->dtype != device_pool->dtype)
    return fail(PA_ERR_INVALID, "%s: host and device pools differ in block geometry or dtype", who);
  if (device_pool->dtype == PA_FP8_E4M3 && (host_pool->k_scale != device_pool->k_scale ||
                                            host_pool->v_scale != device_pool->v_scale))
    return fail(PA_ERR_INVALID, "%s: FP8 pools with different scales", who);
  if (num_pairs < 0) return fail(PA_ERR_INVALID, "%s: num_pairs=%d", who, num_pairs);
  if (num_pairs == 0) return PA_OK;
  if (!src_dst) return fail(PA_ERR_INVALID, "%s: src_dst is NULL", who);
  const bool out = direction == PA_SWAP_OUT;
  const pa_pool* src = out ? device_pool : host_pool;
  const pa_pool* dst = out ? host_pool : device_pool;
  // every id in range and no destination twice (host array, read here)
  std::vector<unsigned char> taken(size_t(dst->num_blocks), 0);
  for (int32_t i = 0; i < num_pairs; ++i) {
    const int32_t s = src_dst[2 * i], d = src_dst[2 * i + 1];
    if (s < 0 || s >= src->num_blocks || d < 0 || d >= dst->num_blocks)
      return fail(PA_ERR_INVALID, "%s: pair %d = (%d, %d) outside the pools (%d source, %d "
                  "destination blocks)", who, i, s, d, src->num_blocks, dst->num_blocks);
    if (taken[d]) return fail(PA_ERR_INVALID, "%s: destination block %d named twice", who, d);
    taken[d] = 1;
  }
  // the device pool must be device memory, the host pool pinned host memory
  // that the device can address (hipHostMalloc); its device address is used
  void* host_k = nullptr;
  void* host_v = nullptr;
  for (int which = 0; which < 4; ++which) {
    const void* ptr = which == 0 ? device_pool->k_pool : which == 1 ? device_pool->v_pool
                    : which == 2 ? host_pool->k_pool : host_pool->v_pool;
    hipPointerAttribute_t attr{};
    const hipError_t e = hipPointerGetAttributes(&attr, ptr);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return fail(PA_ERR_INVALID, "%s: %s pool memory unknown to HIP (%s)", who,
                  which < 2 ? "device" : "host (needs pinned memory)", hipGetErrorString(e));
    }
    if (which < 2 && attr.type != hipMemoryTypeDevice)
      return fail(PA_ERR_INVALID, "%s: device_pool is not device memory", who);
    if (which >= 2) {
      if (attr.type != hipMemoryTypeHost || !attr.devicePointer)
        return fail(PA_ERR_INVALID, "%s: host_pool is not pinned, device-mapped host memory", who);
      (which == 2 ? host_k : host_v) = attr.devicePointer;
    }
  }
  const int64_t block_bytes = int64_t(device_pool->num_kv_heads) * device_pool->block_size *
                              device_pool->head_dim * pa::elt_bytes(device_pool->dtype);
  const void* sk = out ? device_pool->k_pool : host_k;
  const void* sv = out ? device_pool->v_pool : host_v;
  void* dk = out ? host_k : device_pool->k_pool;
  void* dv = out ? host_v : device_pool->v_pool;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  for (int32_t i0 = 0; i0 < num_pairs; i0 += pa::kSwapBatch) {
    const int32_t n = num_pairs - i0 < pa::kSwapBatch ? num_pairs - i0 : pa::kSwapBatch;
    pa::SwapBatch b{};
    std::memcpy(b.pairs, src_dst + 2 * i0, sizeof(int32_t) * 2 * n);
    if (pa_status s = pa::hip_status(pa::launch_swap_blocks(b, n, sk, sv, dk, dv, block_bytes, st),
                                     who))
      return s;
  }
  return PA_OK;
}

pa_status pa_probe_stream_read(const void* buf, size_t bytes, int32_t grid, uint32_t* sink,
                               void* stream) {
  pa::clear_error();
  if (bytes == 0) return PA_OK;
  if (!buf || !sink) return fail(PA_ERR_INVALID, "pa_probe_stream_read: buf/sink is NULL");
  if ((reinterpret_cast<uintptr_t>(buf) & 15) || (bytes & 15))
    return fail(PA_ERR_INVALID, "pa_probe_stream_read: buf and bytes must be 16-byte aligned");
  const int g = grid > 0 ? grid : pa::device_cus() * 16;
  return pa::hip_status(pa::launch_stream_read(buf, bytes, g, sink, static_cast<hipStream_t>(stream)),
                        "pa_probe_stream_read");
}

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t num_workers) {
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      num_workers < 0 || num_q_heads % num_kv_heads)
    return 0;
  return pa::decode_layout(num_seqs, num_q_heads, num_kv_heads, head_dim, num_workers).total();
}

size_t pa_attention_mixed_workspace_bytes(int32_t num_decode, int32_t num_prefill,
                                          int32_t num_q_heads, int32_t num_kv_heads,
                                          int32_t head_dim, int32_t max_q_len,
                                          int32_t num_workers) {
  if (num_decode < 0 || num_prefill < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      head_dim <= 0 || max_q_len < 0 || num_workers < 0 || num_q_heads % num_kv_heads)
    return 0;
  const int32_t G = num_q_heads / num_kv_heads;
  size_t need = 16;
  if (pa::multirow_fits(PA_BF16, head_dim, G, num_prefill, max_q_len))
    return std::max(need, pa::multirow_layout(head_dim, num_workers,
                                              pa::multirow_pair(G, max_q_len)).total());
  if (num_decode > 0) {
    const bool both = num_prefill > 0 && max_q_len > 0;
    const int32_t workers =
        num_workers > 0 ? num_workers : (both ? pa::device_cus() * pa::kMixedDecodeWavesPerCU : 0);
    need = std::max(need, pa::decode_layout(num_decode, num_q_heads, num_kv_heads, head_dim,
                                            workers).total());
  }
  return need;
}

pa_status pa_decode(void* out, const void* q, const pa_pool* pool, const int32_t* block_tables,
                    int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t num_seqs,
                    int32_t num_q_heads, float scale, int32_t num_workers, void* workspace,
                    size_t workspace_bytes, void* stream) {
  pa::clear_error();
  const char* who = "pa_decode";
  const pa::DecodeCall c{out, q, pool, block_tables, max_blocks_per_seq, seq_lens, num_seqs,
                         num_q_heads, scale, num_workers};
  size_t need = 0;
  if (pa_status s = pa::decode_check(c, who, &need)) return s;
  if (num_seqs == 0) return PA_OK;
  if (!workspace || workspace_bytes < need)
    return fail(PA_ERR_WORKSPACE, "pa_decode: workspace of %zu bytes, %zu needed",
                workspace ? workspace_bytes : size_t(0), need);
  if (reinterpret_cast<uintptr_t>(workspace) & 15)
    return fail(PA_ERR_INVALID, "pa_decode: workspace must be 16-byte aligned");
  return pa::decode_launch(c, workspace, stream, who);
}

size_t pa_decode_grouped_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                         int32_t num_kv_heads, int32_t head_dim,
                                         int32_t num_workers) {
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      num_workers < 0 || num_q_heads % num_kv_heads)
    return 0;
  return pa::grouped_layout(head_dim, num_workers).total();
}

pa_status pa_decode_grouped(void* out, const void* q, const pa_pool* pool,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* seq_lens, const int32_t* prefix_lens,
                            int32_t num_seqs, int32_t group_size, int32_t num_q_heads,
                            float scale, int32_t num_workers, void* workspace,
                            size_t workspace_bytes, void* stream) {
  pa::clear_error();
  const char* who = "pa_decode_grouped";
  const pa::DecodeCall c{out, q, pool, block_tables, max_blocks_per_seq, seq_lens, num_seqs,
                         num_q_heads, scale, num_workers};
  size_t plain_need = 0;
  if (pa_status s = pa::decode_check(c, who, &plain_need)) return s;
  if (group_size < 1 || (num_seqs > 0 && num_seqs % group_size))
    return fail(PA_ERR_INVALID, "%s: num_seqs=%d is not a multiple of group_size=%d", who,
                num_seqs, group_size);
  if (num_seqs == 0) return PA_OK;
  if (!prefix_lens) return fail(PA_ERR_INVALID, "%s: prefix_lens is NULL", who);
  if (pool->dtype != PA_BF16 && pool->dtype != PA_FP8_E4M3)
    return fail(PA_ERR_UNSUPPORTED, "%s: dtype=%d not built (bf16 or fp8 pools)", who, pool->dtype);
  const int32_t G = num_q_heads / pool->num_kv_heads;
  const int32_t members = pa::grouped_members(group_size, G);
  if (members == 0)
    return fail(PA_ERR_UNSUPPORTED, "%s: %d query heads per KV head exceed the %d columns of a "
                "unit", who, G, pa::kGroupedCols);
  const pa::DecodeLayout lay = pa::grouped_layout(pool->head_dim, num_workers);
  if (!workspace || workspace_bytes < lay.total())
    return fail(PA_ERR_WORKSPACE, "%s: workspace of %zu bytes, %zu needed", who,
                workspace ? workspace_bytes : size_t(0), lay.total());
  if (reinterpret_cast<uintptr_t>(workspace) & 15)
    return fail(PA_ERR_INVALID, "%s: workspace must be 16-byte aligned", who);
  pa::DecodeArgs a = pa::decode_args(out, q, pool, block_tables, max_blocks_per_seq, seq_lens,
                                     num_seqs, num_q_heads, scale, lay, workspace);
  if (num_workers == 0 && pool->dtype == PA_BF16) a.workers = pa::matrix_default_workers(lay.workers);
  a.prefix_lens = prefix_lens;
  a.group_size = members;
  a.num_groups = num_seqs / members;
  return pa::hip_status(pa::launch_decode(a, static_cast<hipStream_t>(stream)), who);
}

size_t pa_decode_shared_prefix_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                               int32_t num_kv_heads, int32_t head_dim,
                                               int32_t block_size, int32_t num_prefix_blocks,
                                               int32_t num_workers) {
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      block_size <= 0 || num_prefix_blocks < 0 || num_workers < 0 || num_q_heads % num_kv_heads)
    return 0;
  return pa::prefix_layout(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                           num_prefix_blocks, num_workers).total();
}

pa_status pa_decode_shared_prefix(void* out, const void* q, const pa_pool* pool,
                                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                                  const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                                  float scale, int32_t num_prefix_blocks, int32_t num_workers,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  pa::clear_error();
  const char* who = "pa_decode_shared_prefix";
  if (pa_status s = pa::check_pool(pool, who)) return s;
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || num_q_heads <= 0)
    return fail(PA_ERR_INVALID, "%s: num_seqs=%d max_blocks_per_seq=%d num_q_heads=%d", who,
                num_seqs, max_blocks_per_seq, num_q_heads);
  if (num_prefix_blocks < 0 || num_prefix_blocks > max_blocks_per_seq)
    return fail(PA_ERR_INVALID, "%s: num_prefix_blocks=%d outside [0, max_blocks_per_seq=%d]", who,
                num_prefix_blocks, max_blocks_per_seq);
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !block_tables || !seq_lens)
    return fail(PA_ERR_INVALID, "%s: out/q/block_tables/seq_lens is NULL", who);
  if (num_q_heads % pool->num_kv_heads)
    return fail(PA_ERR_INVALID, "%s: num_q_heads=%d not a multiple of num_kv_heads=%d", who,
                num_q_heads, pool->num_kv_heads);
  if (pa_status s = pa::check_scale(scale, who)) return s;
  if (num_workers < 0 || num_workers > (1 << 24))
    return fail(PA_ERR_INVALID, "%s: num_workers=%d out of range", who, num_workers);
  if ((reinterpret_cast<uintptr_t>(out) | reinterpret_cast<uintptr_t>(q) |
       reinterpret_cast<uintptr_t>(pool->k_pool) | reinterpret_cast<uintptr_t>(pool->v_pool)) & 15)
    return fail(PA_ERR_INVALID, "%s: out/q/pools must be 16-byte aligned", who);
  const int32_t G = num_q_heads / pool->num_kv_heads;
  if ((pool->dtype != PA_BF16 && pool->dtype != PA_FP8_E4M3) ||
      (pool->head_dim != 64 && pool->head_dim != 128))
    return fail(PA_ERR_UNSUPPORTED, "%s: dtype=%d head_dim=%d not built (bf16 or fp8, 64 or 128)",
                who, pool->dtype, pool->head_dim);
  if (int64_t(num_seqs) * G >= (int64_t(1) << 30))
    return fail(PA_ERR_UNSUPPORTED, "%s: num_seqs * group too large", who);
  const pa::PrefixLayout lay =
      pa::prefix_layout(num_seqs, num_q_heads, pool->num_kv_heads, pool->head_dim,
                        pool->block_size, num_prefix_blocks, num_workers);
  if (!workspace || workspace_bytes < lay.total())
    return fail(PA_ERR_WORKSPACE, "%s: workspace of %zu bytes, %zu needed", who,
                workspace ? workspace_bytes : size_t(0), lay.total());
  if (reinterpret_cast<uintptr_t>(workspace) & 15)
    return fail(PA_ERR_INVALID, "%s: workspace must be 16-byte aligned", who);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  if (num_prefix_blocks == 0) {  // nothing shared: the plain decode
    const pa::DecodeArgs a = pa::decode_args(out, q, pool, block_tables, max_blocks_per_seq,
                                             seq_lens, num_seqs, num_q_heads, scale, lay.dec, ws);
    return pa::hip_status(pa::launch_decode(a, st), who);
  }
  float* lse = reinterpret_cast<float*>(ws + lay.lse_off);
  // the tails: tokens after the shared blocks, table rows from entry P on
  // (same row stride)
  pa::DecodeArgs a = pa::decode_args(out, q, pool, block_tables + num_prefix_blocks,
                                     max_blocks_per_seq, seq_lens, num_seqs, num_q_heads, scale,
                                     lay.dec, ws);
  a.len_offset = num_prefix_blocks * pool->block_size;
  a.lse = lse;
  if (pa_status s = pa::hip_status(pa::launch_decode(a, st), who)) return s;
  pa::PrefixArgs p{};
  p.out = out;
  p.q = q;
  p.k_pool = pool->k_pool;
  p.v_pool = pool->v_pool;
  p.block_tables = block_tables;
  p.lse = lse;
  p.p_acc = reinterpret_cast<uint16_t*>(ws + lay.acc_off);
  p.p_ml = reinterpret_cast<float2*>(ws + lay.ml_off);
  p.num_seqs = num_seqs;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = pool->num_kv_heads;
  p.head_dim = pool->head_dim;
  p.block_size = pool->block_size;
  p.dtype = pool->dtype;
  p.num_prefix_blocks = num_prefix_blocks;
  p.n_split = lay.plan.n_split;
  p.scale = scale;
  p.k_scale = a.k_scale;
  p.v_scale = a.v_scale;
  return pa::hip_status(pa::launch_prefix(p, lay.plan, st), who);
}

pa_status pa_attention_mixed(void* out, const void* q, const int32_t* q_start_loc,
                             const int32_t* seq_lens, const pa_pool* pool,
                             const int32_t* block_tables, int32_t max_blocks_per_seq,
                             int32_t num_decode, int32_t num_prefill, int32_t num_q_heads,
                             int32_t max_q_len, float scale, int32_t num_workers, void* workspace,
                             size_t workspace_bytes, void* stream) {
  pa::clear_error();
  const char* who = "pa_attention_mixed";
  if (pa_status s = pa::check_pool(pool, who)) return s;
  if (num_decode < 0 || num_prefill < 0 || max_blocks_per_seq <= 0 || num_q_heads <= 0 ||
      max_q_len < 0)
    return fail(PA_ERR_INVALID, "%s: bad sizes", who);
  if (num_decode == 0 && num_prefill == 0) return PA_OK;
  if (num_prefill > 65535) return fail(PA_ERR_UNSUPPORTED, "%s: num_prefill > 65535", who);
  if (!out || !q || !seq_lens || !block_tables || (num_prefill > 0 && !q_start_loc))
    return fail(PA_ERR_INVALID, "%s: NULL pointer argument", who);
  if (num_q_heads % pool->num_kv_heads)
    return fail(PA_ERR_INVALID, "%s: num_q_heads=%d not a multiple of num_kv_heads=%d", who,
                num_q_heads, pool->num_kv_heads);
  if (pa_status s = pa::check_scale(scale, who)) return s;
  if (num_workers < 0 || num_workers > (1 << 24))
    return fail(PA_ERR_INVALID, "%s: num_workers=%d out of range", who, num_workers);
  if ((reinterpret_cast<uintptr_t>(out) | reinterpret_cast<uintptr_t>(q) |
       reinterpret_cast<uintptr_t>(pool->k_pool) | reinterpret_cast<uintptr_t>(pool->v_pool)) & 15)
    return fail(PA_ERR_INVALID, "%s: out/q/pools must be 16-byte aligned", who);
  const int32_t G = num_q_heads / pool->num_kv_heads;
  const bool multirow = pa::multirow_fits(pool->dtype, pool->head_dim, G, num_prefill, max_q_len);
  if (num_prefill > 0 && !multirow &&
      !pa::prefill_supported(pool->dtype, pool->head_dim, pool->block_size, G))
    return fail(PA_ERR_UNSUPPORTED, "%s: chunks longer than the multi-row path takes need a bf16 "
                "pool (dtype=%d head_dim=%d max_q_len=%d)", who, pool->dtype, pool->head_dim,
                max_q_len);
  if (num_decode > 0 && !pa::decode_supported(pool->dtype, pool->head_dim, G))
    return fail(PA_ERR_UNSUPPORTED, "%s: dtype=%d head_dim=%d group=%d not built", who,
                pool->dtype, pool->head_dim, G);
  const bool chunks = num_prefill > 0 && max_q_len > 0;
  if (multirow) {
    // short chunks (speculative verification, small prompt pieces): decode
    // rows and chunk rows in one multi-row decode over all the sequences
    const bool pair = pa::multirow_pair(G, max_q_len);
    const pa::DecodeLayout lay = pa::multirow_layout(pool->head_dim, num_workers, pair);
    if (!workspace || workspace_bytes < lay.total())
      return fail(PA_ERR_WORKSPACE, "%s: workspace of %zu bytes, %zu needed "
                  "(pa_attention_mixed_workspace_bytes)", who,
                  workspace ? workspace_bytes : size_t(0), lay.total());
    if (reinterpret_cast<uintptr_t>(workspace) & 15)
      return fail(PA_ERR_INVALID, "%s: workspace must be 16-byte aligned", who);
    if (int64_t(num_decode) + num_prefill >= (int64_t(1) << 30))
      return fail(PA_ERR_UNSUPPORTED, "%s: too many sequences", who);
    pa::DecodeArgs a = pa::decode_args(out, q, pool, block_tables, max_blocks_per_seq, seq_lens,
                                       num_decode + num_prefill, num_q_heads, scale, lay,
                                       workspace);
    a.q_start_loc = q_start_loc;
    a.mr_pair = pair ? 1 : 0;
    return pa::hip_status(pa::launch_decode(a, static_cast<hipStream_t>(stream)), who);
  }
  const bool both = chunks && num_decode > 0;
  // With both kinds of rows, the chunks (bound by the compute units) run on a
  // second stream beside the decode rows (bound by HBM), joined before return.
  // The decode then takes fewer waves per compute unit by default, which
  // leaves each SIMD room for a prefill wave: the two kernels share the chip
  // instead of queueing behind each other.
  const int32_t workers =
      num_workers > 0 ? num_workers : (both ? pa::device_cus() * pa::kMixedDecodeWavesPerCU : 0);
  const pa::DecodeLayout lay = pa::decode_layout(num_decode > 0 ? num_decode : 1, num_q_heads,
                                                 pool->num_kv_heads, pool->head_dim, workers);
  if (num_decode > 0) {
    if (!workspace || workspace_bytes < lay.total())
      return fail(PA_ERR_WORKSPACE, "%s: workspace of %zu bytes, %zu needed", who,
                  workspace ? workspace_bytes : size_t(0), lay.total());
    if (reinterpret_cast<uintptr_t>(workspace) & 15)
      return fail(PA_ERR_INVALID, "%s: workspace must be 16-byte aligned", who);
  }
  const hipStream_t st = static_cast<hipStream_t>(stream);
  pa::SideStream* side = nullptr;
  if (both) {
    if (pa_status s = pa::hip_status(pa::side_stream(&side), who)) return s;
    if (pa_status s = pa::hip_status(hipEventRecord(side->fork, st), who)) return s;
    if (pa_status s = pa::hip_status(hipStreamWaitEvent(side->stream, side->fork, 0), who))
      return s;
  }
  auto run_decode = [&]() -> pa_status {  // rows 0 .. num_decode-1, one per sequence
    pa::DecodeArgs a = pa::decode_args(out, q, pool, block_tables, max_blocks_per_seq, seq_lens,
                                       num_decode, num_q_heads, scale, lay, workspace);
    // decode rows alone: pa_decode's defaults
    if (num_workers == 0 && !both && pool->dtype == PA_BF16 && pa::decode_heads_per_unit(G) >= 4)
      a.workers = pa::matrix_default_workers(lay.workers);
    return pa::hip_status(pa::launch_decode(a, st), who);
  };
  auto run_chunks = [&]() -> pa_status {
    // sequences num_decode.. : their rows start at q_start_loc[num_decode]
    pa::PrefillArgs a{};
    a.out = out;
    a.q = q;
    a.q_start_loc = q_start_loc + num_decode;
    a.seq_lens = seq_lens + num_decode;
    a.k_pool = pool->k_pool;
    a.v_pool = pool->v_pool;
    a.block_tables = block_tables + int64_t(num_decode) * max_blocks_per_seq;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.num_seqs = num_prefill;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = pool->num_kv_heads;
    a.head_dim = pool->head_dim;
    a.block_size = pool->block_size;
    a.max_q_len = max_q_len;
    a.scale = scale;
    return pa::hip_status(pa::launch_prefill(a, side ? side->stream : st), who);
  };
  pa_status result = PA_OK;
  if (pa::kMixedDecodeFirst) {
    if (num_decode > 0) result = run_decode();
    if (chunks && result == PA_OK) result = run_chunks();
  } else {
    if (chunks) result = run_chunks();
    if (num_decode > 0 && result == PA_OK) result = run_decode();
  }
  if (side) {
    // Join the side stream back into the caller's stream whatever happened
    // above, so that no work of this call is left unordered with later work
    // on `stream`. A launch error is reported in preference to a join error.
    hipError_t e = hipEventRecord(side->join, side->stream);
    if (e == hipSuccess) e = hipStreamWaitEvent(st, side->join, 0);
    if (result == PA_OK) result = pa::hip_status(e, who);
  }
  return result;
}

pa_status pa_prefill_chunk(void* out, const void* q, const int32_t* q_start_loc,
                           const int32_t* seq_lens, const pa_pool* pool,
                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                           int32_t num_seqs, int32_t num_q_heads, int32_t max_q_len, float scale,
                           void* stream) {
  pa::clear_error();
  if (pa_status s = pa::check_pool(pool, "pa_prefill_chunk")) return s;
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || num_q_heads <= 0 || max_q_len < 0)
    return fail(PA_ERR_INVALID, "pa_prefill_chunk: bad sizes");
  if (num_seqs == 0 || max_q_len == 0) return PA_OK;
  if (num_seqs > 65535) return fail(PA_ERR_UNSUPPORTED, "pa_prefill_chunk: num_seqs > 65535");
  if (!out || !q || !q_start_loc || !seq_lens || !block_tables)
    return fail(PA_ERR_INVALID, "pa_prefill_chunk: NULL pointer argument");
  if (num_q_heads % pool->num_kv_heads)
    return fail(PA_ERR_INVALID, "pa_prefill_chunk: num_q_heads not a multiple of num_kv_heads");
  if (pa_status s = pa::check_scale(scale, "pa_prefill_chunk")) return s;
  if ((reinterpret_cast<uintptr_t>(out) | reinterpret_cast<uintptr_t>(q) |
       reinterpret_cast<uintptr_t>(pool->k_pool) | reinterpret_cast<uintptr_t>(pool->v_pool)) & 15)
    return fail(PA_ERR_INVALID, "pa_prefill_chunk: out/q/pools must be 16-byte aligned");
  const int32_t G = num_q_heads / pool->num_kv_heads;
  if (!pa::prefill_supported(pool->dtype, pool->head_dim, pool->block_size, G))
    return fail(PA_ERR_UNSUPPORTED, "pa_prefill_chunk: dtype=%d head_dim=%d block_size=%d not built",
                pool->dtype, pool->head_dim, pool->block_size);
  pa::PrefillArgs a{};
  a.out = out;
  a.q = q;
  a.q_start_loc = q_start_loc;
  a.seq_lens = seq_lens;
  a.k_pool = pool->k_pool;
  a.v_pool = pool->v_pool;
  a.block_tables = block_tables;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = pool->num_kv_heads;
  a.head_dim = pool->head_dim;
  a.block_size = pool->block_size;
  a.max_q_len = max_q_len;
  a.scale = scale;
  return pa::hip_status(pa::launch_prefill(a, static_cast<hipStream_t>(stream)),
                        "pa_prefill_chunk");
}

}  // extern "C"
