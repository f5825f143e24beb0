// Cache write (slot scatter) and whole-block copy. For F32 and BF16 pools both
// are byte copies in 16-byte units, so they are bit-exact; an FP8 pool's cache
// write quantizes bf16 rows to E4M3 codes (see cache_write_fp8_kernel).
//
// Slot rule ("LLM inference engine internals", section 2.3): slot =
// block * B + offset. Pool layout [num_blocks][Hkv][B][D]: the row of token
// (block b, offset o) for head h starts at element ((b * Hkv + h) * B + o) * D.
#include "device.h"

namespace pa {
namespace {

// One thread per 16-byte chunk of one (token, head) row; K and V together.
__global__ __launch_bounds__(256) void cache_write_kernel(
    const uint4* __restrict__ k_new, const uint4* __restrict__ v_new,
    const int64_t* __restrict__ slots, uint4* __restrict__ k_pool, uint4* __restrict__ v_pool,
    int64_t total_chunks, int32_t chunks_per_token, int32_t chunks_per_row, int32_t heads,
    int32_t block_size) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < total_chunks; i += stride) {
    const int64_t t = i / chunks_per_token;
    const int32_t rem = int32_t(i - t * chunks_per_token);
    const int32_t h = rem / chunks_per_row;
    const int32_t c = rem - h * chunks_per_row;
    const int64_t slot = slots[t];
    if (slot < 0) continue;  // padding token
    const int64_t b = slot / block_size;
    const int64_t o = slot - b * block_size;
    const int64_t dst = ((b * heads + h) * block_size + o) * chunks_per_row + c;
    k_pool[dst] = k_new[i];
    v_pool[dst] = v_new[i];
  }
}

// Four values -> four E4M3 codes (first value in the low byte): x / scale (an
// IEEE division), clamped to the largest finite magnitude (a quotient of
// +-inf included), rounded to nearest even by v_cvt_pk_fp8_f32 (OCP E4M3 on
// gfx950). A NaN input is stored as the NaN code 0x7F whatever its sign or
// payload: it is converted as 0 and its byte replaced afterwards.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d, float s) {
  auto q = [s](float x) { return x != x ? 0.f : fminf(fmaxf(x / s, -448.f), 448.f); };
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(q(a), q(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(q(c), q(d), w, true);
  const uint32_t nan = (a != a ? 0xffu : 0u) | (b != b ? 0xff00u : 0u) |
                       (c != c ? 0xff0000u : 0u) | (d != d ? 0xff000000u : 0u);
  return (uint32_t(w) & ~nan) | (0x7f7f7f7fu & nan);
}

// 16 bf16 values (two 16-byte chunks) -> 16 codes.
__device__ __forceinline__ uint4 e4m3x16(const uint4& lo, const uint4& hi, float s) {
  return make_uint4(e4m3x4(bf16_lo(lo.x), bf16_hi(lo.x), bf16_lo(lo.y), bf16_hi(lo.y), s),
                    e4m3x4(bf16_lo(lo.z), bf16_hi(lo.z), bf16_lo(lo.w), bf16_hi(lo.w), s),
                    e4m3x4(bf16_lo(hi.x), bf16_hi(hi.x), bf16_lo(hi.y), bf16_hi(hi.y), s),
                    e4m3x4(bf16_lo(hi.z), bf16_hi(hi.z), bf16_lo(hi.w), bf16_hi(hi.w), s));
}

// FP8 pools: one thread per 16 codes of one (token, head) row, i.e. 32 bytes of
// bf16 input (input chunks 2i and 2i+1 of the flat [T][Hkv][D] rows); K and V.
__global__ __launch_bounds__(256) void cache_write_fp8_kernel(
    const uint4* __restrict__ k_new, const uint4* __restrict__ v_new,
    const int64_t* __restrict__ slots, uint4* __restrict__ k_pool, uint4* __restrict__ v_pool,
    int64_t total_chunks, int32_t chunks_per_token, int32_t chunks_per_row, int32_t heads,
    int32_t block_size, float k_scale, float v_scale) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < total_chunks; i += stride) {
    const int64_t t = i / chunks_per_token;
    const int32_t rem = int32_t(i - t * chunks_per_token);
    const int32_t h = rem / chunks_per_row;
    const int32_t c = rem - h * chunks_per_row;
    const int64_t slot = slots[t];
    if (slot < 0) continue;  // padding token
    const int64_t b = slot / block_size;
    const int64_t o = slot - b * block_size;
    const int64_t dst = ((b * heads + h) * block_size + o) * chunks_per_row + c;
    k_pool[dst] = e4m3x16(k_new[2 * i], k_new[2 * i + 1], k_scale);
    v_pool[dst] = e4m3x16(v_new[2 * i], v_new[2 * i + 1], v_scale);
  }
}

// grid.y = pair index; each thread copies 16-byte chunks of one block, K and V.
__global__ __launch_bounds__(256) void copy_blocks_kernel(
    const int32_t* __restrict__ src_dst, uint4* __restrict__ k_pool, uint4* __restrict__ v_pool,
    int64_t chunks_per_block) {
  const int64_t src = src_dst[2 * blockIdx.y];
  const int64_t dst = src_dst[2 * blockIdx.y + 1];
  const uint4* ks = k_pool + src * chunks_per_block;
  const uint4* vs = v_pool + src * chunks_per_block;
  uint4* kd = k_pool + dst * chunks_per_block;
  uint4* vd = v_pool + dst * chunks_per_block;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < chunks_per_block;
       i += int64_t(gridDim.x) * blockDim.x) {
    kd[i] = ks[i];
    vd[i] = vs[i];
  }
}

// Block swap between the device pool and a pool in pinned host memory: one
// launch moves up to kSwapBatch blocks, whose (src, dst) ids travel in the
// kernel arguments (checked on the host). grid.y = pair; 4 independent 16-byte
// chunks per thread keep many transfers across the host link in flight.
__global__ __launch_bounds__(256) void swap_blocks_kernel(
    SwapBatch b, const uint4* __restrict__ src_k, const uint4* __restrict__ src_v,
    uint4* __restrict__ dst_k, uint4* __restrict__ dst_v, int64_t chunks_per_block) {
  constexpr int U = 4;
  const int64_t src = b.pairs[2 * blockIdx.y];
  const int64_t dst = b.pairs[2 * blockIdx.y + 1];
  const uint4* ks = src_k + src * chunks_per_block;
  const uint4* vs = src_v + src * chunks_per_block;
  uint4* kd = dst_k + dst * chunks_per_block;
  uint4* vd = dst_v + dst * chunks_per_block;
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t i0 = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i0 < chunks_per_block;
       i0 += U * stride) {
    uint4 k[U], v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = i0 + u * stride;
      if (i < chunks_per_block) {
        k[u] = ks[i];
        v[u] = vs[i];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = i0 + u * stride;
      if (i < chunks_per_block) {
        kd[i] = k[u];
        vd[i] = v[u];
      }
    }
  }
}

int elt_bytes(int dtype) { return dtype == PA_F32 ? 4 : dtype == PA_BF16 ? 2 : 1; }

}  // namespace

hipError_t launch_cache_write(const pa_pool& pool, const void* k_new, const void* v_new,
                              const int64_t* slots, int32_t T, hipStream_t stream) {
  const int32_t cpr = pool.head_dim * elt_bytes(pool.dtype) / 16;
  const int32_t cpt = cpr * pool.num_kv_heads;
  const int64_t total = int64_t(T) * cpt;
  const int64_t want = (total + 255) / 256;
  const int grid = int(want < 8192 ? want : 8192);
  if (pool.dtype == PA_FP8_E4M3) {
    cache_write_fp8_kernel<<<grid, 256, 0, stream>>>(
        static_cast<const uint4*>(k_new), static_cast<const uint4*>(v_new), slots,
        static_cast<uint4*>(pool.k_pool), static_cast<uint4*>(pool.v_pool), total, cpt, cpr,
        pool.num_kv_heads, pool.block_size, pool.k_scale, pool.v_scale);
    return hipGetLastError();
  }
  cache_write_kernel<<<grid, 256, 0, stream>>>(
      static_cast<const uint4*>(k_new), static_cast<const uint4*>(v_new), slots,
      static_cast<uint4*>(pool.k_pool), static_cast<uint4*>(pool.v_pool), total, cpt, cpr,
      pool.num_kv_heads, pool.block_size);
  return hipGetLastError();
}

// Streaming read for measuring the device's read ceiling. Each wave reads
// contiguous 8 KB runs (64 lanes x 16 bytes x 8 non-temporal loads in
// flight), runs dealt round-robin over the waves; the bytes past the last
// whole run are read by a grid-stride loop. Of the patterns measured on
// MI355X (grid-stride, 4 or 8 loads per lane, plain or non-temporal, 4 or
// 8 KB runs per wave) this one read fastest.
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* p, int64_t n, uint32_t* sink) {
  constexpr int kLoads = 8;
  constexpr int64_t kRun = int64_t(kWave) * kLoads;  // 16-byte chunks per run
  const int lane = threadIdx.x % kWave;
  const int64_t wave = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) / kWave;
  const int64_t waves = int64_t(gridDim.x) * blockDim.x / kWave;
  const int64_t runs = n / kRun;
  uint32_t acc = 0;
  for (int64_t r = wave; r < runs; r += waves) {
    const uint4* q = p + r * kRun + lane;
    uint4 v[kLoads];
#pragma unroll
    for (int k = 0; k < kLoads; ++k) v[k] = load_stream16(q + kWave * k);
#pragma unroll
    for (int k = 0; k < kLoads; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t i = runs * kRun + int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
    const uint4 a = load_stream16(p + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9e3779b9u) *sink = acc;
}

hipError_t launch_stream_read(const void* buf, size_t bytes, int grid, uint32_t* sink,
                              hipStream_t stream) {
  stream_read_kernel<<<grid, 256, 0, stream>>>(static_cast<const uint4*>(buf),
                                               int64_t(bytes / 16), sink);
  return hipGetLastError();
}

hipError_t launch_swap_blocks(const SwapBatch& b, int32_t n, const void* src_k, const void* src_v,
                              void* dst_k, void* dst_v, int64_t block_bytes, hipStream_t stream) {
  if (n <= 0 || n > kSwapBatch || block_bytes % 16) return hipErrorInvalidValue;
  const int64_t cpb = block_bytes / 16;
  const int64_t want = (cpb + 4 * 256 - 1) / (4 * 256);
  const int gx = int(want < 64 ? want : 64);
  swap_blocks_kernel<<<dim3(gx, n), 256, 0, stream>>>(
      b, static_cast<const uint4*>(src_k), static_cast<const uint4*>(src_v),
      static_cast<uint4*>(dst_k), static_cast<uint4*>(dst_v), cpb);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(const pa_pool& pool, const int32_t* src_dst, int32_t n,
                              hipStream_t stream) {
  const int64_t cpb = int64_t(pool.num_kv_heads) * pool.block_size * pool.head_dim *
                      elt_bytes(pool.dtype) / 16;
  const int64_t want = (cpb + 255) / 256;
  const int gx = int(want < 64 ? want : 64);
  copy_blocks_kernel<<<dim3(gx, n), 256, 0, stream>>>(
      src_dst, static_cast<uint4*>(pool.k_pool), static_cast<uint4*>(pool.v_pool), cpb);
  return hipGetLastError();
}

}  // namespace pa
