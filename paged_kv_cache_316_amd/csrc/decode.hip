// Decode-step paged attention for gfx950.
//
// What it computes: for each sequence s and query head h,
//   out[s][h] = sum_t softmax_t(scale * q.K_s[t]) V_s[t]
// over the seq_lens[s] tokens of s, reading K_s[t] / V_s[t] through the block
// table (logical block t / B -> physical block, offset t % B). This completes
// the kernel outline of "LLM inference engine internals" (section 2.4: grid
// over heads, two-level lookup, q.k; softmax and the V step left as a
// comment) and follows "vLLM PagedAttention explained", section 3.3 step 2
// (the request sees contiguous KV; the lookup translates addresses).
//
// How (MI355X design, not the outline's):
//  * One wavefront owns (sequence, KV head, partition of P tokens) and all the
//    query heads that share that KV head (grouped heads), so each K/V row is
//    read from HBM once per step.
//  * Lane layout: a token row of D elements is LPR lanes x 16 bytes; a
//    wave-wide 16-byte load covers NR = 64 / LPR token rows (bf16, D = 128:
//    16 lanes per row, 4 rows per load, 4 loads per 16-token tile). Loads are
//    fully coalesced 16-byte accesses.
//  * q.k: per-lane partial dot over its 16 bytes (v_dot2 for bf16), then a
//    sum over the LPR lanes of the row with DPP (quad_perm, row_half_mirror,
//    row_mirror).
//  * Online softmax in base 2, kept per row group (lanes with the same token
//    row index), so the hot loop has no cross-row traffic; the NR row groups
//    are merged once per partition.
//  * The block-table slice of the partition is staged once per workgroup in
//    LDS and shared by its four waves (four KV heads of one sequence).
//  * Tiles are double-buffered: the K/V loads of tile i+1 are in flight while
//    tile i is computed.
//  * Sequences longer than P are split into partitions; each writes
//    (max, denominator, unnormalised sum) and a second kernel combines them
//    with the log-sum-exp rule. A sequence with one partition writes its
//    output directly.
#include <math.h>

#include "device.h"

namespace pa {
namespace {

constexpr int kWavesPerGroup = 4;
constexpr int kTile = 16;             // tokens per wave iteration
constexpr int kMaxPartBlocks = 1024;  // LDS table-slice capacity (P / B)
constexpr float kLog2e = 1.4426950408889634f;

template <int DTYPE, int D, int HPW>
struct Tile {
  using RS = RowShape<DTYPE, D>;
  static constexpr int VEC = RS::VEC, LPR = RS::LPR, NR = RS::NR;
  static constexpr int U = kTile / NR;  // 16-byte loads per lane per tile, for K and for V
  static_assert(kTile % NR == 0, "tile must cover whole load rows");
};

typedef short bf16x2_t __attribute__((__vector_size__(2 * sizeof(short))));

// Partial dot product of this lane's 16 bytes of k with its slice of q.
template <int DTYPE>
__device__ __forceinline__ float dot16(const uint4& k, const float* qf, const uint4& qb);

template <>
__device__ __forceinline__ float dot16<PA_F32>(const uint4& k, const float* qf, const uint4&) {
  float s = qf[0] * __uint_as_float(k.x);
  s = fmaf(qf[1], __uint_as_float(k.y), s);
  s = fmaf(qf[2], __uint_as_float(k.z), s);
  s = fmaf(qf[3], __uint_as_float(k.w), s);
  return s;
}

template <>
__device__ __forceinline__ float dot16<PA_BF16>(const uint4& k, const float*, const uint4& qb) {
  float s = 0.f;
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.x),
                                      __builtin_bit_cast(bf16x2_t, qb.x), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.y),
                                      __builtin_bit_cast(bf16x2_t, qb.y), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.z),
                                      __builtin_bit_cast(bf16x2_t, qb.z), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.w),
                                      __builtin_bit_cast(bf16x2_t, qb.w), s, false);
  return s;
}

template <int DTYPE>
__device__ __forceinline__ void unpack16(const uint4& v, float* f);

template <>
__device__ __forceinline__ void unpack16<PA_F32>(const uint4& v, float* f) {
  f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
  f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
}

template <>
__device__ __forceinline__ void unpack16<PA_BF16>(const uint4& v, float* f) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z); f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

// Store VEC fp32 values as one 16-byte chunk of the output dtype.
template <int DTYPE>
__device__ __forceinline__ uint4 pack16(const float* f);

template <>
__device__ __forceinline__ uint4 pack16<PA_F32>(const float* f) {
  return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                    __float_as_uint(f[3]));
}

template <>
__device__ __forceinline__ uint4 pack16<PA_BF16>(const float* f) {
  return make_uint4(pack_bf16(f[0], f[1]), pack_bf16(f[2], f[3]), pack_bf16(f[4], f[5]),
                    pack_bf16(f[6], f[7]));
}

template <int DTYPE, int D, int HPW>
__global__ __launch_bounds__(kWave * kWavesPerGroup) void decode_partition_kernel(
    DecodeArgs a, int32_t b_shift, int32_t n_hchunk, float scale_log2) {
  using TL = Tile<DTYPE, D, HPW>;
  constexpr int VEC = TL::VEC, LPR = TL::LPR, NR = TL::NR, U = TL::U;
  constexpr int ELT = Elt<DTYPE>::bytes;
  __shared__ int32_t s_bt[kMaxPartBlocks];

  const int part = blockIdx.x;
  const int seq = blockIdx.z;
  const int L = a.seq_lens[seq];
  const int P = a.partition_tokens;
  const int start = part * P;
  const int Hq = a.num_q_heads, Hkv = a.num_kv_heads;
  const int G = Hq / Hkv;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int unit = blockIdx.y * kWavesPerGroup + wave;
  const int kvh = unit / n_hchunk;
  const int head0 = kvh * G + (unit % n_hchunk) * HPW;
  const bool active = kvh < Hkv;
  const int r = lane / LPR, c = lane % LPR;

  if (L <= 0) {  // empty sequence: output zeros
    if (part == 0 && active && r == 0) {
      uint4* o = static_cast<uint4*>(a.out) + ((int64_t(seq) * Hq + head0) * D) / VEC + c;
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh) o[hh * (D / VEC)] = make_uint4(0, 0, 0, 0);
    }
    return;
  }
  if (start >= L) return;  // uniform over the workgroup
  const int end = min(L, start + P);
  const int first_blk = start >> b_shift;
  const int nblk = ((end - 1) >> b_shift) - first_blk + 1;
  const int32_t* bt_row = a.block_tables + int64_t(seq) * a.max_blocks_per_seq + first_blk;
  for (int i = threadIdx.x; i < nblk; i += blockDim.x) s_bt[i] = bt_row[i];
  __syncthreads();
  if (!active) return;

  // This lane's slice of the HPW query heads.
  float qf[HPW][VEC > 4 ? 4 : VEC];
  uint4 qb[HPW];
  {
    const uint4* qp = static_cast<const uint4*>(a.q) + ((int64_t(seq) * Hq + head0) * D) / VEC + c;
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      qb[hh] = qp[hh * (D / VEC)];
      if constexpr (DTYPE == PA_F32) {
        qf[hh][0] = __uint_as_float(qb[hh].x) * scale_log2;
        qf[hh][1] = __uint_as_float(qb[hh].y) * scale_log2;
        qf[hh][2] = __uint_as_float(qb[hh].z) * scale_log2;
        qf[hh][3] = __uint_as_float(qb[hh].w) * scale_log2;
      }
    }
  }
  const float zmul = DTYPE == PA_F32 ? 1.f : scale_log2;

  float m[HPW], l[HPW], acc[HPW][VEC];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[hh][e] = 0.f;
  }

  const uint4* kp = static_cast<const uint4*>(a.k_pool);
  const uint4* vp = static_cast<const uint4*>(a.v_pool);
  const int Bm1 = a.block_size - 1;
  const int64_t head_rows = int64_t(Hkv) * a.block_size;

  auto chunk_index = [&](int lt) -> int64_t {
    const int64_t pb = s_bt[(lt >> b_shift) - first_blk];
    return ((pb * Hkv + kvh) * a.block_size + (lt & Bm1)) * LPR + c;
  };
  (void)head_rows;

  auto load_full = [&](int base, uint4* kr, uint4* vr) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t idx = chunk_index(base + u * NR + r);
      kr[u] = load_stream16(kp + idx);
      vr[u] = load_stream16(vp + idx);
    }
  };
  auto load_tail = [&](int base, uint4* kr, uint4* vr) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int lt = base + u * NR + r;
      if (lt < end) {
        const int64_t idx = chunk_index(lt);
        kr[u] = load_stream16(kp + idx);
        vr[u] = load_stream16(vp + idx);
      } else {
        kr[u] = make_uint4(0, 0, 0, 0);
        vr[u] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto compute = [&](int base, const uint4* kr, const uint4* vr, bool masked) {
    float z[HPW][U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool valid = !masked || (base + u * NR + r < end);
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh) {
        const float s = group_sum<LPR>(dot16<DTYPE>(kr[u], qf[hh], qb[hh])) * zmul;
        z[hh][u] = valid ? s : -INFINITY;
      }
    }
    float p[HPW][U];
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      float mx = z[hh][0];
#pragma unroll
      for (int u = 1; u < U; ++u) mx = fmaxf(mx, z[hh][u]);
      const float mn = fmaxf(m[hh], mx);
      const float ms = mn == -INFINITY ? 0.f : mn;
      const float alpha = __builtin_amdgcn_exp2f(m[hh] - ms);
      m[hh] = mn;
      float lsum = l[hh] * alpha;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        p[hh][u] = __builtin_amdgcn_exp2f(z[hh][u] - ms);
        lsum += p[hh][u];
      }
      l[hh] = lsum;
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[hh][e] *= alpha;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float vf[VEC];
      unpack16<DTYPE>(vr[u], vf);
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh)
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[hh][e] = fmaf(p[hh][u], vf[e], acc[hh][e]);
    }
  };

  const int ntok = end - start;
  const int nfull = ntok / kTile;
  uint4 ka[U], va[U], kb[U], vb[U];
  int it = 0;
  if (nfull > 0) load_full(start, ka, va);
  for (; it + 2 <= nfull; it += 2) {
    load_full(start + (it + 1) * kTile, kb, vb);
    compute(start + it * kTile, ka, va, false);
    if (it + 2 < nfull) load_full(start + (it + 2) * kTile, ka, va);
    compute(start + (it + 1) * kTile, kb, vb, false);
  }
  if (it < nfull) {  // one full tile left, already in ka/va
    compute(start + it * kTile, ka, va, false);
    ++it;
  }
  if (ntok % kTile) {
    load_tail(start + it * kTile, kb, vb);
    compute(start + it * kTile, kb, vb, true);
  }

  // Merge the NR row groups: each holds the softmax state of its own tokens.
#pragma unroll
  for (int off = LPR; off < kWave; off <<= 1) {
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      const float mo = __shfl_xor(m[hh], off);
      const float lo = __shfl_xor(l[hh], off);
      const float mn = fmaxf(m[hh], mo);
      const float ms = mn == -INFINITY ? 0.f : mn;
      const float fa = __builtin_amdgcn_exp2f(m[hh] - ms);
      const float fb = __builtin_amdgcn_exp2f(mo - ms);
      l[hh] = l[hh] * fa + lo * fb;
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[hh][e] = acc[hh][e] * fa + __shfl_xor(acc[hh][e], off) * fb;
      m[hh] = mn;
    }
  }
  if (r != 0) return;

  const int nparts = (L + P - 1) / P;
  if (nparts == 1) {
    uint4* o = static_cast<uint4*>(a.out) + ((int64_t(seq) * Hq + head0) * D) / VEC + c;
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      const float inv = 1.f / l[hh];
      float f[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) f[e] = acc[hh][e] * inv;
      o[hh * (D / VEC)] = pack16<DTYPE>(f);
    }
  } else {
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      const int64_t row = (int64_t(seq) * Hq + head0 + hh) * a.max_parts + part;
      float4* w = reinterpret_cast<float4*>(a.ws_acc + row * D + c * VEC);
#pragma unroll
      for (int e = 0; e < VEC; e += 4)
        w[e / 4] = make_float4(acc[hh][e], acc[hh][e + 1], acc[hh][e + 2], acc[hh][e + 3]);
      if (c == 0) a.ws_ml[row] = make_float2(m[hh], l[hh]);
    }
  }
  (void)ELT;
}

// Log-sum-exp combination of the partitions of one (sequence, head):
// M = max_p m_p; out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p.
template <int DTYPE, int D>
__global__ __launch_bounds__(kWave) void decode_reduce_kernel(DecodeArgs a) {
  constexpr int PER = D / kWave;
  const int h = blockIdx.x, seq = blockIdx.y;
  const int L = a.seq_lens[seq];
  const int P = a.partition_tokens;
  const int np = (L + P - 1) / P;
  if (np <= 1) return;
  const int64_t row0 = (int64_t(seq) * a.num_q_heads + h) * a.max_parts;
  const float2* ml = a.ws_ml + row0;
  float M = -INFINITY;
  for (int p = 0; p < np; ++p) M = fmaxf(M, ml[p].x);
  float den = 0.f, num[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) num[j] = 0.f;
  for (int p = 0; p < np; ++p) {
    const float2 v = ml[p];
    const float w = __builtin_amdgcn_exp2f(v.x - M);
    den = fmaf(v.y, w, den);
    const float* src = a.ws_acc + (row0 + p) * D + threadIdx.x * PER;
#pragma unroll
    for (int j = 0; j < PER; ++j) num[j] = fmaf(src[j], w, num[j]);
  }
  const float inv = 1.f / den;
  const int64_t o = (int64_t(seq) * a.num_q_heads + h) * D + threadIdx.x * PER;
  if constexpr (DTYPE == PA_F32) {
    float* out = static_cast<float*>(a.out) + o;
#pragma unroll
    for (int j = 0; j < PER; ++j) out[j] = num[j] * inv;
  } else {
    uint16_t* out = static_cast<uint16_t*>(a.out) + o;
#pragma unroll
    for (int j = 0; j < PER; ++j) out[j] = uint16_t(f32_to_bf16(num[j] * inv));
  }
}

template <int DTYPE, int D, int HPW>
hipError_t run(const DecodeArgs& a, hipStream_t st) {
  int b_shift = 0;
  while ((1 << b_shift) < a.block_size) ++b_shift;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int n_hchunk = G / HPW;
  const int units = a.num_kv_heads * n_hchunk;
  dim3 grid(a.max_parts, (units + kWavesPerGroup - 1) / kWavesPerGroup, a.num_seqs);
  const float scale_log2 = a.scale * kLog2e;
  decode_partition_kernel<DTYPE, D, HPW>
      <<<grid, kWave * kWavesPerGroup, 0, st>>>(a, b_shift, n_hchunk, scale_log2);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.max_parts <= 1) return e;
  decode_reduce_kernel<DTYPE, D><<<dim3(a.num_q_heads, a.num_seqs), kWave, 0, st>>>(a);
  return hipGetLastError();
}

int heads_per_wave(int G) {
  for (int h : {8, 4, 2, 1})
    if (G % h == 0) return h;
  return 1;
}

template <int DTYPE, int D>
hipError_t run_d(const DecodeArgs& a, hipStream_t st) {
  switch (heads_per_wave(a.num_q_heads / a.num_kv_heads)) {
    case 8: return run<DTYPE, D, 8>(a, st);
    case 4: return run<DTYPE, D, 4>(a, st);
    case 2: return run<DTYPE, D, 2>(a, st);
    default: return run<DTYPE, D, 1>(a, st);
  }
}

}  // namespace

bool decode_supported(int dtype, int head_dim, int group) {
  return (dtype == PA_F32 || dtype == PA_BF16) && (head_dim == 64 || head_dim == 128) &&
         group >= 1;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) {
  if (a.partition_tokens / a.block_size > kMaxPartBlocks) return hipErrorInvalidValue;
  if (a.dtype == PA_BF16) {
    if (a.head_dim == 128) return run_d<PA_BF16, 128>(a, st);
    if (a.head_dim == 64) return run_d<PA_BF16, 64>(a, st);
  } else if (a.dtype == PA_F32) {
    if (a.head_dim == 128) return run_d<PA_F32, 128>(a, st);
    if (a.head_dim == 64) return run_d<PA_F32, 64>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
