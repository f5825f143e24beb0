// Decode for a batch whose block tables all begin with the same full blocks.
//
// Prefix caching maps an identical prompt start of many requests onto the same
// physical blocks ("Why PagedAttention multiplies LLM serving throughput",
// section "Automatic prefix caching"; "LLM inference engine internals",
// section 2.3). Plain decode still reads those blocks once per sequence. Here
// the shared part is read once per KV head for all sequences, and the
// softmax over the whole sequence is put back together exactly:
//
//  1. the regular decode over the tails (tokens P*B .. L_s - 1, table rows
//     offset by P), which also writes each row's log-sum-exp;
//  2. prefix_partial_kernel: for every KV head, the queries of all sequences
//     (S * G columns: sequence s, query head kvh*G + hh is column s*G + hh)
//     against the P*B shared keys, on the matrix cores. The keys are cut into
//     n_split ranges; a workgroup takes one (KV head, key range) and a few
//     column blocks, one per wave, whose waves share the range's K/V tiles
//     through LDS; each wave writes unnormalised partials
//     (sum_t 2^(x_t - m) v_t as bf16, m, l).
//  3. prefix_merge_kernel: per row, M = max of the partial maxima and the
//     suffix log-sum-exp, and out = (sum_c acc_c 2^(m_c-M) + o_s l_s 2^(m_s-M)) /
//     (sum_c l_c 2^(m_c-M) + l_s 2^(m_s-M)), o_s being the suffix output.
// Scores are kept in log2 units (scale * log2(e) folded into the exponent).
#include "device.h"

namespace pa {

namespace {

constexpr int kPTile = 16;           // keys per tile
// 16-column groups per wave, at most. More groups share each K/V tile among
// more columns, but the pass is bound by the per-score softmax work, not by
// re-reading tiles: two groups measured best on the prefix-cached batch.
constexpr int kPMaxGroups = 2;
// column blocks of one (KV head, key range) per workgroup: 8 waves, or 4 when
// a wave needs more than 256 registers (more groups, or FP8 widening)
constexpr int waves_per_group(int ng, bool fp8) { return ng >= 4 || (ng >= 2 && fp8) ? 4 : 8; }
constexpr float kPLog2e = 1.4426950408889634f;
constexpr int kPChunk = 4;  // 16-key tiles per LDS stage of the shared pass

// One workgroup: KV head kvh, key tiles [t0, t1), WPG column blocks of NG
// groups of 16 columns (one block per wave). The key range is walked in
// chunks of kPChunk tiles: the waves split each chunk's wave-wide K/V loads
// between them and write them, widened for FP8 pools, into one of two LDS
// stages, so every tile is read from the pool once per workgroup; one
// barrier per chunk, and the next chunk's loads stay in flight across it.
// Every wave of the workgroup loads and meets the barriers; only those with
// columns compute. Operand layouts as in the GQA decode kernel (rows swizzled
// so that the reads below are conflict-free): S^T = K Q^T on
// v_mfma_f32_16x16x32_bf16 (16 keys x 16 columns); the accumulator is
// already the B operand of O^T = V^T P^T (v_mfma_f32_16x16x16_bf16, V^T read
// with ds_read_b64_tr_b16); the exponent base of a column moves only when its
// max grows by more than 2^8.
template <int D, int NG, bool BIG_B, int KV>
__global__ __launch_bounds__(kWave * waves_per_group(NG, KV == PA_FP8_E4M3)) void prefix_partial_kernel(
    PrefixArgs a, int32_t b_shift, int32_t n_cblk, int32_t n_cgrp, int32_t tiles_per_split,
    float scale_log2) {
  constexpr bool FP8 = KV == PA_FP8_E4M3;
  constexpr int WPG = waves_per_group(NG, FP8);
  constexpr int ROW = 2 * D;           // bytes per bf16 row in LDS
  constexpr int GROW = FP8 ? D : ROW;  // bytes per row in the pool
  constexpr int KS = D / 32;
  constexpr int DT = D / 16;
  constexpr int CPR = ROW / 16;
  constexpr int GCPR = GROW / 16;
  constexpr int RPI = 1024 / GROW;     // rows per wave-wide 16-byte load
  constexpr int NI = kPTile / RPI;     // such loads per tile
  constexpr int RPL = 256 / ROW;
  constexpr int TB = kPTile * ROW;     // one bf16 tile in LDS
  constexpr int CB = kPChunk * TB;     // the K (or V) half of a stage
  constexpr int NLD = 2 * kPChunk * NI;  // wave-wide loads per chunk, K then V
  static_assert(NLD % WPG == 0, "a chunk's loads split evenly over the waves");
  constexpr int NL = NLD / WPG;        // this wave's share
  extern __shared__ __align__(16) unsigned char smem[];

  const int lane = threadIdx.x % kWave;
  const int wig = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  // Workgroup i runs on XCD i % 8: renumber so that neighbouring work items
  // (same KV head and key range, hence the same K/V) share an XCD's L2.
  int wg = blockIdx.x;
  if (gridDim.x % 8 == 0) wg = (blockIdx.x % 8) * (gridDim.x / 8) + blockIdx.x / 8;
  const int cg = wg % n_cgrp;
  const int rest = wg / n_cgrp;
  const int sp = rest % a.n_split;
  const int kvh = rest / a.n_split;
  const int cb = cg * WPG + wig;
  const bool active = cb < n_cblk;  // wave-uniform

  const int S = a.num_seqs, Hq = a.num_q_heads, Hkv = a.num_kv_heads;
  const int G = Hq / Hkv;
  const int N = S * G;
  const int g = lane / 16, i16 = lane % 16;
  const int B = a.block_size, Bm1 = B - 1;
  const int Lp = a.num_prefix_blocks * B;
  const int n_tiles = (Lp + kPTile - 1) / kPTile;
  const int t0 = sp * tiles_per_split;
  const int t1 = min(t0 + tiles_per_split, n_tiles);
  const int nch = (t1 - t0 + kPChunk - 1) / kPChunk;

  auto swz = [](int r) { return (r / RPL) % CPR; };
  const int lrow = lane / GCPR, lch = lane % GCPR;
  // this wave's loads of a chunk: load li = wig + WPG * k is the K load li
  // (li < NLD / 2) or the V load li - NLD / 2; load kk of a kind reads rows
  // (kk % NI) * RPI + lrow of the chunk's tile kk / NI
  int ltile[NL];
  uint32_t wr[NL], wr2[NL];
#pragma unroll
  for (int k = 0; k < NL; ++k) {
    const int li = wig + WPG * k;
    const int kk = li % (NLD / 2);
    ltile[k] = kk / NI;
    const int r = (kk % NI) * RPI + lrow;
    const int c0 = FP8 ? 2 * lch : lch;
    const uint32_t base = uint32_t((li >= NLD / 2 ? CB : 0) + ltile[k] * TB + r * ROW);
    wr[k] = base + uint32_t((c0 ^ swz(r)) * 16);
    wr2[k] = base + uint32_t(((c0 + 1) ^ swz(r)) * 16);
  }
  const uint32_t kr0 = uint32_t(i16 * ROW + ((g ^ swz(i16)) * 16));
  const int rr = 4 * g + i16 / 4;
  const uint32_t rd0 = uint32_t(rr * ROW + 8 * (i16 % 2) + (((i16 % 4) / 2) ^ swz(rr)) * 16);

  // this lane's column in group q: sequence s, query head kvh*G + hh
  // (clamped to a real column; columns past N multiply zeros and write nothing)
  bool valid[NG];
  int64_t orow[NG];  // row of out / lse / partials
  uint4 qop[NG][KS];
#pragma unroll
  for (int q = 0; q < NG; ++q) {
    const int col = (cb * NG + q) * 16 + i16;
    valid[q] = active && col < N;
    const int cc = max(min(col, N - 1), 0);
    orow[q] = int64_t(cc / G) * Hq + kvh * G + cc % G;
    const unsigned char* qp = static_cast<const unsigned char*>(a.q) + orow[q] * ROW + 16 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint4 qv = *reinterpret_cast<const uint4*>(qp + 64 * ks);
      qop[q][ks] = valid[q] ? qv : make_uint4(0, 0, 0, 0);
    }
  }
  f32x4_t o[NG][DT];
  float m[NG], lpart[NG];
#pragma unroll
  for (int q = 0; q < NG; ++q) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[q][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    m[q] = -INFINITY;
    lpart[q] = 0.f;
  }
  const float c2 = FP8 ? scale_log2 * a.k_scale : scale_log2;
  const float vsc = FP8 ? a.v_scale : 1.f;

  // one 16-key tile (tile j, at kt / kt + CB in LDS) for the NG column
  // groups: the K and V operands are read from LDS once and shared by them
  auto compute = [&](int j, const unsigned char* kt) {
    uint4 kop[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kop[ks] = *reinterpret_cast<const uint4*>(kt + (kr0 ^ (64u * ks)));
    v4i16_t va[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      va[dt] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(kt + CB + (rd0 ^ (32u * dt))));
    const int key0 = j * kPTile + 4 * g;
#pragma unroll
    for (int q = 0; q < NG; ++q) {
      f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kop[ks]),
                                                    __builtin_bit_cast(bf16x8_t, qop[q][ks]), sc,
                                                    0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (key0 + i >= Lp) sc[i] = -INFINITY;
      float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
      {  // max over the 4 lanes of column l%16
        const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                          false, false);
        mx = fmaxf(__uint_as_float(s16[0]), __uint_as_float(s16[1]));
        const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                          false, false);
        mx = fmaxf(__uint_as_float(s32[0]), __uint_as_float(s32[1]));
      }
      const bool moved = m[q] == -INFINITY ? mx != -INFINITY : (mx - m[q]) * c2 > 8.f;
      const float mn = moved ? mx : m[q];
      const float nms = mn == -INFINITY ? 0.f : -mn * c2;
      const float alpha = moved ? __builtin_amdgcn_exp2f(fmaf(m[q], c2, nms)) : 1.f;
      m[q] = mn;
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(fmaf(sc[i], c2, nms));
      const uint2 pb = make_uint2(pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3]));
      typedef short bf16x2_v __attribute__((ext_vector_type(2)));
      const bf16x2_v ones = __builtin_bit_cast(bf16x2_v, 0x3f803f80u);
      float ps = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_v, pb.x), ones, 0.f, false);
      ps = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_v, pb.y), ones, ps, false);
      lpart[q] = lpart[q] * alpha + ps;
      if (__ballot(moved)) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[q][dt] *= alpha;
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        o[q][dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va[dt], __builtin_bit_cast(bf16x4_t, pb),
                                                           o[q][dt], 0, 0, 0);
    }
  };

  // Row 0 of the block tables holds the shared blocks. A chunk's 64 keys
  // lie in at most 64 blocks, whose ids one 64-entry window of that row holds
  // (one entry per lane), loaded a chunk ahead of its K/V loads. Keys past
  // the split's last tile re-read that tile (not computed); keys past the
  // prefix are clamped to its last token and masked.
  const int32_t* row = a.block_tables;
  const int nblk = a.num_prefix_blocks;
  const unsigned char* kp = static_cast<const unsigned char*>(a.k_pool);
  const unsigned char* vp = static_cast<const unsigned char*>(a.v_pool);
  const int64_t block_bytes = int64_t(Hkv) * B * GROW;
  const int64_t head_off = int64_t(kvh) * B * GROW + lch * 16;
  const int Lm1 = Lp - 1;
  auto window = [&](int c) -> int {
    const int jb0 = ((t0 + c * kPChunk) * kPTile) >> b_shift;
    return c < nch && jb0 + lane < nblk ? row[jb0 + lane] : 0;
  };
  uint4 st[NL];  // this wave's share of the next chunk, on its way from the pool
  auto load_chunk = [&](int c, int win) {
    const int jc = t0 + c * kPChunk;
    const int jb0 = (jc * kPTile) >> b_shift;
#pragma unroll
    for (int k = 0; k < NL; ++k) {
      const int j = min(jc + ltile[k], t1 - 1);
      const int li = wig + WPG * k;
      const int t = min(j * kPTile + ((li % (NLD / 2)) % NI) * RPI + lrow, Lm1);
      int pb;
      if constexpr (BIG_B) pb = __builtin_amdgcn_readlane(win, ((j * kPTile) >> b_shift) - jb0);
      else pb = __shfl(win, (t >> b_shift) - jb0);
      const int64_t off = int64_t(pb) * block_bytes + head_off + int64_t(t & Bm1) * GROW;
      st[k] = load_stream16(reinterpret_cast<const uint4*>((li >= NLD / 2 ? vp : kp) + off));
    }
  };
  auto store_chunk = [&](int stage) {
    unsigned char* dst = smem + stage * 2 * CB;
#pragma unroll
    for (int k = 0; k < NL; ++k) {
      if constexpr (FP8) {
        uint4 lo, hi;
        widen_e4m3(st[k], lo, hi);
        *reinterpret_cast<uint4*>(dst + wr[k]) = lo;
        *reinterpret_cast<uint4*>(dst + wr2[k]) = hi;
      } else {
        *reinterpret_cast<uint4*>(dst + wr[k]) = st[k];
      }
    }
  };
  // LDS writes of every wave done; the loads in flight stay so. The empty asm
  // statements keep LDS accesses on their side of the barrier.
  auto meet = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));  // lgkmcnt(0) only
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  int win = window(0);
  int win_next = window(1);
  load_chunk(0, win);
  store_chunk(0);
  win = win_next;
  win_next = window(2);
  if (nch > 1) load_chunk(1, win);
  meet();
  for (int c = 0; c < nch; ++c) {
    if (active) {
      const unsigned char* kt = smem + (c & 1) * 2 * CB;
      const int jc = t0 + c * kPChunk;
#pragma unroll
      for (int t = 0; t < kPChunk; ++t)
        if (jc + t < t1) compute(jc + t, kt + t * TB);
    }
    if (c + 1 < nch) {
      // stage (c + 1) & 1 was last read in chunk c - 1, before the last barrier
      store_chunk((c + 1) & 1);
      if (c + 2 < nch) {
        win = win_next;
        win_next = window(c + 3);
        load_chunk(c + 2, win);
      }
      meet();
    }
  }

#pragma unroll
  for (int q = 0; q < NG; ++q) {
    float l = lpart[q] + __shfl_xor(lpart[q], 16);
    l += __shfl_xor(l, 32);
    if (!valid[q]) continue;
    const int64_t prow = int64_t(sp) * S * Hq + orow[q];
    uint2* dst = reinterpret_cast<uint2*>(a.p_acc + prow * D);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      dst[(16 * dt + 4 * g) / 4] = make_uint2(pack_bf16(o[q][dt][0] * vsc, o[q][dt][1] * vsc),
                                              pack_bf16(o[q][dt][2] * vsc, o[q][dt][3] * vsc));
    if (g == 0) a.p_ml[prow] = make_float2(m[q] * c2, l);
  }
}

// One thread per 8 output elements of one (sequence, query head) row.
template <int D>
__global__ __launch_bounds__(256) void prefix_merge_kernel(PrefixArgs a) {
  constexpr int C = D / 8;
  const int64_t rows = int64_t(a.num_seqs) * a.num_q_heads;
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t r = i / C;
  const int c = int(i % C);
  if (r >= rows) return;
  const float lse = a.lse[r];
  float M = lse;
  for (int sp = 0; sp < a.n_split; ++sp) M = fmaxf(M, a.p_ml[sp * rows + r].x);
  const float Ms = M == -INFINITY ? 0.f : M;
  // the suffix output is normalised: its weight is l_s 2^(m_s - M) = 2^(lse - M)
  const float fs = __builtin_amdgcn_exp2f(lse - Ms);
  uint4* o = static_cast<uint4*>(a.out) + r * C + c;
  const uint4 os = *o;
  float num[8] = {bf16_lo(os.x) * fs, bf16_hi(os.x) * fs, bf16_lo(os.y) * fs, bf16_hi(os.y) * fs,
                  bf16_lo(os.z) * fs, bf16_hi(os.z) * fs, bf16_lo(os.w) * fs, bf16_hi(os.w) * fs};
  float den = fs;
  for (int sp = 0; sp < a.n_split; ++sp) {
    const float2 ml = a.p_ml[sp * rows + r];
    const float f = __builtin_amdgcn_exp2f(ml.x - Ms);
    den = fmaf(ml.y, f, den);
    const uint4 x = *reinterpret_cast<const uint4*>(a.p_acc + (sp * rows + r) * D + c * 8);
    num[0] = fmaf(bf16_lo(x.x), f, num[0]);
    num[1] = fmaf(bf16_hi(x.x), f, num[1]);
    num[2] = fmaf(bf16_lo(x.y), f, num[2]);
    num[3] = fmaf(bf16_hi(x.y), f, num[3]);
    num[4] = fmaf(bf16_lo(x.z), f, num[4]);
    num[5] = fmaf(bf16_hi(x.z), f, num[5]);
    num[6] = fmaf(bf16_lo(x.w), f, num[6]);
    num[7] = fmaf(bf16_hi(x.w), f, num[7]);
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  *o = make_uint4(pack_bf16(num[0] * inv, num[1] * inv), pack_bf16(num[2] * inv, num[3] * inv),
                  pack_bf16(num[4] * inv, num[5] * inv), pack_bf16(num[6] * inv, num[7] * inv));
}

template <int D, int NG, int KV>
hipError_t run_prefix(const PrefixArgs& a, const PrefixPlan& p, hipStream_t st) {
  int b_shift = 0;
  while ((1 << b_shift) < a.block_size) ++b_shift;
  constexpr int WPG = waves_per_group(NG, KV == PA_FP8_E4M3);
  const int wpg = WPG;  // every wave takes a share of the loads, with or without columns
  const int n_cgrp = (p.n_cblk + wpg - 1) / wpg;
  const int groups = a.num_kv_heads * a.n_split * n_cgrp;
  const size_t lds = size_t(2) * 2 * kPChunk * kPTile * 2 * D;  // 2 stages of K and V
  const float scale_log2 = a.scale * kPLog2e;
  if (a.block_size >= kPTile)
    prefix_partial_kernel<D, NG, true, KV><<<groups, kWave * wpg, lds, st>>>(
        a, b_shift, p.n_cblk, n_cgrp, p.tiles_per_split, scale_log2);
  else
    prefix_partial_kernel<D, NG, false, KV><<<groups, kWave * wpg, lds, st>>>(
        a, b_shift, p.n_cblk, n_cgrp, p.tiles_per_split, scale_log2);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t threads = int64_t(a.num_seqs) * a.num_q_heads * (D / 8);
  prefix_merge_kernel<D><<<int((threads + 255) / 256), 256, 0, st>>>(a);
  return hipGetLastError();
}

template <int D, int KV>
hipError_t run_prefix_ng(const PrefixArgs& a, const PrefixPlan& p, hipStream_t st) {
  static_assert(kPMaxGroups == 2, "one instantiation per group count");
  return p.groups_per_wave == 2 ? run_prefix<D, 2, KV>(a, p, st) : run_prefix<D, 1, KV>(a, p, st);
}

}  // namespace

PrefixPlan prefix_plan(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t block_size, int32_t num_prefix_blocks, int32_t num_cus) {
  PrefixPlan p{};
  const int64_t cols = int64_t(num_seqs) * (num_q_heads / num_kv_heads);
  // column groups per wave: as many as the columns fill, up to kPMaxGroups
  p.groups_per_wave = 1;
  while (p.groups_per_wave < kPMaxGroups && cols >= 32 * p.groups_per_wave) p.groups_per_wave *= 2;
  p.n_cblk = int32_t((cols + 16 * p.groups_per_wave - 1) / (16 * p.groups_per_wave));
  p.n_tiles = int32_t((int64_t(num_prefix_blocks) * block_size + kPTile - 1) / kPTile);
  if (p.n_tiles <= 0) return p;
  // as many key ranges as one round of resident waves (8 per compute unit)
  // holds, but no key range under 8 tiles
  const int64_t per_split = int64_t(num_kv_heads) * p.n_cblk;
  const int64_t want = int64_t(8) * (num_cus > 0 ? num_cus : 256) / per_split;
  const int64_t cap = p.n_tiles / 8 > 1 ? p.n_tiles / 8 : 1;
  const int64_t n = want < 1 ? 1 : (want > cap ? cap : want);
  p.tiles_per_split = int32_t((p.n_tiles + n - 1) / n);
  p.n_split = (p.n_tiles + p.tiles_per_split - 1) / p.tiles_per_split;
  return p;
}

hipError_t launch_prefix(const PrefixArgs& a, const PrefixPlan& p, hipStream_t st) {
  if (a.n_split != p.n_split || p.n_split <= 0) return hipErrorInvalidValue;
  if (a.dtype == PA_BF16) {
    if (a.head_dim == 128) return run_prefix_ng<128, PA_BF16>(a, p, st);
    if (a.head_dim == 64) return run_prefix_ng<64, PA_BF16>(a, p, st);
  } else if (a.dtype == PA_FP8_E4M3) {
    if (a.head_dim == 128) return run_prefix_ng<128, PA_FP8_E4M3>(a, p, st);
    if (a.head_dim == 64) return run_prefix_ng<64, PA_FP8_E4M3>(a, p, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
