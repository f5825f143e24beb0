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
//  * Work list. A segment is (sequence, head unit), where a head unit is a KV
//    head together with up to 8 of the query heads that read it, so each K/V
//    row is read from HBM once per step. Segment (s, u) is cut into 16-token
//    tiles; all tiles of all segments form one list, ordered by sequence,
//    then unit, then tile, and each of W wavefronts takes an equal contiguous
//    slice of it. Ragged lengths therefore cost nothing in balance: every
//    wave streams the same number of bytes, and no workgroup is launched
//    empty. Each wave finds its slice from a prefix sum of the tile counts
//    of all sequences, computed at its start.
//  * Lane layout: a token row of D elements is LPR lanes x 16 bytes; a
//    wave-wide 16-byte load covers NR = 64 / LPR token rows (bf16, D = 128:
//    16 lanes per row, 4 rows per load, 4 loads per tile). All K/V loads are
//    fully coalesced 16-byte accesses, marked non-temporal.
//  * Block-table entries are fetched two tiles ahead of use and the K/V of
//    the next tile are in flight while the current tile is computed, across
//    segment boundaries.
//  * q.k: per-lane partial dot over its 16 bytes (v_dot2 for bf16), then a
//    sum over the LPR lanes of the row with DPP (quad_perm, row_half_mirror,
//    row_mirror).
//  * Online softmax in base 2, kept per row group (lanes with the same token
//    row index), so the hot loop has no cross-row traffic; the NR row groups
//    are merged when a segment ends.
//  * A segment that lies inside one wave's slice is finished by that wave.
//    A segment split between waves leaves one partial (running max,
//    denominator, unnormalised sum) per wave, and its first wave records
//    where it is. A second, small kernel then combines each split segment's
//    partials with the log-sum-exp rule M = max m_p,
//    out = sum 2^(m_p-M) acc_p / sum 2^(m_p-M) l_p. Doing this after the
//    kernel boundary needs no atomics or device-wide fences: on this chip a
//    device-scope fence writes back and invalidates a whole L2, and issuing
//    one per split segment cost more than a third of the bandwidth.
#include <math.h>

#include "device.h"

namespace pa {
namespace {

constexpr int kMaxWavesPerGroup = 8;  // one workgroup per CU holds that CU's waves
constexpr int kTile = 16;  // tokens per tile
// Weights of the work split: a tile counts kTileW, the start of a segment
// kSegW (its query and table loads and the first tile's round trip). Timing
// each wave put a segment start at about 60 % of a tile; of the weights 2, 4
// and 6 (in quarters of a tile), 4 gave the best rates over the batches.
constexpr int kTileW = 4;
constexpr int kSegW = 4;
constexpr float kLog2e = 1.4426950408889634f;

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

// VEC fp32 values as one 16-byte chunk of the output dtype.
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

__device__ __forceinline__ int tiles_of(int L) { return L > 0 ? (L + kTile - 1) / kTile : 0; }

__device__ __forceinline__ int wave_sum_i32(int x) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) x += __shfl_xor(x, off);
  return x;
}

__device__ __forceinline__ int wave_incl_scan_i32(int x, int lane) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x;
}

__device__ __forceinline__ int64_t uniform64(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(uint64_t(x)));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(uint64_t(x) >> 32));
  return int64_t((uint64_t(hi) << 32) | lo);
}

// Position of one tile in the work list: tile j of segment (sequence s, unit u);
// unit u reads KV heads kvh .. kvh+kvp-1; the sequence has n tiles and L tokens; seg0 = list
// index of the segment's tile 0. All fields are wave-uniform.
struct Cursor {
  int s, u, kvh, hc, j, n, L;
  int64_t seg0;
};

// This wave's slice of the work list, walked segment by segment: for each
// segment (sequence, unit) it calls prefetch(cursor), which issues the
// segment's query loads and the load of the block-table window of its first
// tile and returns that window, then begin(cursor), run(cursor, j0, j1, window)
// for the slice's tiles [j0, j1) of it, and end(cursor, owns_start, owns_end),
// which stores the result; finally it records the segment the slice starts and
// leaves open (if any) for the combine kernel (when `record`: of two waves
// walking one slice, only one records it). Also writes zeros for empty
// sequences. VEC: elements of the output dtype per 16 bytes; hpw: query heads
// per unit.
// Order at a segment boundary: the next segment's prefetch comes before the
// current segment's end. Stores and loads share one counter of outstanding
// vector memory operations, which completes in issue order; loads issued
// after a segment's stores could only be waited for together with those
// stores, whose completion is slow while the chip streams K/V. Issued before
// them, the next segment's first loads are awaited while the stores drain.
// tokens of sequence s this call attends to: those after the first len_offset
__device__ __forceinline__ int len_of(const DecodeArgs& a, int s) {
  return max(a.seq_lens[s] - a.len_offset, 0);
}

// Tiles of group g in the grouped decode: its shared prefix once, then the
// tokens after the prefix of each member.
__device__ __forceinline__ int group_tiles(const DecodeArgs& a, int g) {
  const int s0 = g * a.group_size;
  const int P = a.prefix_lens[s0];
  int n = tiles_of(P);
  for (int m = 0; m < a.group_size; ++m) n += tiles_of(a.seq_lens[s0 + m] - P);
  return n;
}

// GROUPED: the walk's items are groups of sequences (their length in tiles),
// else sequences (their length in tokens).
template <int D, int VEC, bool GROUPED, class Prefetch, class Begin, class Run, class End>
__device__ __forceinline__ void walk_slice(const DecodeArgs& a, int w, int lane, int n_hchunk,
                                           int hpw, int kvp, Prefetch prefetch, Begin begin,
                                           Run run, End end, bool record = true) {
  const int S = GROUPED ? a.num_groups : a.num_seqs;
  const int Hq = a.num_q_heads;
  const int G = Hq / a.num_kv_heads;
  const int units = (a.num_kv_heads / kvp) * n_hchunk;
  auto item_len = [&](int s) -> int { return GROUPED ? group_tiles(a, s) : len_of(a, s); };
  auto item_tiles = [&](int v) -> int { return GROUPED ? v : tiles_of(v); };

  // Positions along the work list: a unit of n tiles spans kTileW * n +
  // kSegW of them, its tile j starting at kSegW + kTileW * j; kSegW stands for
  // the start-up cost of a segment, in the same quarters of a tile's time, so
  // that slices full of short units get fewer tiles. Slice w covers positions
  // [total * w / W, total * (w + 1) / W) and walks the tiles that start in it.
  // Slices are at least a tile wide, so every slice that lies inside a unit's
  // tiles walks at least one of them (the combine relies on that).
  auto unit_w = [&](int n) -> int64_t { return int64_t(kTileW) * n + kSegW; };
  int64_t total = 0;
  for (int base = 0; base < S; base += kWave) {
    const int s = base + lane;
    const int t = s < S ? item_tiles(item_len(s)) : 0;
    total += wave_sum_i32(t > 0 ? kTileW * t + kSegW : 0);
  }
  total = uniform64(total * units);
  // every active slice is at least a tile wide
  const int64_t W = total / kTileW < a.workers ? total / kTileW : a.workers;

  // empty sequences: zeros, written by wave (s mod Wz) (a multi-row batch
  // has no rows for them: a sequence's rows are already in its length)
  const int Wz = W > 0 ? int(W) : a.workers;
  for (int s = w; s < (a.q_start_loc ? 0 : a.num_seqs); s += Wz) {
    if ((GROUPED ? a.seq_lens[s] : len_of(a, s)) > 0) continue;
    uint4* o = static_cast<uint4*>(a.out) + (int64_t(s) * Hq * D) / VEC;
    for (int i = lane; i < Hq * D / VEC; i += kWave) o[i] = make_uint4(0, 0, 0, 0);
    if (a.lse)
      for (int h = lane; h < Hq; h += kWave) a.lse[int64_t(s) * Hq + h] = -INFINITY;
  }
  if (w >= W) {
    if (lane == 0 && record) a.ws_seg[w] = make_int4(-1, 0, 0, 0);
    return;
  }
  const int64_t g_begin = total * w / W, g_end = total * (w + 1) / W;

  // lengths of 64 consecutive items, one per lane, read with v_readlane so
  // that moving to the next item issues no memory load in the common case
  int lwin_base = S, lwin = 0;
  auto seq_len = [&](int s) -> int {
    if (s - lwin_base >= kWave || s < lwin_base) {
      lwin_base = s;
      lwin = s + lane < S ? item_len(s + lane) : 0;
    }
    return __builtin_amdgcn_readlane(lwin, s - lwin_base);
  };

  // locate g_begin: the item whose units contain it, then the unit and the
  // first of its tiles that starts at or after g_begin
  Cursor cur{};
  {
    int64_t before = 0;  // positions before this chunk of items
    for (int base = 0; base < S; base += kWave) {
      const int s = base + lane;
      const int t = s < S ? item_tiles(item_len(s)) : 0;
      const int tw = t > 0 ? kTileW * t + kSegW : 0;
      const int64_t incl = before + int64_t(wave_incl_scan_i32(tw, lane)) * units;
      const int64_t excl = incl - int64_t(tw) * units;
      const unsigned long long hit = __ballot(s < S && t > 0 && excl <= g_begin && g_begin < incl);
      if (hit) {
        const int l = __builtin_ctzll(hit);
        const int64_t seq0 = uniform64(__shfl(excl, l));
        cur.s = base + l;
        cur.n = __builtin_amdgcn_readfirstlane(__shfl(t, l));
        cur.L = seq_len(cur.s);
        const int64_t uw = unit_w(cur.n);
        const int64_t off = g_begin - seq0;
        cur.u = int(off / uw);
        const int64_t r = off - int64_t(cur.u) * uw;  // position inside the unit
        cur.j = r <= kSegW ? 0 : int((r - kSegW + kTileW - 1) / kTileW);
        cur.kvh = (cur.u / n_hchunk) * kvp;
        cur.hc = cur.u % n_hchunk;
        cur.seg0 = seq0 + int64_t(cur.u) * uw;
        break;
      }
      before = uniform64(__shfl(incl, kWave - 1));
    }
  }
  // to tile 0 of the next unit: of this sequence, or of the next non-empty one
  auto advance = [&]() {
    cur.j = 0;
    cur.seg0 += unit_w(cur.n);
    ++cur.u;
    if (++cur.hc == n_hchunk) {
      cur.hc = 0;
      cur.kvh += kvp;
    }
    if (cur.u == units) {
      cur.u = cur.kvh = cur.hc = 0;
      do {
        ++cur.s;
        cur.L = seq_len(cur.s);
        cur.n = item_tiles(cur.L);
      } while (cur.n == 0 && cur.s + 1 < S);
    }
  };
  // tiles of the current unit that start before g_end
  auto tiles_before_end = [&]() -> int {
    const int64_t room = g_end - cur.seg0 - kSegW;
    return room <= 0 ? 0 : int(min(int64_t(cur.n), (room + kTileW - 1) / kTileW));
  };
  if (cur.j >= cur.n) advance();  // no tile of that unit starts in the slice
  if (tiles_before_end() <= cur.j) {  // no tile at all starts in the slice
    if (lane == 0 && record) a.ws_seg[w] = make_int4(-1, 0, 0, 0);
    return;
  }

  // walk the segments of this slice
  int4 split = make_int4(-1, 0, 0, 0);  // the segment this slice starts and leaves unfinished
  int win = prefetch(cur);
  begin(cur);
  while (true) {
    const int j1 = tiles_before_end();
    const bool owns_start = cur.j == 0, owns_end = j1 == cur.n;
    run(cur, cur.j, j1, win);
    if (owns_start && !owns_end) {  // only the last segment of a slice can be left open
      const int64_t last = cur.seg0 + unit_w(cur.n) - kTileW;  // start of the unit's last tile
      split = make_int4(cur.s, cur.u, int(((last + 1) * W - 1) / total),
                        cur.kvh * G + cur.hc * hpw);
    }
    // another segment follows when the next unit's first tile starts in the slice
    const bool more = owns_end && cur.seg0 + unit_w(cur.n) + kSegW < g_end;
    const Cursor done = cur;
    if (more) {
      advance();
      win = prefetch(cur);  // its loads go out before the stores of `done`
    }
    end(done, owns_start, owns_end);
    if (!more) break;
    begin(cur);
  }
  if (lane == 0 && record) a.ws_seg[w] = split;
}

template <int DTYPE, int D, int HPW, bool BIG_B>
__global__ __launch_bounds__(kWave * kMaxWavesPerGroup) void decode_balanced_kernel(
    DecodeArgs a, int32_t b_shift, int32_t n_hchunk, float scale_log2) {
  using RS = RowShape<DTYPE, D>;
  constexpr int VEC = RS::VEC, LPR = RS::LPR, NR = RS::NR;
  constexpr int U = kTile / NR;  // 16-byte loads per lane per tile, for K and for V
  static_assert(kTile % NR == 0, "a tile must cover whole load rows");
  constexpr int QF = VEC > 4 ? 4 : VEC;

  const int lane = threadIdx.x % kWave;
  const int w = blockIdx.x * (blockDim.x / kWave) + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int Hq = a.num_q_heads, Hkv = a.num_kv_heads;
  const int G = Hq / Hkv;
  const int r = lane / LPR, c = lane % LPR;
  const int B = a.block_size, Bm1 = B - 1;
  if (w >= a.workers) return;

  const uint4* kp = static_cast<const uint4*>(a.k_pool);
  const uint4* vp = static_cast<const uint4*>(a.v_pool);
  const int64_t block_chunks = int64_t(Hkv) * B * LPR;  // 16-byte chunks per physical block

  // ---- per-segment state ------------------------------------------------------
  float qf[HPW][QF];
  uint4 qb[HPW], qnext[HPW];
  float m[HPW], l[HPW], acc[HPW][VEC];
  auto head_of = [&](const Cursor& x) { return x.kvh * G + x.hc * HPW; };
  // the segment's query loads and the block-table window of its tile x.j
  auto prefetch = [&](const Cursor& x) -> int {
    const uint4* qp = static_cast<const uint4*>(a.q) + ((int64_t(x.s) * Hq + head_of(x)) * D) / VEC + c;
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) qnext[hh] = qp[hh * (D / VEC)];
    const int32_t* row = a.block_tables + int64_t(x.s) * a.max_blocks_per_seq;
    const int nblk = (x.L + Bm1) >> b_shift;
    const int jb0 = (x.j * kTile) >> b_shift;
    return jb0 + lane < nblk ? row[jb0 + lane] : 0;
  };
  auto begin_segment = [&](const Cursor& x) {
    (void)x;
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      qb[hh] = qnext[hh];
      if constexpr (DTYPE == PA_F32) {
        qf[hh][0] = __uint_as_float(qb[hh].x) * scale_log2;
        qf[hh][1] = __uint_as_float(qb[hh].y) * scale_log2;
        qf[hh][2] = __uint_as_float(qb[hh].z) * scale_log2;
        qf[hh][3] = __uint_as_float(qb[hh].w) * scale_log2;
      }
      m[hh] = -INFINITY;
      l[hh] = 0.f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[hh][e] = 0.f;
    }
  };
  const float zmul = DTYPE == PA_F32 ? 1.f : scale_log2;

  auto compute = [&](int j, int L, const uint4* kr, const uint4* vr) {
    float z[HPW][U];
#pragma unroll
    for (int uu = 0; uu < U; ++uu) {
      const bool valid = j * kTile + uu * NR + r < L;
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh) {
        const float sv = group_sum<LPR>(dot16<DTYPE>(kr[uu], qf[hh], qb[hh])) * zmul;
        z[hh][uu] = valid ? sv : -INFINITY;
      }
    }
    float p[HPW][U];
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      float mx = z[hh][0];
#pragma unroll
      for (int uu = 1; uu < U; ++uu) mx = fmaxf(mx, z[hh][uu]);
      const float mn = fmaxf(m[hh], mx);
      const float ms = mn == -INFINITY ? 0.f : mn;
      const float alpha = __builtin_amdgcn_exp2f(m[hh] - ms);
      m[hh] = mn;
      float lsum = l[hh] * alpha;
#pragma unroll
      for (int uu = 0; uu < U; ++uu) {
        p[hh][uu] = __builtin_amdgcn_exp2f(z[hh][uu] - ms);
        lsum += p[hh][uu];
      }
      l[hh] = lsum;
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[hh][e] *= alpha;
    }
    // clamped rows hold a real token's V, finite, and their weight p is 0
#pragma unroll
    for (int uu = 0; uu < U; ++uu) {
      float vf[VEC];
      unpack16<DTYPE>(vr[uu], vf);
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh)
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[hh][e] = fmaf(p[hh][uu], vf[e], acc[hh][e]);
    }
  };

  // merge the NR row groups, then write the output or this wave's partial
  auto end_segment = [&](const Cursor& x, bool owns_start, bool owns_end) {
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
        for (int e = 0; e < VEC; ++e)
          acc[hh][e] = acc[hh][e] * fa + __shfl_xor(acc[hh][e], off) * fb;
        m[hh] = mn;
      }
    }
    uint4* o = static_cast<uint4*>(a.out) + ((int64_t(x.s) * Hq + head_of(x)) * D) / VEC + c;
    if (owns_start && owns_end) {  // whole segment in this wave
      if (r == 0) {
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh) {
          if (a.lse && c == 0)
            a.lse[int64_t(x.s) * Hq + head_of(x) + hh] = m[hh] + __builtin_amdgcn_logf(l[hh]);
          const float inv = 1.f / l[hh];
          float f[VEC];
#pragma unroll
          for (int e = 0; e < VEC; ++e) f[e] = acc[hh][e] * inv;
          o[hh * (D / VEC)] = pack16<DTYPE>(f);
        }
      }
      return;
    }
    // split segment: this wave's partial goes to slot 2w (segment began before
    // the slice) or 2w+1 (segment continues after the slice)
    const int slot = 2 * w + (owns_start ? 1 : 0);
    if (r == 0) {
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh) {
        float4* dst = reinterpret_cast<float4*>(a.ws_acc + (int64_t(slot) * HPW + hh) * D + c * VEC);
#pragma unroll
        for (int e = 0; e < VEC; e += 4)
          dst[e / 4] = make_float4(acc[hh][e], acc[hh][e + 1], acc[hh][e + 2], acc[hh][e + 3]);
        if (c == 0) a.ws_ml[int64_t(slot) * kMLStride + hh] = make_float2(m[hh], l[hh]);
      }
    }
  };

  // Tiles [j0, j1) of one segment, in chunks whose blocks fit a 64-entry window
  // of the block table (one entry per lane, read back with v_readlane / a lane
  // shuffle). Inside a chunk the loop is branch-free and double-buffered:
  // tile j+1 is loading while tile j is computed. Rows past the end of the
  // sequence are clamped to its last token (a valid, written slot) and masked
  // out in compute, so no load sits under divergent control flow.
  // win0: the window of tile j0's chunk (prefetched)
  auto run_tiles = [&](const Cursor& x, int j0, int j1, int win0) {
    const int32_t* row = a.block_tables + int64_t(x.s) * a.max_blocks_per_seq;
    const int nblk = (x.L + Bm1) >> b_shift;
    const int Lm1 = x.L - 1;
    for (int jc = j0; jc < j1;) {
      const int jb0 = (jc * kTile) >> b_shift;
      const int win = jc == j0 ? win0 : (jb0 + lane < nblk ? row[jb0 + lane] : 0);
      const int jc_end = min(j1, ((jb0 + kWave) << b_shift) / kTile);
      auto load_tile = [&](int j, uint4* kr, uint4* vr) {
        if constexpr (BIG_B) {
          const int pb = __builtin_amdgcn_readlane(win, ((j * kTile) >> b_shift) - jb0);
          const int64_t blk = int64_t(pb) * block_chunks;
          const uint4* kb = kp + blk;
          const uint4* vb = vp + blk;
#pragma unroll
          for (int uu = 0; uu < U; ++uu) {
            const int t = min(j * kTile + uu * NR + r, Lm1);
            const int off = (x.kvh * B + (t & Bm1)) * LPR + c;
            kr[uu] = load_stream16(kb + off);
            vr[uu] = load_stream16(vb + off);
          }
        } else {
#pragma unroll
          for (int uu = 0; uu < U; ++uu) {
            const int t = min(j * kTile + uu * NR + r, Lm1);
            const int pb = __shfl(win, (t >> b_shift) - jb0);
            const int64_t idx = int64_t(pb) * block_chunks + (x.kvh * B + (t & Bm1)) * LPR + c;
            kr[uu] = load_stream16(kp + idx);
            vr[uu] = load_stream16(vp + idx);
          }
        }
      };
      // Every load is unconditional (a prefetch past the chunk re-reads its last
      // tile, an L2 hit): with conditional loads the compiler cannot count the
      // loads in flight and waits for all of them before each tile.
      uint4 kA[U], vA[U], kB[U], vB[U];
      int j = jc;
      load_tile(j, kA, vA);
      for (; j + 2 <= jc_end; j += 2) {
        load_tile(j + 1, kB, vB);
        __builtin_amdgcn_sched_barrier(0);  // keep the next tile's loads ahead of this math
        compute(j, x.L, kA, vA);
        load_tile(min(j + 2, jc_end - 1), kA, vA);
        __builtin_amdgcn_sched_barrier(0);
        compute(j + 1, x.L, kB, vB);
      }
      if (j < jc_end) compute(j, x.L, kA, vA);  // odd count: last tile already in A
      jc = jc_end;
    }
  };

  walk_slice<D, VEC, false>(a, w, lane, n_hchunk, HPW, 1, prefetch, begin_segment, run_tiles,
                            end_segment);
}

// GQA decode on the matrix cores (bf16, HPW >= 4 query heads per KV head).
// Same work list, partials and combine as decode_balanced_kernel; per 16-token
// tile of a unit:
//  * K and V tiles are loaded with whole rows per lane group (each 16-byte
//    load instruction covers 1 KB of consecutive rows), which the memory
//    system serves far better than operand-shaped loads that touch every
//    cache line of the tile, and written to the wave's own 8 KB of LDS (16-byte
//    chunk c of row r kept at c ^ f(r), f a bijection over the rows that
//    share a bank line position, so that every read below is conflict-free).
//  * S^T = K Q^T with v_mfma_f32_16x16x32_bf16: M = the 16 keys, N = the
//    unit's query heads (HPW of 16 columns used), K = head_dim in D/32 steps;
//    lane l reads its A operand (key l%16, 8 dims) from LDS.
//  * The accumulator gives lane l the scores of head l%16 for keys
//    4(l/16) + i, which is exactly the B operand (P^T) of
//    v_mfma_f32_16x16x16_bf16 for O^T = V^T P^T, so p needs no shuffle.
//  * V^T, the A operand of that product, needs 4 consecutive keys of one dim
//    per lane: ds_read_b64_tr_b16 reads it from the V tile transposed.
//  * Online softmax per head with the exponent base moved only when a head's
//    max grows by more than 2^8 (exact, as numerator and denominator share
//    it); the row sum adds the bf16 weights the product uses.
// The MFMA work is a small fraction of the time the tile's bytes take to
// arrive, so the kernel streams K/V like the MHA kernel while the per-head
// VALU work of that kernel (dot products, reductions) disappears.
// KV = PA_BF16, or PA_FP8_E4M3: the pool holds E4M3 codes, which are widened
// exactly to bf16 on their way into LDS; k_scale then multiplies the scores and
// v_scale the output, and everything from LDS on is the bf16 kernel.
// KVP = 2 (FP8 MHA, HPW = 2): a unit is two adjacent KV heads with their one
// query head each. Columns c < HPW/2 belong to KV head kvh, the others to
// kvh + 1; each column is scored against, and weights, its own head's K and V
// tiles. The two heads' rows of a block are adjacent in the pool, so each tile
// reads one contiguous run of 2*16 rows per pool instead of two of 16: the
// memory system serves short runs (2 KB for 16 FP8 rows of 128 B) much more
// slowly than long ones. (bf16 groups of 8 paired the same way, 16 columns,
// ran no faster: their 4 KB runs are long enough.)
// GROUPED (HPW = 16, KVP = 1): a unit is one KV head of a group of sequences
// whose first prefix_lens[s] tokens are the same blocks ("vLLM PagedAttention
// explained", sections 4.1-4.2: parallel samples and beams share the blocks of
// their common start). Column c < group_size * G is query head kvh*G + c%G of
// member c/G. A segment's tiles are the shared prefix (every column scores it)
// and then each member's tokens after the prefix, which only that member's
// columns score (the others get -inf); so each shared K/V tile is read once
// for the whole group, and each column's softmax runs over exactly its own
// sequence's tokens.
// LDS of one wave of decode_mfma_kernel: a K and a V tile (bf16 rows) per KV
// head of the unit, then (units of >= 4 columns) two hold slots of HPW result
// rows; smaller units stage their rows in the idle K tile instead.
template <int D, int HPW, int KVP>
constexpr size_t mfma_wave_lds() {
  return size_t(KVP) * 2 * kTile * 2 * D + (HPW >= 4 ? size_t(2) * HPW * 2 * D : 0);
}

// LDS of a pair of multi-row waves (one workgroup): two stages of a K and a V
// tile that both waves read, then each wave's two hold slots of 16 rows.
template <int D>
constexpr size_t mr_pair_lds() {
  return size_t(2) * 2 * kTile * 2 * D + size_t(2) * 2 * 16 * 2 * D;
}
constexpr int kMRPairTiles = 2;  // tiles in flight per wave of a pair (3-4 measured slower)

template <int D, int HPW, bool BIG_B, int KV, int KVP, bool GROUPED, bool MR = false,
          bool PAIR = false>
__global__ __launch_bounds__(kWave * (MR ? kMultiRowWaves : kMaxWavesPerGroup)) void decode_mfma_kernel(
    DecodeArgs a, int32_t b_shift, int32_t n_hchunk, float scale_log2) {
  static_assert(!PAIR || MR, "pairs of waves are a multi-row launch");
  static_assert(!PAIR || (KV == PA_FP8_E4M3 ? D : 2 * D) * kTile >= 2048,
                "a pair splits each tile's rows: at least two wave-wide loads per tile");
  static_assert(!GROUPED || (KVP == 1 && HPW == kGroupedCols), "grouped units: 16 columns");
  static_assert(!MR || (KVP == 1 && !GROUPED && HPW == 16), "multi-row waves: 16 columns");
  constexpr bool FP8 = KV == PA_FP8_E4M3;
  // columns of a workspace slot: a multi-row unit's (up to 32, split over a
  // pair of waves), else the wave's own
  constexpr int UC = MR ? kMultiRowCols : HPW;
  constexpr int MLS = UC > kMLStride ? UC : kMLStride;  // (m, l) records per workspace slot
  constexpr int ROW = 2 * D;        // bytes per bf16 K/V row in LDS
  constexpr int GROW = FP8 ? D : ROW;  // bytes per row in the pool
  constexpr int KS = D / 32;        // 16x16x32 k-steps over head_dim
  constexpr int DT = D / 16;        // 16-dim tiles of O^T
  constexpr int CPR = ROW / 16;     // 16-byte chunks per LDS row
  constexpr int GCPR = GROW / 16;   // 16-byte chunks per pool row
  constexpr int RPI = 1024 / GROW;  // rows per wave-wide 16-byte load
  constexpr int NI = kTile / RPI;   // loads per lane per tile and KV head, for K and for V
  constexpr int NIT = NI * KVP;     // loads per lane per tile, for K and for V
  static_assert(HPW % KVP == 0, "a unit's columns split evenly over its KV heads");
  constexpr int CPH = HPW / KVP;    // MFMA columns (query heads) per KV head of the unit
  constexpr int RPL = 256 / ROW;    // rows per 256-byte LDS bank line
  constexpr int TB = kTile * ROW;   // bytes of one K or V tile in LDS
  // PAIR: the two waves of a workgroup share each K/V tile, each loading half
  // of its rows (NL loads per tensor) into a stage both read
  constexpr int NL = PAIR ? NI / 2 : NI;
  constexpr int NLT = PAIR ? NL : NIT;
  // tiles in flight per wave: an FP8 tile is half the bytes, so more of them
  // are needed to keep as many bytes in flight (a paired tile is twice the
  // bytes; a wave of a pair loads half a tile)
  constexpr int NB = PAIR ? kMRPairTiles : FP8 && KVP == 1 ? 4 : 2;
  static_assert(HPW <= 16, "one MFMA N tile holds the wave's columns");
  extern __shared__ __align__(16) unsigned char smem[];

  const int lane = threadIdx.x % kWave;
  const int wig = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int w = blockIdx.x * (blockDim.x / kWave) + wig;
  const int Hq = a.num_q_heads, Hkv = a.num_kv_heads;
  const int G = Hq / Hkv;
  const int g = lane / 16, i16 = lane % 16;
  const int B = a.block_size, Bm1 = B - 1;
  // Multi-row pairs: the two waves of workgroup k walk work slice k; wave ct
  // holds unit columns [16 ct, 16 ct + 16) of its units and loads rows
  // [ct * NL * RPI, (ct + 1) * NL * RPI) of each tile.
  const int ct = PAIR ? wig : 0;
  const int wk = PAIR ? int(blockIdx.x) : w;  // this wave's work slice
  const int cb = 16 * ct;                     // unit column of the wave's column 0
  const int row0 = ct * NL * RPI;
  if (wk >= a.workers) return;  // (both waves of a pair)

  // this wave's K tiles (one per KV head of the unit), then its V tiles
  // (pairs: the workgroup's two stages, taken in turn)
  unsigned char* kt_lds = PAIR ? smem : smem + wig * mfma_wave_lds<D, HPW, KVP>();
  unsigned char* vt = kt_lds + KVP * TB;
  int tcount = 0;  // pairs: tiles computed so far (the same in both waves)
  auto swz = [](int r) { return (r / RPL) % CPR; };
  // load u of lane l: row u*RPI + l/GCPR, pool chunk l%GCPR; in LDS that is
  // chunk l%GCPR of the bf16 row (two chunks, 2c and 2c+1, for FP8 codes)
  const int lrow = lane / GCPR, lch = lane % GCPR;
  uint32_t wr[NI], wr2[NI];
#pragma unroll
  for (int u = 0; u < NI; ++u) {
    const int r = row0 + u * RPI + lrow;
    const int c0 = FP8 ? 2 * lch : lch;
    wr[u] = uint32_t(r * ROW + ((c0 ^ swz(r)) * 16));
    wr2[u] = uint32_t(r * ROW + (((c0 + 1) ^ swz(r)) * 16));
  }
  // K operand of k-step ks: row i16, chunk 4ks + g  ->  kr0 ^ (64 ks)
  const uint32_t kr0 = uint32_t(i16 * ROW + ((g ^ swz(i16)) * 16));
  // V, read transposed: lane (g, 4k+q) points at row 4g + k, dims 16 dt + 4q .. +3
  const int rr = 4 * g + i16 / 4;
  const uint32_t rd0 = uint32_t(rr * ROW + 8 * (i16 % 2) + (((i16 % 4) / 2) ^ swz(rr)) * 16);

  const unsigned char* kp = static_cast<const unsigned char*>(a.k_pool);
  const unsigned char* vp = static_cast<const unsigned char*>(a.v_pool);
  const int64_t block_bytes = int64_t(Hkv) * B * GROW;

  uint4 qop[KS], qnext[KS];
  f32x4_t o[KVP][DT];
  float m, lpart;
  int lim = 0;  // multi-row: keys this lane's column attends (its row's position + 1)
  const float c2 = FP8 ? scale_log2 * a.k_scale : scale_log2;
  const float vsc = FP8 ? a.v_scale : 1.f;
  // columns in use (multi-row: of the current segment, rows of its sequence x G)
  int ncols = GROUPED ? a.group_size * G : HPW;
  auto rows_of = [&](int sq) { return a.q_start_loc[sq + 1] - a.q_start_loc[sq]; };
  auto head_of = [&](const Cursor& x) { return x.kvh * G + x.hc * HPW; };
  // (row, query head) row of q / out of column c (c < ncols)
  auto row_of = [&](const Cursor& x, int c) -> int64_t {
    if constexpr (GROUPED) return int64_t(x.s * a.group_size + c / G) * Hq + x.kvh * G + c % G;
    else if constexpr (MR) return int64_t(a.q_start_loc[x.s] + c / G) * Hq + x.kvh * G + c % G;
    else return int64_t(x.s) * Hq + head_of(x) + c;
  };
  // Where tile j of a segment lies: the table row of its part (the sequence's
  // row; grouped: the shared prefix through the first member's row, or a
  // member's tokens after it through that member's row from the prefix's end
  // on), the part's length and the tile's index inside the part.
  struct Part {
    const int32_t* row;
    int L, j;
  };
  auto part_of = [&](const Cursor& x, int j) -> Part {
    if constexpr (!GROUPED) {
      return Part{a.block_tables + int64_t(x.s) * a.max_blocks_per_seq, x.L, j};
    } else {
      const int s0 = x.s * a.group_size;
      const int P = a.prefix_lens[s0];
      const int np = tiles_of(P);
      if (j < np) return Part{a.block_tables + int64_t(s0) * a.max_blocks_per_seq, P, j};
      j -= np;
      int mb = 0;
      int Lm = max(a.seq_lens[s0] - P, 0);
      while (j >= tiles_of(Lm) && mb + 1 < a.group_size) {
        j -= tiles_of(Lm);
        ++mb;
        Lm = max(a.seq_lens[s0 + mb] - P, 0);
      }
      return Part{a.block_tables + int64_t(s0 + mb) * a.max_blocks_per_seq + (P >> b_shift), Lm, j};
    }
  };
  // the segment's query loads and the block-table window of its tile x.j
  auto prefetch = [&](const Cursor& x) -> int {
    // columns past the unit's heads multiply zeros (their load is clamped to a
    // real column); a multi-row wave with no column in the unit loads nothing
    const int nc = MR ? rows_of(x.s) * G : ncols;
    if (!MR || cb < nc) {
      const unsigned char* qp = static_cast<const unsigned char*>(a.q) +
                                row_of(x, min(cb + i16, nc - 1)) * ROW + 16 * g;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qnext[ks] = *reinterpret_cast<const uint4*>(qp + 64 * ks);
    }
    const Part pt = part_of(x, x.j);
    const int nblk = (pt.L + Bm1) >> b_shift;
    const int jb0 = (pt.j * kTile) >> b_shift;
    return jb0 + lane < nblk ? pt.row[jb0 + lane] : 0;
  };
  auto begin_segment = [&](const Cursor& x) {
    const int c = cb + i16;  // this lane's unit column
    if constexpr (MR) {
      const int nrows = rows_of(x.s);
      ncols = nrows * G;
      // row c / G of the sequence sits at position L - nrows + c / G
      lim = c < ncols ? x.L - nrows + c / G + 1 : 0;
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qop[ks] = c < ncols ? qnext[ks] : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int p = 0; p < KVP; ++p)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[p][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    m = -INFINITY;
    lpart = 0.f;
  };

  // colok: this lane's column scores the tile (false: its scores are -inf)
  auto compute = [&](int j, int L, const uint4* kr, const uint4* vr, bool colok) {
    unsigned char* ktile = kt_lds;
    unsigned char* vtile = vt;
    if constexpr (PAIR) {
      // stage tcount % 2: both waves read the other stage last, and each
      // passed the last barrier after its reads of this one completed
      ktile = smem + (tcount & 1) * 2 * TB;
      vtile = ktile + TB;
      ++tcount;
    }
    // tiles -> LDS (the previous tile's reads were issued earlier by this
    // wave, and LDS serves one wave's accesses in order)
#pragma unroll
    for (int ut = 0; ut < NLT; ++ut) {
      const int u = ut % NI;
      unsigned char* kd = ktile + (ut / NI) * TB;  // tile of KV head ut / NI
      unsigned char* vd = vtile + (ut / NI) * TB;
      if constexpr (FP8) {
        uint4 k0, k1, v0, v1;
        widen_e4m3(kr[ut], k0, k1);
        widen_e4m3(vr[ut], v0, v1);
        *reinterpret_cast<uint4*>(kd + wr[u]) = k0;
        *reinterpret_cast<uint4*>(kd + wr2[u]) = k1;
        *reinterpret_cast<uint4*>(vd + wr[u]) = v0;
        *reinterpret_cast<uint4*>(vd + wr2[u]) = v1;
      } else {
        *reinterpret_cast<uint4*>(kd + wr[u]) = kr[ut];
        *reinterpret_cast<uint4*>(vd + wr[u]) = vr[ut];
      }
    }
    if constexpr (PAIR) {
      // the other half of the tile is the partner's: meet once both halves
      // are written (LDS writes done; the K/V loads in flight stay so). The
      // empty asm statements keep LDS accesses on their side of the barrier.
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));  // lgkmcnt(0) only
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    }
    f32x4_t scp[KVP];
#pragma unroll
    for (int p = 0; p < KVP; ++p) {
      scp[p] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint4 kop = *reinterpret_cast<const uint4*>(ktile + p * TB + (kr0 ^ (64u * ks)));
        scp[p] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kop),
                                                        __builtin_bit_cast(bf16x8_t, qop[ks]),
                                                        scp[p], 0, 0, 0);
      }
    }
    // column i16 is scored against the K tile of its own KV head
    f32x4_t sc = scp[0];
    if constexpr (KVP == 2) sc = i16 >= CPH ? scp[1] : scp[0];
    // keys past the end, and (multi-row) past this lane's row, score -inf
    const int key0 = j * kTile + 4 * g;
    const int Lc = MR ? lim : L;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (key0 + i >= Lc || !colok) sc[i] = -INFINITY;
    float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    {  // max over lanes l, l^16, l^32, l^48 (the 4 lanes of head l%16), on the VALU
      const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                        false, false);
      mx = fmaxf(__uint_as_float(s16[0]), __uint_as_float(s16[1]));
      const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                        false, false);
      mx = fmaxf(__uint_as_float(s32[0]), __uint_as_float(s32[1]));
    }
    const bool moved = m == -INFINITY ? mx != -INFINITY : (mx - m) * c2 > 8.f;
    const float mn = moved ? mx : m;
    const float nms = mn == -INFINITY ? 0.f : -mn * c2;
    const float alpha = moved ? __builtin_amdgcn_exp2f(fmaf(m, c2, nms)) : 1.f;
    m = mn;
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(fmaf(sc[i], c2, nms));
    const uint2 pb = make_uint2(pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3]));
    const bf16x2_t ones = __builtin_bit_cast(bf16x2_t, 0x3f803f80u);
    float ps = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pb.x), ones, 0.f, false);
    ps = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pb.y), ones, ps, false);
    lpart = lpart * alpha + ps;
    if (__ballot(moved)) {
#pragma unroll
      for (int p = 0; p < KVP; ++p)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[p][dt] *= alpha;
    }
    // O^T of KV head p weights that head's V tile (its column is the one kept)
#pragma unroll
    for (int p = 0; p < KVP; ++p)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const v4i16_t va = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16_t*)(vtile + p * TB + (rd0 ^ (32u * dt))));
        o[p][dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, __builtin_bit_cast(bf16x4_t, pb),
                                                           o[p][dt], 0, 0, 0);
      }
  };

  // Units of 4 or more columns hold their results in the wave's LDS until
  // the wave has streamed all its K/V: each segment's rows (bf16 output, or
  // bf16 partial sums of a segment split between waves) go to one of two
  // hold slots after the wave's tiles, and are written out when the wave is
  // done (or when a third result needs a slot), 16 contiguous bytes per lane,
  // each store instruction covering whole rows. Writes issued while the chip
  // streams K/V cost the stream far more than their own bytes: with the rows
  // written at each segment's end, straight from the accumulators, units of 8
  // query heads lost 9 % of the rate on the Llama-2-70B-shaped batch
  // (timing-only variants: the same instructions writing one line, or
  // partials kept in a 256 KB region, ran at the rate of one-head units).
  // Units of fewer than 4 columns write little per segment: they stage one
  // segment's rows in the wave's K tile, idle at a segment's end (LDS serves
  // one wave's accesses in order, so the reads of the last tile come first),
  // and write them once the next segment's first K/V loads are issued, before
  // any of that segment's tiles reach LDS (measured better for the two-head
  // units of FP8 pools, which are at the register limit).
  constexpr bool kHoldToEnd = HPW >= 4;
  constexpr int kSlots = kHoldToEnd ? 2 : 1;
  static_assert(kHoldToEnd || HPW * ROW <= KVP * TB, "staged rows must fit the K tile");
  // kSlots x HPW rows (pairs: after the two shared stages, one set per wave)
  unsigned char* hold = PAIR         ? smem + 4 * TB + ct * kSlots * HPW * ROW
                        : kHoldToEnd ? kt_lds + 2 * KVP * TB
                                     : kt_lds;
  // What each hold slot holds (wave-uniform, plain registers): kind 1 = output
  // rows (bit c of rows: column c's row is written), 2 = partial rows for the
  // workspace slot `slot`; s, kvh, hc: the segment.
  int held = 0;
  int kind0 = 0, s0 = 0, kvh0 = 0, hc0 = 0, slot0 = 0;
  int kind1 = 0, s1 = 0, kvh1 = 0, hc1 = 0, slot1 = 0;
  uint64_t rows0 = 0, rows1 = 0;
  float2 ml0 = make_float2(0.f, 0.f), ml1 = make_float2(0.f, 0.f);  // partials' (m, l)
  auto write_held = [&](int kind, int sq, int kvh, int hc, uint64_t rows, int slot,
                        const unsigned char* rows_lds, float2 ml) {
    Cursor x{};
    x.s = sq;
    x.kvh = kvh;
    x.hc = hc;
    constexpr int LPRW = ROW / 16;     // lanes per row
    constexpr int RPW = kWave / LPRW;  // rows per store instruction
    unsigned char* part = reinterpret_cast<unsigned char*>(a.ws_acc);  // bf16 partial rows
    // multi-row waves: output rows by the mask, all partial rows (the combine
    // reads only the columns of the sequence's rows); held row cc is the
    // wave's column cc, unit column cb + cc
    const int nc = MR ? HPW : ncols;
#pragma unroll 1
    for (int it = 0; it < (HPW + RPW - 1) / RPW; ++it) {
      const int cc = it * RPW + lane / LPRW;
      const bool use = cc < nc && (kind == 2 || ((rows >> cc) & 1));
      if (use) {
        const uint4 v = *reinterpret_cast<const uint4*>(rows_lds + cc * ROW + (lane % LPRW) * 16);
        unsigned char* dst = kind == 1
                                 ? static_cast<unsigned char*>(a.out) + row_of(x, cb + cc) * ROW
                                 : part + (int64_t(slot) * UC + cb + cc) * ROW;
        *reinterpret_cast<uint4*>(dst + (lane % LPRW) * 16) = v;
      }
    }
    if (!MR && kind == 2 && g == 0 && i16 < ncols) a.ws_ml[int64_t(slot) * MLS + i16] = ml;
  };
  auto flush = [&]() {
    if (held > 0) write_held(kind0, s0, kvh0, hc0, rows0, slot0, hold, ml0);
    if (kSlots > 1 && held > 1)
      write_held(kind1, s1, kvh1, hc1, rows1, slot1, hold + HPW * ROW, ml1);
    held = 0;
  };
  auto end_segment = [&](const Cursor& x, bool owns_start, bool owns_end) {
    float l = lpart + __shfl_xor(lpart, 16);
    l += __shfl_xor(l, 32);
    const int c = cb + i16;  // this lane's unit column
    const bool col = c < ncols;
    // this lane's column: with paired KV heads, column 1 is in the second set
    f32x4_t oc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oc[dt] = KVP == 2 && i16 >= CPH ? o[KVP - 1][dt] : o[0][dt];
    if (held == kSlots) flush();
    const int h = kSlots == 1 ? 0 : held;
    ++held;
    unsigned char* rows_lds = hold + h * HPW * ROW;
    int kind, slot = 0;
    uint64_t rows = 0;
    float2 ml = make_float2(0.f, 0.f);
    if (owns_start && owns_end) {
      // a grouped member without tokens scored nothing: the walk wrote its zeros
      const bool keep = col && (!GROUPED || l > 0.f);
      if (a.lse && g == 0 && keep) a.lse[row_of(x, c)] = m * c2 + __builtin_amdgcn_logf(l);
      const float inv = vsc / l;
      if (keep) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          *reinterpret_cast<uint2*>(rows_lds + i16 * ROW + (16 * dt + 4 * g) * 2) =
              make_uint2(pack_bf16(oc[dt][0] * inv, oc[dt][1] * inv),
                         pack_bf16(oc[dt][2] * inv, oc[dt][3] * inv));
      }
      kind = 1;
      rows = __ballot(g == 0 && keep);
    } else {
      // partial sums of a split segment go to the combine as bf16 (the (max,
      // denominator) record stays fp32); accumulation in the wave was fp32
      if (col) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          *reinterpret_cast<uint2*>(rows_lds + i16 * ROW + (16 * dt + 4 * g) * 2) =
              make_uint2(pack_bf16(oc[dt][0] * vsc, oc[dt][1] * vsc),
                         pack_bf16(oc[dt][2] * vsc, oc[dt][3] * vsc));
      }
      kind = 2;
      slot = 2 * wk + (owns_start ? 1 : 0);
      ml = make_float2(m * c2, l);
      // multi-row waves write their (max, denominator) records now (the
      // columns in use change from one segment to the next); the others keep
      // theirs with the held rows
      if (MR && g == 0 && col) a.ws_ml[int64_t(slot) * MLS + c] = ml;
    }
    if (kSlots == 1 || h == 0) {
      kind0 = kind; s0 = x.s; kvh0 = x.kvh; hc0 = x.hc; rows0 = rows; slot0 = slot; ml0 = ml;
    } else {
      kind1 = kind; s1 = x.s; kvh1 = x.kvh; hc1 = x.hc; rows1 = rows; slot1 = slot; ml1 = ml;
    }
  };

  // Tiles [j0, j1) of a run of L tokens whose blocks are row[0], row[1], ...,
  // in chunks whose blocks fit a 64-entry window of the block table;
  // branch-free, with NB tiles in flight. Keys past the end are clamped to the
  // last token (a valid, written slot) and masked out in compute.
  // win0 (when have_win0): the window of tile j0's chunk, already loaded
  auto run_part = [&](const int32_t* row, int L, int j0, int j1, int kvh, bool colok, int win0,
                      bool have_win0) {
    const int nblk = (L + Bm1) >> b_shift;
    const int Lm1 = L - 1;
    const int64_t head_off = int64_t(kvh) * B * GROW + lch * 16;
    for (int jc = j0; jc < j1;) {
      const int jb0 = (jc * kTile) >> b_shift;
      const int win = have_win0 && jc == j0 ? win0 : (jb0 + lane < nblk ? row[jb0 + lane] : 0);
      const int jc_end = min(j1, ((jb0 + kWave) << b_shift) / kTile);
      auto load_tile = [&](int j, uint4* kr, uint4* vr) {
        int pb = 0;
        if constexpr (BIG_B) pb = __builtin_amdgcn_readlane(win, ((j * kTile) >> b_shift) - jb0);
#pragma unroll
        for (int ut = 0; ut < NLT; ++ut) {  // rows of KV head kvh + ut / NI
          const int t = min(j * kTile + row0 + (ut % NI) * RPI + lrow, Lm1);
          if constexpr (!BIG_B) pb = __shfl(win, (t >> b_shift) - jb0);
          const int64_t off = int64_t(pb) * block_bytes + head_off +
                              int64_t(ut / NI) * B * GROW + int64_t(t & Bm1) * GROW;
          kr[ut] = load_stream16(reinterpret_cast<const uint4*>(kp + off));
          vr[ut] = load_stream16(reinterpret_cast<const uint4*>(vp + off));
        }
      };
      // NB tiles in flight: tile j + NB - 1 loads while tile j is computed
      // (buffer b holds the tiles j with j % NB == b relative to jc). Every
      // load is unconditional (past the chunk it re-reads the chunk's last
      // tile, an L2 hit): with conditional loads the compiler cannot count the
      // loads in flight and waits for all of them.
      uint4 kb[NB][NLT], vb[NB][NLT];
      int j = jc;
#pragma unroll
      for (int b = 0; b < NB - 1; ++b) load_tile(min(j + b, jc_end - 1), kb[b], vb[b]);
      if constexpr (!kHoldToEnd) flush();  // the previous segment's staged rows
      for (; j + NB <= jc_end; j += NB) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const int jl = min(j + b + NB - 1, jc_end - 1);
          load_tile(jl, kb[(b + NB - 1) % NB], vb[(b + NB - 1) % NB]);
          __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of this tile's math
          compute(j + b, L, kb[b], vb[b], colok);
        }
      }
#pragma unroll
      for (int b = 0; b < NB - 1; ++b)  // the last tiles, already loaded
        if (j + b < jc_end) compute(j + b, L, kb[b], vb[b], colok);
      jc = jc_end;
    }
  };

  // Tiles [j0, j1) of one segment. Plain: the sequence's tokens. Grouped: the
  // group's shared prefix (read through the first member's table row), then
  // the tokens after it of member 0, 1, ... (through that member's row, from
  // the entry of the prefix's end on), each scored by that member's columns.
  auto run_tiles = [&](const Cursor& x, int j0, int j1, int win0) {
    if constexpr (MR) {
      // none of this wave's columns has a row here (pairs: skip only together,
      // when the sequence has no rows; a wave without columns scores -inf)
      if (PAIR ? ncols == 0 : cb >= ncols) return;
    }
    if constexpr (!GROUPED) {
      run_part(a.block_tables + int64_t(x.s) * a.max_blocks_per_seq, x.L, j0, j1, x.kvh, true,
               win0, true);
    } else {
      const int s0 = x.s * a.group_size;
      const int P = a.prefix_lens[s0];
      int first = 0;  // the part's first tile in the segment
      for (int mb = -1; mb < a.group_size && first < j1; ++mb) {
        const int s = mb < 0 ? s0 : s0 + mb;
        const int Lp = mb < 0 ? P : max(a.seq_lens[s] - P, 0);
        const int np = tiles_of(Lp);
        const int lo = max(j0, first), hi = min(j1, first + np);
        if (lo < hi) {
          const int32_t* row = a.block_tables + int64_t(s) * a.max_blocks_per_seq +
                               (mb < 0 ? 0 : (P >> b_shift));
          // the part holding tile j0 starts from the prefetched window
          run_part(row, Lp, lo - first, hi - first, x.kvh, mb < 0 || i16 / G == mb, win0,
                   lo == j0);
        }
        first += np;
      }
    }
  };

  walk_slice<D, 8, GROUPED>(a, wk, lane, n_hchunk, HPW, KVP, prefetch, begin_segment, run_tiles,
                            end_segment, ct == 0);
  flush();  // the wave is done: its held results
}

// Combine the partials of each split segment. Wave w looks at the segment
// that wave w of the decode kernel started and left open (if any); its
// partials are in slot 2w+1 (wave w) and slots 2v for the waves v in
// (w, last] that continued it.
// PART_BF16: the partial sums are bf16 rows (written by the matrix-core
// kernel), else fp32 rows.
// MR: multi-row units (columns = (row, query head) pairs of the sequence's rows).
template <int DTYPE, int D, int HPW, bool GROUPED, bool PART_BF16, bool MR = false>
__global__ __launch_bounds__(kWave * kMaxWavesPerGroup) void decode_combine_kernel(DecodeArgs a) {
  constexpr int MLS = HPW > kMLStride ? HPW : kMLStride;
  using RS = RowShape<DTYPE, D>;
  constexpr int VEC = RS::VEC, LPR = RS::LPR;
  const int lane = threadIdx.x % kWave;
  const int w = blockIdx.x * (blockDim.x / kWave) + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  if (w >= a.workers) return;
  const int4 seg = a.ws_seg[w];
  if (seg.x < 0) return;
  const int wb = seg.z, head0 = seg.w;
  // one lane group of LPR lanes per query head of the unit; with more heads
  // than lane groups a lane takes several heads, whose loads are issued
  // together. The partials are merged online (running max M, rescaled sums),
  // two of them per step so that their loads are in flight together.
  constexpr int GROUPS = kWave / LPR;
  constexpr int HPL = (HPW + GROUPS - 1) / GROUPS;  // heads per lane
  const int c = lane % LPR;
  float M[HPL], den[HPL], num[HPL][VEC];
#pragma unroll
  for (int k = 0; k < HPL; ++k) {
    M[k] = -INFINITY;
    den[k] = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) num[k][e] = 0.f;
  }
  auto slot_of = [&](int v) { return v == w ? 2 * v + 1 : 2 * v; };
  for (int v = w; v <= wb; v += 2) {
    const int nv = v + 1 <= wb ? 2 : 1;  // wave-uniform
    float2 ml[2][HPL];
    float4 x[2][HPL][VEC / 4];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int sl = slot_of(q < nv ? v + q : v);
#pragma unroll
      for (int k = 0; k < HPL; ++k) {
        const int hh = min(lane / LPR + k * GROUPS, HPW - 1);
        ml[q][k] = a.ws_ml[int64_t(sl) * MLS + hh];
        if constexpr (PART_BF16) {
          static_assert(VEC == 8, "bf16 partials: one 16-byte load per lane");
          const uint4 b = *reinterpret_cast<const uint4*>(
              reinterpret_cast<const uint16_t*>(a.ws_acc) + (int64_t(sl) * HPW + hh) * D + c * VEC);
          x[q][k][0] = make_float4(bf16_lo(b.x), bf16_hi(b.x), bf16_lo(b.y), bf16_hi(b.y));
          x[q][k][1] = make_float4(bf16_lo(b.z), bf16_hi(b.z), bf16_lo(b.w), bf16_hi(b.w));
        } else {
          const float4* src =
              reinterpret_cast<const float4*>(a.ws_acc + (int64_t(sl) * HPW + hh) * D + c * VEC);
#pragma unroll
          for (int e = 0; e < VEC; e += 4) x[q][k][e / 4] = src[e / 4];
        }
      }
    }
#pragma unroll
    for (int k = 0; k < HPL; ++k) {
      const float m2 = nv == 2 ? ml[1][k].x : -INFINITY;
      const float Mn = fmaxf(M[k], fmaxf(ml[0][k].x, m2));
      // A partial that scored nothing has m = -inf (in the grouped decode, a
      // wave that only saw other members' tokens): weight 0. While every
      // partial so far is such, the base is 0 so no -inf - -inf arises.
      const float Ms = Mn == -INFINITY ? 0.f : Mn;
      const float fo = M[k] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M[k] - Ms);
      const float f0 = __builtin_amdgcn_exp2f(ml[0][k].x - Ms);
      const float f1 = nv == 2 ? __builtin_amdgcn_exp2f(m2 - Ms) : 0.f;
      den[k] = den[k] * fo + ml[0][k].y * f0 + (nv == 2 ? ml[1][k].y * f1 : 0.f);
#pragma unroll
      for (int e = 0; e < VEC; e += 4) {
        const float4 x0 = x[0][k][e / 4], x1 = x[1][k][e / 4];
        num[k][e] = num[k][e] * fo + x0.x * f0 + x1.x * f1;
        num[k][e + 1] = num[k][e + 1] * fo + x0.y * f0 + x1.y * f1;
        num[k][e + 2] = num[k][e + 2] * fo + x0.z * f0 + x1.z * f1;
        num[k][e + 3] = num[k][e + 3] * fo + x0.w * f0 + x1.w * f1;
      }
      M[k] = Mn;
    }
  }
  const int G = a.num_q_heads / a.num_kv_heads;
  const int ncols = GROUPED ? a.group_size * G
                             : MR ? (a.q_start_loc[seg.x + 1] - a.q_start_loc[seg.x]) * G : HPW;
#pragma unroll
  for (int k = 0; k < HPL; ++k) {
    const int hh = lane / LPR + k * GROUPS;
    if (hh >= ncols) continue;
    // grouped: a member without tokens has no partials (the walk wrote its zeros)
    if (GROUPED && !(den[k] > 0.f)) continue;
    const float inv = 1.f / den[k];
    const int64_t row = GROUPED ? int64_t(seg.x * a.group_size + hh / G) * a.num_q_heads +
                                      head0 + hh % G
                        : MR    ? int64_t(a.q_start_loc[seg.x] + hh / G) * a.num_q_heads +
                                      head0 + hh % G
                                : int64_t(seg.x) * a.num_q_heads + head0 + hh;
    if (a.lse && c == 0) a.lse[row] = M[k] + __builtin_amdgcn_logf(den[k]);
    float f[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) f[e] = num[k][e] * inv;
    uint4* o = static_cast<uint4*>(a.out) + (row * D) / VEC + c;
    *o = pack16<DTYPE>(f);
  }
}

template <int DTYPE, int D, int HPW>
hipError_t run(const DecodeArgs& a, hipStream_t st) {
  int b_shift = 0;
  while ((1 << b_shift) < a.block_size) ++b_shift;
  const int n_hchunk = (a.num_q_heads / a.num_kv_heads) / HPW;
  // Persistent waves: size workgroups so that there is about one per compute
  // unit; the dispatcher then spreads the waves evenly over the chip.
  const int cus = a.num_cus > 0 ? a.num_cus : 1;
  int wpg = (a.workers + cus - 1) / cus;
  wpg = wpg < 1 ? 1 : (wpg > kMaxWavesPerGroup ? kMaxWavesPerGroup : wpg);
  const int groups = (a.workers + wpg - 1) / wpg;
  const float scale_log2 = a.scale * kLog2e;
  // FP8 MHA with an even number of heads: units of two adjacent KV heads
  // (one contiguous run of both heads' rows per tile), combined as 2 heads
  if constexpr (DTYPE == PA_FP8_E4M3 && HPW == 1) {
    if (a.num_q_heads == a.num_kv_heads && a.num_kv_heads % 2 == 0) {
      const size_t lds = size_t(wpg) * mfma_wave_lds<D, 2, 2>();
      if (a.block_size >= kTile)
        decode_mfma_kernel<D, 2, true, DTYPE, 2, false>
            <<<groups, kWave * wpg, lds, st>>>(a, b_shift, 1, scale_log2);
      else
        decode_mfma_kernel<D, 2, false, DTYPE, 2, false>
            <<<groups, kWave * wpg, lds, st>>>(a, b_shift, 1, scale_log2);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      decode_combine_kernel<PA_BF16, D, 2, false, true><<<groups, kWave * wpg, 0, st>>>(a);
      return hipGetLastError();
    }
  }
  // bf16 groups of >= 4 heads and every FP8 pool run on the matrix cores
  if constexpr (DTYPE == PA_FP8_E4M3 || (DTYPE == PA_BF16 && HPW >= 4)) {
    const size_t lds = size_t(wpg) * mfma_wave_lds<D, HPW, 1>();
    if (a.block_size >= kTile)
      decode_mfma_kernel<D, HPW, true, DTYPE, 1, false>
          <<<groups, kWave * wpg, lds, st>>>(a, b_shift, n_hchunk, scale_log2);
    else
      decode_mfma_kernel<D, HPW, false, DTYPE, 1, false>
          <<<groups, kWave * wpg, lds, st>>>(a, b_shift, n_hchunk, scale_log2);
  } else {
    if (a.block_size >= kTile)
      decode_balanced_kernel<DTYPE, D, HPW, true>
          <<<groups, kWave * wpg, 0, st>>>(a, b_shift, n_hchunk, scale_log2);
    else
      decode_balanced_kernel<DTYPE, D, HPW, false>
          <<<groups, kWave * wpg, 0, st>>>(a, b_shift, n_hchunk, scale_log2);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int OUT = DTYPE == PA_F32 ? PA_F32 : PA_BF16;  // FP8 pools give bf16 output
  // the matrix-core kernel hands over bf16 partials
  constexpr bool PART_BF16 = DTYPE == PA_FP8_E4M3 || (DTYPE == PA_BF16 && HPW >= 4);
  decode_combine_kernel<OUT, D, HPW, false, PART_BF16><<<groups, kWave * wpg, 0, st>>>(a);
  return hipGetLastError();
}

// Grouped decode: one unit per (group, KV head) of 16 columns, on the matrix
// cores (bf16 and FP8 pools).
template <int DTYPE, int D>
hipError_t run_grouped(const DecodeArgs& a, hipStream_t st) {
  int b_shift = 0;
  while ((1 << b_shift) < a.block_size) ++b_shift;
  const int cus = a.num_cus > 0 ? a.num_cus : 1;
  int wpg = (a.workers + cus - 1) / cus;
  wpg = wpg < 1 ? 1 : (wpg > kMaxWavesPerGroup ? kMaxWavesPerGroup : wpg);
  const int groups = (a.workers + wpg - 1) / wpg;
  const float scale_log2 = a.scale * kLog2e;
  constexpr int H = kGroupedCols;
  const size_t lds = size_t(wpg) * mfma_wave_lds<D, H, 1>();
  if (a.block_size >= kTile)
    decode_mfma_kernel<D, H, true, DTYPE, 1, true><<<groups, kWave * wpg, lds, st>>>(a, b_shift, 1, scale_log2);
  else
    decode_mfma_kernel<D, H, false, DTYPE, 1, true><<<groups, kWave * wpg, lds, st>>>(a, b_shift, 1, scale_log2);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  decode_combine_kernel<PA_BF16, D, H, true, true><<<groups, kWave * wpg, 0, st>>>(a);
  return hipGetLastError();
}

// Multi-row decode (bf16 and FP8 pools): units of (sequence, KV head) with up to
// kMultiRowCols (row, query head) columns, 16 per wave: units of more than 16
// run on a workgroup of two waves that share each K/V tile in LDS; two waves
// per SIMD.
template <int KV, int D>
hipError_t run_multirow(const DecodeArgs& a, hipStream_t st) {
  int b_shift = 0;
  while ((1 << b_shift) < a.block_size) ++b_shift;
  const float scale_log2 = a.scale * kLog2e;
  constexpr int H = 16;
  if (a.mr_pair) {
    // one workgroup of two waves per work slice (not for FP8 rows of 64 dims,
    // whose tile is one wave-wide load)
    if constexpr (KV == PA_FP8_E4M3 && D == 64) {
      return hipErrorInvalidValue;
    } else {
      const size_t lds = mr_pair_lds<D>();
      if (a.block_size >= kTile)
        decode_mfma_kernel<D, H, true, KV, 1, false, true, true>
            <<<a.workers, 2 * kWave, lds, st>>>(a, b_shift, 1, scale_log2);
      else
        decode_mfma_kernel<D, H, false, KV, 1, false, true, true>
            <<<a.workers, 2 * kWave, lds, st>>>(a, b_shift, 1, scale_log2);
    }
  } else {
    const int cus = a.num_cus > 0 ? a.num_cus : 1;
    int wpg = (a.workers + cus - 1) / cus;
    wpg = wpg < 1 ? 1 : (wpg > kMultiRowWaves ? kMultiRowWaves : wpg);
    const int groups = (a.workers + wpg - 1) / wpg;
    const size_t lds = size_t(wpg) * mfma_wave_lds<D, H, 1>();
    if (a.block_size >= kTile)
      decode_mfma_kernel<D, H, true, KV, 1, false, true>
          <<<groups, kWave * wpg, lds, st>>>(a, b_shift, 1, scale_log2);
    else
      decode_mfma_kernel<D, H, false, KV, 1, false, true>
          <<<groups, kWave * wpg, lds, st>>>(a, b_shift, 1, scale_log2);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int cwpg = a.workers < kMaxWavesPerGroup ? a.workers : kMaxWavesPerGroup;
  decode_combine_kernel<PA_BF16, D, kMultiRowCols, false, true, true>
      <<<(a.workers + cwpg - 1) / cwpg, kWave * cwpg, 0, st>>>(a);
  return hipGetLastError();
}

template <int DTYPE, int D>
hipError_t run_d(const DecodeArgs& a, hipStream_t st) {
  switch (decode_heads_per_unit(a.num_q_heads / a.num_kv_heads)) {
    // fp32 rows of 128 dims with 8 heads per unit would spill registers: two
    // units of 4 heads per KV head instead (each reads the KV head's rows)
    case 8:
      if constexpr (DTYPE == PA_F32 && D == 128) return run<DTYPE, D, 4>(a, st);
      else return run<DTYPE, D, 8>(a, st);
    case 4: return run<DTYPE, D, 4>(a, st);
    case 2: return run<DTYPE, D, 2>(a, st);
    default: return run<DTYPE, D, 1>(a, st);
  }
}

}  // namespace

int decode_heads_per_unit(int group) {
  for (int h : {8, 4, 2, 1})
    if (group % h == 0) return h;
  return 1;
}

bool decode_supported(int dtype, int head_dim, int group) {
  return (dtype == PA_F32 || dtype == PA_BF16 || dtype == PA_FP8_E4M3) &&
         (head_dim == 64 || head_dim == 128) && group >= 1;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) {
  if (a.q_start_loc) {
    if (a.prefix_lens || a.len_offset) return hipErrorInvalidValue;
    if (a.dtype == PA_BF16) {
      if (a.head_dim == 128) return run_multirow<PA_BF16, 128>(a, st);
      if (a.head_dim == 64) return run_multirow<PA_BF16, 64>(a, st);
    } else if (a.dtype == PA_FP8_E4M3) {
      if (a.head_dim == 128) return run_multirow<PA_FP8_E4M3, 128>(a, st);
      if (a.head_dim == 64) return run_multirow<PA_FP8_E4M3, 64>(a, st);
    }
    return hipErrorInvalidValue;
  }
  if (a.prefix_lens) {
    if (a.group_size < 1 || a.group_size * (a.num_q_heads / a.num_kv_heads) > kGroupedCols)
      return hipErrorInvalidValue;
    if (a.dtype == PA_BF16) {
      if (a.head_dim == 128) return run_grouped<PA_BF16, 128>(a, st);
      if (a.head_dim == 64) return run_grouped<PA_BF16, 64>(a, st);
    } else if (a.dtype == PA_FP8_E4M3) {
      if (a.head_dim == 128) return run_grouped<PA_FP8_E4M3, 128>(a, st);
      if (a.head_dim == 64) return run_grouped<PA_FP8_E4M3, 64>(a, st);
    }
    return hipErrorInvalidValue;
  }
  if (a.dtype == PA_BF16) {
    if (a.head_dim == 128) return run_d<PA_BF16, 128>(a, st);
    if (a.head_dim == 64) return run_d<PA_BF16, 64>(a, st);
  } else if (a.dtype == PA_F32) {
    if (a.head_dim == 128) return run_d<PA_F32, 128>(a, st);
    if (a.head_dim == 64) return run_d<PA_F32, 64>(a, st);
  } else if (a.dtype == PA_FP8_E4M3) {
    if (a.head_dim == 128) return run_d<PA_FP8_E4M3, 128>(a, st);
    if (a.head_dim == 64) return run_d<PA_FP8_E4M3, 64>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
