// Chunked-prefill attention over paged K/V with bf16 MFMA (gfx950).
//
// What it computes ("vLLM PagedAttention explained", section 7.2: a long
// prompt is processed in chunks that join the sequence's block table): for
// each sequence s with a chunk of C = q_len rows whose keys are already in the
// pool, row i sits at absolute position a_i = seq_lens[s] - C + i and
//   out[row i][h] = sum_{t <= a_i} softmax_t(scale * q_i.K_s[t]) V_s[t],
// K_s/V_s read through the block table. Query head h reads KV head h / G.
//
// How. This is the one place where the work is a dense contraction (queries x
// keys x head_dim), so it runs on the matrix cores:
//  * v_mfma_f32_32x32x16_bf16 computes S^T = K Q^T (keys x rows) and then
//    O^T = V^T P^T (head_dim x rows). In both accumulators a lane holds one
//    query row (lane % 32), so the online softmax of a row lives in two lanes
//    (lane and lane ^ 32), and P^T is fed to the second product straight from
//    the first product's accumulators, converted to bf16, with no shuffles.
//  * A workgroup is (sequence, KV head, 32-row tile, up to 4 query heads of
//    the group): its four waves share every K/V tile of 64 keys.
//  * K/V tiles go from the pool straight into LDS (global_load_lds_dwordx4:
//    a wave's 64 lanes fill 1 KB of LDS, lane l at byte 16 l), double
//    buffered: the loads of tile t+1 and the block-table entries of tile t+2
//    are in flight while tile t is computed; one barrier per tile. No
//    registers stage the data and no LDS store instructions run.
//  * LDS rows are unpadded, [key][head_dim]; the 16-byte chunk c of row r is
//    kept at chunk c ^ swz(r). A lane picks the global chunk that lands in
//    its LDS slot, so the swizzle costs nothing on the way in, and swz is
//    chosen so that both operand reads below touch every LDS bank at most
//    once per pass.
//  * The K operand of S^T is a 16-byte read (one key, 8 dims). The V operand
//    of O^T needs 4 consecutive keys of one dim per lane: ds_read_b64_tr_b16
//    reads it transposed. Within 16 lanes, lane 4k+q points at
//    V[key0+k][dim0+4q .. +3] and lane i receives V[key0..key0+3][dim0+i].
//  * The softmax scale is folded into the exponent (one FMA per score);
//    causal masking (keys past a row's position get -inf) is applied only on
//    tiles that reach the diagonal; the exponent base of a row only moves when
//    its max grows by more than 2^8, so the output rescale is rare. Tiles
//    beyond a wave's last row are skipped.
//  * Workgroups that read the same (sequence, KV head) stream are placed on
//    the same XCD (workgroup i runs on XCD i mod 8), so its L2 serves the
//    repeated K/V reads, and these groups are dealt round-robin over the
//    XCDs so that sequences of different lengths load them evenly; within a
//    group the longest (last) row tiles are dispatched first.
#include <math.h>

#include "device.h"

namespace pa {
namespace {

constexpr int kWaves = 4;
constexpr int kRows = 32;     // query rows per wave (MFMA N)
constexpr int kKeys = 64;     // keys per K/V tile
constexpr int kXcds = 8;
constexpr float kLog2e = 1.4426950408889634f;

typedef short bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;
typedef short bf16x2_t __attribute__((__vector_size__(2 * sizeof(short))));
typedef __attribute__((address_space(4))) const int32_t const_i32;

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ f32x16_t mfma32(const uint4& a, const uint4& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

template <int D>
struct PrefillShape {
  static constexpr int KSTEPS = D / 16;               // MFMA k-steps over head_dim
  static constexpr int DTILES = D / 32;               // 32-row tiles of head_dim in O^T
  static constexpr int CPR = D / 8;                   // 16-byte chunks per K/V row
  static constexpr int ROW = D * 2;                   // bytes per K/V row in LDS
  static constexpr int RPI = 1024 / ROW;              // rows one wave-wide load fills
  static constexpr int NI = kKeys / (RPI * kWaves);   // loads per wave per tensor per tile
  static constexpr int TILE = kKeys * ROW;            // bytes of one K or V tile
  static constexpr int STAGE = 2 * TILE;              // K tile then V tile
  static constexpr int LDS = 2 * STAGE;               // two stages
  static_assert(NI >= 1 && kKeys % (RPI * kWaves) == 0, "tile must split evenly over waves");
};

// Chunk swizzle. For 16 chunks per row: swz(r) = 4 (r % 4) + (r / 4) % 4, a
// bijection on 16 consecutive rows (K reads: 16 rows, one chunk) whose upper
// two bits differ over any 4 consecutive rows (V reads: 4 rows x 4 aligned
// chunks). For 8 chunks per row (two rows per 256-byte bank line) the same
// two properties hold per row parity.
template <int CPR>
__device__ __forceinline__ int swz(int r) {
  if constexpr (CPR == 16) return 4 * (r % 4) + (r / 4) % 4;
  else return 4 * ((r / 2) % 2) + (r / 4) % 4;
}

// 16 bytes per lane from global memory into LDS at lds_addr + 16 * lane.
// Issued from inline assembly so that the compiler does not put a wait for
// it in front of every later LDS read; completion is awaited explicitly
// (vmcnt) before the barrier that publishes the tile. M0 holds the LDS
// address; nothing else in this kernel uses M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void load_lds16(const void* gptr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gptr), "s"(lds_addr)
               : "memory", "m0");
}
// Same, from a wave-uniform base plus a 32-bit per-lane byte offset.
__device__ __forceinline__ void load_lds16(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds_addr)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Wait for every outstanding load of this wave (including the direct-to-LDS
// ones) and every LDS access, then meet the other waves. The wait is the
// compiler's own s_waitcnt, so its bookkeeping of outstanding loads restarts
// from zero here and it adds no waits of its own for older loads later in the
// loop; the empty asm keeps LDS reads from moving above the barrier.
__device__ __forceinline__ void drain_and_barrier() {
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// WAVE_BLOCK: blocks of at least 16 tokens, so that a wave's 16 keys of a
// tile lie in one block.
template <int D, bool WAVE_BLOCK>
__global__ __launch_bounds__(kWave * kWaves, 2) void prefill_kernel(
    PrefillArgs a, int32_t b_shift, int32_t heads_per_group, int32_t n_hchunk, int32_t n_rtiles,
    int32_t chunk_wgs, int32_t chunks_per_group, float scale_log2) {
  using PS = PrefillShape<D>;
  constexpr int NI = PS::NI;
  extern __shared__ __align__(16) unsigned char smem[];

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int g = lane / 32;  // which half of the wave
  const int Hq = a.num_q_heads, Hkv = a.num_kv_heads;
  const int G = Hq / Hkv;
  const int R = kWaves / heads_per_group;  // row tiles per workgroup

  // Workgroup -> (sequence, KV head, head chunk, row tile). The workgroups of
  // one (sequence, KV head) group read the same K/V and are cut into chunks
  // of chunk_wgs; hardware workgroup i runs on XCD i % 8, and XCD x takes
  // chunks x, x+8, x+16, ... so that every chunk stays on one XCD (its L2
  // serves the repeated K/V reads) and the groups are dealt out evenly.
  const int gs = n_hchunk * n_rtiles;  // workgroups per group
  const int x = blockIdx.x % kXcds, j = blockIdx.x / kXcds;
  const int c = (j / chunk_wgs) * kXcds + x;
  const int group = c / chunks_per_group;
  const int member = (c % chunks_per_group) * chunk_wgs + j % chunk_wgs;
  if (group >= a.num_seqs * a.num_kv_heads || member >= gs) return;  // grid padding
  const int rt_rev = member % n_rtiles;
  const int hc = member / n_rtiles;
  const int kvh = group % a.num_kv_heads;
  const int s = group / a.num_kv_heads;
  const int rt = n_rtiles - 1 - rt_rev;  // longest rows first

  const int q0 = a.q_start_loc[s];
  const int q_len = a.q_start_loc[s + 1] - q0;
  const int L = a.seq_lens[s];
  const int wg_row0 = rt * R * kRows;
  if (wg_row0 >= q_len || L <= 0) return;  // uniform over the workgroup
  const int start = L - q_len;                 // absolute position of chunk row 0
  const int wg_last_key = start + min(q_len, wg_row0 + R * kRows) - 1;
  const int n_ktiles = wg_last_key / kKeys + 1;

  const int row0 = wg_row0 + (wave / heads_per_group) * kRows;  // this wave's first row
  const int head = kvh * G + hc * heads_per_group + wave % heads_per_group;
  const bool wave_active = row0 < q_len;
  const int wave_last_key = wave_active ? start + min(q_len, row0 + kRows) - 1 : -1;
  const bool wave_ragged = row0 + kRows > q_len;  // has rows past the chunk: always mask
  const int my_row = row0 + lane % kRows;
  const int my_pos = my_row < q_len ? start + my_row : -1;

  // Q^T operands: row my_row, dims 16*ks + 8*g .. +7 (rows past the chunk read its last row)
  uint4 qop[PS::KSTEPS];
  {
    const int qr = q0 + min(my_row, q_len - 1);
    const uint4* qp = static_cast<const uint4*>(a.q) + (int64_t(qr) * Hq + head) * PS::CPR;
#pragma unroll
    for (int ks = 0; ks < PS::KSTEPS; ++ks) qop[ks] = qp[2 * ks + g];
  }

  // Tile loads: load i of this wave fills LDS rows (wave*NI + i)*RPI + lane/CPR
  // of a K or V tile, lane l the chunk slot l % CPR. A wave's loads cover the
  // 16 consecutive keys t*64 + 16*wave .. +15 of tile t.
  const int32_t* bt = a.block_tables + int64_t(s) * a.max_blocks_per_seq;
  const unsigned char* kpool = static_cast<const unsigned char*>(a.k_pool);
  const unsigned char* vpool = static_cast<const unsigned char*>(a.v_pool);
  const int B = a.block_size, Bm1 = B - 1;
  const uint32_t lds0 = static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) unsigned char*)smem));
  int ld_row[NI], ld_chunk[NI];
  uint32_t ld_off[NI];  // byte offset of this lane's chunk from the wave's first row
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    ld_row[i] = (wave * NI + i) * PS::RPI + lane / PS::CPR;
    ld_chunk[i] = (lane % PS::CPR) ^ swz<PS::CPR>(ld_row[i]);
    ld_off[i] = uint32_t((i * PS::RPI + lane / PS::CPR) * PS::ROW + ld_chunk[i] * 16);
  }
  // WAVE_BLOCK: the wave's block is found with one scalar load; clamped keys
  // (past the end) stay in it, since it is looked up for min(first key, L-1).
  // Otherwise each lane looks up the block of each of its keys.
  const_i32* btc = (const_i32*)bt;
  const int64_t head_bytes = int64_t(kvh) * B * PS::ROW;
  const int64_t block_bytes = int64_t(Hkv) * B * PS::ROW;
  auto load_table = [&](int t, int32_t (&tab)[NI]) {
    if constexpr (WAVE_BLOCK) {
      tab[0] = btc[min(t * kKeys + 16 * wave, L - 1) >> b_shift];
    } else {
#pragma unroll
      for (int i = 0; i < NI; ++i) tab[i] = bt[min(t * kKeys + ld_row[i], L - 1) >> b_shift];
    }
  };
  // tile t of one tensor (pool) into the LDS tile at byte offset tile_off
  auto issue_tile = [&](const unsigned char* pool, int t, const int32_t (&tab)[NI],
                        uint32_t tile_off) {
    const uint32_t st = lds0 + tile_off + uint32_t(wave * NI * 1024);
    const int key0 = t * kKeys + 16 * wave;
    if constexpr (WAVE_BLOCK) {
      const int64_t base = int64_t(tab[0]) * block_bytes + head_bytes;
      if (key0 + 16 <= L) {  // no clamping: every offset is a per-lane constant
        const int64_t wb = base + int64_t(key0 & Bm1) * PS::ROW;
#pragma unroll
        for (int i = 0; i < NI; ++i) load_lds16(pool + wb, ld_off[i], st + uint32_t(i * 1024));
      } else {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const int tk = min(t * kKeys + ld_row[i], L - 1);  // past the end: a valid, masked key
          const uint32_t off = uint32_t((tk & Bm1) * PS::ROW + ld_chunk[i] * 16);
          load_lds16(pool + base, off, st + uint32_t(i * 1024));
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int tk = min(t * kKeys + ld_row[i], L - 1);  // past the end: a valid, masked key
        const int64_t off = int64_t(tab[i]) * block_bytes + head_bytes +
                            int64_t((tk & Bm1) * PS::ROW + ld_chunk[i] * 16);
        load_lds16(pool + off, st + uint32_t(i * 1024));
      }
    }
  };

  // LDS: K tiles in stages 0, 1 (bytes 0, TILE), V tiles in stages 0, 1 (bytes
  // 2 TILE, 3 TILE); tile t of either tensor uses stage t % 2.
  // Operand-read byte addresses inside a tile.
  // K: row mt*32 + lane%32, chunk 2ks + g  ->  (k_addr ^ 32 ks) + mt * 32 rows.
  const int kr = lane % 32;
  const uint32_t k_addr = uint32_t(kr * PS::ROW + ((g ^ swz<PS::CPR>(kr)) * 16));
  // V, read transposed: rows 16kk + 4g + (lane%16)/4 (+8 for the upper four
  // keys), dims 32dt + 16((lane/16)%2) + 4(lane%4) .. +3, i.e. chunk 4dt + cl,
  // half lane%2  ->  (v_lo ^ 64 dt) + 16 kk rows.
  const int vr = 4 * g + (lane % 16) / 4;
  const int cl = 2 * ((lane / 16) % 2) + (lane % 4) / 2;
  const uint32_t v_lo = uint32_t(vr * PS::ROW + ((cl ^ swz<PS::CPR>(vr)) * 16) + 8 * (lane % 2));
  const uint32_t v_hi =
      uint32_t((vr + 8) * PS::ROW + ((cl ^ swz<PS::CPR>(vr + 8)) * 16) + 8 * (lane % 2));

  f32x16_t o[PS::DTILES];
#pragma unroll
  for (int dt = 0; dt < PS::DTILES; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;
  float m = -INFINITY, lsum = 0.f;  // running max in raw score units

  // S^T = K Q^T for the 64 keys of the K tile at tile_off (two 32-key m-tiles)
  auto qk = [&](uint32_t tile_off, f32x16_t (&sacc)[2]) {
    const unsigned char* kt_lds = smem + tile_off;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[mt][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < PS::KSTEPS; ++ks)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const uint4 kop = *reinterpret_cast<const uint4*>(
            kt_lds + ((k_addr ^ (32u * ks)) + mt * 32 * PS::ROW));
        sacc[mt] = mfma32(kop, qop[ks], sacc[mt]);
      }
  };

  // One tile of the loop, software-pipelined: the scores of tile kt are in
  // cur.s (computed one step earlier); this step computes the scores of tile
  // kt+1 into nxt.s on the matrix cores while the VALU runs the softmax of
  // tile kt, then multiplies tile kt's weights with its V tile. Loads run two
  // tiles ahead for K and one for V; block-table entries one step before
  // their loads. The state of consecutive steps alternates between two sets
  // of registers (the loop is unrolled by two), so no value is copied.
  struct Step {
    f32x16_t s[2];    // scores of the tile this step works on
    int32_t tk[NI];   // block-table entries for the K tile this step loads
    int32_t tv[NI];   // ... and for the V tile
  };
  auto step = [&](int kt, int par, Step& cur, Step& nxt) {
    // K(kt+1) and V(kt) are in LDS for every wave, and every wave is done
    // with K(kt) and V(kt-1), whose stages the loads below overwrite
    drain_and_barrier();
    if (kt + 2 < n_ktiles) issue_tile(kpool, kt + 2, cur.tk, uint32_t(par * PS::TILE));
    if (kt + 1 < n_ktiles) issue_tile(vpool, kt + 1, cur.tv, uint32_t((3 - par) * PS::TILE));
    if (kt + 3 < n_ktiles) load_table(kt + 3, nxt.tk);
    if (kt + 2 < n_ktiles) load_table(kt + 2, nxt.tv);
    const int t0 = kt * kKeys;
    if (!wave_active || t0 > wave_last_key) return;  // uniform per wave

    // causal mask only where the tile reaches the diagonal (or rows past the chunk)
    if (wave_ragged || t0 + kKeys - 1 > start + row0) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = t0 + mt * 32 + 8 * (i / 4) + 4 * g + (i % 4);
          if (key > my_pos) cur.s[mt][i] = -INFINITY;
        }
    }
    // scores of tile kt+1 (unused when this wave stops at kt; the K stage then
    // holds an older tile, which is harmless)
    qk(uint32_t((1 - par) * PS::TILE), nxt.s);

    // Weights of tile kt against the current exponent base m, while those
    // MFMAs run. The base only moves when a row's max exceeds it by more than
    // 2^8 (or on a row's first scores): until then weights up to 256 are
    // taken as they are. Numerator and denominator share the base, so this
    // is exact, and the rare move redoes the weights below.
    uint4 pop[4];  // P^T operands for the four 16-key k-steps
    float ps;
    auto weights = [&](float nms) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float p[8];
#pragma unroll
          for (int j = 0; j < 8; ++j)
            p[j] = __builtin_amdgcn_exp2f(fmaf(cur.s[mt][8 * h + j], scale_log2, nms));
          pop[2 * mt + h] = make_uint4(pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3]),
                                       pack_bf16(p[4], p[5]), pack_bf16(p[6], p[7]));
        }
      // the row sum adds up the same bf16 weights that the PV product uses
      const bf16x2_t ones = __builtin_bit_cast(bf16x2_t, 0x3f803f80u);
      float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        ps0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pop[k].x), ones, ps0, false);
        ps1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pop[k].y), ones, ps1, false);
        ps0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pop[k].z), ones, ps0, false);
        ps1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pop[k].w), ones, ps1, false);
      }
      ps = ps0 + ps1;
    };
    weights(m == -INFINITY ? 0.f : -m * scale_log2);
    // keep this work before the branch below (next to the MFMAs above) rather
    // than let it sink into the common path after it
    asm volatile("" ::"v"(pop[0].x), "v"(pop[0].y), "v"(pop[0].z), "v"(pop[0].w),
                 "v"(pop[1].x), "v"(pop[1].y), "v"(pop[1].z), "v"(pop[1].w),
                 "v"(pop[2].x), "v"(pop[2].y), "v"(pop[2].z), "v"(pop[2].w),
                 "v"(pop[3].x), "v"(pop[3].y), "v"(pop[3].z), "v"(pop[3].w), "v"(ps));

    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, cur.s[mt][i]);
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                       false, false);
      mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));  // max over lanes l, l^32
    }
    const bool moved = m == -INFINITY ? mx != -INFINITY : (mx - m) * scale_log2 > 8.f;
    if (__ballot(moved)) {  // rare: new base for the rows that moved, weights again
      const float mn = moved ? mx : m;
      const float nms = mn == -INFINITY ? 0.f : -mn * scale_log2;
      const float alpha = moved ? __builtin_amdgcn_exp2f(fmaf(m, scale_log2, nms)) : 1.f;
      m = mn;
      weights(nms);
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < PS::DTILES; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[dt][i] *= alpha;
    }
    lsum += ps;
    // O^T += V^T P^T; operand j of half g in k-step kk = (mt, h) is key
    // 16 kk + 8 (j / 4) + 4 g + j % 4, matching the S^T accumulator order
    // The V^T operands are read kVAhead products ahead of their use, and the
    // order (reads first, then one product per pair of reads) is pinned, so
    // each product waits only for reads issued several products earlier.
    const unsigned char* vt_lds = smem + (2 + par) * PS::TILE;
    constexpr int NPV = 4 * PS::DTILES;  // products of this tile: (kk, dt), dt fastest
    constexpr int kVAhead = 3;
    auto vread = [&](int i) {
      const int kk = i / PS::DTILES, dt = i % PS::DTILES;
      const uint32_t rows = uint32_t(kk * 16 * PS::ROW);
      const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_v4i16_t*)(vt_lds + ((v_lo ^ (64u * dt)) + rows)));
      const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_v4i16_t*)(vt_lds + ((v_hi ^ (64u * dt)) + rows)));
      const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
      return make_uint4(l2.x, l2.y, h2.x, h2.y);
    };
    uint4 vop[NPV];
#pragma unroll
    for (int i = 0; i < kVAhead; ++i) vop[i] = vread(i);
#pragma unroll
    for (int i = 0; i < NPV; ++i) {
      if (i + kVAhead < NPV) vop[i + kVAhead] = vread(i + kVAhead);
      o[i % PS::DTILES] = mfma32(vop[i], pop[i / PS::DTILES], o[i % PS::DTILES]);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * kVAhead, 0);  // DS reads
#pragma unroll
    for (int i = 0; i < NPV - kVAhead; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kVAhead, 0);
  };

  // prologue: K(0), V(0), K(1) in flight, then the scores of tile 0
  Step st_a, st_b;
  {
    int32_t t0[NI], t1[NI];
    load_table(0, t0);
    if (n_ktiles > 1) load_table(1, t1);
    issue_tile(kpool, 0, t0, 0u);
    issue_tile(vpool, 0, t0, uint32_t(2 * PS::TILE));
    if (n_ktiles > 1) issue_tile(kpool, 1, t1, uint32_t(PS::TILE));
  }
  if (n_ktiles > 2) load_table(2, st_a.tk);
  if (n_ktiles > 1) load_table(1, st_a.tv);
  drain_and_barrier();
  if (wave_active) qk(0u, st_a.s);
  for (int kt = 0; kt < n_ktiles; kt += 2) {
    step(kt, 0, st_a, st_b);
    if (kt + 1 < n_ktiles) step(kt + 1, 1, st_b, st_a);
  }

  if (!wave_active || my_pos < 0) return;
  const auto lsw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lsum), __float_as_uint(lsum),
                                                    false, false);
  const float l_row = __uint_as_float(lsw[0]) + __uint_as_float(lsw[1]);  // lanes l and l^32
  const float inv = 1.f / l_row;
  uint2* orow = reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) +
                                         (int64_t(q0 + my_row) * Hq + head) * D);
#pragma unroll
  for (int dt = 0; dt < PS::DTILES; ++dt)
#pragma unroll
    for (int bq = 0; bq < 4; ++bq) {
      const int d0 = dt * 32 + 8 * bq + 4 * g;
      orow[d0 / 4] = make_uint2(pack_bf16(o[dt][4 * bq] * inv, o[dt][4 * bq + 1] * inv),
                                pack_bf16(o[dt][4 * bq + 2] * inv, o[dt][4 * bq + 3] * inv));
    }
}

int gcd_pos(int x, int y) {
  while (y) {
    const int t = x % y;
    x = y;
    y = t;
  }
  return x;
}

}  // namespace

bool prefill_supported(int dtype, int head_dim, int block_size, int group) {
  return dtype == PA_BF16 && (head_dim == 64 || head_dim == 128) && block_size >= 1 && group >= 1;
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t st) {
  int b_shift = 0;
  while ((1 << b_shift) < a.block_size) ++b_shift;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int hpg = gcd_pos(G, kWaves);       // query heads per workgroup
  const int n_hchunk = G / hpg;
  const int rows_per_wg = (kWaves / hpg) * kRows;
  const int n_rtiles = (a.max_q_len + rows_per_wg - 1) / rows_per_wg;
  // deal (sequence, KV head) groups to the XCDs; split groups when there are
  // too few of them to give every XCD several chunks
  const int64_t n_groups = int64_t(a.num_seqs) * a.num_kv_heads;
  const int gs = n_hchunk * n_rtiles;
  int split = 1;
  while (n_groups * split < 4 * kXcds && split < gs) split *= 2;
  const int chunk_wgs = (gs + split - 1) / split;
  const int chunks_per_group = (gs + chunk_wgs - 1) / chunk_wgs;
  const int64_t n_chunks = n_groups * chunks_per_group;
  const int64_t blocks = (n_chunks + kXcds - 1) / kXcds * kXcds * chunk_wgs;
  if (n_groups <= 0 || gs <= 0 || blocks > 0x7fffffff) return hipErrorInvalidValue;
  const float scale_log2 = a.scale * kLog2e;
  const bool wave_block = b_shift >= 4;
  const dim3 grid{unsigned(blocks)}, block{unsigned(kWave * kWaves)};
  if (a.head_dim == 128) {
    constexpr int lds = PrefillShape<128>::LDS;
    if (wave_block)
      prefill_kernel<128, true><<<grid, block, lds, st>>>(a, b_shift, hpg, n_hchunk, n_rtiles, chunk_wgs, chunks_per_group, scale_log2);
    else
      prefill_kernel<128, false><<<grid, block, lds, st>>>(a, b_shift, hpg, n_hchunk, n_rtiles, chunk_wgs, chunks_per_group, scale_log2);
  } else if (a.head_dim == 64) {
    constexpr int lds = PrefillShape<64>::LDS;
    if (wave_block)
      prefill_kernel<64, true><<<grid, block, lds, st>>>(a, b_shift, hpg, n_hchunk, n_rtiles, chunk_wgs, chunks_per_group, scale_log2);
    else
      prefill_kernel<64, false><<<grid, block, lds, st>>>(a, b_shift, hpg, n_hchunk, n_rtiles, chunk_wgs, chunks_per_group, scale_log2);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa
