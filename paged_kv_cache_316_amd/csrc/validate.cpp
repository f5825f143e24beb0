// Host-side checks of the preconditions that the device calls cannot check
// themselves: the contents of block tables, lengths, slots, copy pairs and
// chunk offsets, which live in device memory during a call. Also the host
// helper that finds the blocks a group of sequences shares. A caller (or a
// debug mode of a binding) copies those arrays to the host and passes them
// here before launching; every function reports the first violation it finds
// through pa_last_error() and returns PA_ERR_INVALID. Plain host C++.
//
// What is checked follows the slot rule and the block-table reading of the
// attention calls ("LLM inference engine internals", section 2.3: slot =
// block * B + offset; "Why PagedAttention multiplies LLM serving throughput",
// section "Block Table: the GPU page table": logical block j of a sequence is
// its table entry j).
#include <algorithm>
#include <cstdint>
#include <utility>
#include <vector>

#include "pagedkv.h"
#include "status.h"

using pa::fail;

namespace {

pa_status check_geometry(const pa_pool* p, const char* who) {
  if (!p) return fail(PA_ERR_INVALID, "%s: pool is NULL", who);
  if (p->num_blocks <= 0) return fail(PA_ERR_INVALID, "%s: num_blocks=%d", who, p->num_blocks);
  if (p->block_size <= 0 || (p->block_size & (p->block_size - 1)))
    return fail(PA_ERR_INVALID, "%s: block_size=%d is not a power of two", who, p->block_size);
  return PA_OK;
}

}  // namespace

extern "C" {

pa_status pa_check_batch(const pa_pool* pool, const int32_t* block_tables,
                         int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t num_seqs) {
  pa::clear_error();
  const char* who = "pa_check_batch";
  if (pa_status s = check_geometry(pool, who)) return s;
  if (num_seqs < 0 || max_blocks_per_seq <= 0)
    return fail(PA_ERR_INVALID, "%s: num_seqs=%d max_blocks_per_seq=%d", who, num_seqs,
                max_blocks_per_seq);
  if (num_seqs == 0) return PA_OK;
  if (!block_tables || !seq_lens) return fail(PA_ERR_INVALID, "%s: NULL array", who);
  const int64_t B = pool->block_size;
  const int64_t cap = int64_t(max_blocks_per_seq) * B;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int32_t L = seq_lens[s];
    if (L < 0 || L > cap)
      return fail(PA_ERR_INVALID, "%s: seq_lens[%d]=%d outside [0, max_blocks_per_seq * B = %lld]",
                  who, s, L, static_cast<long long>(cap));
    const int64_t nblk = (L + B - 1) / B;
    const int32_t* row = block_tables + int64_t(s) * max_blocks_per_seq;
    for (int64_t j = 0; j < nblk; ++j)
      if (row[j] < 0 || row[j] >= pool->num_blocks)
        return fail(PA_ERR_INVALID, "%s: block_tables[%d][%lld]=%d outside the pool of %d blocks",
                    who, s, static_cast<long long>(j), row[j], pool->num_blocks);
  }
  return PA_OK;
}

pa_status pa_check_slots(const pa_pool* pool, const int64_t* slot_mapping, int32_t num_tokens) {
  pa::clear_error();
  const char* who = "pa_check_slots";
  if (pa_status s = check_geometry(pool, who)) return s;
  if (num_tokens < 0) return fail(PA_ERR_INVALID, "%s: num_tokens=%d", who, num_tokens);
  if (num_tokens == 0) return PA_OK;
  if (!slot_mapping) return fail(PA_ERR_INVALID, "%s: slot_mapping is NULL", who);
  const int64_t n_slots = int64_t(pool->num_blocks) * pool->block_size;
  // (slot, token) of every written token, sorted: a slot named twice shows up
  // as two neighbours (memory and time follow the tokens, not the pool)
  std::vector<std::pair<int64_t, int32_t>> named;
  named.reserve(size_t(num_tokens));
  for (int32_t t = 0; t < num_tokens; ++t) {
    const int64_t slot = slot_mapping[t];
    if (slot < 0) continue;  // padding: skipped by the write
    if (slot >= n_slots)
      return fail(PA_ERR_INVALID, "%s: slot_mapping[%d]=%lld >= num_blocks * B = %lld", who, t,
                  static_cast<long long>(slot), static_cast<long long>(n_slots));
    named.emplace_back(slot, t);
  }
  std::sort(named.begin(), named.end());
  for (size_t i = 1; i < named.size(); ++i)
    if (named[i].first == named[i - 1].first)
      return fail(PA_ERR_INVALID, "%s: slot %lld named by tokens %d and %d", who,
                  static_cast<long long>(named[i].first), named[i - 1].second, named[i].second);
  return PA_OK;
}

pa_status pa_check_copies(const pa_pool* pool, const int32_t* src_dst, int32_t num_pairs) {
  pa::clear_error();
  const char* who = "pa_check_copies";
  if (pa_status s = check_geometry(pool, who)) return s;
  if (num_pairs < 0) return fail(PA_ERR_INVALID, "%s: num_pairs=%d", who, num_pairs);
  if (num_pairs == 0) return PA_OK;
  if (!src_dst) return fail(PA_ERR_INVALID, "%s: src_dst is NULL", who);
  // 1 = read by a pair, 2 = written by a pair
  std::vector<unsigned char> role(size_t(pool->num_blocks), 0);
  for (int32_t i = 0; i < num_pairs; ++i) {
    const int32_t s = src_dst[2 * i], d = src_dst[2 * i + 1];
    if (s < 0 || s >= pool->num_blocks || d < 0 || d >= pool->num_blocks)
      return fail(PA_ERR_INVALID, "%s: pair %d = (%d, %d) outside the pool of %d blocks", who, i,
                  s, d, pool->num_blocks);
    if (role[size_t(d)] == 2)
      return fail(PA_ERR_INVALID, "%s: block %d is the destination of two pairs", who, d);
    if (role[size_t(d)] == 1 || role[size_t(s)] == 2 || s == d)
      return fail(PA_ERR_INVALID, "%s: pair %d = (%d, %d): a block is both a source and a "
                  "destination", who, i, s, d);
    role[size_t(s)] = 1;
    role[size_t(d)] = 2;
  }
  return PA_OK;
}

pa_status pa_check_chunks(const int32_t* q_start_loc, const int32_t* seq_lens, int32_t num_seqs,
                          int32_t num_decode, int32_t max_q_len, int64_t total_rows) {
  pa::clear_error();
  const char* who = "pa_check_chunks";
  if (num_seqs < 0 || num_decode < 0 || num_decode > num_seqs || max_q_len < 0 || total_rows < 0)
    return fail(PA_ERR_INVALID, "%s: num_seqs=%d num_decode=%d max_q_len=%d total_rows=%lld", who,
                num_seqs, num_decode, max_q_len, static_cast<long long>(total_rows));
  if (num_seqs == 0) return PA_OK;
  if (!q_start_loc || !seq_lens) return fail(PA_ERR_INVALID, "%s: NULL array", who);
  if (q_start_loc[0] != 0) return fail(PA_ERR_INVALID, "%s: q_start_loc[0]=%d, not 0", who, q_start_loc[0]);
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int64_t q_len = int64_t(q_start_loc[s + 1]) - q_start_loc[s];
    if (seq_lens[s] < 0) return fail(PA_ERR_INVALID, "%s: seq_lens[%d]=%d < 0", who, s, seq_lens[s]);
    if (s < num_decode) {
      if (q_len != 1)
        return fail(PA_ERR_INVALID, "%s: decode sequence %d has %lld rows, not 1", who, s,
                    static_cast<long long>(q_len));
      continue;
    }
    if (q_len < 0)
      return fail(PA_ERR_INVALID, "%s: q_start_loc decreases at sequence %d", who, s);
    if (q_len > max_q_len)
      return fail(PA_ERR_INVALID, "%s: chunk of sequence %d has %lld rows > max_q_len=%d", who, s,
                  static_cast<long long>(q_len), max_q_len);
    if (q_len > seq_lens[s])
      return fail(PA_ERR_INVALID, "%s: chunk of sequence %d has %lld rows but seq_lens=%d (its "
                  "rows must already be in the pool)", who, s, static_cast<long long>(q_len),
                  seq_lens[s]);
  }
  if (q_start_loc[num_seqs] > total_rows)
    return fail(PA_ERR_INVALID, "%s: q_start_loc[%d]=%d beyond the %lld rows of q", who, num_seqs,
                q_start_loc[num_seqs], static_cast<long long>(total_rows));
  return PA_OK;
}

pa_status pa_check_shared_prefix(const pa_pool* pool, const int32_t* block_tables,
                                 int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                 int32_t num_seqs, int32_t num_prefix_blocks) {
  if (pa_status s = pa_check_batch(pool, block_tables, max_blocks_per_seq, seq_lens, num_seqs))
    return s;
  const char* who = "pa_check_shared_prefix";
  if (num_prefix_blocks < 0 || num_prefix_blocks > max_blocks_per_seq)
    return fail(PA_ERR_INVALID, "%s: num_prefix_blocks=%d outside [0, %d]", who, num_prefix_blocks,
                max_blocks_per_seq);
  const int64_t need = int64_t(num_prefix_blocks) * pool->block_size;
  for (int32_t s = 0; s < num_seqs; ++s) {
    if (seq_lens[s] < need)
      return fail(PA_ERR_INVALID, "%s: seq_lens[%d]=%d shorter than the %lld shared tokens", who,
                  s, seq_lens[s], static_cast<long long>(need));
    const int32_t* row = block_tables + int64_t(s) * max_blocks_per_seq;
    for (int32_t j = 0; j < num_prefix_blocks; ++j)
      if (row[j] != block_tables[j])
        return fail(PA_ERR_INVALID, "%s: block_tables[%d][%d]=%d differs from row 0 (%d)", who, s,
                    j, row[j], block_tables[j]);
  }
  return PA_OK;
}

pa_status pa_group_prefix_lens(const int32_t* block_tables, int32_t max_blocks_per_seq,
                               const int32_t* seq_lens, int32_t num_seqs, int32_t group_size,
                               int32_t block_size, int32_t* prefix_lens) {
  pa::clear_error();
  const char* who = "pa_group_prefix_lens";
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || group_size < 1 || block_size <= 0 ||
      num_seqs % group_size)
    return fail(PA_ERR_INVALID, "%s: num_seqs=%d max_blocks_per_seq=%d group_size=%d "
                "block_size=%d", who, num_seqs, max_blocks_per_seq, group_size, block_size);
  if (num_seqs == 0) return PA_OK;
  if (!block_tables || !seq_lens || !prefix_lens) return fail(PA_ERR_INVALID, "%s: NULL array", who);
  for (int32_t s0 = 0; s0 < num_seqs; s0 += group_size) {
    // blocks full in every member
    int64_t full = max_blocks_per_seq;
    for (int32_t m = 0; m < group_size; ++m) {
      const int32_t L = seq_lens[s0 + m];
      if (L < 0) return fail(PA_ERR_INVALID, "%s: seq_lens[%d]=%d < 0", who, s0 + m, L);
      full = std::min<int64_t>(full, L / block_size);
    }
    const int32_t* r0 = block_tables + int64_t(s0) * max_blocks_per_seq;
    int64_t j = 0;
    for (; j < full; ++j) {
      bool same = true;
      for (int32_t m = 1; m < group_size && same; ++m)
        same = block_tables[int64_t(s0 + m) * max_blocks_per_seq + j] == r0[j];
      if (!same) break;
    }
    for (int32_t m = 0; m < group_size; ++m) prefix_lens[s0 + m] = int32_t(j * block_size);
  }
  return PA_OK;
}

pa_status pa_check_grouped(const pa_pool* pool, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, const int32_t* seq_lens,
                           const int32_t* prefix_lens, int32_t num_seqs, int32_t group_size) {
  if (pa_status s = pa_check_batch(pool, block_tables, max_blocks_per_seq, seq_lens, num_seqs))
    return s;
  const char* who = "pa_check_grouped";
  if (group_size < 1 || num_seqs % group_size)
    return fail(PA_ERR_INVALID, "%s: num_seqs=%d is not a multiple of group_size=%d", who,
                num_seqs, group_size);
  if (num_seqs > 0 && !prefix_lens) return fail(PA_ERR_INVALID, "%s: prefix_lens is NULL", who);
  const int32_t B = pool->block_size;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int32_t s0 = s - s % group_size;
    const int32_t P = prefix_lens[s];
    if (P < 0 || P % B || P > seq_lens[s])
      return fail(PA_ERR_INVALID, "%s: prefix_lens[%d]=%d is not a multiple of B=%d in [0, "
                  "seq_lens=%d]", who, s, P, B, seq_lens[s]);
    if (P != prefix_lens[s0])
      return fail(PA_ERR_INVALID, "%s: prefix_lens[%d]=%d differs from its group's first "
                  "member (%d)", who, s, P, prefix_lens[s0]);
    const int32_t* row = block_tables + int64_t(s) * max_blocks_per_seq;
    const int32_t* r0 = block_tables + int64_t(s0) * max_blocks_per_seq;
    for (int32_t j = 0; j < P / B; ++j)
      if (row[j] != r0[j])
        return fail(PA_ERR_INVALID, "%s: block_tables[%d][%d]=%d differs from its group's "
                    "first member (%d) inside the shared prefix", who, s, j, row[j], r0[j]);
  }
  return PA_OK;
}

}  // extern "C"
