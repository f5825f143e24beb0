// Host block allocator: free list, reference counts, fork + copy-on-write,
// hash-based prefix sharing. Produces block tables, slots and block copies;
// touches no device memory.
//
// Rules (each from the pages):
//  - FIFO free list, take from the front, return to the back; ceil(n/B) blocks
//    for an n-token prompt; append_slot gives last*B + n%B while the last block
//    has room, else takes a new block, and reports out-of-memory without
//    changing state ("LLM inference engine internals", section 2.3).
//  - Reference counts, fork, copy-on-write of a shared partially filled last
//    block on append; release in table order, a block returns to the free list
//    when its count reaches zero ("vLLM PagedAttention explained", sections
//    4.1 and 4.2).
//  - Prefix sharing by a hash of (previous block's hash, block tokens)
//    ("Why PagedAttention multiplies LLM serving throughput", section
//    "Automatic prefix caching"). Readings where the pages are silent: 64-bit
//    FNV-1a over the previous hash (8 bytes little-endian, 0 before the first
//    block) then the int32 tokens (4 bytes little-endian each); a hit also
//    compares the stored tokens; only full blocks laid down by allocate are
//    registered, the first registration of a hash wins, and an entry is
//    dropped when its block's count reaches zero.
#include <cstdint>
#include <cstring>
#include <deque>
#include <new>
#include <unordered_map>
#include <utility>
#include <vector>

#include "pagedkv.h"
#include "status.h"

namespace {

constexpr uint64_t kFnvOffset = 0xcbf29ce484222325ull;
constexpr uint64_t kFnvPrime = 0x100000001b3ull;

uint64_t fnv1a_bytes(uint64_t h, const uint8_t* p, size_t n) {
  for (size_t i = 0; i < n; ++i) {
    h ^= p[i];
    h *= kFnvPrime;
  }
  return h;
}

uint64_t chain_hash(uint64_t prev, const int32_t* tok, int32_t B) {
  uint8_t buf[8];
  for (int i = 0; i < 8; ++i) buf[i] = uint8_t(prev >> (8 * i));
  uint64_t h = fnv1a_bytes(kFnvOffset, buf, 8);
  for (int32_t j = 0; j < B; ++j) {
    uint32_t t = uint32_t(tok[j]);
    uint8_t b4[4] = {uint8_t(t), uint8_t(t >> 8), uint8_t(t >> 16), uint8_t(t >> 24)};
    h = fnv1a_bytes(h, b4, 4);
  }
  return h;
}

struct Seq {
  std::vector<int32_t> table;
  int32_t len = 0;
};

}  // namespace

struct pa_alloc {
  int32_t num_blocks = 0, B = 0;
  std::deque<int32_t> free_list;
  std::vector<int32_t> ref;
  std::unordered_map<int64_t, Seq> seqs;
  std::unordered_map<uint64_t, int32_t> block_of_hash;
  std::vector<uint64_t> hash_of_block;          // valid where registered[b]
  std::vector<uint8_t> registered;
  std::vector<std::vector<int32_t>> tokens_of_block;
  std::vector<std::pair<int32_t, int32_t>> copies;

  int32_t take_block() {
    int32_t b = free_list.front();
    free_list.pop_front();
    ref[b] = 1;
    return b;
  }
};

extern "C" {

pa_status pa_alloc_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                          pa_alloc** out) {
  pa::clear_error();
  if (!out) return pa::fail(PA_ERR_INVALID, "pa_alloc_create: out is NULL");
  *out = nullptr;
  if (num_blocks <= 0 || block_size <= 0)
    return pa::fail(PA_ERR_INVALID, "pa_alloc_create: num_blocks=%d block_size=%d must be > 0",
                    num_blocks, block_size);
  pa_alloc* a = new (std::nothrow) pa_alloc();
  if (!a) return pa::fail(PA_ERR_OOM, "pa_alloc_create: host allocation failed");
  a->num_blocks = num_blocks;
  a->B = block_size;
  a->ref.assign(num_blocks, 0);
  a->hash_of_block.assign(num_blocks, 0);
  a->registered.assign(num_blocks, 0);
  a->tokens_of_block.resize(num_blocks);
  if (free_order) {
    std::vector<uint8_t> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      int32_t b = free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete a;
        return pa::fail(PA_ERR_INVALID, "pa_alloc_create: free_order is not a permutation (entry %d = %d)",
                        i, b);
      }
      seen[b] = 1;
      a->free_list.push_back(b);
    }
  } else {
    for (int32_t b = 0; b < num_blocks; ++b) a->free_list.push_back(b);
  }
  *out = a;
  return PA_OK;
}

void pa_alloc_destroy(pa_alloc* a) { delete a; }

pa_status pa_alloc_allocate(pa_alloc* a, int64_t seq_id, const int32_t* tokens, int32_t n,
                            int32_t* cached_out, int64_t* slots_out) {
  pa::clear_error();
  if (!a || n < 0 || (n > 0 && !tokens))
    return pa::fail(PA_ERR_INVALID, "pa_alloc_allocate: bad arguments");
  if (a->seqs.count(seq_id))
    return pa::fail(PA_ERR_STATE, "pa_alloc_allocate: sequence %lld already exists",
                    (long long)seq_id);
  const int32_t B = a->B;
  const int32_t nblk = (n + B - 1) / B, nfull = n / B;
  std::vector<uint64_t> hashes(nfull);
  uint64_t prev = 0;
  for (int32_t j = 0; j < nfull; ++j) hashes[j] = prev = chain_hash(prev, tokens + j * B, B);
  int32_t hits = 0;
  for (; hits < nfull; ++hits) {
    auto it = a->block_of_hash.find(hashes[hits]);
    if (it == a->block_of_hash.end()) break;
    const auto& stored = a->tokens_of_block[it->second];
    if (std::memcmp(stored.data(), tokens + hits * B, sizeof(int32_t) * B) != 0) break;
  }
  if (size_t(nblk - hits) > a->free_list.size())
    return pa::fail(PA_ERR_OOM, "pa_alloc_allocate: need %d blocks, %zu free", nblk - hits,
                    a->free_list.size());
  Seq s;
  s.table.reserve(nblk);
  for (int32_t j = 0; j < hits; ++j) {
    int32_t b = a->block_of_hash[hashes[j]];
    a->ref[b] += 1;
    s.table.push_back(b);
  }
  for (int32_t j = hits; j < nblk; ++j) {
    int32_t b = a->take_block();
    s.table.push_back(b);
    if (j < nfull && !a->block_of_hash.count(hashes[j])) {
      a->block_of_hash[hashes[j]] = b;
      a->hash_of_block[b] = hashes[j];
      a->registered[b] = 1;
      a->tokens_of_block[b].assign(tokens + j * B, tokens + (j + 1) * B);
    }
  }
  s.len = n;
  if (slots_out)
    for (int32_t t = 0; t < n; ++t) slots_out[t] = int64_t(s.table[t / B]) * B + t % B;
  a->seqs.emplace(seq_id, std::move(s));
  if (cached_out) *cached_out = hits * B;
  return PA_OK;
}

static pa_status append_one(pa_alloc* a, Seq& s, int64_t* slot_out) {
  const int32_t B = a->B, L = s.len;
  int64_t slot;
  if (L % B) {
    int32_t last = s.table.back();
    if (a->ref[last] > 1) {  // shared partial last block: copy on write
      if (a->free_list.empty()) return pa::fail(PA_ERR_OOM, "append: no free block for copy-on-write");
      int32_t nb = a->take_block();
      a->ref[last] -= 1;
      s.table.back() = nb;
      a->copies.emplace_back(last, nb);
      slot = int64_t(nb) * B + L % B;
    } else {
      slot = int64_t(last) * B + L % B;
    }
  } else {
    if (a->free_list.empty()) return pa::fail(PA_ERR_OOM, "append: no free block");
    int32_t nb = a->take_block();
    s.table.push_back(nb);
    slot = int64_t(nb) * B;
  }
  s.len = L + 1;
  if (slot_out) *slot_out = slot;
  return PA_OK;
}

pa_status pa_alloc_append_slot(pa_alloc* a, int64_t seq_id, int32_t token, int64_t* slot_out) {
  (void)token;
  pa::clear_error();
  if (!a) return pa::fail(PA_ERR_INVALID, "pa_alloc_append_slot: allocator is NULL");
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end())
    return pa::fail(PA_ERR_STATE, "pa_alloc_append_slot: unknown sequence %lld", (long long)seq_id);
  return append_one(a, it->second, slot_out);
}

pa_status pa_alloc_extend(pa_alloc* a, int64_t seq_id, const int32_t* tokens, int32_t n,
                          int64_t* slots_out) {
  (void)tokens;
  pa::clear_error();
  if (!a || n < 0) return pa::fail(PA_ERR_INVALID, "pa_alloc_extend: bad arguments");
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end())
    return pa::fail(PA_ERR_STATE, "pa_alloc_extend: unknown sequence %lld", (long long)seq_id);
  Seq& s = it->second;
  const int32_t B = a->B, L = s.len;
  int64_t need = (int64_t(L) + n + B - 1) / B - (int64_t(L) + B - 1) / B;
  if (n > 0 && L % B && a->ref[s.table.back()] > 1) need += 1;
  if (need > int64_t(a->free_list.size()))
    return pa::fail(PA_ERR_OOM, "pa_alloc_extend: need %lld blocks, %zu free", (long long)need,
                    a->free_list.size());
  for (int32_t i = 0; i < n; ++i) append_one(a, s, slots_out ? slots_out + i : nullptr);
  return PA_OK;
}

pa_status pa_alloc_fork(pa_alloc* a, int64_t parent, int64_t child) {
  pa::clear_error();
  if (!a) return pa::fail(PA_ERR_INVALID, "pa_alloc_fork: allocator is NULL");
  auto it = a->seqs.find(parent);
  if (it == a->seqs.end())
    return pa::fail(PA_ERR_STATE, "pa_alloc_fork: unknown parent %lld", (long long)parent);
  if (a->seqs.count(child))
    return pa::fail(PA_ERR_STATE, "pa_alloc_fork: child %lld already exists", (long long)child);
  Seq c = it->second;
  for (int32_t b : c.table) a->ref[b] += 1;
  a->seqs.emplace(child, std::move(c));
  return PA_OK;
}

pa_status pa_alloc_free(pa_alloc* a, int64_t seq_id) {
  pa::clear_error();
  if (!a) return pa::fail(PA_ERR_INVALID, "pa_alloc_free: allocator is NULL");
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end())
    return pa::fail(PA_ERR_STATE, "pa_alloc_free: unknown sequence %lld", (long long)seq_id);
  for (int32_t b : it->second.table) {
    if (--a->ref[b] == 0) {
      a->free_list.push_back(b);
      if (a->registered[b]) {
        a->block_of_hash.erase(a->hash_of_block[b]);
        a->registered[b] = 0;
        a->tokens_of_block[b].clear();
      }
    }
  }
  a->seqs.erase(it);
  return PA_OK;
}

pa_status pa_alloc_take_copies(pa_alloc* a, int32_t* src_dst, int32_t cap, int32_t* n_out) {
  pa::clear_error();
  if (!a || !n_out || cap < 0) return pa::fail(PA_ERR_INVALID, "pa_alloc_take_copies: bad arguments");
  int32_t n = int32_t(a->copies.size());
  *n_out = n;
  if (n > cap) return pa::fail(PA_ERR_INVALID, "pa_alloc_take_copies: %d copies queued, cap %d", n, cap);
  if (n > 0 && !src_dst) return pa::fail(PA_ERR_INVALID, "pa_alloc_take_copies: src_dst is NULL");
  for (int32_t i = 0; i < n; ++i) {
    src_dst[2 * i] = a->copies[i].first;
    src_dst[2 * i + 1] = a->copies[i].second;
  }
  a->copies.clear();
  return PA_OK;
}

pa_status pa_alloc_block_table(const pa_alloc* a, int64_t seq_id, int32_t* out, int32_t cap,
                               int32_t* n_out) {
  pa::clear_error();
  if (!a || !n_out || cap < 0) return pa::fail(PA_ERR_INVALID, "pa_alloc_block_table: bad arguments");
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end())
    return pa::fail(PA_ERR_STATE, "pa_alloc_block_table: unknown sequence %lld", (long long)seq_id);
  const auto& t = it->second.table;
  *n_out = int32_t(t.size());
  if (int32_t(t.size()) > cap)
    return pa::fail(PA_ERR_INVALID, "pa_alloc_block_table: table has %zu entries, cap %d", t.size(), cap);
  if (!t.empty() && !out) return pa::fail(PA_ERR_INVALID, "pa_alloc_block_table: out is NULL");
  for (size_t i = 0; i < t.size(); ++i) out[i] = t[i];
  return PA_OK;
}

pa_status pa_alloc_seq_len(const pa_alloc* a, int64_t seq_id, int32_t* len_out) {
  pa::clear_error();
  if (!a || !len_out) return pa::fail(PA_ERR_INVALID, "pa_alloc_seq_len: bad arguments");
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end())
    return pa::fail(PA_ERR_STATE, "pa_alloc_seq_len: unknown sequence %lld", (long long)seq_id);
  *len_out = it->second.len;
  return PA_OK;
}

pa_status pa_alloc_batch_tables(const pa_alloc* a, const int64_t* seq_ids, int32_t n,
                                int32_t* tables, int32_t max_blocks, int32_t* seq_lens) {
  pa::clear_error();
  if (!a || n < 0 || max_blocks < 0 || (n > 0 && (!seq_ids || !tables || !seq_lens)))
    return pa::fail(PA_ERR_INVALID, "pa_alloc_batch_tables: bad arguments");
  for (int32_t i = 0; i < n; ++i) {  // validate everything before writing
    auto it = a->seqs.find(seq_ids[i]);
    if (it == a->seqs.end())
      return pa::fail(PA_ERR_STATE, "pa_alloc_batch_tables: unknown sequence %lld",
                      (long long)seq_ids[i]);
    if (int32_t(it->second.table.size()) > max_blocks)
      return pa::fail(PA_ERR_INVALID, "pa_alloc_batch_tables: sequence %lld has %zu blocks > %d",
                      (long long)seq_ids[i], it->second.table.size(), max_blocks);
  }
  for (int32_t i = 0; i < n; ++i) {
    const Seq& s = a->seqs.find(seq_ids[i])->second;
    int32_t* row = tables + int64_t(i) * max_blocks;
    size_t k = 0;
    for (; k < s.table.size(); ++k) row[k] = s.table[k];
    for (; k < size_t(max_blocks); ++k) row[k] = 0;
    seq_lens[i] = s.len;
  }
  return PA_OK;
}

int32_t pa_alloc_num_free(const pa_alloc* a) { return a ? int32_t(a->free_list.size()) : -1; }

pa_status pa_alloc_ref_count(const pa_alloc* a, int32_t block, int32_t* out) {
  pa::clear_error();
  if (!a || !out || block < 0 || block >= a->num_blocks)
    return pa::fail(PA_ERR_INVALID, "pa_alloc_ref_count: bad arguments");
  *out = a->ref[block];
  return PA_OK;
}

}  // extern "C"
