// Host cache manager: block allocator, per-sequence block tables, slot mapping, shared blocks.
//
// The pool is a set of fixed-size physical blocks; a sequence lists the blocks it owns in order (its block
// table) and takes one more block when its last one is full, without moving data ("Paged Attention 基础 –
// 原理与实现进度", §1 problems 1-2; §3.1 A: block allocator, block table, slot mapping).  Several tables
// may list the same block (§1 problem 3, the §2 figure's block 7): sharing is counted by references, and
// a write into a shared, partly filled last block first copies it (copy on write).  One append call covers
// a fresh sequence and an extension; tables are kept per sequence id and released by free; prefixes are
// registered and reused by key (ADR 004 "Paged Attention Serving Integration", Decision 5 and
// Consequences: update, free(seq_id), add_prefix / try_get_prefix_blocks).
//
// Allocation takes the lowest-numbered free block, so the allocation sequence is a pure function of the
// calls.  Every call either completes or changes nothing.  Not thread-safe: one manager per thread, or
// external locking.
#include <cstdint>
#include <map>
#include <set>
#include <string>
#include <unordered_map>
#include <vector>

#include "host_status.h"
#include "paged_kv.h"

struct pkv_cache_manager {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> ref;   // references per block (sequences and prefixes listing it)
  std::set<int32_t> free;     // blocks with no reference, lowest first
  struct Seq {
    std::vector<int32_t> blocks;
    int32_t len = 0;
  };
  std::unordered_map<int64_t, Seq> seqs;
  struct Prefix {
    std::vector<int32_t> blocks;
    int32_t tokens = 0;
  };
  std::unordered_map<uint64_t, Prefix> prefixes;

  int32_t take() {
    const int32_t b = *free.begin();
    free.erase(free.begin());
    ref[b] = 1;
    return b;
  }
  void release(int32_t b) {
    if (--ref[b] == 0) free.insert(b);
  }
};

namespace {

using pkv::host_fail;
using pkv::host_ok;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

extern "C" {

pkv_cache_manager* pkv_cm_create(int32_t num_blocks, int32_t block_size) {
  if (num_blocks < 1 || block_size < 1) {
    host_fail(PKV_ERR_INVALID_ARG, "num_blocks and block_size must be >= 1");
    return nullptr;
  }
  if (static_cast<int64_t>(num_blocks) * block_size > INT32_MAX) {
    host_fail(PKV_ERR_UNSUPPORTED, "num_blocks * block_size must be < 2^31 (slots are int32)");
    return nullptr;
  }
  auto* m = new pkv_cache_manager;
  m->num_blocks = num_blocks;
  m->block_size = block_size;
  m->ref.assign(num_blocks, 0);
  for (int32_t b = 0; b < num_blocks; ++b) m->free.insert(m->free.end(), b);
  host_ok();
  return m;
}

void pkv_cm_destroy(pkv_cache_manager* m) { delete m; }

int32_t pkv_cm_num_free(const pkv_cache_manager* m) {
  return m ? static_cast<int32_t>(m->free.size()) : -1;
}

int32_t pkv_cm_seq_len(const pkv_cache_manager* m, int64_t seq_id) {
  if (!m) return -1;
  const auto it = m->seqs.find(seq_id);
  return it == m->seqs.end() ? -1 : it->second.len;
}

int pkv_cm_append(pkv_cache_manager* m, int64_t seq_id, int32_t num_tokens, int32_t* slots_out,
                  int32_t* cow_out) {
  if (!m || !cow_out || num_tokens < 0 || (num_tokens > 0 && !slots_out))
    return host_fail(PKV_ERR_INVALID_ARG, "append needs a manager, cow_out[2], num_tokens >= 0 and slots_out");
  const auto it = m->seqs.find(seq_id);
  const pkv_cache_manager::Seq empty;
  const pkv_cache_manager::Seq& cur = it == m->seqs.end() ? empty : it->second;
  const int64_t bs = m->block_size;
  if (static_cast<int64_t>(cur.len) + num_tokens > INT32_MAX)
    return host_fail(PKV_ERR_INVALID_ARG, "sequence length would exceed 2^31 - 1");
  const int64_t need = ceil_div(cur.len + static_cast<int64_t>(num_tokens), bs) -
                       static_cast<int64_t>(cur.blocks.size());
  const bool cow = num_tokens > 0 && cur.len % bs != 0 && m->ref[cur.blocks.back()] > 1;
  if (need + (cow ? 1 : 0) > static_cast<int64_t>(m->free.size()))
    return host_fail(PKV_ERR_NO_BLOCKS, "out of blocks: need " + std::to_string(need + (cow ? 1 : 0)) +
                                            ", free " + std::to_string(m->free.size()));
  pkv_cache_manager::Seq next = cur;
  cow_out[0] = cow_out[1] = -1;
  if (cow) {
    const int32_t src = next.blocks.back();
    const int32_t dst = m->take();
    m->release(src);
    next.blocks.back() = dst;
    cow_out[0] = src;
    cow_out[1] = dst;
  }
  for (int64_t i = 0; i < need; ++i) next.blocks.push_back(m->take());
  for (int32_t i = 0; i < num_tokens; ++i) {
    const int64_t pos = static_cast<int64_t>(cur.len) + i;
    slots_out[i] = static_cast<int32_t>(next.blocks[pos / bs] * bs + pos % bs);
  }
  next.len = cur.len + num_tokens;
  m->seqs[seq_id] = std::move(next);
  return host_ok();
}

int pkv_cm_free(pkv_cache_manager* m, int64_t seq_id) {
  if (!m) return host_fail(PKV_ERR_INVALID_ARG, "null manager");
  const auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return host_fail(PKV_ERR_INVALID_ARG, "unknown sequence " + std::to_string(seq_id));
  for (const int32_t b : it->second.blocks) m->release(b);
  m->seqs.erase(it);
  return host_ok();
}

int pkv_cm_fork(pkv_cache_manager* m, int64_t parent, int64_t child) {
  if (!m) return host_fail(PKV_ERR_INVALID_ARG, "null manager");
  const auto it = m->seqs.find(parent);
  if (it == m->seqs.end() || m->seqs.count(child))
    return host_fail(PKV_ERR_INVALID_ARG, "fork needs a known parent and a new child");
  for (const int32_t b : it->second.blocks) ++m->ref[b];
  const pkv_cache_manager::Seq copy = it->second;
  m->seqs[child] = copy;
  return host_ok();
}

int pkv_cm_add_prefix(pkv_cache_manager* m, uint64_t key, int64_t seq_id, int32_t num_tokens) {
  if (!m) return host_fail(PKV_ERR_INVALID_ARG, "null manager");
  const auto it = m->seqs.find(seq_id);
  if (m->prefixes.count(key) || it == m->seqs.end())
    return host_fail(PKV_ERR_INVALID_ARG, "prefix key taken or unknown sequence");
  if (num_tokens <= 0 || num_tokens > it->second.len)
    return host_fail(PKV_ERR_INVALID_ARG, "prefix length must be in [1, sequence length]");
  pkv_cache_manager::Prefix pre;
  pre.tokens = num_tokens;
  pre.blocks.assign(it->second.blocks.begin(), it->second.blocks.begin() + ceil_div(num_tokens, m->block_size));
  for (const int32_t b : pre.blocks) ++m->ref[b];
  m->prefixes[key] = std::move(pre);
  return host_ok();
}

int pkv_cm_attach_prefix(pkv_cache_manager* m, uint64_t key, int64_t seq_id, int32_t* tokens_out) {
  if (!m || !tokens_out) return host_fail(PKV_ERR_INVALID_ARG, "attach needs a manager and tokens_out");
  if (m->seqs.count(seq_id)) return host_fail(PKV_ERR_INVALID_ARG, "the sequence already exists");
  *tokens_out = 0;
  const auto it = m->prefixes.find(key);
  if (it == m->prefixes.end()) return host_ok();
  for (const int32_t b : it->second.blocks) ++m->ref[b];
  pkv_cache_manager::Seq seq;
  seq.blocks = it->second.blocks;
  seq.len = it->second.tokens;
  m->seqs[seq_id] = std::move(seq);
  *tokens_out = it->second.tokens;
  return host_ok();
}

int pkv_cm_drop_prefix(pkv_cache_manager* m, uint64_t key) {
  if (!m) return host_fail(PKV_ERR_INVALID_ARG, "null manager");
  const auto it = m->prefixes.find(key);
  if (it == m->prefixes.end()) return host_fail(PKV_ERR_INVALID_ARG, "unknown prefix key");
  for (const int32_t b : it->second.blocks) m->release(b);
  m->prefixes.erase(it);
  return host_ok();
}

int pkv_cm_build_tables(const pkv_cache_manager* m, const int64_t* seq_ids, int32_t num_seqs,
                        int32_t max_blocks_per_seq, int32_t* block_tables_out, int32_t* context_lens_out) {
  if (!m || num_seqs < 0 || max_blocks_per_seq < 1 ||
      (num_seqs > 0 && (!seq_ids || !block_tables_out || !context_lens_out)))
    return host_fail(PKV_ERR_INVALID_ARG, "build_tables needs a manager, seq_ids, outputs and max_blocks_per_seq >= 1");
  for (int32_t i = 0; i < num_seqs; ++i) {  // check everything before writing anything
    const auto it = m->seqs.find(seq_ids[i]);
    if (it == m->seqs.end()) return host_fail(PKV_ERR_INVALID_ARG, "unknown sequence " + std::to_string(seq_ids[i]));
    if (static_cast<int64_t>(it->second.blocks.size()) > max_blocks_per_seq)
      return host_fail(PKV_ERR_INVALID_ARG, "sequence " + std::to_string(seq_ids[i]) + " holds more blocks than a table row");
  }
  for (int32_t i = 0; i < num_seqs; ++i) {
    const pkv_cache_manager::Seq& seq = m->seqs.find(seq_ids[i])->second;
    int32_t* row = block_tables_out + static_cast<int64_t>(i) * max_blocks_per_seq;
    const int32_t nb = static_cast<int32_t>(seq.blocks.size());
    for (int32_t j = 0; j < max_blocks_per_seq; ++j) row[j] = j < nb ? seq.blocks[j] : -1;
    context_lens_out[i] = seq.len;
  }
  return host_ok();
}

}  // extern "C"
