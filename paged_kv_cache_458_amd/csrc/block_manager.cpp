// Host block manager of the paged KV cache (C ABI in include/paged_block_manager.h).
//
// vLLM PagedAttention, page 1 ("LLM inference framework evaluation ... PagedAttention"), section 3.2: the cache
// is a pool of fixed-size blocks; a sequence takes a new block only when a token needs one; freed blocks go
// back to the pool; sequences may share physical blocks, and a shared block is copied before it is written.
// Page 2 ("vLLM-v0.11.0 ... how much memory does PagedAttention save"), section 4.2: a sequence of length L
// holds ceil(L / block_size) blocks, and requests with the same prefix reuse the same blocks.
//
// Swap (page 1 section 5: swap space on the host; page 2 section 7.2: inactive blocks moved to host memory): a
// sequence can leave the device pool for blocks of a host pool and come back later into fresh device blocks.
//
// Host code only: it decides where tokens go; the kernels move the bytes.
#include <stdint.h>

#include <algorithm>
#include <new>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "../../include/pa.h"
#include "../../include/paged_block_manager.h"

namespace {

struct Sequence {
  std::vector<int32_t> blocks;  // physical blocks in logical order
  int64_t len = 0;              // tokens
};

// 64-bit FNV-1a over a block's predecessor id and its tokens: the key of the prefix-sharing index. Hits are
// confirmed by comparing the predecessor and the tokens themselves, so a collision never shares a block.
uint64_t block_key(int32_t parent, const int32_t* tokens, int32_t n) {
  uint64_t h = 1469598103934665603ull;
  auto mix = [&h](uint32_t v) {
    for (int i = 0; i < 4; ++i) {
      h ^= (v >> (8 * i)) & 0xffu;
      h *= 1099511628211ull;
    }
  };
  mix((uint32_t)parent);
  for (int32_t i = 0; i < n; ++i) mix((uint32_t)tokens[i]);
  return h;
}

}  // namespace

struct pa_block_manager {
  int32_t num_blocks, block_size, max_blocks, reserved;
  std::vector<int32_t> ref;        // sequences referencing each block
  std::vector<int32_t> free_list;  // stack: the most recently freed block is reused first
  std::unordered_map<int64_t, Sequence> seqs;
  // prefix-sharing index over full prompt blocks: key -> blocks; per cached block its predecessor and tokens
  std::unordered_map<uint64_t, std::vector<int32_t>> index;
  std::vector<char> cached;
  std::vector<int32_t> cached_parent;
  std::vector<std::vector<int32_t>> cached_tokens;
  std::vector<uint64_t> cached_key;
  std::vector<int32_t> copies;  // pending copy-on-write pairs {src, dst}
  int64_t cow_total = 0;
  // host pool for swapped-out sequences: their block lists hold host block ids
  int32_t num_host_blocks = 0;
  std::vector<int32_t> host_free;  // stack, like free_list
  std::unordered_map<int64_t, Sequence> swapped;
  int64_t moved_total = 0;

  bool known(int64_t id) const { return seqs.count(id) || swapped.count(id); }

  int32_t pop_free() {
    const int32_t b = free_list.back();
    free_list.pop_back();
    ref[b] = 1;
    return b;
  }

  void release(int32_t b) {
    if (--ref[b] > 0) return;
    if (cached[b]) {
      auto it = index.find(cached_key[b]);
      if (it != index.end()) {
        auto& v = it->second;
        v.erase(std::remove(v.begin(), v.end(), b), v.end());
        if (v.empty()) index.erase(it);
      }
      cached[b] = 0;
      cached_tokens[b].clear();
    }
    free_list.push_back(b);
  }

  // a cached full block with predecessor `parent` and exactly these tokens, or -1
  int32_t find_shared(int32_t parent, const int32_t* tokens) const {
    auto it = index.find(block_key(parent, tokens, block_size));
    if (it == index.end()) return -1;
    for (int32_t b : it->second) {
      if (cached_parent[b] == parent && std::equal(tokens, tokens + block_size, cached_tokens[b].begin()))
        return b;
    }
    return -1;
  }

  void add_to_index(int32_t b, int32_t parent, const int32_t* tokens) {
    const uint64_t k = block_key(parent, tokens, block_size);
    cached[b] = 1;
    cached_parent[b] = parent;
    cached_tokens[b].assign(tokens, tokens + block_size);
    cached_key[b] = k;
    index[k].push_back(b);
  }
};

extern "C" {

pa_block_manager* pa_bm_create(int32_t num_blocks, int32_t block_size, int32_t max_blocks_per_seq,
                               int32_t reserved_block) {
  if (num_blocks <= 0 || block_size <= 0 || max_blocks_per_seq <= 0 || reserved_block < -1 ||
      reserved_block >= num_blocks || (int64_t)num_blocks * block_size > INT32_MAX)
    return nullptr;
  pa_block_manager* bm = new (std::nothrow) pa_block_manager();
  if (!bm) return nullptr;
  try {
    bm->num_blocks = num_blocks;
    bm->block_size = block_size;
    bm->max_blocks = max_blocks_per_seq;
    bm->reserved = reserved_block;
    bm->ref.assign(num_blocks, 0);
    bm->cached.assign(num_blocks, 0);
    bm->cached_parent.assign(num_blocks, -1);
    bm->cached_tokens.resize(num_blocks);
    bm->cached_key.assign(num_blocks, 0);
    bm->free_list.reserve(num_blocks);
    for (int32_t b = num_blocks - 1; b >= 0; --b)
      if (b != reserved_block) bm->free_list.push_back(b);  // pops hand out 0, 1, 2, ...
  } catch (...) {
    delete bm;
    return nullptr;
  }
  return bm;
}

void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

int32_t pa_bm_add_sequence(pa_block_manager* bm, int64_t seq_id, const int32_t* tokens, int32_t num_tokens,
                           int32_t* slots_out) {
  if (!bm) return PA_ERR_NULL;
  if (num_tokens < 0 || (num_tokens > 0 && !slots_out)) return num_tokens < 0 ? PA_ERR_SHAPE : PA_ERR_NULL;
  if (bm->known(seq_id)) return PA_ERR_SEQ;
  const int32_t bs = bm->block_size;
  const int32_t nblk = (num_tokens + bs - 1) / bs;
  if (nblk > bm->max_blocks) return PA_ERR_SHAPE;
  try {
    // leading full blocks already in the pool with the same tokens after the same predecessors
    std::vector<int32_t> blocks;
    int32_t parent = -1;
    if (tokens) {
      for (int32_t i = 0; i < num_tokens / bs; ++i) {
        const int32_t b = bm->find_shared(parent, tokens + (int64_t)i * bs);
        if (b < 0) break;
        blocks.push_back(b);
        parent = b;
      }
    }
    const int32_t shared = (int32_t)blocks.size();
    const int32_t fresh = nblk - shared;
    if (fresh > (int32_t)bm->free_list.size()) return PA_ERR_NOMEM;
    Sequence seq;
    seq.blocks.reserve(nblk);
    for (int32_t b : blocks) {
      ++bm->ref[b];
      seq.blocks.push_back(b);
    }
    for (int32_t i = shared; i < nblk; ++i) {
      const int32_t b = bm->pop_free();
      seq.blocks.push_back(b);
      if (tokens && (int64_t)(i + 1) * bs <= num_tokens) {  // a full prompt block becomes shareable
        bm->add_to_index(b, parent, tokens + (int64_t)i * bs);
        parent = b;
      }
    }
    seq.len = num_tokens;
    for (int32_t t = 0; t < num_tokens; ++t) {
      const int32_t i = t / bs;
      slots_out[t] = i < shared ? -1 : seq.blocks[i] * bs + t % bs;
    }
    bm->seqs.emplace(seq_id, std::move(seq));
    return fresh;
  } catch (...) {
    return PA_ERR_NOMEM;
  }
}

int32_t pa_bm_fork(pa_block_manager* bm, int64_t parent_id, int64_t child_id) {
  if (!bm) return PA_ERR_NULL;
  auto it = bm->seqs.find(parent_id);
  if (it == bm->seqs.end() || bm->known(child_id)) return PA_ERR_SEQ;
  try {
    Sequence child = it->second;
    for (int32_t b : child.blocks) ++bm->ref[b];
    bm->seqs.emplace(child_id, std::move(child));
  } catch (...) {
    return PA_ERR_NOMEM;
  }
  return PA_OK;
}

int32_t pa_bm_append_slots(pa_block_manager* bm, const int64_t* seq_ids, int32_t n, int32_t* slots_out) {
  if (!bm) return PA_ERR_NULL;
  if (n < 0) return PA_ERR_SHAPE;
  if (n == 0) return PA_OK;
  if (!seq_ids || !slots_out) return PA_ERR_NULL;
  const int32_t bs = bm->block_size;
  try {
    // count the blocks this step needs, following the reference counts as earlier appends change them
    std::vector<Sequence*> seq(n);
    std::unordered_set<int64_t> seen;
    std::unordered_map<int32_t, int32_t> ref_drop;
    int64_t need = 0;
    for (int32_t i = 0; i < n; ++i) {
      auto it = bm->seqs.find(seq_ids[i]);
      if (it == bm->seqs.end() || !seen.insert(seq_ids[i]).second) return PA_ERR_SEQ;
      seq[i] = &it->second;
      const Sequence& q = *seq[i];
      if (q.len % bs == 0) {  // no room in the last block (or no block yet)
        if ((int32_t)q.blocks.size() >= bm->max_blocks) return PA_ERR_SHAPE;
        ++need;
      } else {
        const int32_t last = q.blocks.back();
        if (bm->ref[last] - ref_drop[last] > 1) {  // shared: this sequence gets its own copy
          ++need;
          ++ref_drop[last];
        }
      }
    }
    if (need > (int64_t)bm->free_list.size()) return PA_ERR_NOMEM;
    bm->copies.reserve(bm->copies.size() + 2 * need);
    for (int32_t i = 0; i < n; ++i) {
      Sequence& q = *seq[i];
      const int32_t off = (int32_t)(q.len % bs);
      int32_t b;
      if (off == 0) {
        b = bm->pop_free();
        q.blocks.push_back(b);
      } else {
        b = q.blocks.back();
        if (bm->ref[b] > 1) {
          const int32_t dst = bm->pop_free();
          --bm->ref[b];
          bm->copies.push_back(b);
          bm->copies.push_back(dst);
          ++bm->cow_total;
          q.blocks.back() = dst;
          b = dst;
        }
      }
      slots_out[i] = b * bs + off;
      ++q.len;
    }
  } catch (...) {
    return PA_ERR_NOMEM;
  }
  return PA_OK;
}

int32_t pa_bm_take_copies(pa_block_manager* bm, int32_t* pairs_out, int32_t max_pairs) {
  if (!bm) return PA_ERR_NULL;
  const int32_t n = (int32_t)(bm->copies.size() / 2);
  if (n > max_pairs) return PA_ERR_SHAPE;
  if (n > 0 && !pairs_out) return PA_ERR_NULL;
  std::copy(bm->copies.begin(), bm->copies.end(), pairs_out);
  bm->copies.clear();
  return n;
}

int32_t pa_bm_free_sequence(pa_block_manager* bm, int64_t seq_id) {
  if (!bm) return PA_ERR_NULL;
  auto sw = bm->swapped.find(seq_id);
  if (sw != bm->swapped.end()) {  // a swapped-out sequence gives back its host blocks
    try {
      bm->host_free.reserve(bm->host_free.size() + sw->second.blocks.size());
    } catch (...) {
      return PA_ERR_NOMEM;
    }
    for (int32_t b : sw->second.blocks) bm->host_free.push_back(b);
    bm->swapped.erase(sw);
    return PA_OK;
  }
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PA_ERR_SEQ;
  // the free list grows by at most the sequence's block count; reserve first so nothing below can throw
  try {
    bm->free_list.reserve(bm->free_list.size() + it->second.blocks.size());
  } catch (...) {
    return PA_ERR_NOMEM;
  }
  for (int32_t b : it->second.blocks) bm->release(b);
  bm->seqs.erase(it);
  return PA_OK;
}

int32_t pa_bm_block_tables(const pa_block_manager* bm, const int64_t* seq_ids, int32_t n, int32_t* table_out,
                           int32_t* lens_out, int32_t pad) {
  if (!bm) return PA_ERR_NULL;
  if (n < 0) return PA_ERR_SHAPE;
  if (n == 0) return PA_OK;
  if (!seq_ids || !table_out || !lens_out) return PA_ERR_NULL;
  for (int32_t i = 0; i < n; ++i)
    if (!bm->seqs.count(seq_ids[i])) return PA_ERR_SEQ;
  const int32_t mb = bm->max_blocks;
  for (int32_t i = 0; i < n; ++i) {
    const Sequence& q = bm->seqs.at(seq_ids[i]);
    int32_t* row = table_out + (int64_t)i * mb;
    std::fill(row, row + mb, pad);
    std::copy(q.blocks.begin(), q.blocks.end(), row);
    lens_out[i] = (int32_t)q.len;
  }
  return PA_OK;
}

int32_t pa_bm_set_host_pool(pa_block_manager* bm, int32_t num_host_blocks) {
  if (!bm) return PA_ERR_NULL;
  if (num_host_blocks < 0) return PA_ERR_SHAPE;
  if (!bm->swapped.empty()) return PA_ERR_SEQ;  // blocks of the current host pool are in use
  try {
    std::vector<int32_t> fl;
    fl.reserve(num_host_blocks);
    for (int32_t b = num_host_blocks - 1; b >= 0; --b) fl.push_back(b);
    bm->host_free.swap(fl);
  } catch (...) {
    return PA_ERR_NOMEM;
  }
  bm->num_host_blocks = num_host_blocks;
  return PA_OK;
}

int32_t pa_bm_swap_out(pa_block_manager* bm, int64_t seq_id, int32_t* pairs_out, int32_t max_pairs) {
  if (!bm) return PA_ERR_NULL;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PA_ERR_SEQ;
  if (!bm->copies.empty()) return PA_ERR_SHAPE;  // pending copy-on-write pairs must be taken and applied first
  const int32_t n = (int32_t)it->second.blocks.size();
  if (n > max_pairs) return PA_ERR_SHAPE;
  if (n > 0 && !pairs_out) return PA_ERR_NULL;
  if (n > (int32_t)bm->host_free.size()) return PA_ERR_NOMEM;
  try {
    bm->free_list.reserve(bm->free_list.size() + n);
    Sequence out;
    out.len = it->second.len;
    out.blocks.reserve(n);
    bm->swapped.reserve(bm->swapped.size() + 1);
    for (int32_t i = 0; i < n; ++i) {
      const int32_t h = bm->host_free.back();
      bm->host_free.pop_back();
      pairs_out[2 * i] = it->second.blocks[i];
      pairs_out[2 * i + 1] = h;
      out.blocks.push_back(h);
    }
    // nothing below throws: the device blocks are released (shared ones stay with their other users)
    for (int32_t b : it->second.blocks) bm->release(b);
    bm->seqs.erase(it);
    bm->swapped.emplace(seq_id, std::move(out));
    bm->moved_total += n;
    return n;
  } catch (...) {
    return PA_ERR_NOMEM;
  }
}

int32_t pa_bm_swap_in(pa_block_manager* bm, int64_t seq_id, int32_t* pairs_out, int32_t max_pairs) {
  if (!bm) return PA_ERR_NULL;
  auto it = bm->swapped.find(seq_id);
  if (it == bm->swapped.end()) return PA_ERR_SEQ;
  const int32_t n = (int32_t)it->second.blocks.size();
  if (n > max_pairs) return PA_ERR_SHAPE;
  if (n > 0 && !pairs_out) return PA_ERR_NULL;
  if (n > (int32_t)bm->free_list.size()) return PA_ERR_NOMEM;
  try {
    bm->host_free.reserve(bm->host_free.size() + n);
    Sequence back;
    back.len = it->second.len;
    back.blocks.reserve(n);
    bm->seqs.reserve(bm->seqs.size() + 1);
    for (int32_t i = 0; i < n; ++i) {
      const int32_t b = bm->pop_free();
      pairs_out[2 * i] = it->second.blocks[i];
      pairs_out[2 * i + 1] = b;
      back.blocks.push_back(b);
    }
    for (int32_t h : it->second.blocks) bm->host_free.push_back(h);
    bm->swapped.erase(it);
    bm->seqs.emplace(seq_id, std::move(back));
    bm->moved_total += n;
    return n;
  } catch (...) {
    return PA_ERR_NOMEM;
  }
}

int32_t pa_bm_swap_stats(const pa_block_manager* bm, int64_t* stats_out) {
  if (!bm || !stats_out) return PA_ERR_NULL;
  stats_out[0] = (int64_t)bm->host_free.size();
  stats_out[1] = bm->num_host_blocks - (int64_t)bm->host_free.size();
  stats_out[2] = (int64_t)bm->swapped.size();
  stats_out[3] = bm->moved_total;
  return PA_OK;
}

int32_t pa_bm_stats(const pa_block_manager* bm, int64_t* stats_out) {
  if (!bm || !stats_out) return PA_ERR_NULL;
  const int64_t bs = bm->block_size;
  int64_t used = 0, shared = 0, tokens = 0, filled = 0;
  std::vector<int32_t> fill(bm->num_blocks, 0);  // slots holding a token, per block
  for (const auto& kv : bm->seqs) {
    const Sequence& q = kv.second;
    tokens += q.len;
    for (size_t i = 0; i < q.blocks.size(); ++i) {
      const int64_t f = std::min<int64_t>(bs, q.len - (int64_t)i * bs);
      fill[q.blocks[i]] = std::max<int32_t>(fill[q.blocks[i]], (int32_t)f);
    }
  }
  for (int32_t b = 0; b < bm->num_blocks; ++b) {
    if (bm->ref[b] > 0) ++used;
    if (bm->ref[b] > 1) ++shared;
    filled += fill[b];
  }
  stats_out[0] = (int64_t)bm->free_list.size();
  stats_out[1] = used;
  stats_out[2] = shared;
  stats_out[3] = (int64_t)bm->seqs.size();
  stats_out[4] = tokens;
  stats_out[5] = used * bs;
  stats_out[6] = filled;
  stats_out[7] = bm->cow_total;
  return PA_OK;
}

}  // extern "C"
