// Host block manager: free pool, block tables, reference counts with
// copy-on-write, prefix keys with LRU eviction, and a host pool for swap.
//
// quant67 "PagedAttention 与 Continuous Batching" §3.3 (append into the last
// block, else take a free block), §3.5 / §3.8 (shared prompt blocks and
// copy-on-write), §3.9 / §6.1 (swap), §5.2 (chained block keys, shared hits,
// LRU eviction of unreferenced blocks); lpnh.cn "大模型推理架构演进：从
// PagedAttention 到 Prefill-Decode 分离的深度解析" §二 2.2, third step (blocks
// go back to the global pool when a request ends).  The rules where the pages leave a
// step open are listed in pa_blocks.h.
//
// Every operation checks that it can complete before it changes anything,
// so a PA_ERR_NO_BLOCKS leaves the manager as it was.
#include <cstring>
#include <deque>
#include <new>
#include <unordered_map>
#include <vector>

#include "../../include/pa_blocks.h"

namespace {

struct Key {
  uint64_t a = 0, b = 0;
  bool operator==(const Key& o) const { return a == o.a && b == o.b; }
};

struct KeyHash {
  size_t operator()(const Key& k) const { return size_t(k.a ^ (k.b * 0x9e3779b97f4a7c15ULL)); }
};

// SplitMix64 output function (Steele, Lea and Flood, "Fast splittable
// pseudorandom number generators", 2014).
inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
  return z ^ (z >> 31);
}

// Key of a full block: its tokens chained onto the previous block's key
// (§5.2).  Two lanes with different seeds and different token injections.
Key chain_key(const Key& prev, const int32_t* tokens, int32_t bs) {
  uint64_t a = mix64(prev.a ^ 0x243f6a8885a308d3ULL);
  uint64_t b = mix64(prev.b ^ 0x13198a2e03707344ULL);
  for (int32_t i = 0; i < bs; ++i) {
    const uint64_t v = uint32_t(tokens[i]);
    a = mix64(a + v + 0x9e3779b97f4a7c15ULL);
    b = mix64(b ^ (v * 0xff51afd7ed558ccdULL + uint64_t(i)));
  }
  return Key{a, b};
}

struct Seq {
  std::vector<int32_t> tokens;
  std::vector<int32_t> table;
  Key tail_key;         // key of the last full block (root key if none)
  bool swapped = false;
};

}  // namespace

struct pa_block_manager {
  int64_t num_blocks = 0;
  int32_t bs = 0;
  int64_t num_host = 0;
  bool prefix = false;

  std::vector<int32_t> ref;
  std::deque<int32_t> free_q;
  // eviction order of cached blocks with no reference: intrusive list
  std::vector<int32_t> prev, next;
  std::vector<uint8_t> in_lru;
  int32_t lru_head = -1, lru_tail = -1;
  int64_t lru_size = 0;
  // registered full blocks
  std::vector<uint8_t> registered;
  std::vector<Key> key, parent;
  std::vector<int32_t> content;   // [num_blocks][bs] tokens of registered blocks
  std::unordered_map<Key, int32_t, KeyHash> block_of;

  std::deque<int32_t> host_free;
  std::unordered_map<int64_t, Seq> seqs;

  // -- eviction list -------------------------------------------------------
  void lru_push(int32_t b) {
    prev[b] = lru_tail;
    next[b] = -1;
    if (lru_tail >= 0) next[lru_tail] = b; else lru_head = b;
    lru_tail = b;
    in_lru[b] = 1;
    ++lru_size;
  }
  void lru_remove(int32_t b) {
    if (prev[b] >= 0) next[prev[b]] = next[b]; else lru_head = next[b];
    if (next[b] >= 0) prev[next[b]] = prev[b]; else lru_tail = prev[b];
    in_lru[b] = 0;
    --lru_size;
  }

  // -- pool ----------------------------------------------------------------
  int64_t available() const { return int64_t(free_q.size()) + lru_size; }

  int32_t alloc() {   // callers have checked available() first
    int32_t b;
    if (!free_q.empty()) {
      b = free_q.front();
      free_q.pop_front();
    } else {
      b = lru_head;
      lru_remove(b);
      block_of.erase(key[b]);
      registered[b] = 0;
    }
    ref[b] = 1;
    return b;
  }

  void release(int32_t b) {
    if (--ref[b] == 0) {
      if (registered[b]) lru_push(b); else free_q.push_back(b);
    }
  }

  void take(int32_t b) {
    if (ref[b] == 0) lru_remove(b);
    ++ref[b];
  }

  // -- keys ----------------------------------------------------------------
  void register_block(int32_t b, const Key& k, const Key& parent_key, const int32_t* toks) {
    if (!prefix || block_of.count(k)) return;
    block_of.emplace(k, b);
    registered[b] = 1;
    key[b] = k;
    parent[b] = parent_key;
    std::memcpy(&content[size_t(b) * bs], toks, sizeof(int32_t) * bs);
  }

  int32_t lookup(const Key& k, const Key& parent_key, const int32_t* toks) const {
    auto it = block_of.find(k);
    if (it == block_of.end()) return -1;
    const int32_t b = it->second;
    if (!(parent[b] == parent_key) || std::memcmp(&content[size_t(b) * bs], toks, sizeof(int32_t) * bs) != 0)
      return -1;
    return b;
  }

  Seq* resident(int64_t id) {
    auto it = seqs.find(id);
    return (it == seqs.end() || it->second.swapped) ? nullptr : &it->second;
  }
  const Seq* resident(int64_t id) const {
    auto it = seqs.find(id);
    return (it == seqs.end() || it->second.swapped) ? nullptr : &it->second;
  }

  // -- operations ------------------------------------------------------------
  pa_status add_sequence(int64_t id, const int32_t* tokens, int64_t n, int64_t* cached) {
    if (seqs.count(id)) return PA_ERR_STATE;
    const int64_t nblocks = (n + bs - 1) / bs, nfull = n / bs, nlook = (n - 1) / bs;
    if (nblocks > num_blocks) return PA_ERR_NO_BLOCKS;
    std::vector<Key> keys;
    std::vector<int32_t> hits;
    if (prefix) {
      keys.resize(size_t(nfull));
      Key k{};
      for (int64_t i = 0; i < nfull; ++i) keys[size_t(i)] = k = chain_key(k, tokens + i * bs, bs);
      for (int64_t i = 0; i < nlook; ++i) {
        const int32_t b = lookup(keys[size_t(i)], i ? keys[size_t(i - 1)] : Key{}, tokens + i * bs);
        if (b < 0) break;
        hits.push_back(b);
      }
    }
    int64_t cached_free = 0;
    for (int32_t b : hits) cached_free += ref[b] == 0;
    const int64_t need = nblocks - int64_t(hits.size());
    if (need > available() - cached_free) return PA_ERR_NO_BLOCKS;

    Seq s;
    s.tokens.assign(tokens, tokens + n);
    s.table.reserve(size_t(nblocks));
    for (int32_t b : hits) {
      take(b);
      s.table.push_back(b);
    }
    for (int64_t i = 0; i < need; ++i) s.table.push_back(alloc());
    if (prefix) {
      for (int64_t i = int64_t(hits.size()); i < nfull; ++i)
        register_block(s.table[size_t(i)], keys[size_t(i)], i ? keys[size_t(i - 1)] : Key{}, tokens + i * bs);
      if (nfull) s.tail_key = keys[size_t(nfull - 1)];
    }
    if (cached) *cached = int64_t(hits.size()) * bs;
    seqs.emplace(id, std::move(s));
    return PA_OK;
  }

  pa_status fork(int64_t parent_id, int64_t child) {
    const Seq* p = resident(parent_id);
    if (!p || seqs.count(child)) return PA_ERR_STATE;
    for (int32_t b : p->table) ++ref[b];
    Seq c = *p;
    seqs.emplace(child, std::move(c));
    return PA_OK;
  }

  pa_status append_slot(int64_t id, int32_t token, int64_t* slot, int64_t* src, int64_t* dst) {
    Seq* s = resident(id);
    if (!s) return PA_ERR_STATE;
    const int64_t n = int64_t(s->tokens.size());
    int64_t cs = -1, cd = -1;
    if (n % bs == 0) {
      if (available() < 1) return PA_ERR_NO_BLOCKS;
      s->table.push_back(alloc());
    } else if (ref[s->table.back()] > 1) {
      if (available() < 1) return PA_ERR_NO_BLOCKS;
      cs = s->table.back();
      cd = alloc();
      release(int32_t(cs));
      s->table.back() = int32_t(cd);
    }
    s->tokens.push_back(token);
    if ((n + 1) % bs == 0 && prefix) {
      const int32_t* blk = s->tokens.data() + (n + 1 - bs);
      const Key k = chain_key(s->tail_key, blk, bs);
      register_block(s->table.back(), k, s->tail_key, blk);
      s->tail_key = k;
    }
    *slot = int64_t(s->table[size_t(n / bs)]) * bs + n % bs;
    *src = cs;
    *dst = cd;
    return PA_OK;
  }

  pa_status free_seq(int64_t id) {
    auto it = seqs.find(id);
    if (it == seqs.end()) return PA_ERR_STATE;
    const std::vector<int32_t>& t = it->second.table;
    if (it->second.swapped) {
      for (auto r = t.rbegin(); r != t.rend(); ++r) host_free.push_back(*r);
    } else {
      for (auto r = t.rbegin(); r != t.rend(); ++r) release(*r);
    }
    seqs.erase(it);
    return PA_OK;
  }

  pa_status swap_out(int64_t id, int64_t* pairs, int64_t capacity, int64_t* num_pairs) {
    Seq* s = resident(id);
    if (!s) return PA_ERR_STATE;
    const int64_t n = int64_t(s->table.size());
    if (capacity < n) return PA_ERR_SHAPE;
    if (int64_t(host_free.size()) < n) return PA_ERR_NO_BLOCKS;
    std::vector<int32_t> host(static_cast<size_t>(n));
    for (int64_t i = 0; i < n; ++i) {
      host[size_t(i)] = host_free.front();
      host_free.pop_front();
      pairs[2 * i] = s->table[size_t(i)];
      pairs[2 * i + 1] = host[size_t(i)];
    }
    for (auto r = s->table.rbegin(); r != s->table.rend(); ++r) release(*r);
    s->table.swap(host);
    s->swapped = true;
    *num_pairs = n;
    return PA_OK;
  }

  pa_status swap_in(int64_t id, int64_t* pairs, int64_t capacity, int64_t* num_pairs) {
    auto it = seqs.find(id);
    if (it == seqs.end() || !it->second.swapped) return PA_ERR_STATE;
    Seq& s = it->second;
    const int64_t n = int64_t(s.table.size());
    if (capacity < n) return PA_ERR_SHAPE;
    if (available() < n) return PA_ERR_NO_BLOCKS;
    std::vector<int32_t> dev(static_cast<size_t>(n));
    for (int64_t i = 0; i < n; ++i) {
      dev[size_t(i)] = alloc();
      pairs[2 * i] = s.table[size_t(i)];
      pairs[2 * i + 1] = dev[size_t(i)];
    }
    for (auto r = s.table.rbegin(); r != s.table.rend(); ++r) host_free.push_back(*r);
    if (prefix) {
      Key k{};
      const int64_t nfull = int64_t(s.tokens.size()) / bs;
      for (int64_t i = 0; i < nfull; ++i) {
        const Key kk = chain_key(k, s.tokens.data() + i * bs, bs);
        register_block(dev[size_t(i)], kk, k, s.tokens.data() + i * bs);
        k = kk;
      }
    }
    s.table.swap(dev);
    s.swapped = false;
    *num_pairs = n;
    return PA_OK;
  }
};

#define PA_BM_GUARD(expr)                 \
  try {                                   \
    return (expr);                        \
  } catch (const std::bad_alloc&) {       \
    return PA_ERR_HOST_MEMORY;            \
  } catch (...) {                         \
    return PA_ERR_HOST_MEMORY;            \
  }

extern "C" {

pa_status pa_bm_create(int64_t num_blocks, int32_t block_size, int64_t num_host_blocks, int32_t prefix_caching,
                       pa_block_manager** out) {
  if (!out) return PA_ERR_NULL;
  *out = nullptr;
  if (num_blocks < 1 || num_blocks > INT32_MAX || block_size < 1 || num_host_blocks < 0 ||
      num_host_blocks > INT32_MAX)
    return PA_ERR_SHAPE;
  try {
    auto* m = new pa_block_manager;
    m->num_blocks = num_blocks;
    m->bs = block_size;
    m->num_host = num_host_blocks;
    m->prefix = prefix_caching != 0;
    m->ref.assign(size_t(num_blocks), 0);
    for (int64_t b = 0; b < num_blocks; ++b) m->free_q.push_back(int32_t(b));
    for (int64_t b = 0; b < num_host_blocks; ++b) m->host_free.push_back(int32_t(b));
    m->prev.assign(size_t(num_blocks), -1);
    m->next.assign(size_t(num_blocks), -1);
    m->in_lru.assign(size_t(num_blocks), 0);
    m->registered.assign(size_t(num_blocks), 0);
    if (m->prefix) {
      m->key.resize(size_t(num_blocks));
      m->parent.resize(size_t(num_blocks));
      m->content.assign(size_t(num_blocks) * size_t(block_size), 0);
    }
    *out = m;
    return PA_OK;
  } catch (...) {
    return PA_ERR_HOST_MEMORY;
  }
}

void pa_bm_destroy(pa_block_manager* m) { delete m; }

pa_status pa_bm_add_sequence(pa_block_manager* m, int64_t seq_id, const int32_t* tokens, int64_t num_tokens,
                             int64_t* num_cached_tokens) {
  if (!m || !tokens) return PA_ERR_NULL;
  if (num_tokens < 1) return PA_ERR_SHAPE;
  PA_BM_GUARD(m->add_sequence(seq_id, tokens, num_tokens, num_cached_tokens))
}

pa_status pa_bm_fork(pa_block_manager* m, int64_t parent, int64_t child) {
  if (!m) return PA_ERR_NULL;
  PA_BM_GUARD(m->fork(parent, child))
}

pa_status pa_bm_append_slot(pa_block_manager* m, int64_t seq_id, int32_t token, int64_t* slot, int64_t* cow_src,
                            int64_t* cow_dst) {
  if (!m || !slot || !cow_src || !cow_dst) return PA_ERR_NULL;
  PA_BM_GUARD(m->append_slot(seq_id, token, slot, cow_src, cow_dst))
}

pa_status pa_bm_free(pa_block_manager* m, int64_t seq_id) {
  if (!m) return PA_ERR_NULL;
  PA_BM_GUARD(m->free_seq(seq_id))
}

pa_status pa_bm_swap_out(pa_block_manager* m, int64_t seq_id, int64_t* pairs, int64_t capacity,
                         int64_t* num_pairs) {
  if (!m || !pairs || !num_pairs) return PA_ERR_NULL;
  PA_BM_GUARD(m->swap_out(seq_id, pairs, capacity, num_pairs))
}

pa_status pa_bm_swap_in(pa_block_manager* m, int64_t seq_id, int64_t* pairs, int64_t capacity, int64_t* num_pairs) {
  if (!m || !pairs || !num_pairs) return PA_ERR_NULL;
  PA_BM_GUARD(m->swap_in(seq_id, pairs, capacity, num_pairs))
}

pa_status pa_bm_block_table(const pa_block_manager* m, int64_t seq_id, int32_t* table, int64_t capacity,
                            int64_t* num_entries) {
  if (!m || !num_entries) return PA_ERR_NULL;
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return PA_ERR_STATE;
  const std::vector<int32_t>& t = it->second.table;
  *num_entries = int64_t(t.size());
  if (capacity < int64_t(t.size())) return PA_ERR_SHAPE;
  if (!t.empty() && !table) return PA_ERR_NULL;
  if (!t.empty()) std::memcpy(table, t.data(), sizeof(int32_t) * t.size());
  return PA_OK;
}

pa_status pa_bm_block_tables(const pa_block_manager* m, const int64_t* seq_ids, int64_t num_seqs, int32_t* tables,
                             int32_t width, int32_t* seq_lens) {
  if (!m) return PA_ERR_NULL;
  if (num_seqs < 0 || width < 0) return PA_ERR_SHAPE;
  if (num_seqs == 0) return PA_OK;
  if (!seq_ids || (!tables && width > 0)) return PA_ERR_NULL;
  for (int64_t i = 0; i < num_seqs; ++i) {
    const Seq* s = m->resident(seq_ids[i]);
    if (!s) return PA_ERR_STATE;
    if (int64_t(s->table.size()) > width || int64_t(s->tokens.size()) > INT32_MAX) return PA_ERR_SHAPE;
  }
  for (int64_t i = 0; i < num_seqs; ++i) {
    const Seq* s = m->resident(seq_ids[i]);
    int32_t* row = tables + i * width;
    std::memset(row, 0, sizeof(int32_t) * size_t(width));
    if (!s->table.empty()) std::memcpy(row, s->table.data(), sizeof(int32_t) * s->table.size());
    if (seq_lens) seq_lens[i] = int32_t(s->tokens.size());
  }
  return PA_OK;
}

pa_status pa_bm_slot_mapping(const pa_block_manager* m, int64_t seq_id, int64_t start, int64_t count,
                             int64_t* slots) {
  if (!m) return PA_ERR_NULL;
  const Seq* s = m->resident(seq_id);
  if (!s) return PA_ERR_STATE;
  if (start < 0 || count < 0 || start + count > int64_t(s->tokens.size())) return PA_ERR_SHAPE;
  if (count && !slots) return PA_ERR_NULL;
  for (int64_t i = 0; i < count; ++i) {
    const int64_t t = start + i;
    slots[i] = int64_t(s->table[size_t(t / m->bs)]) * m->bs + t % m->bs;
  }
  return PA_OK;
}

pa_status pa_bm_seq_info(const pa_block_manager* m, int64_t seq_id, int64_t* num_tokens, int32_t* swapped) {
  if (!m) return PA_ERR_NULL;
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return PA_ERR_STATE;
  if (num_tokens) *num_tokens = int64_t(it->second.tokens.size());
  if (swapped) *swapped = it->second.swapped ? 1 : 0;
  return PA_OK;
}

pa_status pa_bm_refcount(const pa_block_manager* m, int64_t block, int32_t* count) {
  if (!m || !count) return PA_ERR_NULL;
  if (block < 0 || block >= m->num_blocks) return PA_ERR_SHAPE;
  *count = m->ref[size_t(block)];
  return PA_OK;
}

pa_status pa_bm_stats(const pa_block_manager* m, int64_t* num_free, int64_t* num_cached, int64_t* num_host_free,
                      int64_t* num_seqs) {
  if (!m) return PA_ERR_NULL;
  if (num_free) *num_free = m->available();
  if (num_cached) *num_cached = int64_t(m->block_of.size());
  if (num_host_free) *num_host_free = int64_t(m->host_free.size());
  if (num_seqs) *num_seqs = int64_t(m->seqs.size());
  return PA_OK;
}

}  // extern "C"
