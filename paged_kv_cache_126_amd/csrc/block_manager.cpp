// Host block manager (declared in include/paged_blocks.h): frame pool, block
// tables, slot mapping, fork with copy-on-write and prefix caching of full
// blocks. Plain C++ on the host; the rules it follows are listed in the
// header with the passages they come from.
#include <cstdint>
#include <cstring>
#include <deque>
#include <new>
#include <set>
#include <unordered_map>
#include <utility>
#include <vector>

#include "paged_blocks.h"

namespace {

// 128-bit key of a full block: a chain hash over the key of the block
// before it and the block's token ids. Lookups also compare the stored
// predecessor key and token ids, so a hash collision can cost a reuse but
// never return a frame holding other tokens.
struct Key {
  uint64_t hi = 0, lo = 0;
  bool operator==(const Key& o) const { return hi == o.hi && lo == o.lo; }
};

struct KeyHash {
  size_t operator()(const Key& k) const { return static_cast<size_t>(k.hi ^ (k.lo * 0x9E3779B97F4A7C15ull)); }
};

inline uint64_t mix64(uint64_t x) {  // splitmix64 finaliser
  x ^= x >> 30;
  x *= 0xBF58476D1CE4E5B9ull;
  x ^= x >> 27;
  x *= 0x94D049BB133111EBull;
  x ^= x >> 31;
  return x;
}

Key chain_key(const Key& prev, const int64_t* tokens, int64_t n) {
  uint64_t a = mix64(prev.hi ^ 0x243F6A8885A308D3ull) ^ prev.lo;
  uint64_t b = mix64(prev.lo ^ 0x13198A2E03707344ull) ^ prev.hi;
  for (int64_t i = 0; i < n; ++i) {
    const uint64_t w = static_cast<uint64_t>(tokens[i]);
    a = mix64(a ^ w) + 0x9E3779B97F4A7C15ull;
    b = mix64(b + (w ^ 0xA4093822299F31D0ull)) ^ (b >> 17);
  }
  return Key{mix64(a ^ static_cast<uint64_t>(n)), mix64(b + static_cast<uint64_t>(n))};
}

struct Entry {         // one cached frame
  int32_t frame;
  Key prev;            // key of the block before it (zero for block 0)
  std::vector<int64_t> tokens;
};

struct Seq {
  std::vector<int32_t> table;
  int64_t len = 0;
  std::vector<int64_t> tokens;  // prefix caching only
  std::vector<Key> chain;       // keys of the sequence's full blocks (prefix caching only)
};

}  // namespace

struct pb_manager {
  int64_t num_frames = 0;
  int32_t B = 0;
  bool caching = false;
  std::deque<int32_t> free_list;
  std::vector<int32_t> ref;
  std::unordered_map<int64_t, Seq> seqs;
  // prefix cache
  std::unordered_map<Key, Entry, KeyHash> index;
  std::vector<Key> key_of;            // per frame, valid when cached[f]
  std::vector<uint8_t> cached;
  std::vector<int64_t> last_use;      // per cached frame
  std::set<std::pair<int64_t, int32_t>> idle;  // (last use, frame): cached, referenced by the cache only
  int64_t tick = 0;
  int64_t hit_blocks = 0, miss_blocks = 0, evictions = 0;

  void add_ref(int32_t f) {
    if (cached[f] && ref[f] == 1) idle.erase({last_use[f], f});
    ++ref[f];
  }
  void release(int32_t f) {  // drop one reference
    if (ref[f] <= 0) return;
    --ref[f];
    if (ref[f] == 0)
      free_list.push_back(f);
    else if (ref[f] == 1 && cached[f])
      idle.insert({last_use[f], f});
  }
  void touch(int32_t f) {  // only for frames that are not idle (ref >= 2)
    last_use[f] = ++tick;
  }
  // Take a frame: first in, first out; with an empty free list, drop the
  // cached frame used longest ago that only the cache references.
  bool take(int32_t* out) {
    if (free_list.empty()) {
      if (idle.empty()) return false;
      const int32_t f = idle.begin()->second;
      idle.erase(idle.begin());
      index.erase(key_of[f]);
      cached[f] = 0;
      ++evictions;
      release(f);  // 1 -> 0: joins the free list
    }
    *out = free_list.front();
    free_list.pop_front();
    ref[*out] = 1;
    return true;
  }
  int64_t spare_frames() const { return static_cast<int64_t>(free_list.size() + idle.size()); }

  // Block b of `s` has just filled: key it and cache it if the key is new.
  void enter(Seq& s, int64_t b) {
    const Key prev = b > 0 ? s.chain[b - 1] : Key{};
    const int64_t* toks = s.tokens.data() + b * B;
    const Key k = chain_key(prev, toks, B);
    s.chain.push_back(k);
    if (index.count(k)) return;
    const int32_t f = s.table[b];
    Entry e{f, prev, std::vector<int64_t>(toks, toks + B)};
    index.emplace(k, std::move(e));
    key_of[f] = k;
    cached[f] = 1;
    add_ref(f);  // the cache's own reference
    touch(f);
  }
  // The cached frame for block (prev, tokens), or -1.
  int32_t lookup(const Key& k, const Key& prev, const int64_t* toks) const {
    auto it = index.find(k);
    if (it == index.end()) return -1;
    const Entry& e = it->second;
    if (!(e.prev == prev) || std::memcmp(e.tokens.data(), toks, sizeof(int64_t) * B) != 0) return -1;
    return e.frame;
  }
};

namespace {

bool append_one(pb_manager* m, int64_t sid, const int64_t* token_id, int64_t* slot, int64_t* cow) {
  auto it = m->seqs.find(sid);
  if (it == m->seqs.end()) return false;
  Seq& s = it->second;
  const int64_t t = s.len;
  const int64_t off = t % m->B;
  int64_t c0 = -1, c1 = -1, c2 = 0;
  if (off == 0) {
    int32_t f;
    if (!m->take(&f)) return false;
    s.table.push_back(f);
  } else {
    const int32_t last = s.table.back();
    if (m->ref[last] > 1) {  // shared partial frame: move to a private copy
      int32_t f;
      if (!m->take(&f)) return false;
      m->release(last);
      s.table.back() = f;
      c0 = last, c1 = f, c2 = off;
    }
  }
  s.len = t + 1;
  *slot = static_cast<int64_t>(s.table.back()) * m->B + off;
  if (cow) cow[0] = c0, cow[1] = c1, cow[2] = c2;
  if (m->caching) {
    s.tokens.push_back(*token_id);
    if ((t + 1) % m->B == 0) m->enter(s, t / m->B);
  }
  return true;
}

void fill_slots(const pb_manager* m, const Seq& s, int64_t n, int64_t* slots) {
  for (int64_t p = 0; p < n; ++p) slots[p] = static_cast<int64_t>(s.table[p / m->B]) * m->B + p % m->B;
}

}  // namespace

extern "C" {

pb_status pb_create(int64_t num_frames, int32_t block_size, const int32_t* order,
                    int32_t prefix_caching, pb_manager** out) {
  if (!out || num_frames <= 0 || num_frames > INT32_MAX || block_size <= 0) return PB_EINVAL;
  *out = nullptr;
  if (order) {
    std::vector<uint8_t> seen(num_frames, 0);
    for (int64_t i = 0; i < num_frames; ++i) {
      if (order[i] < 0 || order[i] >= num_frames || seen[order[i]]) return PB_EINVAL;
      seen[order[i]] = 1;
    }
  }
  pb_manager* m = new (std::nothrow) pb_manager;
  if (!m) return PB_ENOMEM;
  m->num_frames = num_frames;
  m->B = block_size;
  m->caching = prefix_caching != 0;
  for (int64_t i = 0; i < num_frames; ++i)
    m->free_list.push_back(order ? order[i] : static_cast<int32_t>(i));
  m->ref.assign(num_frames, 0);
  m->key_of.assign(num_frames, Key{});
  m->cached.assign(num_frames, 0);
  m->last_use.assign(num_frames, 0);
  *out = m;
  return PB_OK;
}

void pb_destroy(pb_manager* m) { delete m; }

pb_status pb_init_sequence(pb_manager* m, int64_t sid, int64_t n_tokens, int64_t* slots_out) {
  if (!m || n_tokens < 0 || (n_tokens > 0 && !slots_out)) return PB_EINVAL;
  if (m->caching) return PB_ESTATE;  // requests need their token ids
  if (m->seqs.count(sid)) return PB_EINVAL;
  const int64_t need = (n_tokens + m->B - 1) / m->B;
  if (need > static_cast<int64_t>(m->free_list.size())) return PB_ENOMEM;
  Seq s;
  s.len = n_tokens;
  for (int64_t i = 0; i < need; ++i) {
    int32_t f;
    m->take(&f);
    s.table.push_back(f);
  }
  fill_slots(m, s, n_tokens, slots_out);
  m->seqs.emplace(sid, std::move(s));
  return PB_OK;
}

pb_status pb_init_sequence_tokens(pb_manager* m, int64_t sid, const int64_t* tokens, int64_t n,
                                  int64_t* reused_out, int64_t* slots_out) {
  if (!m || n < 0 || !reused_out || (n > 0 && (!tokens || !slots_out))) return PB_EINVAL;
  if (!m->caching) {
    *reused_out = 0;
    return pb_init_sequence(m, sid, n, slots_out);
  }
  if (m->seqs.count(sid)) return PB_EINVAL;
  const int64_t B = m->B;
  const int64_t full = n / B;
  std::vector<int32_t> hits;
  std::vector<Key> chain;
  Key prev{};
  for (int64_t b = 0; b < full; ++b) {
    const Key k = chain_key(prev, tokens + b * B, B);
    const int32_t f = m->lookup(k, prev, tokens + b * B);
    if (f < 0) break;
    hits.push_back(f);
    chain.push_back(k);
    prev = k;
  }
  const int64_t need = (n + B - 1) / B - static_cast<int64_t>(hits.size());
  int64_t idle_hits = 0;  // reused frames that are idle now: they stop counting as spare
  for (int32_t f : hits) idle_hits += m->ref[f] == 1;
  if (need > m->spare_frames() - idle_hits) return PB_ENOMEM;
  for (int32_t f : hits) {
    m->add_ref(f);
    m->touch(f);
  }
  Seq s;
  s.table = hits;
  for (int64_t i = 0; i < need; ++i) {
    int32_t f;
    m->take(&f);  // cannot fail: checked above
    s.table.push_back(f);
  }
  s.len = n;
  s.tokens.assign(tokens, tokens + n);
  s.chain = std::move(chain);
  m->hit_blocks += static_cast<int64_t>(hits.size());
  m->miss_blocks += need;
  auto& stored = m->seqs.emplace(sid, std::move(s)).first->second;
  for (int64_t b = static_cast<int64_t>(hits.size()); b < full; ++b) m->enter(stored, b);
  *reused_out = static_cast<int64_t>(hits.size()) * B;
  fill_slots(m, stored, n, slots_out);
  return PB_OK;
}

pb_status pb_append_tokens(pb_manager* m, const int64_t* sids, const int64_t* token_ids, int64_t n,
                           int64_t* slots_out, int64_t* cow_out, int64_t* done_out) {
  if (done_out) *done_out = 0;
  if (!m || n < 0 || (n > 0 && (!sids || !slots_out))) return PB_EINVAL;
  if (m->caching && n > 0 && !token_ids) return PB_ESTATE;
  for (int64_t i = 0; i < n; ++i)
    if (!m->seqs.count(sids[i])) return PB_EINVAL;
  for (int64_t i = 0; i < n; ++i) {
    if (!append_one(m, sids[i], token_ids ? token_ids + i : nullptr, slots_out + i,
                    cow_out ? cow_out + 3 * i : nullptr))
      return PB_ENOMEM;
    if (done_out) *done_out = i + 1;
  }
  return PB_OK;
}

pb_status pb_fork(pb_manager* m, int64_t parent, int64_t child) {
  if (!m) return PB_EINVAL;
  auto it = m->seqs.find(parent);
  if (it == m->seqs.end() || m->seqs.count(child)) return PB_EINVAL;
  Seq c = it->second;  // copy: table, length, tokens, chain
  for (int32_t f : c.table) m->add_ref(f);
  m->seqs.emplace(child, std::move(c));
  return PB_OK;
}

pb_status pb_free_sequence(pb_manager* m, int64_t sid) {
  if (!m) return PB_EINVAL;
  auto it = m->seqs.find(sid);
  if (it == m->seqs.end()) return PB_OK;
  for (int32_t f : it->second.table) m->release(f);
  m->seqs.erase(it);
  return PB_OK;
}

pb_status pb_block_tables(const pb_manager* m, const int64_t* sids, int64_t n, int32_t pad,
                          int32_t max_blocks, int32_t* tables_out, int32_t* lens_out) {
  if (!m || n < 0 || max_blocks <= 0 || (n > 0 && (!sids || !tables_out))) return PB_EINVAL;
  for (int64_t i = 0; i < n; ++i) {
    auto it = m->seqs.find(sids[i]);
    if (it == m->seqs.end() || static_cast<int64_t>(it->second.table.size()) > max_blocks ||
        it->second.len > INT32_MAX)
      return PB_EINVAL;
  }
  for (int64_t i = 0; i < n; ++i) {
    const Seq& s = m->seqs.find(sids[i])->second;
    int32_t* row = tables_out + i * static_cast<int64_t>(max_blocks);
    const int64_t k = static_cast<int64_t>(s.table.size());
    for (int64_t b = 0; b < max_blocks; ++b) row[b] = b < k ? s.table[b] : pad;
    if (lens_out) lens_out[i] = static_cast<int32_t>(s.len);
  }
  return PB_OK;
}

pb_status pb_table_length(const pb_manager* m, int64_t sid, int64_t* out) {
  if (!m || !out) return PB_EINVAL;
  auto it = m->seqs.find(sid);
  if (it == m->seqs.end()) return PB_EINVAL;
  *out = static_cast<int64_t>(it->second.table.size());
  return PB_OK;
}

pb_status pb_free_list(const pb_manager* m, int32_t* out, int64_t cap, int64_t* count_out) {
  if (!m || cap < 0 || (cap > 0 && !out) || !count_out) return PB_EINVAL;
  *count_out = static_cast<int64_t>(m->free_list.size());
  int64_t i = 0;
  for (auto it = m->free_list.begin(); it != m->free_list.end() && i < cap; ++it) out[i++] = *it;
  return PB_OK;
}

pb_status pb_ref_counts(const pb_manager* m, int32_t* out) {
  if (!m || !out) return PB_EINVAL;
  std::memcpy(out, m->ref.data(), sizeof(int32_t) * m->ref.size());
  return PB_OK;
}

pb_status pb_get_stats(const pb_manager* m, pb_stats* out) {
  if (!m || !out) return PB_EINVAL;
  out->free_frames = static_cast<int64_t>(m->free_list.size());
  out->cached_frames = static_cast<int64_t>(m->index.size());
  out->hit_blocks = m->hit_blocks;
  out->miss_blocks = m->miss_blocks;
  out->evictions = m->evictions;
  out->sequences = static_cast<int64_t>(m->seqs.size());
  return PB_OK;
}

}  // extern "C"
