// Host-side manager of a paged KV pool's pages: fixed-size pages taken
// from and returned to a free pool in O(1), one page list per sequence
// (its block-table row), sequences forked by sharing their full pages, and
// a prefix cache that lets a new sequence take over the full pages of an
// earlier one whose tokens match (the rkmt page, "从零构建 Qwen3-8B 推理引擎",
// sections 4.3.1 on the paged KV cache and 4.4.4 on the automatic prefix
// cache).  Plain C++ behind the C ABI in qd.h; no GPU work.
//
// Page states: referenced by one or more sequences (refcount > 0); cached
// (refcount 0, its content registered under a prefix key, kept for reuse
// until the pool runs out); free.  A page is shared only while full, so a
// sequence appends only to pages it owns alone.
#include <cstdint>
#include <cstring>
#include <list>
#include <map>
#include <string>
#include <unordered_map>
#include <vector>

#include "qd.h"

namespace {

constexpr int kPageTokens = 16;

// Key of a full cached page: the serial number its predecessor in the
// sequence got when it was cached (0 for a first page) and its own 16
// tokens, so that a key names the whole prefix exactly in constant size.
// Serial numbers are never reused: evicting a page makes every key built on
// it unreachable (those pages age out of the cache in turn).
struct PrefixKey {
  uint64_t parent;
  int32_t tokens[kPageTokens];
  bool operator==(const PrefixKey& o) const {
    return parent == o.parent && std::memcmp(tokens, o.tokens, sizeof(tokens)) == 0;
  }
};
struct PrefixHash {
  size_t operator()(const PrefixKey& k) const {
    uint64_t h = 1469598103934665603ull ^ k.parent;  // FNV-1a over the key's words
    for (int32_t t : k.tokens) {
      h ^= (uint32_t)t;
      h *= 1099511628211ull;
    }
    return (size_t)h;
  }
};

struct Page {
  int refs = 0;
  bool cached = false;
  uint64_t serial = 0;               // while cached
  std::list<int32_t>::iterator lru;  // position in the eviction order while cached and unreferenced
  const PrefixKey* key = nullptr;    // its entry in the prefix table while cached
};

struct Seq {
  std::vector<int32_t> pages;
  int32_t tokens = 0;  // token positions reserved: its pages cover [0, tokens)
};

}  // namespace

struct qd_blocks {
  int32_t num_pages = 0, max_pages = 0;
  std::vector<Page> page;
  std::vector<int32_t> free_stack;  // free pages, next taken from the back
  std::list<int32_t> lru;            // cached, unreferenced pages: front = evicted first
  std::unordered_map<PrefixKey, int32_t, PrefixHash> table;
  uint64_t next_serial = 1;
  std::map<int64_t, Seq> seqs;
};

namespace {

// Pages obtainable now: free ones, then cached unreferenced ones.
int32_t available(const qd_blocks* m) {
  return (int32_t)m->free_stack.size() + (int32_t)m->lru.size();
}

// Take one page (refcount 1); the caller checked availability.
int32_t take(qd_blocks* m) {
  int32_t p;
  if (!m->free_stack.empty()) {
    p = m->free_stack.back();
    m->free_stack.pop_back();
  } else {  // evict the least recently released cached page
    p = m->lru.front();
    m->lru.pop_front();
    Page& pg = m->page[p];
    m->table.erase(*pg.key);
    pg.key = nullptr;
    pg.cached = false;
    pg.serial = 0;
  }
  m->page[p].refs = 1;
  return p;
}

void add_ref(qd_blocks* m, int32_t p) {
  Page& pg = m->page[p];
  if (pg.refs == 0 && pg.cached) m->lru.erase(pg.lru);
  ++pg.refs;
}

void drop_ref(qd_blocks* m, int32_t p) {
  Page& pg = m->page[p];
  if (--pg.refs > 0) return;
  if (pg.cached) {
    m->lru.push_back(p);
    pg.lru = std::prev(m->lru.end());
  } else {
    m->free_stack.push_back(p);
  }
}

}  // namespace

extern "C" {

int qd_blocks_create(int32_t num_pages, int32_t max_pages_per_seq, qd_blocks** out) {
  if (!out) return QD_EINVAL;
  *out = nullptr;
  if (num_pages < 1 || max_pages_per_seq < 1) return QD_EINVAL;
  qd_blocks* m = new qd_blocks();
  m->num_pages = num_pages;
  m->max_pages = max_pages_per_seq;
  m->page.resize(num_pages);
  m->free_stack.reserve(num_pages);
  for (int32_t p = num_pages - 1; p >= 0; --p) m->free_stack.push_back(p);  // page 0 first
  *out = m;
  return QD_OK;
}

void qd_blocks_destroy(qd_blocks* m) { delete m; }

int qd_blocks_add(qd_blocks* m, int64_t seq) {
  if (!m) return QD_EINVAL;
  if (m->seqs.count(seq)) return QD_EINVAL;
  m->seqs[seq] = Seq{};
  return QD_OK;
}

int qd_blocks_reserve(qd_blocks* m, int64_t seq, int32_t n_tokens) {
  if (!m || n_tokens < 0) return QD_EINVAL;
  auto it = m->seqs.find(seq);
  if (it == m->seqs.end()) return QD_EINVAL;
  Seq& s = it->second;
  if (n_tokens > m->max_pages * kPageTokens) return QD_EUNSUPPORTED;
  const int32_t need = (n_tokens + kPageTokens - 1) / kPageTokens;
  const int32_t more = need - (int32_t)s.pages.size();
  if (more > available(m)) return QD_ENOMEM;  // nothing changes
  for (int32_t i = 0; i < more; ++i) s.pages.push_back(take(m));
  if (n_tokens > s.tokens) s.tokens = n_tokens;
  return QD_OK;
}

int qd_blocks_release(qd_blocks* m, int64_t seq) {
  if (!m) return QD_EINVAL;
  auto it = m->seqs.find(seq);
  if (it == m->seqs.end()) return QD_EINVAL;
  // last page first: a cached chain is evicted from its end, so that its
  // prefix stays reachable longest
  const std::vector<int32_t>& pg = it->second.pages;
  for (auto r = pg.rbegin(); r != pg.rend(); ++r) drop_ref(m, *r);
  m->seqs.erase(it);
  return QD_OK;
}

int qd_blocks_fork(qd_blocks* m, int64_t src, int64_t dst, int32_t* copy_src,
                   int32_t* copy_dst) {
  if (!m || !copy_src || !copy_dst) return QD_EINVAL;
  auto si = m->seqs.find(src);
  if (si == m->seqs.end() || m->seqs.count(dst)) return QD_EINVAL;
  const Seq& s = si->second;
  const int32_t full = s.tokens / kPageTokens;
  const bool partial = (int32_t)s.pages.size() > full;
  if (partial && available(m) < 1) return QD_ENOMEM;
  Seq d;
  d.tokens = s.tokens;
  for (int32_t i = 0; i < full; ++i) {
    add_ref(m, s.pages[i]);
    d.pages.push_back(s.pages[i]);
  }
  *copy_src = *copy_dst = -1;
  if (partial) {  // the page being filled is never shared: a fresh one to copy into
    const int32_t p = take(m);
    d.pages.push_back(p);
    *copy_src = s.pages[full];
    *copy_dst = p;
  }
  // pages reserved past the partial one stay with the source
  m->seqs[dst] = std::move(d);
  return partial ? 1 : 0;
}

int qd_blocks_tables(const qd_blocks* m, const int64_t* seqs, int32_t n, int32_t pad_page,
                     int32_t* out) {
  if (!m || n < 0 || (n > 0 && (!seqs || !out))) return QD_EINVAL;
  for (int32_t i = 0; i < n; ++i) {
    auto it = m->seqs.find(seqs[i]);
    if (it == m->seqs.end()) return QD_EINVAL;
  }
  for (int32_t i = 0; i < n; ++i) {
    const Seq& s = m->seqs.find(seqs[i])->second;
    int32_t* row = out + (size_t)i * m->max_pages;
    for (int32_t j = 0; j < m->max_pages; ++j)
      row[j] = j < (int32_t)s.pages.size() ? s.pages[j] : pad_page;
  }
  return QD_OK;
}

int qd_blocks_length(const qd_blocks* m, int64_t seq) {
  if (!m) return QD_EINVAL;
  auto it = m->seqs.find(seq);
  return it == m->seqs.end() ? QD_EINVAL : it->second.tokens;
}

int qd_blocks_available(const qd_blocks* m) { return m ? available(m) : QD_EINVAL; }

int qd_blocks_publish(qd_blocks* m, int64_t seq, const int32_t* tokens, int32_t n) {
  if (!m || n < 0 || (n > 0 && !tokens)) return QD_EINVAL;
  auto it = m->seqs.find(seq);
  if (it == m->seqs.end()) return QD_EINVAL;
  const Seq& s = it->second;
  if (n > s.tokens) return QD_EINVAL;
  int32_t added = 0;
  PrefixKey key{};
  key.parent = 0;
  for (int32_t i = 0; i < n / kPageTokens; ++i) {
    std::memcpy(key.tokens, tokens + i * kPageTokens, sizeof(key.tokens));
    auto hit = m->table.find(key);
    if (hit != m->table.end()) {  // this prefix is cached already (possibly as this very page)
      key.parent = m->page[hit->second].serial;
      continue;
    }
    Page& pg = m->page[s.pages[i]];
    if (pg.cached) break;  // the page holds another prefix's content: the chain ends here
    auto ins = m->table.emplace(key, s.pages[i]);
    pg.cached = true;
    pg.key = &ins.first->first;
    pg.serial = m->next_serial++;
    key.parent = pg.serial;
    ++added;
  }
  return added;
}

int qd_blocks_match(qd_blocks* m, int64_t seq, const int32_t* tokens, int32_t n) {
  if (!m || n < 0 || (n > 0 && !tokens)) return QD_EINVAL;
  auto it = m->seqs.find(seq);
  if (it == m->seqs.end() || !it->second.pages.empty()) return QD_EINVAL;
  Seq& s = it->second;
  PrefixKey key{};
  key.parent = 0;
  int32_t i = 0;
  for (; i < n / kPageTokens && i < m->max_pages; ++i) {
    std::memcpy(key.tokens, tokens + i * kPageTokens, sizeof(key.tokens));
    auto hit = m->table.find(key);
    if (hit == m->table.end()) break;
    add_ref(m, hit->second);
    s.pages.push_back(hit->second);
    key.parent = m->page[hit->second].serial;
  }
  s.tokens = i * kPageTokens;
  return s.tokens;
}

}  // extern "C"
