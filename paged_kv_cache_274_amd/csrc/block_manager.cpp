// Block manager: which physical 16-token block holds each token of each
// sequence, with prefix sharing, copy on write and swapping (host-only C++; the
// C ABI is in pkv.h).
//
// The pool is the fixed set of 16-token physical blocks reached through a
// per-sequence block table (LLM Inference Server page, Optional Stretch
// Challenges, "Paged KV-Cache Block Allocator"; Mini inference engine page,
// section 2: blocks shared across requests).  Prompts that start with an
// already prefilled prefix reuse its blocks and skip prefill on those tokens,
// with hit/miss counts (LLM Inference Server page, Stage 1 prefix-cache task;
// From Scratch page, "Take it further").  The pool is a fixed budget: an
// operation that needs more blocks than are free fails and changes nothing, so
// the caller can queue the request (Stage 1, footprint-calculator task).
// Sequences can be swapped out to host blocks and back (the preempt/swap of
// the Scheduler box, pipeline figure, From Scratch page).
//
// Policy (the pages leave it open):
//   - free blocks form one FIFO queue, initially 0..n-1; allocation takes the
//     head, a block whose reference count reaches 0 joins the tail, and a freed
//     sequence releases its blocks last block first;
//   - a block that holds tokens stays indexed by (all tokens before it, the
//     tokens it holds) until it is reallocated;
//   - a prompt is matched block by block against the indexed blocks with the
//     same preceding tokens: the longest run of leading tokens wins (ties: the
//     lowest block id); a whole-block match continues, a shorter one ends it;
//     the match never takes the prompt's last token, so at least one query
//     row is always prefilled (the one that yields the first output token);
//   - writing at offset o of a block held by another sequence as well copies
//     it first to a new block (copy on write); a block held alone that has
//     more than o tokens drops them and is written in place;
//   - swap out copies every block of a sequence to host blocks (a FIFO queue
//     of its own) and releases the device blocks; swap in allocates new device
//     blocks.
// "All tokens before it" is an exact identity, never a hash: each distinct
// run of whole blocks from the start of a sequence is interned as a node of a
// prefix trie (key: the parent node and the 16 token ids, compared in full),
// and a block is indexed under the node of its preceding tokens.  A node lives
// while a sequence, an indexed block or a child node refers to it.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <new>
#include <unordered_map>
#include <vector>

#include "pkv.h"

namespace {

constexpr int kB = 16;
constexpr int32_t kRoot = 0;  // the node of the empty prefix

// Trie node key: the node of the tokens before a whole block, and the block's
// 16 token ids.  Equality compares every field; the hash only picks buckets.
struct NodeKey {
  int32_t parent;
  int32_t tok[kB];
  bool operator==(const NodeKey& o) const {
    return parent == o.parent && memcmp(tok, o.tok, sizeof(tok)) == 0;
  }
};
struct NodeKeyHash {
  size_t operator()(const NodeKey& k) const {
    uint64_t h = 0xcbf29ce484222325ull ^ (uint32_t)k.parent;
    for (int i = 0; i < kB; ++i) {
      h ^= (uint32_t)k.tok[i];
      h *= 0x100000001b3ull;
    }
    return (size_t)(h ^ (h >> 29));
  }
};

struct Node {
  NodeKey key;
  int64_t refs = 0;  // sequences' key lists, indexed blocks and child nodes
  bool live = false;
};

struct Block {
  int32_t ref = 0;
  int32_t n_held = 0;
  int32_t held[kB];
  bool indexed = false;
  int32_t before = 0;  // node of the tokens before this block, when indexed
  int32_t prev = -1, next = -1;
  bool in_free = false;
};

struct Seq {
  std::vector<int32_t> table;
  std::vector<int32_t> tokens;
  std::vector<int32_t> keys;  // keys[j] = node of tokens[0 .. 16 j), one reference each
  bool swapped = false;
};

}  // namespace

struct pkv_block_manager {
  std::vector<Block> blocks;
  int32_t free_head = -1, free_tail = -1, n_free = 0;
  std::vector<int32_t> host_free;  // FIFO ring over a vector: [host_pos, end)
  size_t host_pos = 0;
  int32_t n_host = 0;
  bool prefix_cache = true;
  std::unordered_map<int32_t, std::vector<int32_t>> index;  // node -> blocks indexed under it
  std::vector<Node> nodes;
  std::vector<int32_t> free_nodes;
  std::unordered_map<NodeKey, int32_t, NodeKeyHash> node_of;
  std::unordered_map<int64_t, Seq> seqs;
  int64_t hit_tokens = 0, query_tokens = 0, hit_requests = 0, requests = 0;

  // -- free queue ---------------------------------------------------------------
  void push_free(int32_t b) {
    Block& x = blocks[b];
    x.prev = free_tail;
    x.next = -1;
    if (free_tail >= 0) blocks[free_tail].next = b;
    else free_head = b;
    free_tail = b;
    x.in_free = true;
    ++n_free;
  }
  void unlink_free(int32_t b) {
    Block& x = blocks[b];
    if (x.prev >= 0) blocks[x.prev].next = x.next;
    else free_head = x.next;
    if (x.next >= 0) blocks[x.next].prev = x.prev;
    else free_tail = x.prev;
    x.prev = x.next = -1;
    x.in_free = false;
    --n_free;
  }

  // -- prefix trie ------------------------------------------------------------------
  void init_trie() {
    nodes.assign(1, Node());
    nodes[kRoot].live = true;
    nodes[kRoot].refs = 1;  // the root is never released
  }
  static NodeKey key_of(int32_t parent, const int32_t* t) {
    NodeKey k;
    k.parent = parent;
    memcpy(k.tok, t, sizeof(k.tok));
    return k;
  }
  // The node of prefix `parent` followed by the whole block t[0..16), or -1.
  int32_t find_node(int32_t parent, const int32_t* t) const {
    auto it = node_of.find(key_of(parent, t));
    return it == node_of.end() ? -1 : it->second;
  }
  // The same node, created if needed, with one reference taken for the caller.
  int32_t intern(int32_t parent, const int32_t* t) {
    const NodeKey k = key_of(parent, t);
    auto it = node_of.find(k);
    int32_t id;
    if (it != node_of.end()) {
      id = it->second;
    } else {
      if (!free_nodes.empty()) {
        id = free_nodes.back();
        free_nodes.pop_back();
      } else {
        id = (int32_t)nodes.size();
        nodes.emplace_back();
      }
      Node& n = nodes[id];
      n.key = k;
      n.refs = 0;
      n.live = true;
      node_of.emplace(k, id);
      ++nodes[parent].refs;  // the child's reference
    }
    ++nodes[id].refs;
    return id;
  }
  void ref_node(int32_t id) { ++nodes[id].refs; }
  void unref_node(int32_t id) {
    while (id != kRoot && --nodes[id].refs == 0) {
      Node& n = nodes[id];
      node_of.erase(n.key);
      n.live = false;
      free_nodes.push_back(id);
      id = n.key.parent;  // drop the child's reference to its parent
    }
  }
  void release_keys(Seq& s) {
    for (int32_t k : s.keys) unref_node(k);
    s.keys.clear();
  }

  // -- index ----------------------------------------------------------------------
  void unindex(int32_t b) {
    Block& x = blocks[b];
    if (!x.indexed) return;
    auto it = index.find(x.before);
    if (it != index.end()) {
      auto& v = it->second;
      v.erase(std::find(v.begin(), v.end(), b));
      if (v.empty()) index.erase(it);
    }
    x.indexed = false;
    unref_node(x.before);
  }
  void set_index(int32_t b, int32_t before) {
    Block& x = blocks[b];
    if (x.indexed && x.before == before) return;
    ref_node(before);
    unindex(b);
    x.before = before;
    x.indexed = true;
    index[before].push_back(b);
  }
  // Indexed block under node `before` sharing the longest run of leading
  // tokens with t[0..n); returns the run length (0: none).
  int lookup(int32_t before, const int32_t* t, int n, int32_t* best) const {
    auto it = index.find(before);
    if (it == index.end()) return 0;
    int best_m = 0;
    for (int32_t b : it->second) {
      const Block& x = blocks[b];
      int m = 0;
      const int lim = std::min(n, (int)x.n_held);
      while (m < lim && x.held[m] == t[m]) ++m;
      if (m > best_m || (m == best_m && m > 0 && b < *best)) {
        best_m = m;
        *best = b;
      }
    }
    return best_m;
  }

  // -- blocks ---------------------------------------------------------------------
  int32_t alloc() {
    const int32_t b = free_head;
    unlink_free(b);
    unindex(b);
    blocks[b].n_held = 0;
    blocks[b].ref = 1;
    return b;
  }
  void release(int32_t b) {
    if (--blocks[b].ref == 0) push_free(b);
  }
  void claim(int32_t b) {
    if (blocks[b].ref == 0) unlink_free(b);
    ++blocks[b].ref;
  }

  // Blocks the free queue must supply to write n_new more tokens to s.
  int64_t needs(const Seq& s, int64_t n_new) const {
    const int64_t L = (int64_t)s.tokens.size();
    const int64_t fresh = (L + n_new + kB - 1) / kB - (int64_t)s.table.size();
    const bool cow = n_new > 0 && (L % kB) != 0 && blocks[s.table[L / kB]].ref > 1;
    return fresh + (cow ? 1 : 0);
  }

  // The write path: tokens t[0..n) go to positions len(s) ...; slots[i] gets
  // token i's slot; a copy on write is reported in pairs (at most one).
  void write(Seq& s, const int32_t* t, int n, int64_t* slots, int32_t* pairs, int* n_pairs) {
    for (int i = 0; i < n; ++i) {
      const int64_t p = (int64_t)s.tokens.size();
      const int64_t j = p / kB;
      const int o = (int)(p % kB);
      if (j == (int64_t)s.table.size()) s.table.push_back(alloc());
      int32_t b = s.table[j];
      if (blocks[b].ref > 1) {
        const int32_t d = alloc();
        pairs[2 * *n_pairs] = b;
        pairs[2 * *n_pairs + 1] = d;
        ++*n_pairs;
        memcpy(blocks[d].held, blocks[b].held, sizeof(int32_t) * o);
        blocks[d].n_held = o;
        release(b);
        s.table[j] = b = d;
      } else if (blocks[b].n_held > o) {
        blocks[b].n_held = o;
      }
      Block& x = blocks[b];
      x.held[x.n_held++] = t[i];
      s.tokens.push_back(t[i]);
      if (prefix_cache) set_index(b, s.keys[j]);
      if (o == kB - 1) s.keys.push_back(intern(s.keys[j], &s.tokens[j * kB]));
      slots[i] = (int64_t)b * kB + o;
    }
  }
};

namespace {

bool pairs_fit(int need, int max_pairs, const int32_t* pairs) {
  return need <= max_pairs && (need == 0 || pairs != nullptr);
}

}  // namespace

extern "C" {

pkv_block_manager* pkv_bm_create(int n_blocks, int n_host_blocks, int prefix_cache) {
  if (n_blocks < 1 || n_host_blocks < 0) return nullptr;
  pkv_block_manager* m = new (std::nothrow) pkv_block_manager();
  if (!m) return nullptr;
  try {
    m->blocks.resize((size_t)n_blocks);
    m->host_free.reserve((size_t)n_host_blocks);
  } catch (...) {
    delete m;
    return nullptr;
  }
  m->init_trie();
  for (int32_t b = 0; b < n_blocks; ++b) m->push_free(b);
  for (int32_t h = 0; h < n_host_blocks; ++h) m->host_free.push_back(h);
  m->n_host = n_host_blocks;
  m->prefix_cache = prefix_cache != 0;
  return m;
}

void pkv_bm_destroy(pkv_block_manager* m) { delete m; }

int pkv_bm_add_sequence(pkv_block_manager* m, int64_t seq_id, const int32_t* tokens,
                        int n_tokens, int64_t* slots, int32_t* cow_pairs, int* n_cow,
                        int* n_cached) {
  if (!m || n_tokens < 0 || (n_tokens > 0 && (!tokens || !slots)) || !n_cow || !n_cached)
    return PKV_ERR_INVALID_ARG;
  if (m->seqs.count(seq_id)) return PKV_ERR_INVALID_ARG;
  Seq s;
  int pos = 0;
  std::vector<int32_t> matched;
  if (m->prefix_cache) {
    // The match stops short of the last token: its query row must be prefilled.
    const int limit = n_tokens - 1;
    int32_t key = kRoot;
    while (pos < limit) {
      int32_t b = -1;
      const int len = std::min(kB, limit - pos);
      const int mlen = m->lookup(key, tokens + pos, len, &b);
      if (mlen == 0) break;
      matched.push_back(b);
      pos += mlen;
      if (mlen < kB) break;
      key = m->find_node(key, tokens + pos - kB);
      if (key < 0) break;  // no block is indexed after this prefix
    }
  }
  int64_t from_free = 0;
  for (int32_t b : matched) from_free += m->blocks[b].ref == 0;
  const int64_t fresh = ((int64_t)n_tokens + kB - 1) / kB - (int64_t)matched.size();
  const bool cow = pos < n_tokens && (pos % kB) != 0 && m->blocks[matched.back()].ref >= 1;
  if (cow && !cow_pairs) return PKV_ERR_INVALID_ARG;
  if (from_free + fresh + (cow ? 1 : 0) > m->n_free) return PKV_ERR_NO_BLOCKS;
  try {
    s.table.reserve(matched.size() + (size_t)fresh);
    s.tokens.reserve((size_t)n_tokens);
    s.keys.reserve((size_t)n_tokens / kB + 2);
  } catch (...) {
    return PKV_ERR_INVALID_ARG;
  }
  for (int32_t b : matched) {
    m->claim(b);
    s.table.push_back(b);
  }
  m->ref_node(kRoot);
  s.keys.push_back(kRoot);
  for (int i = 0; i < pos; ++i) {
    s.tokens.push_back(tokens[i]);
    if (i % kB == kB - 1) s.keys.push_back(m->intern(s.keys[i / kB], &s.tokens[i + 1 - kB]));
    slots[i] = -1;
  }
  *n_cow = 0;
  m->write(s, tokens + pos, n_tokens - pos, slots + pos, cow_pairs, n_cow);
  m->seqs.emplace(seq_id, std::move(s));
  ++m->requests;
  m->query_tokens += n_tokens;
  m->hit_tokens += pos;
  m->hit_requests += pos > 0;
  *n_cached = pos;
  return PKV_OK;
}

int pkv_bm_append(pkv_block_manager* m, int64_t seq_id, const int32_t* tokens, int n_tokens,
                  int64_t* slots, int32_t* cow_pairs, int* n_cow) {
  if (!m || n_tokens < 0 || (n_tokens > 0 && (!tokens || !slots)) || !n_cow)
    return PKV_ERR_INVALID_ARG;
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end() || it->second.swapped) return PKV_ERR_INVALID_ARG;
  Seq& s = it->second;
  const int64_t need = m->needs(s, n_tokens);
  const int64_t L = (int64_t)s.tokens.size();
  if (n_tokens > 0 && (L % kB) != 0 && m->blocks[s.table[L / kB]].ref > 1 && !cow_pairs)
    return PKV_ERR_INVALID_ARG;
  if (need > m->n_free) return PKV_ERR_NO_BLOCKS;
  *n_cow = 0;
  m->write(s, tokens, n_tokens, slots, cow_pairs, n_cow);
  return PKV_OK;
}

int pkv_bm_append_batch(pkv_block_manager* m, int n, const int64_t* seq_ids,
                        const int32_t* tokens, int64_t* slots, int32_t* cow_pairs, int* n_cow) {
  if (!m || n < 0 || !n_cow || (n > 0 && (!seq_ids || !tokens || !slots || !cow_pairs)))
    return PKV_ERR_INVALID_ARG;
  std::vector<Seq*> ss((size_t)n);
  std::unordered_map<int64_t, int> seen;
  // Blocks the whole step takes from the free queue, in order: a sequence at a
  // block boundary takes a new block; one writing into a block that others
  // still hold takes a copy, after which that block has one holder fewer.
  std::unordered_map<int32_t, int32_t> copied;  // block -> holders gone to copies
  int64_t need = 0;
  for (int i = 0; i < n; ++i) {
    auto it = m->seqs.find(seq_ids[i]);
    if (it == m->seqs.end() || it->second.swapped || seen.count(seq_ids[i]))
      return PKV_ERR_INVALID_ARG;
    seen[seq_ids[i]] = i;
    Seq& s = it->second;
    ss[(size_t)i] = &s;
    const int64_t L = (int64_t)s.tokens.size();
    if (L % kB == 0) {
      ++need;
    } else {
      const int32_t b = s.table[L / kB];
      if (m->blocks[b].ref - copied[b] > 1) {
        ++need;
        ++copied[b];
      }
    }
  }
  if (need > m->n_free) return PKV_ERR_NO_BLOCKS;
  *n_cow = 0;
  for (int i = 0; i < n; ++i) m->write(*ss[(size_t)i], tokens + i, 1, slots + i, cow_pairs, n_cow);
  return PKV_OK;
}

int pkv_bm_block_tables(const pkv_block_manager* m, int n, const int64_t* seq_ids,
                        int32_t* tables, int max_blocks, int32_t* context_lens) {
  if (!m || n < 0 || max_blocks < 0 ||
      (n > 0 && (!seq_ids || !context_lens || (max_blocks > 0 && !tables))))
    return PKV_ERR_INVALID_ARG;
  for (int i = 0; i < n; ++i) {
    auto it = m->seqs.find(seq_ids[i]);
    if (it == m->seqs.end() || it->second.swapped ||
        (int64_t)it->second.table.size() > max_blocks)
      return PKV_ERR_INVALID_ARG;
  }
  for (int i = 0; i < n; ++i) {
    const Seq& s = m->seqs.find(seq_ids[i])->second;
    int32_t* row = tables + (size_t)i * max_blocks;
    const size_t nb = s.table.size();
    if (nb) memcpy(row, s.table.data(), sizeof(int32_t) * nb);
    for (size_t j = nb; j < (size_t)max_blocks; ++j) row[j] = 0;
    context_lens[i] = (int32_t)s.tokens.size();
  }
  return PKV_OK;
}

int pkv_bm_fork(pkv_block_manager* m, int64_t parent, int64_t child) {
  if (!m) return PKV_ERR_INVALID_ARG;
  auto it = m->seqs.find(parent);
  if (it == m->seqs.end() || it->second.swapped || m->seqs.count(child))
    return PKV_ERR_INVALID_ARG;
  Seq c = it->second;
  for (int32_t b : c.table) ++m->blocks[b].ref;
  for (int32_t k : c.keys) m->ref_node(k);
  m->seqs.emplace(child, std::move(c));
  return PKV_OK;
}

int pkv_bm_free(pkv_block_manager* m, int64_t seq_id) {
  if (!m) return PKV_ERR_INVALID_ARG;
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return PKV_ERR_INVALID_ARG;
  Seq& s = it->second;
  for (auto b = s.table.rbegin(); b != s.table.rend(); ++b) {
    if (s.swapped) m->host_free.push_back(*b);
    else m->release(*b);
  }
  m->release_keys(s);
  m->seqs.erase(it);
  return PKV_OK;
}

int pkv_bm_swap_out(pkv_block_manager* m, int64_t seq_id, int32_t* pairs, int max_pairs,
                    int* n_pairs) {
  if (!m || !n_pairs) return PKV_ERR_INVALID_ARG;
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end() || it->second.swapped) return PKV_ERR_INVALID_ARG;
  Seq& s = it->second;
  const int n = (int)s.table.size();
  if (!pairs_fit(n, max_pairs, pairs)) return PKV_ERR_INVALID_ARG;
  if ((size_t)n > m->host_free.size() - m->host_pos) return PKV_ERR_NO_BLOCKS;
  std::vector<int32_t> host(s.table.size());
  for (int j = 0; j < n; ++j) {
    host[j] = m->host_free[m->host_pos++];
    pairs[2 * j] = s.table[j];
    pairs[2 * j + 1] = host[j];
  }
  for (int j = n - 1; j >= 0; --j) m->release(s.table[j]);
  s.table.swap(host);
  s.swapped = true;
  *n_pairs = n;
  // keep the host queue's storage bounded: drop the consumed head
  if (m->host_pos > 4096 && m->host_pos * 2 > m->host_free.size()) {
    m->host_free.erase(m->host_free.begin(), m->host_free.begin() + (long)m->host_pos);
    m->host_pos = 0;
  }
  return PKV_OK;
}

int pkv_bm_swap_in(pkv_block_manager* m, int64_t seq_id, int32_t* pairs, int max_pairs,
                   int* n_pairs) {
  if (!m || !n_pairs) return PKV_ERR_INVALID_ARG;
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end() || !it->second.swapped) return PKV_ERR_INVALID_ARG;
  Seq& s = it->second;
  const int n = (int)s.table.size();
  if (!pairs_fit(n, max_pairs, pairs)) return PKV_ERR_INVALID_ARG;
  if (n > m->n_free) return PKV_ERR_NO_BLOCKS;
  std::vector<int32_t> dev(s.table.size());
  for (int j = 0; j < n; ++j) {
    const int32_t d = m->alloc();
    dev[j] = d;
    Block& x = m->blocks[d];
    const int64_t lo = (int64_t)j * kB;
    const int64_t hi = std::min((int64_t)s.tokens.size(), lo + kB);
    x.n_held = (int32_t)(hi - lo);
    memcpy(x.held, s.tokens.data() + lo, sizeof(int32_t) * (size_t)x.n_held);
    if (m->prefix_cache) m->set_index(d, s.keys[j]);
    pairs[2 * j] = s.table[j];
    pairs[2 * j + 1] = d;
  }
  for (int j = n - 1; j >= 0; --j) m->host_free.push_back(s.table[j]);
  s.table.swap(dev);
  s.swapped = false;
  *n_pairs = n;
  return PKV_OK;
}

int pkv_bm_block_table(const pkv_block_manager* m, int64_t seq_id, int32_t* table,
                       int max_blocks, int* n_blocks, int* seq_len) {
  if (!m || !n_blocks || !seq_len) return PKV_ERR_INVALID_ARG;
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return PKV_ERR_INVALID_ARG;
  const Seq& s = it->second;
  *n_blocks = (int)s.table.size();
  *seq_len = (int)s.tokens.size();
  if (s.swapped || (int)s.table.size() > max_blocks || (!table && !s.table.empty()))
    return PKV_ERR_INVALID_ARG;
  if (!s.table.empty()) memcpy(table, s.table.data(), sizeof(int32_t) * s.table.size());
  return PKV_OK;
}

int pkv_bm_get_stats(const pkv_block_manager* m, pkv_bm_stats* out) {
  if (!m || !out) return PKV_ERR_INVALID_ARG;
  memset(out, 0, sizeof(*out));
  out->n_blocks = (int32_t)m->blocks.size();
  out->free_blocks = m->n_free;
  for (const Block& x : m->blocks) {
    out->cached_blocks += x.indexed;
    out->cached_free_blocks += x.indexed && x.in_free;
  }
  out->n_host_blocks = m->n_host;
  out->host_free_blocks = (int32_t)(m->host_free.size() - m->host_pos);
  out->n_sequences = (int32_t)m->seqs.size();
  out->hit_tokens = m->hit_tokens;
  out->query_tokens = m->query_tokens;
  out->hit_requests = m->hit_requests;
  out->requests = m->requests;
  return PKV_OK;
}

int64_t pkv_kv_cache_bytes(int n_layers, int h_kv, int d_h, int64_t batch, int64_t seq_len,
                           int dtype, int paged) {
  if (n_layers < 0 || h_kv < 0 || d_h < 0 || batch < 0 || seq_len < 0) return -1;
  int64_t row;  // bytes of one token's row of one KV head, K or V
  if (dtype == PKV_F32) row = 4 * (int64_t)d_h;
  else if (dtype == PKV_BF16) row = 2 * (int64_t)d_h;
  else if (dtype == PKV_INT8) row = (int64_t)d_h + 4;  // codes and one float32 scale
  else return -1;
  const int64_t L = paged ? (seq_len + kB - 1) / kB * kB : seq_len;
  return 2 * (int64_t)n_layers * h_kv * row * L * batch;
}

}  // extern "C"
