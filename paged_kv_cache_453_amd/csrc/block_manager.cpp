// Block manager: which physical block holds which tokens of which sequence.
//
// Host-side bookkeeping in front of the attention kernels ("vLLM 基本原理",
// section PagedAttention, items 1-3): a pool of fixed-size physical blocks, a
// block table per sequence, blocks taken only when a sequence's last block is
// full ("按需分配"), blocks shared between sequences with reference counts and
// copied when a sharer writes into a partly filled one (intelliparadigm.com
// article, sections 2.2 and 3.3; "vLLM 基本原理", 内存共享), the three sharing
// modes of the same article's section 2.3 (whole sequence, prefix, chosen
// blocks), blocks returned as soon as a sequence ends (xdnf.cn article, section
// 六.1), and a second pool in host memory to swap sequences out to
// (intelliparadigm.com article, section 5.1, swap space).
//
// Policy choices the pages leave open:
//  * free blocks form a stack (the most recently released block is reused
//    first; at the start ids come out in increasing order), and a released
//    table goes back last entry first;
//  * every operation is all-or-nothing;
//  * data movement is recorded as (src, dst) pairs and handed out by
//    pa_bm_take_moves(); a block named by a pending pair that drops to zero
//    references is held back from the free stack until then, and an operation
//    that would read a pending destination is refused, so the pairs of one
//    batch never overlap and can run in any order -- all at once on the GPU;
//  * a sequence that reserved slots since the last take cannot be forked,
//    shared from or swapped out, since its new tokens are not in its blocks yet.
//
// Prefix cache (xdnf.cn article, section 六.3: a hash per KV block; a request
// whose prefix blocks hit reuses them; a hit needs the same model, precision,
// quantisation and adapter, the same tokens from position 0, and whole
// blocks):
//  * a block's key chains FNV-1a 64 over (previous key, salt, its 16 token
//    ids); the salt stands for everything besides the tokens that must match;
//  * a full block enters the cache at the end of the batch that filled it,
//    if the sequence that filled it still holds it; a hit is verified exactly
//    (salt, the 16 tokens, and the parent being the previous hit), and a key
//    whose entry fails that check is taken over by the new block;
//  * a prompt reuses at most the full blocks before its last token;
//  * cached blocks nobody holds stay cached; allocation takes uncached idle
//    blocks first and only then evicts the cached block idle the longest.
#include <stdint.h>

#include <algorithm>
#include <new>
#include <unordered_map>
#include <utility>
#include <vector>

#include "pa.h"

namespace {

struct Pool {
  std::vector<int32_t> free_stack;   // idle blocks without cached contents; back() is the top
  std::vector<int32_t> ref;
  std::vector<int32_t> held;         // released while named by a pending pair
  std::vector<uint8_t> pending;      // named by a pending pair
  std::vector<uint8_t> pending_dst;  // destination of a pending pair
  std::vector<int32_t> marked;       // blocks whose pending flags are set
  // idle blocks with cached contents, oldest first: a doubly linked list
  std::vector<int32_t> lru_prev, lru_next;
  std::vector<uint8_t> in_lru;
  int32_t lru_head = -1, lru_tail = -1;
  int64_t lru_size = 0;
  const std::vector<uint8_t>* cached = nullptr;   // per block: holds a cache entry
  void (*evict)(void*, int32_t) = nullptr;        // drops a block's cache entry
  void* evict_ctx = nullptr;

  void init(int64_t n) {
    free_stack.resize((size_t)n);
    for (int64_t i = 0; i < n; ++i) free_stack[(size_t)i] = (int32_t)(n - 1 - i);
    ref.assign((size_t)n, 0);
    pending.assign((size_t)n, 0);
    pending_dst.assign((size_t)n, 0);
    lru_prev.assign((size_t)n, -1);
    lru_next.assign((size_t)n, -1);
    in_lru.assign((size_t)n, 0);
  }
  int64_t size() const { return (int64_t)ref.size(); }
  int64_t num_idle() const { return (int64_t)free_stack.size() + lru_size; }
  bool is_cached(int32_t b) const { return cached && (*cached)[b]; }
  void lru_push(int32_t b) {
    lru_prev[b] = lru_tail;
    lru_next[b] = -1;
    if (lru_tail >= 0) lru_next[lru_tail] = b; else lru_head = b;
    lru_tail = b;
    in_lru[b] = 1;
    ++lru_size;
  }
  void lru_remove(int32_t b) {
    const int32_t p = lru_prev[b], n = lru_next[b];
    if (p >= 0) lru_next[p] = n; else lru_head = n;
    if (n >= 0) lru_prev[n] = p; else lru_tail = p;
    in_lru[b] = 0;
    --lru_size;
  }
  int32_t take() {
    int32_t b;
    if (!free_stack.empty()) {
      b = free_stack.back();
      free_stack.pop_back();
    } else {
      b = lru_head;
      lru_remove(b);
      evict(evict_ctx, b);
    }
    ref[b] = 1;
    return b;
  }
  void park(int32_t b) {
    if (is_cached(b)) lru_push(b); else free_stack.push_back(b);
  }
  void release(int32_t b) {
    if (--ref[b] == 0) {
      if (pending[b]) held.push_back(b); else park(b);
    }
  }
  void revive(int32_t b) {
    const auto it = std::find(held.begin(), held.end(), b);
    if (it != held.end()) held.erase(it); else lru_remove(b);
    ref[b] = 1;
  }
  void mark(int32_t b, bool dst) {
    if (!pending[b]) {
      pending[b] = 1;
      marked.push_back(b);
    }
    if (dst) pending_dst[b] = 1;
  }
  void settle() {
    for (int32_t b : held) park(b);
    held.clear();
    for (int32_t b : marked) pending[b] = pending_dst[b] = 0;
    marked.clear();
  }
};

struct Sequence {
  std::vector<int32_t> table;
  int64_t num_tokens = 0;
  bool on_host = false;
  bool dirty = false;  // reserved slots since the last take of the moves
  uint64_t serial = 0;  // creation number
  // prefix cache: the token ids (sequences created from a prompt, or forked
  // from one), the salt and the keys of the full blocks
  bool tracks_tokens = false;
  std::vector<int32_t> tokens;
  uint64_t salt = 0;
  std::vector<uint64_t> keys;
};

using Pair = std::pair<int32_t, int32_t>;
constexpr int kBs = 16;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// FNV-1a, 64 bits: for each byte, xor it in, then multiply by the prime.
constexpr uint64_t kFnvOffset = 0xCBF29CE484222325ull;
constexpr uint64_t kFnvPrime = 0x100000001B3ull;
uint64_t fnv1a64_bytes(const uint8_t* p, size_t n, uint64_t h = kFnvOffset) {
  for (size_t i = 0; i < n; ++i) {
    h ^= p[i];
    h *= kFnvPrime;
  }
  return h;
}

// Chained key of one full block: FNV-1a over the parent key, the salt (both
// 8 bytes) and the 16 token ids (4 bytes each), little-endian.
uint64_t block_key(uint64_t parent, uint64_t salt, const int32_t* tokens) {
  uint8_t buf[16 + 4 * kBs];
  for (int i = 0; i < 8; ++i) {
    buf[i] = (uint8_t)(parent >> (8 * i));
    buf[8 + i] = (uint8_t)(salt >> (8 * i));
  }
  for (int t = 0; t < kBs; ++t)
    for (int i = 0; i < 4; ++i) buf[16 + 4 * t + i] = (uint8_t)((uint32_t)tokens[t] >> (8 * i));
  return fnv1a64_bytes(buf, sizeof buf);
}

struct Registration {     // a block filled in the current batch
  uint64_t serial;
  int64_t seq;
  int32_t j, block, parent;
  uint64_t key, salt;
  int32_t tokens[kBs];
};

}  // namespace

struct pa_block_manager {
  int block_size = 16;
  Pool dev, host;
  std::unordered_map<int64_t, Sequence> seqs;
  std::vector<int64_t> dirty;
  std::vector<Pair> copies, swapped_out, swapped_in;
  uint64_t next_serial = 0;
  // prefix cache over the device pool
  std::unordered_map<uint64_t, int32_t> cache;   // key -> block
  std::vector<uint8_t> cached;                   // per block: holds a cache entry
  std::vector<uint64_t> meta_key, meta_salt;
  std::vector<int32_t> meta_parent, meta_tokens; // meta_tokens: 16 per block
  std::vector<Registration> to_register;

  void init_cache(int64_t n) {
    cached.assign((size_t)n, 0);
    meta_key.assign((size_t)n, 0);
    meta_salt.assign((size_t)n, 0);
    meta_parent.assign((size_t)n, -1);
    meta_tokens.assign((size_t)n * kBs, 0);
    dev.cached = &cached;
    dev.evict = [](void* ctx, int32_t b) { static_cast<pa_block_manager*>(ctx)->evict_block(b); };
    dev.evict_ctx = this;
  }
  void evict_block(int32_t b) {
    cache.erase(meta_key[b]);
    cached[b] = 0;
  }
  // b loses its entry; an idle b moves from the cached list to the plain stack
  void uncache(int32_t b) {
    cached[b] = 0;
    if (dev.in_lru[b]) {
      dev.lru_remove(b);
      dev.free_stack.push_back(b);
    }
  }
  bool meta_matches(int32_t b, int32_t parent, uint64_t salt, const int32_t* tokens) const {
    return meta_parent[b] == parent && meta_salt[b] == salt &&
           std::equal(tokens, tokens + kBs, meta_tokens.begin() + (size_t)b * kBs);
  }
  Sequence& create(int64_t id) {
    Sequence& s = seqs[id];
    s.serial = next_serial++;
    return s;
  }
  void lookup(const int32_t* tokens, int64_t max_blocks, uint64_t salt,
              std::vector<int32_t>& hits, std::vector<uint64_t>& keys) const;
  void commit_registrations();

  Sequence* find(int64_t id) {
    auto it = seqs.find(id);
    return it == seqs.end() ? nullptr : &it->second;
  }
  const Sequence* find(int64_t id) const {
    auto it = seqs.find(id);
    return it == seqs.end() ? nullptr : &it->second;
  }
  // A copy on write is due when the last block is partly filled and shared.
  bool cow_needed(const Sequence& s, int64_t n) const {
    return n > 0 && s.num_tokens % block_size != 0 && dev.ref[s.table.back()] > 1;
  }
  int64_t blocks_needed(const Sequence& s, int64_t n) const {
    const int64_t fresh = ceil_div(s.num_tokens + n, block_size) - ceil_div(s.num_tokens, block_size);
    return fresh + (cow_needed(s, n) ? 1 : 0);
  }
  void mark_dirty(int64_t id, Sequence& s) {
    if (!s.dirty) {
      s.dirty = true;
      dirty.push_back(id);
    }
  }
  int append(int64_t id, int64_t n, int64_t* slots);
  int swap(const int64_t* ids, int32_t count, bool to_host);
};

void pa_block_manager::lookup(const int32_t* tokens, int64_t max_blocks, uint64_t salt,
                              std::vector<int32_t>& hits, std::vector<uint64_t>& keys) const {
  uint64_t key = 0;
  int32_t parent = -1;
  for (int64_t j = 0; j < max_blocks; ++j) {
    const int32_t* blk = tokens + j * kBs;
    key = block_key(key, salt, blk);
    const auto it = cache.find(key);
    if (it == cache.end() || !meta_matches(it->second, parent, salt, blk)) break;
    hits.push_back(it->second);
    keys.push_back(key);
    parent = it->second;
  }
}

void pa_block_manager::commit_registrations() {
  for (const Registration& r : to_register) {
    const Sequence* s = find(r.seq);
    if (!s || s->serial != r.serial || s->on_host || s->table[(size_t)r.j] != r.block) continue;
    const auto it = cache.find(r.key);
    if (it != cache.end()) {
      if (meta_matches(it->second, r.parent, r.salt, r.tokens)) continue;
      uncache(it->second);          // a stale or colliding entry gives way
    }
    cache[r.key] = r.block;
    cached[r.block] = 1;
    meta_key[r.block] = r.key;
    meta_salt[r.block] = r.salt;
    meta_parent[r.block] = r.parent;
    std::copy(r.tokens, r.tokens + kBs, meta_tokens.begin() + (size_t)r.block * kBs);
  }
  to_register.clear();
}

int pa_block_manager::append(int64_t id, int64_t n, int64_t* slots) {
  Sequence* s = find(id);
  if (!s || s->on_host) return PA_ERR_SEQ;
  if (n < 0) return PA_ERR_SHAPE;
  if (n > 0 && !slots) return PA_ERR_NULL;
  if (cow_needed(*s, n) && dev.pending_dst[s->table.back()]) return PA_ERR_BUSY;
  if (blocks_needed(*s, n) > dev.num_idle()) return PA_ERR_NO_BLOCKS;
  const int64_t bs = block_size;
  for (int64_t i = 0; i < n; ++i) {
    const int64_t pos = s->num_tokens;
    if (pos % bs == 0) {
      s->table.push_back(dev.take());
    } else if (dev.ref[s->table.back()] > 1) {
      const int32_t old = s->table.back();
      const int32_t fresh = dev.take();
      copies.emplace_back(old, fresh);
      dev.mark(old, false);
      dev.mark(fresh, true);
      dev.release(old);
      s->table.back() = fresh;
    }
    slots[i] = (int64_t)s->table.back() * bs + pos % bs;
    s->num_tokens = pos + 1;
  }
  if (n > 0) mark_dirty(id, *s);
  return PA_OK;
}

int pa_block_manager::swap(const int64_t* ids, int32_t count, bool to_host) {
  Pool& src = to_host ? dev : host;
  Pool& dst = to_host ? host : dev;
  std::vector<Sequence*> list;
  list.reserve((size_t)count);
  for (int32_t i = 0; i < count; ++i) {
    for (int32_t j = 0; j < i; ++j)
      if (ids[j] == ids[i]) return PA_ERR_SEQ;
    Sequence* s = find(ids[i]);
    if (!s || s->on_host == to_host) return PA_ERR_SEQ;
    list.push_back(s);
  }
  for (Sequence* s : list)
    if (s->dirty) return PA_ERR_BUSY;
  std::unordered_map<int32_t, int32_t> moved;
  int64_t distinct = 0;
  for (Sequence* s : list)
    for (int32_t b : s->table)
      if (moved.emplace(b, -1).second) {
        if (src.pending_dst[b]) return PA_ERR_BUSY;
        ++distinct;
      }
  if (distinct > dst.num_idle()) return PA_ERR_NO_BLOCKS;
  std::vector<Pair>& record = to_host ? swapped_out : swapped_in;
  for (Sequence* s : list) {
    for (int32_t& b : s->table) {
      int32_t& to = moved[b];
      if (to >= 0) {
        ++dst.ref[to];
      } else {
        to = dst.take();
        record.emplace_back(b, to);
        src.mark(b, false);
        dst.mark(to, true);
      }
      src.release(b);
      b = to;
    }
    s->on_host = to_host;
  }
  return PA_OK;
}

extern "C" {

int pa_bm_create(int64_t num_blocks, int64_t num_host_blocks, int block_size,
                 pa_block_manager** out) {
  if (!out) return PA_ERR_NULL;
  *out = nullptr;
  if (block_size != 16) return PA_ERR_UNSUPPORTED;
  if (num_blocks < 1 || num_blocks > INT32_MAX || num_host_blocks < 0 ||
      num_host_blocks > INT32_MAX)
    return PA_ERR_SHAPE;
  pa_block_manager* bm = new (std::nothrow) pa_block_manager;
  if (!bm) return PA_ERR_NO_MEMORY;
  try {
    bm->block_size = block_size;
    bm->dev.init(num_blocks);
    bm->host.init(num_host_blocks);
    bm->init_cache(num_blocks);
  } catch (...) {
    delete bm;
    return PA_ERR_NO_MEMORY;
  }
  *out = bm;
  return PA_OK;
}

void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

int pa_bm_add_sequence(pa_block_manager* bm, int64_t seq) {
  if (!bm) return PA_ERR_NULL;
  if (bm->find(seq)) return PA_ERR_SEQ;
  try {
    bm->create(seq);
  } catch (...) {
    return PA_ERR_NO_MEMORY;
  }
  return PA_OK;
}

int pa_bm_fork(pa_block_manager* bm, int64_t parent, int64_t child) {
  if (!bm) return PA_ERR_NULL;
  const Sequence* p = bm->find(parent);
  if (!p || p->on_host) return PA_ERR_SEQ;
  if (p->dirty) return PA_ERR_BUSY;
  if (bm->find(child)) return PA_ERR_SEQ;
  try {
    const Sequence parent_copy = *p;
    Sequence& c = bm->create(child);
    c.table = parent_copy.table;
    c.num_tokens = parent_copy.num_tokens;
    c.tracks_tokens = parent_copy.tracks_tokens;
    c.tokens = parent_copy.tokens;
    c.salt = parent_copy.salt;
    c.keys = parent_copy.keys;
  } catch (...) {
    bm->seqs.erase(child);
    return PA_ERR_NO_MEMORY;
  }
  for (int32_t b : bm->find(child)->table) ++bm->dev.ref[b];
  return PA_OK;
}

int pa_bm_share(pa_block_manager* bm, int64_t src, int64_t dst, const int32_t* logical_blocks,
                int32_t count) {
  if (!bm) return PA_ERR_NULL;
  if (count > 0 && !logical_blocks) return PA_ERR_NULL;
  const Sequence* s = bm->find(src);
  if (!s || s->on_host) return PA_ERR_SEQ;
  if (s->dirty) return PA_ERR_BUSY;
  if (bm->find(dst)) return PA_ERR_SEQ;
  if (count < 0) return PA_ERR_SHAPE;
  const int64_t full = s->num_tokens / bm->block_size;
  for (int32_t i = 0; i < count; ++i)
    if (logical_blocks[i] < 0 || logical_blocks[i] >= full) return PA_ERR_SHAPE;
  try {
    std::vector<int32_t> table;
    table.reserve((size_t)count);
    for (int32_t i = 0; i < count; ++i) table.push_back(s->table[(size_t)logical_blocks[i]]);
    Sequence& d = bm->create(dst);
    d.table = std::move(table);
    d.num_tokens = (int64_t)count * bm->block_size;
  } catch (...) {
    bm->seqs.erase(dst);
    return PA_ERR_NO_MEMORY;
  }
  for (int32_t b : bm->find(dst)->table) ++bm->dev.ref[b];
  return PA_OK;
}

int pa_bm_free_sequence(pa_block_manager* bm, int64_t seq) {
  if (!bm) return PA_ERR_NULL;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return PA_ERR_SEQ;
  Pool& pool = it->second.on_host ? bm->host : bm->dev;
  const std::vector<int32_t>& t = it->second.table;
  for (auto b = t.rbegin(); b != t.rend(); ++b) pool.release(*b);
  bm->seqs.erase(it);
  return PA_OK;
}

int pa_bm_append_slots(pa_block_manager* bm, int64_t seq, int32_t count, int64_t* slots) {
  if (!bm) return PA_ERR_NULL;
  try {
    return bm->append(seq, count, slots);
  } catch (...) {
    return PA_ERR_NO_MEMORY;
  }
}

int pa_bm_append_batch(pa_block_manager* bm, const int64_t* seqs, const int32_t* counts,
                       int32_t num_seqs, int64_t* slot_mapping, int32_t* num_done) {
  if (!bm || !num_done) return PA_ERR_NULL;
  *num_done = 0;
  if (num_seqs < 0) return PA_ERR_SHAPE;
  if (num_seqs > 0 && (!seqs || !counts)) return PA_ERR_NULL;
  int64_t total = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    if (counts[i] < 0) return PA_ERR_SHAPE;
    total += counts[i];
  }
  if (total > 0 && !slot_mapping) return PA_ERR_NULL;
  int64_t off = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    int st;
    try {
      st = bm->append(seqs[i], counts[i], slot_mapping + off);
    } catch (...) {
      st = PA_ERR_NO_MEMORY;
    }
    if (st != PA_OK) return st;
    off += counts[i];
    *num_done = i + 1;
  }
  return PA_OK;
}

int pa_bm_swap_out(pa_block_manager* bm, const int64_t* seqs, int32_t count) {
  if (!bm) return PA_ERR_NULL;
  if (count < 0) return PA_ERR_SHAPE;
  if (count > 0 && !seqs) return PA_ERR_NULL;
  try {
    return bm->swap(seqs, count, true);
  } catch (...) {
    return PA_ERR_NO_MEMORY;
  }
}

int pa_bm_swap_in(pa_block_manager* bm, const int64_t* seqs, int32_t count) {
  if (!bm) return PA_ERR_NULL;
  if (count < 0) return PA_ERR_SHAPE;
  if (count > 0 && !seqs) return PA_ERR_NULL;
  try {
    return bm->swap(seqs, count, false);
  } catch (...) {
    return PA_ERR_NO_MEMORY;
  }
}

int pa_bm_pending_moves(const pa_block_manager* bm, int64_t* counts) {
  if (!bm || !counts) return PA_ERR_NULL;
  counts[0] = (int64_t)bm->copies.size();
  counts[1] = (int64_t)bm->swapped_out.size();
  counts[2] = (int64_t)bm->swapped_in.size();
  return PA_OK;
}

int pa_bm_take_moves(pa_block_manager* bm, int32_t* copies, int32_t* swap_out, int32_t* swap_in) {
  if (!bm) return PA_ERR_NULL;
  if ((!bm->copies.empty() && !copies) || (!bm->swapped_out.empty() && !swap_out) ||
      (!bm->swapped_in.empty() && !swap_in))
    return PA_ERR_NULL;
  const std::pair<std::vector<Pair>*, int32_t*> lists[3] = {
      {&bm->copies, copies}, {&bm->swapped_out, swap_out}, {&bm->swapped_in, swap_in}};
  for (const auto& l : lists) {
    for (size_t i = 0; i < l.first->size(); ++i) {
      l.second[2 * i] = (*l.first)[i].first;
      l.second[2 * i + 1] = (*l.first)[i].second;
    }
    l.first->clear();
  }
  for (int64_t id : bm->dirty) {
    Sequence* s = bm->find(id);
    if (s) s->dirty = false;
  }
  bm->dirty.clear();
  bm->commit_registrations();
  bm->dev.settle();
  bm->host.settle();
  return PA_OK;
}

int pa_bm_num_tokens(const pa_block_manager* bm, int64_t seq, int64_t* num_tokens) {
  if (!bm || !num_tokens) return PA_ERR_NULL;
  const Sequence* s = bm->find(seq);
  if (!s) return PA_ERR_SEQ;
  *num_tokens = s->num_tokens;
  return PA_OK;
}

int pa_bm_is_swapped(const pa_block_manager* bm, int64_t seq, int32_t* swapped) {
  if (!bm || !swapped) return PA_ERR_NULL;
  const Sequence* s = bm->find(seq);
  if (!s) return PA_ERR_SEQ;
  *swapped = s->on_host ? 1 : 0;
  return PA_OK;
}

int pa_bm_block_table(const pa_block_manager* bm, int64_t seq, int32_t* table, int32_t capacity,
                      int32_t* length) {
  if (!bm || !length) return PA_ERR_NULL;
  const Sequence* s = bm->find(seq);
  if (!s) return PA_ERR_SEQ;
  const int64_t n = (int64_t)s->table.size();
  if (n > INT32_MAX) return PA_ERR_SHAPE;
  *length = (int32_t)n;
  if (capacity < n) return PA_ERR_SHAPE;
  if (n > 0 && !table) return PA_ERR_NULL;
  std::copy(s->table.begin(), s->table.end(), table);
  return PA_OK;
}

int64_t pa_bm_num_free(const pa_block_manager* bm, int host) {
  if (!bm) return PA_ERR_NULL;
  return (host ? bm->host : bm->dev).num_idle();
}

int pa_bm_prefix_keys(const int32_t* tokens, int64_t num_tokens, uint64_t salt, uint64_t* keys) {
  if (num_tokens < 0) return PA_ERR_SHAPE;
  const int64_t nb = num_tokens / kBs;
  if (nb > 0 && (!tokens || !keys)) return PA_ERR_NULL;
  uint64_t key = 0;
  for (int64_t j = 0; j < nb; ++j) keys[j] = key = block_key(key, salt, tokens + j * kBs);
  return PA_OK;
}

int pa_bm_add_prompt(pa_block_manager* bm, int64_t seq, const int32_t* tokens,
                     int64_t num_tokens, uint64_t salt, int64_t* num_cached_tokens) {
  if (!bm || !num_cached_tokens) return PA_ERR_NULL;
  if (num_tokens < 0) return PA_ERR_SHAPE;
  if (num_tokens > 0 && !tokens) return PA_ERR_NULL;
  if (bm->find(seq)) return PA_ERR_SEQ;
  try {
    std::vector<int32_t> hits;
    std::vector<uint64_t> keys;
    const int64_t max_blocks = num_tokens > 0 ? (num_tokens - 1) / kBs : 0;
    bm->lookup(tokens, max_blocks, salt, hits, keys);
    Sequence s;
    s.num_tokens = (int64_t)hits.size() * kBs;
    s.tracks_tokens = true;
    s.tokens.assign(tokens, tokens + s.num_tokens);
    s.salt = salt;
    s.keys = std::move(keys);
    s.table = hits;
    s.serial = bm->next_serial;
    bm->seqs.emplace(seq, std::move(s));
    ++bm->next_serial;
    for (int32_t b : hits) {
      if (bm->dev.ref[b] == 0) bm->dev.revive(b); else ++bm->dev.ref[b];
    }
    *num_cached_tokens = (int64_t)hits.size() * kBs;
  } catch (...) {
    return PA_ERR_NO_MEMORY;
  }
  return PA_OK;
}

int pa_bm_append_tokens(pa_block_manager* bm, int64_t seq, const int32_t* tokens, int32_t count,
                        int64_t* slots) {
  if (!bm) return PA_ERR_NULL;
  Sequence* s = bm->find(seq);
  if (!s || !s->tracks_tokens) return PA_ERR_SEQ;
  if (count > 0 && !tokens) return PA_ERR_NULL;
  try {
    s->tokens.reserve(s->tokens.size() + (size_t)std::max<int32_t>(count, 0));
    bm->to_register.reserve(bm->to_register.size() + (size_t)std::max<int32_t>(count, 0) / kBs + 1);
    const int st = bm->append(seq, count, slots);
    if (st != PA_OK) return st;
    s->tokens.insert(s->tokens.end(), tokens, tokens + count);
    while ((int64_t)(s->keys.size() + 1) * kBs <= s->num_tokens) {
      const size_t j = s->keys.size();
      Registration r;
      r.serial = s->serial;
      r.seq = seq;
      r.j = (int32_t)j;
      r.block = s->table[j];
      r.parent = j ? s->table[j - 1] : -1;
      r.salt = s->salt;
      std::copy(s->tokens.begin() + (ptrdiff_t)(j * kBs), s->tokens.begin() + (ptrdiff_t)((j + 1) * kBs),
                r.tokens);
      r.key = block_key(j ? s->keys.back() : 0, s->salt, r.tokens);
      s->keys.push_back(r.key);
      bm->to_register.push_back(r);
    }
  } catch (...) {
    return PA_ERR_NO_MEMORY;
  }
  return PA_OK;
}

int64_t pa_bm_num_cached_blocks(const pa_block_manager* bm) {
  if (!bm) return PA_ERR_NULL;
  return (int64_t)bm->cache.size();
}

int pa_bm_build_batch(const pa_block_manager* bm, const int64_t* seqs, int32_t num_seqs,
                      int32_t max_blocks_per_seq, int32_t* block_tables, int32_t* context_lens,
                      int32_t* shared_prefix_blocks) {
  if (!bm) return PA_ERR_NULL;
  if (num_seqs < 0 || max_blocks_per_seq < 1) return PA_ERR_SHAPE;
  if (num_seqs == 0) return PA_OK;
  if (!seqs || !block_tables || !context_lens) return PA_ERR_NULL;
  for (int32_t i = 0; i < num_seqs; ++i) {
    const Sequence* s = bm->find(seqs[i]);
    if (!s || s->on_host) return PA_ERR_SEQ;
    if ((int64_t)s->table.size() > max_blocks_per_seq || s->num_tokens > INT32_MAX)
      return PA_ERR_SHAPE;
  }
  for (int32_t i = 0; i < num_seqs; ++i) {
    const Sequence& s = *bm->find(seqs[i]);
    int32_t* row = block_tables + (int64_t)i * max_blocks_per_seq;
    std::copy(s.table.begin(), s.table.end(), row);
    std::fill(row + s.table.size(), row + max_blocks_per_seq, -1);
    context_lens[i] = (int32_t)s.num_tokens;
    if (shared_prefix_blocks) {
      int32_t n = 0;
      while (n < (int32_t)s.table.size() && bm->dev.ref[s.table[(size_t)n]] > 1) ++n;
      shared_prefix_blocks[i] = n;
    }
  }
  return PA_OK;
}

int pa_bm_prefix_groups(const pa_block_manager* bm, const int64_t* seqs, int32_t num_seqs,
                        int32_t* prefix_group, int32_t* group_blocks, int32_t* max_group_size) {
  if (!bm) return PA_ERR_NULL;
  if (num_seqs < 0) return PA_ERR_SHAPE;
  if (num_seqs > 0 && (!seqs || !prefix_group || !group_blocks)) return PA_ERR_NULL;
  std::vector<const Sequence*> ss((size_t)num_seqs);
  for (int32_t i = 0; i < num_seqs; ++i) {
    ss[(size_t)i] = bm->find(seqs[i]);
    if (!ss[(size_t)i] || ss[(size_t)i]->on_host) return PA_ERR_SEQ;
  }
  int32_t largest = num_seqs > 0 ? 1 : 0;
  for (int32_t i = 0; i < num_seqs;) {
    // a run of consecutive entries whose tables start with entry i's first block
    const std::vector<int32_t>& lead = ss[(size_t)i]->table;
    int32_t end = i + 1;
    while (end < num_seqs && !lead.empty() && !ss[(size_t)end]->table.empty() &&
           ss[(size_t)end]->table[0] == lead[0])
      ++end;
    int32_t most = 0;
    for (int32_t m = i + 1; m < end; ++m) {
      const std::vector<int32_t>& t = ss[(size_t)m]->table;
      int32_t n = 0;
      while (n < (int32_t)t.size() && n < (int32_t)lead.size() && t[(size_t)n] == lead[(size_t)n])
        ++n;
      prefix_group[m] = i;
      group_blocks[m] = n;
      most = std::max(most, n);
    }
    prefix_group[i] = i;
    group_blocks[i] = most;
    largest = std::max(largest, end - i);
    i = end;
  }
  if (max_group_size) *max_group_size = largest;
  return PA_OK;
}

int pa_bm_check(const pa_block_manager* bm) {
  if (!bm) return PA_ERR_NULL;
  for (int side = 0; side < 2; ++side) {
    const Pool& pool = side ? bm->host : bm->dev;
    std::vector<int64_t> count((size_t)pool.size(), 0);
    for (const auto& kv : bm->seqs) {
      if (kv.second.on_host != (side == 1)) continue;
      for (int32_t b : kv.second.table) {
        if (b < 0 || b >= pool.size()) return PA_ERR_STATE;
        ++count[(size_t)b];
      }
    }
    std::vector<uint8_t> idle((size_t)pool.size(), 0);
    std::vector<int32_t> lru;
    for (int32_t b = pool.lru_head; b >= 0; b = pool.lru_next[b]) {
      if ((int64_t)lru.size() > pool.size()) return PA_ERR_STATE;
      lru.push_back(b);
    }
    if ((int64_t)lru.size() != pool.lru_size) return PA_ERR_STATE;
    for (const std::vector<int32_t>* v : {&pool.free_stack, &pool.held, (const std::vector<int32_t>*)&lru})
      for (int32_t b : *v) {
        if (b < 0 || b >= pool.size() || idle[(size_t)b]) return PA_ERR_STATE;
        idle[(size_t)b] = 1;
      }
    for (int32_t b : lru)
      if (!pool.is_cached(b)) return PA_ERR_STATE;
    for (int32_t b : pool.free_stack)
      if (pool.is_cached(b)) return PA_ERR_STATE;
    for (int64_t b = 0; b < pool.size(); ++b) {
      if (count[(size_t)b] != pool.ref[(size_t)b]) return PA_ERR_STATE;
      if ((count[(size_t)b] == 0) != (idle[(size_t)b] == 1)) return PA_ERR_STATE;
    }
  }
  for (const auto& kv : bm->seqs)
    if ((int64_t)kv.second.table.size() != ceil_div(kv.second.num_tokens, bm->block_size))
      return PA_ERR_STATE;
  int64_t ncached = 0;
  for (uint8_t c : bm->cached) ncached += c;
  if (ncached != (int64_t)bm->cache.size()) return PA_ERR_STATE;
  for (const auto& kv : bm->cache)
    if (!bm->cached[(size_t)kv.second] || bm->meta_key[(size_t)kv.second] != kv.first)
      return PA_ERR_STATE;
  return PA_OK;
}

}  // extern "C"
