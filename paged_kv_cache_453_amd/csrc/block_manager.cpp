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
#include <stdint.h>

#include <algorithm>
#include <new>
#include <unordered_map>
#include <utility>
#include <vector>

#include "pa.h"

namespace {

struct Pool {
  std::vector<int32_t> free_stack;   // back() is the top
  std::vector<int32_t> ref;
  std::vector<int32_t> held;         // released while named by a pending pair
  std::vector<uint8_t> pending;      // named by a pending pair
  std::vector<uint8_t> pending_dst;  // destination of a pending pair
  std::vector<int32_t> marked;       // blocks whose pending flags are set

  void init(int64_t n) {
    free_stack.resize((size_t)n);
    for (int64_t i = 0; i < n; ++i) free_stack[(size_t)i] = (int32_t)(n - 1 - i);
    ref.assign((size_t)n, 0);
    pending.assign((size_t)n, 0);
    pending_dst.assign((size_t)n, 0);
  }
  int64_t size() const { return (int64_t)ref.size(); }
  int32_t take() {
    const int32_t b = free_stack.back();
    free_stack.pop_back();
    ref[b] = 1;
    return b;
  }
  void release(int32_t b) {
    if (--ref[b] == 0) (pending[b] ? held : free_stack).push_back(b);
  }
  void mark(int32_t b, bool dst) {
    if (!pending[b]) {
      pending[b] = 1;
      marked.push_back(b);
    }
    if (dst) pending_dst[b] = 1;
  }
  void settle() {
    free_stack.insert(free_stack.end(), held.begin(), held.end());
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
};

using Pair = std::pair<int32_t, int32_t>;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

struct pa_block_manager {
  int block_size = 16;
  Pool dev, host;
  std::unordered_map<int64_t, Sequence> seqs;
  std::vector<int64_t> dirty;
  std::vector<Pair> copies, swapped_out, swapped_in;

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

int pa_block_manager::append(int64_t id, int64_t n, int64_t* slots) {
  Sequence* s = find(id);
  if (!s || s->on_host) return PA_ERR_SEQ;
  if (n < 0) return PA_ERR_SHAPE;
  if (n > 0 && !slots) return PA_ERR_NULL;
  if (cow_needed(*s, n) && dev.pending_dst[s->table.back()]) return PA_ERR_BUSY;
  if (blocks_needed(*s, n) > (int64_t)dev.free_stack.size()) return PA_ERR_NO_BLOCKS;
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
  if (distinct > (int64_t)dst.free_stack.size()) return PA_ERR_NO_BLOCKS;
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
  try {
    if (!bm->seqs.emplace(seq, Sequence()).second) return PA_ERR_SEQ;
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
    Sequence c;
    c.table = p->table;
    c.num_tokens = p->num_tokens;
    bm->seqs.emplace(child, std::move(c));
  } catch (...) {
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
    Sequence d;
    d.table.reserve((size_t)count);
    for (int32_t i = 0; i < count; ++i) d.table.push_back(s->table[(size_t)logical_blocks[i]]);
    d.num_tokens = (int64_t)count * bm->block_size;
    bm->seqs.emplace(dst, std::move(d));
  } catch (...) {
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
  return (int64_t)(host ? bm->host : bm->dev).free_stack.size();
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
    for (const std::vector<int32_t>* v : {&pool.free_stack, &pool.held})
      for (int32_t b : *v) {
        if (b < 0 || b >= pool.size() || idle[(size_t)b]) return PA_ERR_STATE;
        idle[(size_t)b] = 1;
      }
    for (int64_t b = 0; b < pool.size(); ++b) {
      if (count[(size_t)b] != pool.ref[(size_t)b]) return PA_ERR_STATE;
      if ((count[(size_t)b] == 0) != (idle[(size_t)b] == 1)) return PA_ERR_STATE;
    }
  }
  for (const auto& kv : bm->seqs)
    if ((int64_t)kv.second.table.size() != ceil_div(kv.second.num_tokens, bm->block_size))
      return PA_ERR_STATE;
  return PA_OK;
}

}  // extern "C"
