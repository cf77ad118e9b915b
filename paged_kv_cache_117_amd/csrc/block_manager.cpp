// Host block manager: FIFO free list, per-block reference counts, one block
// table per sequence, copy-on-write bookkeeping.
//
// Rules (PagedAttention and vLLM: Paging the KV Cache Like an OS, "Step 3"
// on-demand allocation and request A, "Step 4" reference counts, fork and
// copy-on-write; PagedAttention (tensortonic), "7. Sharing a Prefix Without
// Overwriting It": full prefix blocks stay shared; Paging the KV Cache Like an
// OS, "Step 2": a request gets all its blocks or none):
//   * a block is popped from the front of the free list only when a
//     sequence's last block is full;
//   * fork copies the table and bumps the counts;
//   * an append into a partly filled last block with count > 1 first moves
//     the writer onto a fresh copy (queued as (src, dst) for pa_copy_blocks);
//     count == 1 writes in place;
//   * freed blocks (count 0) go to the back of the free list in table order,
//     unless a queued copy names them: those wait for pa_bm_take_copies, so a
//     block is never reused while a copy that reads or writes it is pending.
#include <cstdint>
#include <deque>
#include <new>
#include <unordered_map>
#include <unordered_set>
#include <utility>
#include <vector>

#include "pa_internal.h"

namespace {

struct Seq {
  std::vector<int32_t> table;
  int64_t ntok = 0;
};

}  // namespace

struct pa_bm {
  int num_blocks = 0;
  int block_size = 16;
  std::deque<int32_t> free_list;
  std::vector<int32_t> ref;
  std::vector<int32_t> pend_uses;  // how many queued copies name each block
  std::unordered_map<int64_t, Seq> seqs;
  std::vector<std::pair<int32_t, int32_t>> pending;
  std::vector<int32_t> held;

  int64_t blocks_for(int64_t ntok) const { return (ntok + block_size - 1) / block_size; }

  int32_t pop_free() {
    int32_t b = free_list.front();
    free_list.pop_front();
    return b;
  }

  // Free blocks `s` needs to take n more tokens (new blocks + a copy).
  int64_t need_for(const Seq& s, int64_t n) const {
    if (n <= 0) return 0;
    int64_t need = blocks_for(s.ntok + n) - blocks_for(s.ntok);
    if (s.ntok % block_size != 0 && ref[s.table.back()] > 1) need += 1;
    return need;
  }

  // Caller has checked that the free list covers need_for(s, n).
  void do_append(Seq& s, int64_t n, int64_t* slots_out) {
    if (n <= 0) return;
    if (s.ntok % block_size != 0 && ref[s.table.back()] > 1) {
      const int32_t src = s.table.back();
      const int32_t dst = pop_free();
      pending.emplace_back(src, dst);
      pend_uses[src] += 1;
      pend_uses[dst] += 1;
      ref[src] -= 1;
      ref[dst] = 1;
      s.table.back() = dst;
    }
    for (int64_t k = 0; k < n; ++k) {
      if (s.ntok % block_size == 0) {
        const int32_t b = pop_free();
        ref[b] = 1;
        s.table.push_back(b);
      }
      if (slots_out)
        slots_out[k] = (int64_t)s.table[s.ntok / block_size] * block_size + s.ntok % block_size;
      s.ntok += 1;
    }
  }
};

extern "C" {

pa_bm_t* pa_bm_create(int num_blocks, int block_size, const int32_t* initial_free_order) {
  if (num_blocks < 0 || block_size <= 0) {
    pa::fail(PA_ERR_SHAPE, "pa_bm_create: num_blocks=%d block_size=%d", num_blocks, block_size);
    return nullptr;
  }
  pa_bm* bm = new (std::nothrow) pa_bm();
  if (!bm) {
    pa::fail(PA_ERR_SHAPE, "pa_bm_create: out of host memory");
    return nullptr;
  }
  bm->num_blocks = num_blocks;
  bm->block_size = block_size;
  bm->ref.assign(num_blocks, 0);
  bm->pend_uses.assign(num_blocks, 0);
  if (initial_free_order) {
    std::vector<char> seen(num_blocks, 0);
    for (int i = 0; i < num_blocks; ++i) {
      const int32_t b = initial_free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        pa::fail(PA_ERR_SHAPE, "pa_bm_create: initial_free_order is not a permutation (entry %d = %d)", i, b);
        delete bm;
        return nullptr;
      }
      seen[b] = 1;
      bm->free_list.push_back(b);
    }
  } else {
    for (int i = 0; i < num_blocks; ++i) bm->free_list.push_back(i);
  }
  return bm;
}

void pa_bm_destroy(pa_bm_t* bm) { delete bm; }

pa_status_t pa_bm_add_seq(pa_bm_t* bm, int64_t seq_id) {
  if (!bm) return pa::fail(PA_ERR_NULL, "pa_bm_add_seq: bm is NULL");
  if (bm->seqs.count(seq_id)) return pa::fail(PA_ERR_EXISTS, "pa_bm_add_seq: sequence %lld exists", (long long)seq_id);
  bm->seqs.emplace(seq_id, Seq());
  return PA_OK;
}

pa_status_t pa_bm_append(pa_bm_t* bm, int64_t seq_id, int n_tokens, int64_t* slots_out) {
  if (!bm) return pa::fail(PA_ERR_NULL, "pa_bm_append: bm is NULL");
  if (n_tokens < 0) return pa::fail(PA_ERR_SHAPE, "pa_bm_append: n_tokens=%d", n_tokens);
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return pa::fail(PA_ERR_NOT_FOUND, "pa_bm_append: unknown sequence %lld", (long long)seq_id);
  const int64_t need = bm->need_for(it->second, n_tokens);
  if ((int64_t)bm->free_list.size() < need)
    return pa::fail(PA_ERR_NO_BLOCKS, "pa_bm_append: need %lld free blocks, have %zu", (long long)need,
                    bm->free_list.size());
  bm->do_append(it->second, n_tokens, slots_out);
  return PA_OK;
}

pa_status_t pa_bm_append_batch(pa_bm_t* bm, const int64_t* seq_ids, int n, int64_t* slots_out) {
  if (!bm) return pa::fail(PA_ERR_NULL, "pa_bm_append_batch: bm is NULL");
  if (n < 0) return pa::fail(PA_ERR_SHAPE, "pa_bm_append_batch: n=%d", n);
  if (n > 0 && (!seq_ids || !slots_out)) return pa::fail(PA_ERR_NULL, "pa_bm_append_batch: NULL array");
  std::vector<Seq*> ptrs(n);
  std::unordered_set<int64_t> ids;
  for (int i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end())
      return pa::fail(PA_ERR_NOT_FOUND, "pa_bm_append_batch: unknown sequence %lld", (long long)seq_ids[i]);
    if (!ids.insert(seq_ids[i]).second)
      return pa::fail(PA_ERR_SHAPE, "pa_bm_append_batch: sequence %lld appears twice", (long long)seq_ids[i]);
    ptrs[i] = &it->second;
  }
  // Exact count: sharers of one partial block copy in turn; the last finds 1.
  int64_t need = 0;
  std::unordered_map<int32_t, int32_t> tentative;
  for (Seq* s : ptrs) {
    if (s->ntok % bm->block_size == 0) {
      need += 1;
      continue;
    }
    const int32_t last = s->table.back();
    auto t = tentative.find(last);
    const int32_t r = t == tentative.end() ? bm->ref[last] : t->second;
    if (r > 1) {
      need += 1;
      tentative[last] = r - 1;
    }
  }
  if ((int64_t)bm->free_list.size() < need)
    return pa::fail(PA_ERR_NO_BLOCKS, "pa_bm_append_batch: need %lld free blocks, have %zu", (long long)need,
                    bm->free_list.size());
  for (int i = 0; i < n; ++i) bm->do_append(*ptrs[i], 1, slots_out + i);
  return PA_OK;
}

pa_status_t pa_bm_fork(pa_bm_t* bm, int64_t parent, int64_t child) {
  if (!bm) return pa::fail(PA_ERR_NULL, "pa_bm_fork: bm is NULL");
  auto it = bm->seqs.find(parent);
  if (it == bm->seqs.end()) return pa::fail(PA_ERR_NOT_FOUND, "pa_bm_fork: unknown parent %lld", (long long)parent);
  if (bm->seqs.count(child)) return pa::fail(PA_ERR_EXISTS, "pa_bm_fork: child %lld exists", (long long)child);
  Seq c = it->second;  // copy before emplace may rehash
  for (int32_t b : c.table) bm->ref[b] += 1;
  bm->seqs.emplace(child, std::move(c));
  return PA_OK;
}

pa_status_t pa_bm_free_seq(pa_bm_t* bm, int64_t seq_id) {
  if (!bm) return pa::fail(PA_ERR_NULL, "pa_bm_free_seq: bm is NULL");
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return pa::fail(PA_ERR_NOT_FOUND, "pa_bm_free_seq: unknown sequence %lld", (long long)seq_id);
  for (int32_t b : it->second.table) {
    if (--bm->ref[b] == 0) {
      if (bm->pend_uses[b] > 0)
        bm->held.push_back(b);
      else
        bm->free_list.push_back(b);
    }
  }
  bm->seqs.erase(it);
  return PA_OK;
}

int pa_bm_table(const pa_bm_t* bm, int64_t seq_id, int32_t* out, int cap) {
  if (!bm) return -1;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return -1;
  const auto& t = it->second.table;
  for (int i = 0; i < cap && i < (int)t.size(); ++i) out[i] = t[i];
  return (int)t.size();
}

pa_status_t pa_bm_tables(const pa_bm_t* bm, const int64_t* seq_ids, int n, int32_t* out, int max_blocks,
                         int32_t pad) {
  if (!bm) return pa::fail(PA_ERR_NULL, "pa_bm_tables: bm is NULL");
  if (n < 0 || max_blocks < 0) return pa::fail(PA_ERR_SHAPE, "pa_bm_tables: n=%d max_blocks=%d", n, max_blocks);
  if (n > 0 && (!seq_ids || !out)) return pa::fail(PA_ERR_NULL, "pa_bm_tables: NULL array");
  for (int i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end())
      return pa::fail(PA_ERR_NOT_FOUND, "pa_bm_tables: unknown sequence %lld", (long long)seq_ids[i]);
    const auto& t = it->second.table;
    if ((int)t.size() > max_blocks)
      return pa::fail(PA_ERR_SHAPE, "pa_bm_tables: sequence %lld has %zu blocks > max_blocks %d",
                      (long long)seq_ids[i], t.size(), max_blocks);
    int32_t* row = out + (size_t)i * max_blocks;
    int j = 0;
    for (; j < (int)t.size(); ++j) row[j] = t[j];
    for (; j < max_blocks; ++j) row[j] = pad;
  }
  return PA_OK;
}

int pa_bm_num_tokens(const pa_bm_t* bm, int64_t seq_id) {
  if (!bm) return -1;
  auto it = bm->seqs.find(seq_id);
  return it == bm->seqs.end() ? -1 : (int)it->second.ntok;
}

int pa_bm_num_pending_copies(const pa_bm_t* bm) { return bm ? (int)bm->pending.size() : 0; }

int pa_bm_take_copies(pa_bm_t* bm, int32_t* pairs_out, int cap) {
  if (!bm) return -1;
  const int n = (int)bm->pending.size();
  if (cap < n || (n > 0 && !pairs_out)) {
    pa::fail(PA_ERR_SHAPE, "pa_bm_take_copies: %d pairs pending, cap %d", n, cap);
    return -1;
  }
  for (int i = 0; i < n; ++i) {
    pairs_out[2 * i] = bm->pending[i].first;
    pairs_out[2 * i + 1] = bm->pending[i].second;
    bm->pend_uses[bm->pending[i].first] -= 1;
    bm->pend_uses[bm->pending[i].second] -= 1;
  }
  bm->pending.clear();
  for (int32_t b : bm->held) bm->free_list.push_back(b);
  bm->held.clear();
  return n;
}

int pa_bm_num_free(const pa_bm_t* bm) { return bm ? (int)bm->free_list.size() : -1; }

int pa_bm_refcount(const pa_bm_t* bm, int32_t block) {
  if (!bm || block < 0 || block >= bm->num_blocks) return -1;
  return bm->ref[block];
}

}  // extern "C"
