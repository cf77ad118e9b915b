// Host block manager: free list, per-block reference counts, one block table
// per sequence, copy-on-write bookkeeping, swapping to a host pool and an
// optional prefix cache.
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
// Swapping (PagedAttention: Virtual Memory for the KV Cache, "Scheduling and
// preemption": a whole group is evicted together, its blocks copied to CPU
// memory and brought back later): swap-out moves every distinct block of a
// group of sequences to a host pool (pairs for pa_swap_blocks), swap-in
// brings them back into fresh device blocks; blocks shared inside the group
// stay shared.
// Prefix cache (vLLM's PagedAttention: How Memory Management Supports Large
// Model Inference, "2.4" and "7"; PagedAttention (tensortonic), "8. Reusing
// Work Across Separate Requests"): a full block is keyed by the chained hash
// SHA-256(parent block's hash || its token ids || extra key); a map from hash
// to block finds earlier requests' blocks; freed blocks keep their entry and
// go to the back of the free queue (a sequence's last blocks first), and a
// block taken from the front for reuse loses its entry, so the queue order
// is the eviction order (least recently freed first).
#include <cstdint>
#include <cstring>
#include <list>
#include <new>
#include <string>
#include <unordered_map>
#include <unordered_set>
#include <utility>
#include <vector>

#include "pa_internal.h"
#include "sha256.h"

namespace {

using pa::Digest;

struct DigestHash {
  size_t operator()(const Digest& d) const {
    size_t h;
    std::memcpy(&h, d.data(), sizeof(h));
    return h;
  }
};

struct Seq {
  std::vector<int32_t> table;  // device block ids, or host block ids while swapped
  int64_t ntok = 0;
  bool swapped = false;
  // prefix cache (cached managers only)
  std::vector<int32_t> tokens;  // token ids of positions 0..ntok-1 while hash_ok
  std::vector<Digest> hashes;   // chained hash of each full block
  std::string extra;
  bool hash_ok = false;
};

}  // namespace

struct pa_bm {
  int num_blocks = 0;
  int block_size = 16;
  bool cached = false;
  std::list<int32_t> free_list;
  std::vector<std::list<int32_t>::iterator> free_pos;
  std::vector<char> in_free;
  std::vector<int32_t> ref;
  std::vector<int32_t> pend_uses;  // how many queued copies name each block
  std::unordered_map<int64_t, Seq> seqs;
  std::vector<std::pair<int32_t, int32_t>> pending;
  std::vector<int32_t> held;
  // host pool for swapping
  int num_host = 0;
  std::list<int32_t> host_free;
  std::vector<int32_t> host_ref;
  // prefix cache
  std::unordered_map<Digest, int32_t, DigestHash> by_hash;
  std::vector<char> has_hash;
  std::vector<Digest> block_hash;

  int64_t blocks_for(int64_t ntok) const { return (ntok + block_size - 1) / block_size; }

  void push_free(int32_t b) {
    free_list.push_back(b);
    free_pos[b] = std::prev(free_list.end());
    in_free[b] = 1;
  }
  void unlink_free(int32_t b) {
    free_list.erase(free_pos[b]);
    in_free[b] = 0;
  }
  void forget_hash(int32_t b) {
    if (!has_hash[b]) return;
    auto it = by_hash.find(block_hash[b]);
    if (it != by_hash.end() && it->second == b) by_hash.erase(it);
    has_hash[b] = 0;
  }
  void remember_hash(int32_t b, const Digest& h) {
    if (by_hash.count(h) || has_hash[b]) return;  // the first block with this content keeps the entry
    by_hash.emplace(h, b);
    has_hash[b] = 1;
    block_hash[b] = h;
  }

  // Front of the free list; a cached block loses its entry (eviction).
  int32_t pop_free() {
    const int32_t b = free_list.front();
    unlink_free(b);
    forget_hash(b);
    return b;
  }

  // A block whose count dropped to 0.
  void release(int32_t b) {
    if (pend_uses[b] > 0)
      held.push_back(b);
    else
      push_free(b);
  }

  // SHA-256 of parent (32 zero bytes for a sequence's first block) || the
  // block's tokens as int32 little-endian || extra key, hashed from one buffer.
  Digest chain_hash(const Digest* parent, const int32_t* toks, const std::string& extra) const {
    uint8_t small[32 + 4 * 64];
    std::vector<uint8_t> big;
    uint8_t* msg = small;
    if (block_size > 64) {
      big.resize(32 + 4 * (size_t)block_size);
      msg = big.data();
    }
    if (parent)
      std::memcpy(msg, parent->data(), 32);
    else
      std::memset(msg, 0, 32);
    for (int i = 0; i < block_size; ++i) {
      const uint32_t t = (uint32_t)toks[i];
      uint8_t* o = msg + 32 + 4 * i;
      o[0] = (uint8_t)t;
      o[1] = (uint8_t)(t >> 8);
      o[2] = (uint8_t)(t >> 16);
      o[3] = (uint8_t)(t >> 24);
    }
    pa::Sha256 s;
    s.update(msg, 32 + 4 * (size_t)block_size);
    s.update(extra.data(), extra.size());
    return s.finish();
  }

  // Free blocks `s` needs to take n more tokens (new blocks + a copy).
  int64_t need_for(const Seq& s, int64_t n) const {
    if (n <= 0) return 0;
    int64_t need = blocks_for(s.ntok + n) - blocks_for(s.ntok);
    if (s.ntok % block_size != 0 && ref[s.table.back()] > 1) need += 1;
    return need;
  }

  // Caller has checked that the free list covers need_for(s, n).  With
  // `toks` (cached managers), each block that fills is hashed and entered.
  void do_append(Seq& s, int64_t n, int64_t* slots_out, const int32_t* toks) {
    if (n <= 0) return;
    if (cached && !toks) s.hash_ok = false;
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
      if (cached && s.hash_ok) {
        s.tokens.push_back(toks[k]);
        if (s.ntok % block_size == 0) {
          const size_t j = (size_t)(s.ntok / block_size) - 1;
          if (j >= s.hashes.size())  // (else: the recomputed last token of a full prefix hit)
            s.hashes.push_back(chain_hash(j ? &s.hashes[j - 1] : nullptr, &s.tokens[j * block_size], s.extra));
          remember_hash(s.table[j], s.hashes[j]);
        }
      }
    }
  }

  // Validates a group for swapping: distinct, known ids whose swapped state
  // is `want_swapped`.  Fills the Seq pointers and the distinct blocks in
  // order of first appearance.
  pa_status_t group(const char* what, const int64_t* ids, int n, bool want_swapped, std::vector<Seq*>& ss,
                    std::vector<int32_t>& blocks, std::unordered_map<int32_t, int32_t>& uses) {
    if (n < 0) return pa::fail(PA_ERR_SHAPE, "%s: n=%d", what, n);
    if (n > 0 && !ids) return pa::fail(PA_ERR_NULL, "%s: NULL ids", what);
    std::unordered_set<int64_t> seen;
    for (int i = 0; i < n; ++i) {
      auto it = seqs.find(ids[i]);
      if (it == seqs.end()) return pa::fail(PA_ERR_NOT_FOUND, "%s: unknown sequence %lld", what, (long long)ids[i]);
      if (!seen.insert(ids[i]).second)
        return pa::fail(PA_ERR_SHAPE, "%s: sequence %lld appears twice", what, (long long)ids[i]);
      if (it->second.swapped != want_swapped)
        return pa::fail(PA_ERR_SHAPE, "%s: sequence %lld is %s", what, (long long)ids[i],
                        want_swapped ? "not swapped out" : "already swapped out");
      ss.push_back(&it->second);
      for (int32_t b : it->second.table)
        if (uses[b]++ == 0) blocks.push_back(b);
    }
    return PA_OK;
  }
};

namespace {

pa_bm* make_bm(int num_blocks, int block_size, const int32_t* order, bool cached, const char* what) {
  if (num_blocks < 0 || block_size <= 0) {
    pa::fail(PA_ERR_SHAPE, "%s: num_blocks=%d block_size=%d", what, num_blocks, block_size);
    return nullptr;
  }
  pa_bm* bm = new (std::nothrow) pa_bm();
  if (!bm) {
    pa::fail(PA_ERR_SHAPE, "%s: out of host memory", what);
    return nullptr;
  }
  bm->num_blocks = num_blocks;
  bm->block_size = block_size;
  bm->cached = cached;
  bm->ref.assign(num_blocks, 0);
  bm->pend_uses.assign(num_blocks, 0);
  bm->free_pos.resize(num_blocks);
  bm->in_free.assign(num_blocks, 0);
  bm->has_hash.assign(num_blocks, 0);
  bm->block_hash.resize(num_blocks);
  std::vector<char> seen(num_blocks, 0);
  for (int i = 0; i < num_blocks; ++i) {
    const int32_t b = order ? order[i] : i;
    if (b < 0 || b >= num_blocks || seen[b]) {
      pa::fail(PA_ERR_SHAPE, "%s: initial_free_order is not a permutation (entry %d = %d)", what, i, b);
      delete bm;
      return nullptr;
    }
    seen[b] = 1;
    bm->push_free(b);
  }
  return bm;
}

}  // namespace

extern "C" {

pa_bm_t* pa_bm_create(int num_blocks, int block_size, const int32_t* initial_free_order) {
  return make_bm(num_blocks, block_size, initial_free_order, false, "pa_bm_create");
}

pa_bm_t* pa_bm_create_cached(int num_blocks, int block_size, const int32_t* initial_free_order) {
  return make_bm(num_blocks, block_size, initial_free_order, true, "pa_bm_create_cached");
}

void pa_bm_destroy(pa_bm_t* bm) { delete bm; }

pa_status_t pa_bm_add_seq(pa_bm_t* bm, int64_t seq_id) {
  if (!bm) return pa::fail(PA_ERR_NULL, "pa_bm_add_seq: bm is NULL");
  if (bm->seqs.count(seq_id)) return pa::fail(PA_ERR_EXISTS, "pa_bm_add_seq: sequence %lld exists", (long long)seq_id);
  Seq s;
  s.hash_ok = bm->cached;
  bm->seqs.emplace(seq_id, std::move(s));
  return PA_OK;
}

pa_status_t pa_bm_add_seq_cached(pa_bm_t* bm, int64_t seq_id, const int32_t* tokens, int n_tokens,
                                 const void* extra_key, int extra_len, int* num_cached_out) {
  if (!bm) return pa::fail(PA_ERR_NULL, "pa_bm_add_seq_cached: bm is NULL");
  if (!bm->cached) return pa::fail(PA_ERR_UNSUPPORTED, "pa_bm_add_seq_cached: manager has no prefix cache");
  if (n_tokens < 0 || extra_len < 0)
    return pa::fail(PA_ERR_SHAPE, "pa_bm_add_seq_cached: n_tokens=%d extra_len=%d", n_tokens, extra_len);
  if ((n_tokens > 0 && !tokens) || (extra_len > 0 && !extra_key))
    return pa::fail(PA_ERR_NULL, "pa_bm_add_seq_cached: NULL array");
  if (bm->seqs.count(seq_id))
    return pa::fail(PA_ERR_EXISTS, "pa_bm_add_seq_cached: sequence %lld exists", (long long)seq_id);
  Seq s;
  s.hash_ok = true;
  s.extra.assign(static_cast<const char*>(extra_key), (size_t)extra_len);
  const int bs = bm->block_size;
  for (int j = 0; (j + 1) * bs <= n_tokens; ++j) {
    const Digest h = bm->chain_hash(j ? &s.hashes[j - 1] : nullptr, tokens + (size_t)j * bs, s.extra);
    auto it = bm->by_hash.find(h);
    if (it == bm->by_hash.end()) break;
    const int32_t b = it->second;
    if (bm->ref[b] == 0) {
      if (bm->in_free[b]) {
        bm->unlink_free(b);
      } else {  // held for a pending copy that reads it; it stays valid
        for (size_t k = 0; k < bm->held.size(); ++k)
          if (bm->held[k] == b) {
            bm->held.erase(bm->held.begin() + k);
            break;
          }
      }
    }
    bm->ref[b] += 1;
    s.table.push_back(b);
    s.hashes.push_back(h);
  }
  int64_t ntok = (int64_t)s.table.size() * bs;
  if (ntok == n_tokens && n_tokens > 0) ntok -= 1;  // a full hit still computes its last token
  s.ntok = ntok;
  s.tokens.assign(tokens, tokens + ntok);
  bm->seqs.emplace(seq_id, std::move(s));
  if (num_cached_out) *num_cached_out = (int)ntok;
  return PA_OK;
}

pa_status_t pa_bm_append(pa_bm_t* bm, int64_t seq_id, int n_tokens, int64_t* slots_out) {
  if (!bm) return pa::fail(PA_ERR_NULL, "pa_bm_append: bm is NULL");
  if (n_tokens < 0) return pa::fail(PA_ERR_SHAPE, "pa_bm_append: n_tokens=%d", n_tokens);
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return pa::fail(PA_ERR_NOT_FOUND, "pa_bm_append: unknown sequence %lld", (long long)seq_id);
  if (it->second.swapped)
    return pa::fail(PA_ERR_SHAPE, "pa_bm_append: sequence %lld is swapped out", (long long)seq_id);
  const int64_t need = bm->need_for(it->second, n_tokens);
  if ((int64_t)bm->free_list.size() < need)
    return pa::fail(PA_ERR_NO_BLOCKS, "pa_bm_append: need %lld free blocks, have %zu", (long long)need,
                    bm->free_list.size());
  bm->do_append(it->second, n_tokens, slots_out, nullptr);
  return PA_OK;
}

pa_status_t pa_bm_append_tokens(pa_bm_t* bm, int64_t seq_id, const int32_t* tokens, int n_tokens,
                                int64_t* slots_out) {
  if (!bm) return pa::fail(PA_ERR_NULL, "pa_bm_append_tokens: bm is NULL");
  if (!bm->cached) return pa::fail(PA_ERR_UNSUPPORTED, "pa_bm_append_tokens: manager has no prefix cache");
  if (n_tokens < 0) return pa::fail(PA_ERR_SHAPE, "pa_bm_append_tokens: n_tokens=%d", n_tokens);
  if (n_tokens > 0 && !tokens) return pa::fail(PA_ERR_NULL, "pa_bm_append_tokens: NULL tokens");
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end())
    return pa::fail(PA_ERR_NOT_FOUND, "pa_bm_append_tokens: unknown sequence %lld", (long long)seq_id);
  if (it->second.swapped)
    return pa::fail(PA_ERR_SHAPE, "pa_bm_append_tokens: sequence %lld is swapped out", (long long)seq_id);
  const int64_t need = bm->need_for(it->second, n_tokens);
  if ((int64_t)bm->free_list.size() < need)
    return pa::fail(PA_ERR_NO_BLOCKS, "pa_bm_append_tokens: need %lld free blocks, have %zu", (long long)need,
                    bm->free_list.size());
  bm->do_append(it->second, n_tokens, slots_out, tokens);
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
    if (it->second.swapped)
      return pa::fail(PA_ERR_SHAPE, "pa_bm_append_batch: sequence %lld is swapped out", (long long)seq_ids[i]);
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
  for (int i = 0; i < n; ++i) bm->do_append(*ptrs[i], 1, slots_out + i, nullptr);
  return PA_OK;
}

pa_status_t pa_bm_fork(pa_bm_t* bm, int64_t parent, int64_t child) {
  if (!bm) return pa::fail(PA_ERR_NULL, "pa_bm_fork: bm is NULL");
  auto it = bm->seqs.find(parent);
  if (it == bm->seqs.end()) return pa::fail(PA_ERR_NOT_FOUND, "pa_bm_fork: unknown parent %lld", (long long)parent);
  if (it->second.swapped) return pa::fail(PA_ERR_SHAPE, "pa_bm_fork: parent %lld is swapped out", (long long)parent);
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
  const auto& t = it->second.table;
  if (it->second.swapped) {
    for (int32_t h : t)
      if (--bm->host_ref[h] == 0) bm->host_free.push_back(h);
  } else if (bm->cached) {
    // last blocks first: a sequence's head blocks (shared prefixes) are evicted last
    for (size_t k = t.size(); k-- > 0;)
      if (--bm->ref[t[k]] == 0) bm->release(t[k]);
  } else {
    for (int32_t b : t)
      if (--bm->ref[b] == 0) bm->release(b);
  }
  bm->seqs.erase(it);
  return PA_OK;
}

pa_status_t pa_bm_set_host_blocks(pa_bm_t* bm, int num_host_blocks) {
  if (!bm) return pa::fail(PA_ERR_NULL, "pa_bm_set_host_blocks: bm is NULL");
  if (num_host_blocks < 0) return pa::fail(PA_ERR_SHAPE, "pa_bm_set_host_blocks: %d blocks", num_host_blocks);
  for (const auto& kv : bm->seqs)
    if (kv.second.swapped) return pa::fail(PA_ERR_SHAPE, "pa_bm_set_host_blocks: a sequence is swapped out");
  bm->num_host = num_host_blocks;
  bm->host_free.clear();
  for (int i = 0; i < num_host_blocks; ++i) bm->host_free.push_back(i);
  bm->host_ref.assign(num_host_blocks, 0);
  return PA_OK;
}

pa_status_t pa_bm_swap_out(pa_bm_t* bm, const int64_t* seq_ids, int n, int32_t* pairs_out, int cap,
                           int* num_pairs_out) {
  if (!bm) return pa::fail(PA_ERR_NULL, "pa_bm_swap_out: bm is NULL");
  std::vector<Seq*> ss;
  std::vector<int32_t> blocks;
  std::unordered_map<int32_t, int32_t> uses;
  pa_status_t st = bm->group("pa_bm_swap_out", seq_ids, n, false, ss, blocks, uses);
  if (st != PA_OK) return st;
  if (!bm->pending.empty())
    return pa::fail(PA_ERR_SHAPE, "pa_bm_swap_out: %zu copy-on-write pairs pending; take them first",
                    bm->pending.size());
  for (int32_t b : blocks)
    if (bm->ref[b] != uses[b])
      return pa::fail(PA_ERR_SHAPE, "pa_bm_swap_out: block %d is shared with a sequence outside the group", b);
  if ((int64_t)bm->host_free.size() < (int64_t)blocks.size())
    return pa::fail(PA_ERR_NO_BLOCKS, "pa_bm_swap_out: need %zu host blocks, have %zu", blocks.size(),
                    bm->host_free.size());
  if (cap < (int)blocks.size() || (!blocks.empty() && !pairs_out))
    return pa::fail(PA_ERR_SHAPE, "pa_bm_swap_out: %zu pairs, cap %d", blocks.size(), cap);
  std::unordered_map<int32_t, int32_t> to_host;
  for (size_t k = 0; k < blocks.size(); ++k) {
    const int32_t b = blocks[k];
    const int32_t h = bm->host_free.front();
    bm->host_free.pop_front();
    bm->host_ref[h] = bm->ref[b];
    bm->ref[b] = 0;
    bm->forget_hash(b);
    bm->push_free(b);
    to_host[b] = h;
    pairs_out[2 * k] = b;
    pairs_out[2 * k + 1] = h;
  }
  for (Seq* s : ss) {
    for (int32_t& b : s->table) b = to_host[b];
    s->swapped = true;
  }
  if (num_pairs_out) *num_pairs_out = (int)blocks.size();
  return PA_OK;
}

pa_status_t pa_bm_swap_in(pa_bm_t* bm, const int64_t* seq_ids, int n, int32_t* pairs_out, int cap,
                          int* num_pairs_out) {
  if (!bm) return pa::fail(PA_ERR_NULL, "pa_bm_swap_in: bm is NULL");
  std::vector<Seq*> ss;
  std::vector<int32_t> hblocks;
  std::unordered_map<int32_t, int32_t> uses;
  pa_status_t st = bm->group("pa_bm_swap_in", seq_ids, n, true, ss, hblocks, uses);
  if (st != PA_OK) return st;
  for (int32_t h : hblocks)
    if (bm->host_ref[h] != uses[h])
      return pa::fail(PA_ERR_SHAPE, "pa_bm_swap_in: host block %d is shared with a sequence outside the group", h);
  if ((int64_t)bm->free_list.size() < (int64_t)hblocks.size())
    return pa::fail(PA_ERR_NO_BLOCKS, "pa_bm_swap_in: need %zu free blocks, have %zu", hblocks.size(),
                    bm->free_list.size());
  if (cap < (int)hblocks.size() || (!hblocks.empty() && !pairs_out))
    return pa::fail(PA_ERR_SHAPE, "pa_bm_swap_in: %zu pairs, cap %d", hblocks.size(), cap);
  std::unordered_map<int32_t, int32_t> to_dev;
  for (size_t k = 0; k < hblocks.size(); ++k) {
    const int32_t h = hblocks[k];
    const int32_t b = bm->pop_free();
    bm->ref[b] = bm->host_ref[h];
    bm->host_ref[h] = 0;
    bm->host_free.push_back(h);
    to_dev[h] = b;
    pairs_out[2 * k] = h;
    pairs_out[2 * k + 1] = b;
  }
  for (Seq* s : ss) {
    for (int32_t& h : s->table) h = to_dev[h];
    s->swapped = false;
    if (bm->cached && s->hash_ok) {
      const size_t full = (size_t)(s->ntok / bm->block_size);
      for (size_t j = 0; j < s->hashes.size() && j < full; ++j) bm->remember_hash(s->table[j], s->hashes[j]);
    }
  }
  if (num_pairs_out) *num_pairs_out = (int)hblocks.size();
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
    if (it->second.swapped)
      return pa::fail(PA_ERR_SHAPE, "pa_bm_tables: sequence %lld is swapped out", (long long)seq_ids[i]);
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
  for (int32_t b : bm->held)
    if (bm->ref[b] == 0) bm->push_free(b);
  bm->held.clear();
  return n;
}

int pa_bm_num_free(const pa_bm_t* bm) { return bm ? (int)bm->free_list.size() : -1; }

int pa_bm_refcount(const pa_bm_t* bm, int32_t block) {
  if (!bm || block < 0 || block >= bm->num_blocks) return -1;
  return bm->ref[block];
}

int pa_bm_is_swapped(const pa_bm_t* bm, int64_t seq_id) {
  if (!bm) return -1;
  auto it = bm->seqs.find(seq_id);
  return it == bm->seqs.end() ? -1 : (int)it->second.swapped;
}

int pa_bm_num_host_free(const pa_bm_t* bm) { return bm ? (int)bm->host_free.size() : -1; }

int pa_bm_host_refcount(const pa_bm_t* bm, int32_t host_block) {
  if (!bm || host_block < 0 || host_block >= bm->num_host) return -1;
  return bm->host_ref[host_block];
}

int pa_bm_num_cached_blocks(const pa_bm_t* bm) { return bm ? (int)bm->by_hash.size() : -1; }

int pa_bm_block_hash(const pa_bm_t* bm, int64_t seq_id, int j, uint8_t* out32) {
  if (!bm || !out32) return -1;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end() || j < 0 || j >= (int)it->second.hashes.size()) return -1;
  std::memcpy(out32, it->second.hashes[j].data(), 32);
  return 0;
}

int pa_bm_cached_block(const pa_bm_t* bm, const uint8_t* hash32) {
  if (!bm || !hash32) return -1;
  Digest d;
  std::memcpy(d.data(), hash32, 32);
  auto it = bm->by_hash.find(d);
  return it == bm->by_hash.end() ? -1 : it->second;
}

}  // extern "C"
