// Host block manager: refcounts, chained prefix hashes, LRU evictable pool,
// all-or-nothing allocate / append_slot, reverse-order free, fork and
// copy-on-write append.
//
// Specification: "P06 · BlockManager: paged KV + prefix cache" -- spec
// overview (slot formula, chained hashes, (len-1)/bs match limit, free and
// eviction policy, atomicity, append registers full blocks), operations
// table (read steps, ordered write steps, single raise point), invariants
// I1-I5, details (fixed sentinel, contiguous match, coarse can_allocate,
// prefix cache switch, duplicate-content rule) and algorithm notes
// (take-block helper, append order, reverse free).  Fork and COW append:
// "day31", toy COW append.  Preemption: "qaqbuyan.com article 130",
// continuous-batching scheduler (the victim's blocks go to host memory and
// are freed); the way back is the allocate path over the saved tokens.
//
// Data layout (all O(1) per step, no allocation on the append path once a
// sequence's vectors have grown):
//   free list  -- ring buffer of capacity num_blocks (FIFO);
//   evictable  -- intrusive doubly linked list over block ids, oldest at
//                 the head, so a revived hit leaves it in O(1);
//   per block  -- ref, has_hash, hash, parent hash and tokens (the tokens
//                 and parent let a hit be verified, so a false hit needs a
//                 64-bit collision of whole prefixes).
#include <algorithm>
#include <cstring>
#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

#include "pagedkv.h"
#include "status.hpp"

namespace {

// h_{-1}: a fixed sentinel shared by allocate and append_slot (first 64
// fractional bits of sqrt(2)).
constexpr uint64_t kChainSentinel = 0x6a09e667f3bcc908ull;
constexpr uint64_t kGolden = 0x9e3779b97f4a7c15ull;

// splitmix64 output mix (S. Vigna, "splitmix64.c", public domain).
inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}

// h_i = H(h_{i-1}, tokens of block i).
uint64_t chain_hash(uint64_t parent, const int32_t* toks, int32_t bs) {
  uint64_t x = mix64(parent ^ kGolden);
  for (int32_t i = 0; i < bs; ++i)
    x = mix64(x + kGolden * (static_cast<uint64_t>(static_cast<uint32_t>(toks[i])) + 1));
  return x;
}

struct Seq {
  std::vector<int32_t> table;
  std::vector<int32_t> tokens;
  std::vector<uint64_t> hashes;  // chain over the full blocks
  int32_t cached = 0;
};

}  // namespace

struct pa_bm {
  int32_t nb = 0, bs = 0;
  bool prefix = true;
  std::vector<int32_t> ref;
  std::vector<uint8_t> has_hash;
  std::vector<uint64_t> block_hash, block_parent;
  std::vector<int32_t> block_tokens;  // [nb][bs], meaningful when has_hash
  std::unordered_map<uint64_t, int32_t> hash_to_block;
  // free list (FIFO ring)
  std::vector<int32_t> ring;
  int32_t head = 0, nfree = 0;
  // evictable pool (LRU: head oldest, tail newest)
  std::vector<int32_t> prv, nxt;
  std::vector<uint8_t> in_pool;
  int32_t ev_head = -1, ev_tail = -1, nevict = 0;
  std::unordered_map<int64_t, Seq> seqs;
  std::unordered_map<int64_t, std::vector<int32_t>> swapped;  // preempted: tokens only
  mutable std::mutex mu;

  int32_t num_free() const { return nfree + nevict; }

  void free_push(int32_t b) {
    ring[(head + nfree) % nb] = b;
    ++nfree;
  }
  int32_t free_pop() {
    int32_t b = ring[head];
    head = (head + 1) % nb;
    --nfree;
    return b;
  }
  void pool_push(int32_t b) {  // newest end
    prv[b] = ev_tail;
    nxt[b] = -1;
    if (ev_tail >= 0) nxt[ev_tail] = b; else ev_head = b;
    ev_tail = b;
    in_pool[b] = 1;
    ++nevict;
  }
  void pool_remove(int32_t b) {
    if (prv[b] >= 0) nxt[prv[b]] = nxt[b]; else ev_head = nxt[b];
    if (nxt[b] >= 0) prv[nxt[b]] = prv[b]; else ev_tail = prv[b];
    prv[b] = nxt[b] = -1;
    in_pool[b] = 0;
    --nevict;
  }
  void unregister(int32_t b) {
    auto it = hash_to_block.find(block_hash[b]);
    if (it != hash_to_block.end() && it->second == b) hash_to_block.erase(it);
    has_hash[b] = 0;
  }
  // Free list first, else the oldest evictable block (dropping its
  // registration); -1 if neither.  The block gets ref 1.
  int32_t take_block() {
    int32_t b;
    if (nfree > 0) {
      b = free_pop();
    } else if (nevict > 0) {
      b = ev_head;
      pool_remove(b);
      unregister(b);
    } else {
      return -1;
    }
    ref[b] = 1;
    return b;
  }
  // Record a full block's hash; an existing mapping for the same hash is
  // kept (duplicate-content rule).
  void register_block(int32_t b, uint64_t h, uint64_t parent, const int32_t* toks) {
    has_hash[b] = 1;
    block_hash[b] = h;
    block_parent[b] = parent;
    std::memcpy(&block_tokens[static_cast<size_t>(b) * bs], toks, sizeof(int32_t) * bs);
    hash_to_block.emplace(h, b);
  }
  // Lookup with verification of parent hash and block tokens.
  int32_t lookup(uint64_t h, uint64_t parent, const int32_t* toks) const {
    auto it = hash_to_block.find(h);
    if (it == hash_to_block.end()) return -1;
    int32_t b = it->second;
    if (!has_hash[b] || block_hash[b] != h || block_parent[b] != parent) return -1;
    if (std::memcmp(&block_tokens[static_cast<size_t>(b) * bs], toks, sizeof(int32_t) * bs) != 0)
      return -1;
    return b;
  }
  void free_seq(Seq& s) {
    for (auto it = s.table.rbegin(); it != s.table.rend(); ++it) {
      int32_t b = *it;
      if (--ref[b] == 0) {
        if (has_hash[b]) pool_push(b); else free_push(b);
      }
    }
  }
};

using pkv::fail;

extern "C" {

pa_bm* pa_bm_create(int32_t num_blocks, int32_t block_size, int32_t enable_prefix_cache) {
  if (num_blocks <= 0 || block_size <= 0) {
    fail(PA_ERR_INVALID, "pa_bm_create: num_blocks and block_size must be positive");
    return nullptr;
  }
  pa_bm* bm = new pa_bm;
  bm->nb = num_blocks;
  bm->bs = block_size;
  bm->prefix = enable_prefix_cache != 0;
  bm->ref.assign(num_blocks, 0);
  bm->has_hash.assign(num_blocks, 0);
  bm->block_hash.assign(num_blocks, 0);
  bm->block_parent.assign(num_blocks, 0);
  bm->block_tokens.assign(static_cast<size_t>(num_blocks) * block_size, 0);
  bm->ring.resize(num_blocks);
  for (int32_t b = 0; b < num_blocks; ++b) bm->ring[b] = b;
  bm->nfree = num_blocks;
  bm->prv.assign(num_blocks, -1);
  bm->nxt.assign(num_blocks, -1);
  bm->in_pool.assign(num_blocks, 0);
  pkv::clear_error();
  return bm;
}

void pa_bm_destroy(pa_bm* bm) { delete bm; }

// The allocate row of the operations table; the caller holds the lock and
// has checked that `seq` is neither live nor swapped out.
static int allocate_locked(pa_bm* bm, int64_t seq, const int32_t* tokens, int32_t n,
                           int32_t* table_out, int32_t cap, int32_t* nblocks_out) {
  const int32_t bs = bm->bs;
  const int32_t nblocks = (n + bs - 1) / bs;
  if (table_out && cap < nblocks) return fail(PA_ERR_INVALID, "pa_bm_allocate: table_out too small");
  // (1) chain hashes of the full blocks.
  const int32_t full = n / bs;
  std::vector<uint64_t> hashes;
  if (bm->prefix) {
    hashes.resize(full);
    uint64_t parent = kChainSentinel;
    for (int32_t i = 0; i < full; ++i) {
      parent = chain_hash(parent, tokens + static_cast<size_t>(i) * bs, bs);
      hashes[i] = parent;
    }
  }
  // (2) contiguous lookups over the first (n-1)/bs blocks.
  std::vector<int32_t> hits;
  if (bm->prefix && n > 0) {
    const int32_t limit = (n - 1) / bs;
    for (int32_t i = 0; i < limit; ++i) {
      uint64_t parent = i ? hashes[i - 1] : kChainSentinel;
      int32_t b = bm->lookup(hashes[i], parent, tokens + static_cast<size_t>(i) * bs);
      if (b < 0) break;
      hits.push_back(b);
    }
  }
  // (3) exact capacity check, before any change.
  const int32_t new_needed = nblocks - static_cast<int32_t>(hits.size());
  int32_t revived = 0;
  for (int32_t b : hits) revived += bm->ref[b] == 0;
  if (new_needed > bm->num_free() - revived)
    return fail(PA_ERR_OUT_OF_BLOCKS, "pa_bm_allocate: need " + std::to_string(new_needed) +
                                          " new blocks, " +
                                          std::to_string(bm->num_free() - revived) + " usable");
  // (4) revive hits; (5) new blocks in logical order; (6) register.
  Seq s;
  s.table.reserve(nblocks);
  for (int32_t b : hits) {
    if (bm->ref[b] == 0) bm->pool_remove(b);
    ++bm->ref[b];
    s.table.push_back(b);
  }
  for (int32_t i = 0; i < new_needed; ++i) s.table.push_back(bm->take_block());
  for (int32_t i = static_cast<int32_t>(hits.size()); i < static_cast<int32_t>(hashes.size()); ++i)
    bm->register_block(s.table[i], hashes[i], i ? hashes[i - 1] : kChainSentinel,
                       tokens + static_cast<size_t>(i) * bs);
  // (7) record the sequence.
  s.tokens.assign(tokens, tokens + n);
  s.hashes = std::move(hashes);
  s.cached = static_cast<int32_t>(hits.size()) * bs;
  if (table_out) std::copy(s.table.begin(), s.table.end(), table_out);
  if (nblocks_out) *nblocks_out = nblocks;
  bm->seqs.emplace(seq, std::move(s));
  return PA_OK;
}

int pa_bm_allocate(pa_bm* bm, int64_t seq, const int32_t* tokens, int32_t n,
                   int32_t* table_out, int32_t cap, int32_t* nblocks_out) {
  if (!bm) return fail(PA_ERR_INVALID, "pa_bm_allocate: null manager");
  std::lock_guard<std::mutex> lock(bm->mu);
  if (n < 0 || (n > 0 && !tokens)) return fail(PA_ERR_INVALID, "pa_bm_allocate: bad tokens");
  if (bm->seqs.count(seq) || bm->swapped.count(seq))
    return fail(PA_ERR_INVALID, "pa_bm_allocate: sequence exists");
  int st = allocate_locked(bm, seq, tokens, n, table_out, cap, nblocks_out);
  if (st == PA_OK) pkv::clear_error();
  return st;
}

static int append_locked(pa_bm* bm, int64_t seq, int32_t token, int64_t* slot_out,
                         int32_t* cow_src, int32_t* cow_dst) {
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return fail(PA_ERR_INVALID, "pa_bm_append_slot: unknown sequence");
  Seq& s = it->second;
  const int32_t bs = bm->bs;
  const int32_t pos = static_cast<int32_t>(s.tokens.size());
  int32_t src = -1, dst = -1;
  // (1) take a block first: the only step that can fail.
  if (pos / bs == static_cast<int32_t>(s.table.size())) {
    int32_t b = bm->take_block();
    if (b < 0) return fail(PA_ERR_OUT_OF_BLOCKS, "pa_bm_append_slot: no free or evictable block");
    s.table.push_back(b);
  } else {
    int32_t last = s.table.back();
    if (bm->ref[last] > 1) {  // shared, partly filled: copy on write
      int32_t b = bm->take_block();
      if (b < 0) return fail(PA_ERR_OUT_OF_BLOCKS, "pa_bm_append_slot: no block for COW");
      --bm->ref[last];
      s.table.back() = b;
      src = last;
      dst = b;
    }
  }
  // (2) the token.
  s.tokens.push_back(token);
  // (3) a block that just filled is hashed from the chain tail and registered.
  if (bm->prefix && (pos + 1) % bs == 0) {
    uint64_t parent = s.hashes.empty() ? kChainSentinel : s.hashes.back();
    const int32_t* blk = s.tokens.data() + (pos + 1 - bs);
    uint64_t h = chain_hash(parent, blk, bs);
    s.hashes.push_back(h);
    bm->register_block(s.table[pos / bs], h, parent, blk);
  }
  if (slot_out) *slot_out = static_cast<int64_t>(s.table[pos / bs]) * bs + pos % bs;
  if (cow_src) *cow_src = src;
  if (cow_dst) *cow_dst = dst;
  return PA_OK;
}

int pa_bm_append_slot(pa_bm* bm, int64_t seq, int32_t token, int64_t* slot_out,
                      int32_t* cow_src_out, int32_t* cow_dst_out) {
  if (!bm) return fail(PA_ERR_INVALID, "pa_bm_append_slot: null manager");
  std::lock_guard<std::mutex> lock(bm->mu);
  int st = append_locked(bm, seq, token, slot_out, cow_src_out, cow_dst_out);
  if (st == PA_OK) pkv::clear_error();
  return st;
}

int pa_bm_append_slots(pa_bm* bm, const int64_t* seqs, const int32_t* tokens, int32_t B,
                       int64_t* slots_out, int32_t* cow_pairs_out, int32_t* n_cow_out,
                       int32_t* n_done_out) {
  if (!bm) return fail(PA_ERR_INVALID, "pa_bm_append_slots: null manager");
  if (B < 0 || (B > 0 && (!seqs || !tokens || !slots_out)))
    return fail(PA_ERR_INVALID, "pa_bm_append_slots: bad arguments");
  std::lock_guard<std::mutex> lock(bm->mu);
  int32_t ncow = 0, done = 0;
  int st = PA_OK;
  for (; done < B; ++done) {
    int32_t src, dst;
    st = append_locked(bm, seqs[done], tokens[done], &slots_out[done], &src, &dst);
    if (st != PA_OK) break;
    if (src >= 0) {
      if (cow_pairs_out) {
        cow_pairs_out[2 * ncow] = src;
        cow_pairs_out[2 * ncow + 1] = dst;
      }
      ++ncow;
    }
  }
  if (n_cow_out) *n_cow_out = ncow;
  if (n_done_out) *n_done_out = done;
  if (st == PA_OK) pkv::clear_error();
  return st;
}

int pa_bm_fork(pa_bm* bm, int64_t parent, int64_t child) {
  if (!bm) return fail(PA_ERR_INVALID, "pa_bm_fork: null manager");
  std::lock_guard<std::mutex> lock(bm->mu);
  auto it = bm->seqs.find(parent);
  if (it == bm->seqs.end()) return fail(PA_ERR_INVALID, "pa_bm_fork: unknown parent");
  if (bm->seqs.count(child) || bm->swapped.count(child))
    return fail(PA_ERR_INVALID, "pa_bm_fork: child exists");
  Seq s = it->second;
  for (int32_t b : s.table) ++bm->ref[b];
  bm->seqs.emplace(child, std::move(s));
  pkv::clear_error();
  return PA_OK;
}

int pa_bm_fork_batch(pa_bm* bm, const int64_t* parents, const int64_t* children, int32_t n,
                     int32_t* n_done_out) {
  if (!bm || n < 0 || (n > 0 && (!parents || !children)))
    return fail(PA_ERR_INVALID, "pa_bm_fork_batch: bad arguments");
  std::lock_guard<std::mutex> lock(bm->mu);
  int32_t done = 0;
  int st = PA_OK;
  for (; done < n; ++done) {
    auto it = bm->seqs.find(parents[done]);
    if (it == bm->seqs.end()) { st = fail(PA_ERR_INVALID, "pa_bm_fork_batch: unknown parent"); break; }
    if (bm->seqs.count(children[done]) || bm->swapped.count(children[done])) {
      st = fail(PA_ERR_INVALID, "pa_bm_fork_batch: child exists");
      break;
    }
    Seq s = it->second;
    for (int32_t b : s.table) ++bm->ref[b];
    bm->seqs.emplace(children[done], std::move(s));
  }
  if (n_done_out) *n_done_out = done;
  if (st == PA_OK) pkv::clear_error();
  return st;
}

int pa_bm_free_batch(pa_bm* bm, const int64_t* seqs, int32_t n) {
  if (!bm || n < 0 || (n > 0 && !seqs)) return fail(PA_ERR_INVALID, "pa_bm_free_batch: bad arguments");
  std::lock_guard<std::mutex> lock(bm->mu);
  for (int32_t i = 0; i < n; ++i) {
    bm->swapped.erase(seqs[i]);
    auto it = bm->seqs.find(seqs[i]);
    if (it != bm->seqs.end()) {
      bm->free_seq(it->second);
      bm->seqs.erase(it);
    }
  }
  pkv::clear_error();
  return PA_OK;
}

int pa_bm_free(pa_bm* bm, int64_t seq) {
  if (!bm) return fail(PA_ERR_INVALID, "pa_bm_free: null manager");
  std::lock_guard<std::mutex> lock(bm->mu);
  bm->swapped.erase(seq);
  auto it = bm->seqs.find(seq);
  if (it != bm->seqs.end()) {
    bm->free_seq(it->second);
    bm->seqs.erase(it);
  }
  pkv::clear_error();
  return PA_OK;
}

int pa_bm_swap_out(pa_bm* bm, int64_t seq, int32_t* table_out, int32_t cap, int32_t* nblocks_out) {
  if (!bm || !nblocks_out) return fail(PA_ERR_INVALID, "pa_bm_swap_out: null argument");
  std::lock_guard<std::mutex> lock(bm->mu);
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return fail(PA_ERR_INVALID, "pa_bm_swap_out: unknown sequence");
  Seq& s = it->second;
  const int32_t nblocks = static_cast<int32_t>(s.table.size());
  if (nblocks > cap || (!table_out && nblocks > 0))
    return fail(PA_ERR_INVALID, "pa_bm_swap_out: table_out too small");
  std::copy(s.table.begin(), s.table.end(), table_out);
  *nblocks_out = nblocks;
  bm->free_seq(s);
  bm->swapped.emplace(seq, std::move(s.tokens));
  bm->seqs.erase(it);
  pkv::clear_error();
  return PA_OK;
}

int pa_bm_swap_in(pa_bm* bm, int64_t seq, int32_t* table_out, int32_t cap, int32_t* nblocks_out,
                  int32_t* first_restore_out) {
  if (!bm || !nblocks_out || !first_restore_out)
    return fail(PA_ERR_INVALID, "pa_bm_swap_in: null argument");
  std::lock_guard<std::mutex> lock(bm->mu);
  auto it = bm->swapped.find(seq);
  if (it == bm->swapped.end()) return fail(PA_ERR_INVALID, "pa_bm_swap_in: sequence is not swapped out");
  const std::vector<int32_t>& toks = it->second;
  const int32_t n = static_cast<int32_t>(toks.size());
  if (!table_out && n > 0) return fail(PA_ERR_INVALID, "pa_bm_swap_in: null table_out");
  int st = allocate_locked(bm, seq, toks.data(), n, table_out, cap, nblocks_out);
  if (st != PA_OK) return st;                 // still swapped out, nothing changed
  *first_restore_out = bm->seqs.at(seq).cached / bm->bs;
  bm->swapped.erase(it);
  pkv::clear_error();
  return PA_OK;
}

int32_t pa_bm_is_swapped(const pa_bm* bm, int64_t seq) {
  if (!bm) return -1;
  std::lock_guard<std::mutex> lock(bm->mu);
  return bm->swapped.count(seq) ? 1 : 0;
}

int pa_bm_swapped(const pa_bm* bm, int64_t* seqs_out, int32_t* lens_out, int32_t cap,
                  int32_t* n_out) {
  if (!bm || !n_out) return fail(PA_ERR_INVALID, "pa_bm_swapped: null argument");
  std::lock_guard<std::mutex> lock(bm->mu);
  const int32_t n = static_cast<int32_t>(bm->swapped.size());
  if (!seqs_out && !lens_out) {   // count only
    *n_out = n;
    pkv::clear_error();
    return PA_OK;
  }
  if (n > cap || (n > 0 && (!seqs_out || !lens_out)))
    return fail(PA_ERR_INVALID, "pa_bm_swapped: output too small");
  std::vector<int64_t> ids;
  ids.reserve(n);
  for (const auto& kv : bm->swapped) ids.push_back(kv.first);
  std::sort(ids.begin(), ids.end());
  for (int32_t i = 0; i < n; ++i) {
    seqs_out[i] = ids[i];
    lens_out[i] = static_cast<int32_t>(bm->swapped.at(ids[i]).size());
  }
  *n_out = n;
  pkv::clear_error();
  return PA_OK;
}

int pa_bm_slot(const pa_bm* bm, int64_t seq, int32_t pos, int64_t* slot_out) {
  if (!bm || !slot_out) return fail(PA_ERR_INVALID, "pa_bm_slot: null argument");
  std::lock_guard<std::mutex> lock(bm->mu);
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return fail(PA_ERR_INVALID, "pa_bm_slot: unknown sequence");
  const Seq& s = it->second;
  if (pos < 0 || pos >= static_cast<int32_t>(s.tokens.size()))
    return fail(PA_ERR_INVALID, "pa_bm_slot: pos out of range");
  *slot_out = static_cast<int64_t>(s.table[pos / bm->bs]) * bm->bs + pos % bm->bs;
  return PA_OK;
}

int32_t pa_bm_block_size(const pa_bm* bm) { return bm ? bm->bs : -1; }
int32_t pa_bm_num_blocks(const pa_bm* bm) { return bm ? bm->nb : -1; }

int32_t pa_bm_num_free_blocks(const pa_bm* bm) {
  if (!bm) return -1;
  std::lock_guard<std::mutex> lock(bm->mu);
  return bm->num_free();
}

int32_t pa_bm_can_allocate(const pa_bm* bm, int32_t n_tokens) {
  if (!bm || n_tokens < 0) return 0;
  std::lock_guard<std::mutex> lock(bm->mu);
  int64_t need = (static_cast<int64_t>(n_tokens) + bm->bs - 1) / bm->bs;
  return need <= bm->num_free() ? 1 : 0;
}

int pa_bm_num_cached_tokens(const pa_bm* bm, int64_t seq, int32_t* out) {
  if (!bm || !out) return fail(PA_ERR_INVALID, "pa_bm_num_cached_tokens: null argument");
  std::lock_guard<std::mutex> lock(bm->mu);
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return fail(PA_ERR_INVALID, "pa_bm_num_cached_tokens: unknown sequence");
  *out = it->second.cached;
  return PA_OK;
}

int pa_bm_seq_len(const pa_bm* bm, int64_t seq, int32_t* out) {
  if (!bm || !out) return fail(PA_ERR_INVALID, "pa_bm_seq_len: null argument");
  std::lock_guard<std::mutex> lock(bm->mu);
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return fail(PA_ERR_INVALID, "pa_bm_seq_len: unknown sequence");
  *out = static_cast<int32_t>(it->second.tokens.size());
  return PA_OK;
}

int pa_bm_get_table(const pa_bm* bm, int64_t seq, int32_t* out, int32_t cap, int32_t* n_out) {
  if (!bm || !n_out) return fail(PA_ERR_INVALID, "pa_bm_get_table: null argument");
  std::lock_guard<std::mutex> lock(bm->mu);
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return fail(PA_ERR_INVALID, "pa_bm_get_table: unknown sequence");
  const auto& t = it->second.table;
  if (static_cast<int32_t>(t.size()) > cap || (!out && !t.empty()))
    return fail(PA_ERR_INVALID, "pa_bm_get_table: output too small");
  std::copy(t.begin(), t.end(), out);
  *n_out = static_cast<int32_t>(t.size());
  return PA_OK;
}

int32_t pa_bm_num_seqs(const pa_bm* bm) {
  if (!bm) return -1;
  std::lock_guard<std::mutex> lock(bm->mu);
  return static_cast<int32_t>(bm->seqs.size());
}

int pa_bm_seq_ids(const pa_bm* bm, int64_t* out, int32_t cap, int32_t* n_out) {
  if (!bm || !n_out) return fail(PA_ERR_INVALID, "pa_bm_seq_ids: null argument");
  std::lock_guard<std::mutex> lock(bm->mu);
  const int32_t n = static_cast<int32_t>(bm->seqs.size());
  if (n > cap || (!out && n > 0)) return fail(PA_ERR_INVALID, "pa_bm_seq_ids: output too small");
  int32_t i = 0;
  for (const auto& kv : bm->seqs) out[i++] = kv.first;
  std::sort(out, out + n);
  *n_out = n;
  return PA_OK;
}

int pa_bm_export_batch(const pa_bm* bm, const int64_t* seqs, int32_t B, int32_t* tables_out,
                       int32_t max_blocks, int32_t pad_block, int32_t* context_lens_out) {
  if (!bm || B < 0 || max_blocks < 0 ||
      (B > 0 && (!seqs || !context_lens_out || (!tables_out && max_blocks > 0))))
    return fail(PA_ERR_INVALID, "pa_bm_export_batch: bad arguments");
  std::lock_guard<std::mutex> lock(bm->mu);
  std::vector<const Seq*> ss(B);
  for (int32_t i = 0; i < B; ++i) {
    auto it = bm->seqs.find(seqs[i]);
    if (it == bm->seqs.end()) return fail(PA_ERR_INVALID, "pa_bm_export_batch: unknown sequence");
    if (static_cast<int32_t>(it->second.table.size()) > max_blocks)
      return fail(PA_ERR_INVALID, "pa_bm_export_batch: table longer than max_blocks");
    ss[i] = &it->second;
  }
  for (int32_t i = 0; i < B; ++i) {
    int32_t* row = tables_out + static_cast<size_t>(i) * max_blocks;
    const auto& t = ss[i]->table;
    std::copy(t.begin(), t.end(), row);
    std::fill(row + t.size(), row + max_blocks, pad_block);
    context_lens_out[i] = static_cast<int32_t>(ss[i]->tokens.size());
  }
  pkv::clear_error();
  return PA_OK;
}

int pa_bm_check_invariants(const pa_bm* bm) {
  if (!bm) return fail(PA_ERR_INVALID, "null manager");
  std::lock_guard<std::mutex> lock(bm->mu);
  const int32_t nb = bm->nb;
  std::vector<int8_t> where(nb, 0);  // 1 free, 2 evictable
  for (int32_t i = 0; i < bm->nfree; ++i) {
    int32_t b = bm->ring[(bm->head + i) % nb];
    if (where[b]) return fail(PA_ERR_INVALID, "I1: block twice in free list");
    where[b] = 1;
  }
  int32_t cnt = 0;
  for (int32_t b = bm->ev_head; b >= 0; b = bm->nxt[b]) {
    if (where[b]) return fail(PA_ERR_INVALID, "I1: free and evictable overlap");
    where[b] = 2;
    if (++cnt > nb) return fail(PA_ERR_INVALID, "evictable list cycles");
  }
  if (cnt != bm->nevict) return fail(PA_ERR_INVALID, "evictable count mismatch");
  for (int32_t b = 0; b < nb; ++b) {
    if (where[b] && bm->ref[b] != 0) return fail(PA_ERR_INVALID, "I1: pooled block with ref != 0");
    bool expect_evict = bm->ref[b] == 0 && bm->has_hash[b];
    if ((where[b] == 2) != expect_evict) return fail(PA_ERR_INVALID, "I2: evictable <=> ref==0 && hashed");
    if ((where[b] == 2) != (bm->in_pool[b] != 0)) return fail(PA_ERR_INVALID, "pool flag mismatch");
  }
  for (const auto& kv : bm->hash_to_block) {
    int32_t b = kv.second;
    if (!bm->has_hash[b] || bm->block_hash[b] != kv.first) return fail(PA_ERR_INVALID, "I3");
  }
  for (const auto& kv : bm->swapped)
    if (bm->seqs.count(kv.first)) return fail(PA_ERR_INVALID, "swapped-out sequence holds blocks");
  std::vector<int32_t> count(nb, 0);
  for (const auto& kv : bm->seqs) {
    const Seq& s = kv.second;
    const int32_t n = static_cast<int32_t>(s.tokens.size());
    if (static_cast<int32_t>(s.table.size()) != (n + bm->bs - 1) / bm->bs)
      return fail(PA_ERR_INVALID, "table not tight");
    for (int32_t b : s.table) ++count[b];
    if (s.cached % bm->bs != 0 || !(s.cached < n || (n == 0 && s.cached == 0)))
      return fail(PA_ERR_INVALID, "I5: cached");
  }
  int32_t held = 0;
  for (int32_t b = 0; b < nb; ++b) {
    if (count[b] != bm->ref[b]) return fail(PA_ERR_INVALID, "I4: ref != table count");
    held += count[b] > 0;
  }
  if (held + bm->num_free() != nb) return fail(PA_ERR_INVALID, "I4: block leak");
  pkv::clear_error();
  return PA_OK;
}

int pa_bm_dump(const pa_bm* bm, int32_t* ref, int8_t* has_hash, int32_t* free_order,
               int32_t* n_free, int32_t* evict_order, int32_t* n_evict) {
  if (!bm) return fail(PA_ERR_INVALID, "pa_bm_dump: null manager");
  std::lock_guard<std::mutex> lock(bm->mu);
  const int32_t nb = bm->nb;
  if (ref) std::copy(bm->ref.begin(), bm->ref.end(), ref);
  if (has_hash)
    for (int32_t b = 0; b < nb; ++b) has_hash[b] = static_cast<int8_t>(bm->has_hash[b]);
  if (free_order)
    for (int32_t i = 0; i < bm->nfree; ++i) free_order[i] = bm->ring[(bm->head + i) % nb];
  if (n_free) *n_free = bm->nfree;
  if (evict_order) {
    int32_t i = 0;
    for (int32_t b = bm->ev_head; b >= 0; b = bm->nxt[b]) evict_order[i++] = b;
  }
  if (n_evict) *n_evict = bm->nevict;
  return PA_OK;
}

}  // extern "C"
