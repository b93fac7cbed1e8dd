// Shared-prefix plan for decode: groups of sequences whose block tables
// start with the same physical blocks.
//
// Forked sequences share the parent's blocks ("day31", fork and
// copy-on-write: a fork takes a reference on every block of the parent and
// copies only a shared, partly filled block it writes into) and prefix-cache
// hits share full blocks ("P06 · BlockManager" spec overview).  Plain decode
// reads a shared block once per sequence that holds it; pa_decode_shared
// reads the shared leading blocks of a group once for all its members.
//
// Grouping (a heuristic: any plan that satisfies the rules in the header is
// correct, this one aims at many members times many shared blocks):
//   * a sequence is a candidate when at least kMinShared full blocks
//     precede its last block (the last block always stays private);
//   * candidates are bucketed by their first block id and sorted
//     lexicographically by table row, so rows with long common prefixes are
//     adjacent and a run's common prefix is that of its first and last row;
//   * runs are cut greedily: a row joins the open group while the group's
//     saving, (members - 1) x shared blocks, does not drop, up to
//     16 / query_group members; a group needs at least two members and
//     kMinShared shared blocks;
//   * groups are listed by shared blocks, most first: the shared pass
//     dispatches its workgroups in group order, so the longest start first
//     and the short ones fill in behind them instead of trailing alone.
#include <algorithm>
#include <numeric>
#include <unordered_map>
#include <vector>

#include "pagedkv.h"
#include "status.hpp"

using pkv::fail;

namespace {

// Fewest shared blocks worth a group: below this the group's extra partial
// result per member costs about what its shared reads save.
constexpr int32_t kMinShared = 2;

struct Cand {
  int32_t seq;
  int32_t cap;   // shareable leading blocks: full, before the last block
};

}  // namespace

extern "C" int pa_shared_plan(const int32_t* tables, int32_t max_blocks, const int32_t* lens,
                              int32_t B, int32_t block_size, int32_t partition_tokens,
                              int32_t query_group, int32_t* seq_group_out, int32_t* groups_out,
                              int32_t* n_groups_out, int32_t* max_parts_out,
                              int32_t* max_private_parts_out, int32_t* max_private_blocks_out) {
  if (B < 0 || max_blocks < 0 || block_size <= 0)
    return fail(PA_ERR_INVALID, "pa_shared_plan: negative size or block_size <= 0");
  if (partition_tokens <= 0 || partition_tokens % block_size != 0)
    return fail(PA_ERR_INVALID,
                "pa_shared_plan: partition_tokens must be a positive multiple of block_size");
  if (query_group != 1 && query_group != 2 && query_group != 4 && query_group != 8)
    return fail(PA_ERR_INVALID, "pa_shared_plan: query_group must be 1, 2, 4 or 8");
  if (!n_groups_out || !max_parts_out || !max_private_parts_out || !max_private_blocks_out ||
      (B > 0 && (!tables || !lens || !seq_group_out)) || (B > 1 && !groups_out))
    return fail(PA_ERR_INVALID, "pa_shared_plan: null pointer");
  const int32_t pb = partition_tokens / block_size;
  const int32_t cap_members = PA_SHARED_MAX_MEMBERS / query_group;
  std::fill(seq_group_out, seq_group_out + B, -1);
  *n_groups_out = 0;
  *max_parts_out = 0;
  *max_private_parts_out = 0;
  *max_private_blocks_out = 0;

  auto row = [&](int32_t b) { return tables + static_cast<size_t>(b) * max_blocks; };
  // Length in blocks of the common prefix of two rows, within both caps.
  auto lcp = [&](const Cand& x, const Cand& y) {
    const int32_t lim = std::min(x.cap, y.cap);
    const int32_t* rx = row(x.seq);
    const int32_t* ry = row(y.seq);
    int32_t j = 0;
    while (j < lim && rx[j] == ry[j]) ++j;
    return j;
  };

  std::vector<int32_t> order;   // bucket keys in first-seen order
  std::unordered_map<int32_t, std::vector<Cand>> buckets;
  for (int32_t b = 0; b < B; ++b) {
    const int32_t n = lens[b];
    if (n <= 0 || n > static_cast<int64_t>(max_blocks) * block_size) continue;
    const int32_t nblk = (n + block_size - 1) / block_size;
    const int32_t cap = nblk - 1;          // every block before the last is full
    if (cap < kMinShared) continue;
    const int32_t first = row(b)[0];
    auto it = buckets.find(first);
    if (it == buckets.end()) {
      order.push_back(first);
      it = buckets.emplace(first, std::vector<Cand>{}).first;
    }
    it->second.push_back(Cand{b, cap});
  }

  int32_t ng = 0, max_parts = 0;
  auto emit = [&](const std::vector<Cand>& c, size_t lo, size_t hi, int32_t shared) {
    int32_t* g = groups_out + static_cast<size_t>(ng) * PA_SHARED_ROW;
    g[0] = shared;
    for (int32_t s = 0; s < PA_SHARED_MAX_MEMBERS; ++s) g[1 + s] = -1;
    for (size_t i = lo; i < hi; ++i) {
      g[1 + (i - lo)] = c[i].seq;
      seq_group_out[c[i].seq] = ng;
    }
    max_parts = std::max(max_parts, (shared + pb - 1) / pb);
    ++ng;
  };
  for (int32_t key : order) {
    std::vector<Cand>& c = buckets[key];
    std::stable_sort(c.begin(), c.end(), [&](const Cand& x, const Cand& y) {
      const int32_t j = lcp(x, y);
      if (j < x.cap && j < y.cap) return row(x.seq)[j] < row(y.seq)[j];
      return x.cap < y.cap;
    });
    size_t lo = 0;
    while (lo < c.size()) {
      // Grow [lo, hi) while the saving does not drop.
      size_t hi = lo + 1;
      int32_t shared = c[lo].cap;
      while (hi < c.size() && static_cast<int32_t>(hi - lo) < cap_members) {
        const int32_t s2 = std::min(shared, lcp(c[lo], c[hi]));
        const int64_t old_save = static_cast<int64_t>(hi - lo - 1) * shared;
        const int64_t new_save = static_cast<int64_t>(hi - lo) * s2;
        if (s2 < kMinShared || new_save < old_save) break;
        shared = s2;
        ++hi;
      }
      if (hi - lo >= 2) emit(c, lo, hi, shared);
      lo = hi;
    }
  }
  // Longest groups first (stable, so equal groups keep their order).
  if (ng > 1) {
    std::vector<int32_t> idx(ng), rank(ng);
    std::iota(idx.begin(), idx.end(), 0);
    std::stable_sort(idx.begin(), idx.end(), [&](int32_t x, int32_t y) {
      return groups_out[static_cast<size_t>(x) * PA_SHARED_ROW] >
             groups_out[static_cast<size_t>(y) * PA_SHARED_ROW];
    });
    std::vector<int32_t> rows(groups_out, groups_out + static_cast<size_t>(ng) * PA_SHARED_ROW);
    for (int32_t i = 0; i < ng; ++i) {
      std::copy_n(rows.data() + static_cast<size_t>(idx[i]) * PA_SHARED_ROW, PA_SHARED_ROW,
                  groups_out + static_cast<size_t>(i) * PA_SHARED_ROW);
      rank[idx[i]] = i;
    }
    for (int32_t b = 0; b < B; ++b)
      if (seq_group_out[b] >= 0) seq_group_out[b] = rank[seq_group_out[b]];
  }
  // Private partitions and blocks left to each sequence: those after its
  // group's shared blocks (all of them when it is in no group; one
  // partition and no block for an empty or invalid length, as in decode).
  int32_t max_private = 0, max_private_blocks = 0;
  for (int32_t b = 0; b < B; ++b) {
    const int32_t n = lens[b];
    const bool ok = n > 0 && n <= static_cast<int64_t>(max_blocks) * block_size;
    const int32_t nblk = ok ? (n + block_size - 1) / block_size : 0;
    const int32_t gi = seq_group_out[b];
    const int32_t shared = gi >= 0 ? groups_out[static_cast<size_t>(gi) * PA_SHARED_ROW] : 0;
    const int32_t priv = nblk == 0 ? 1 : (nblk - shared + pb - 1) / pb;
    max_private = std::max(max_private, priv);
    max_private_blocks = std::max(max_private_blocks, nblk - shared);
  }
  *n_groups_out = ng;
  *max_parts_out = max_parts;
  *max_private_parts_out = max_private;
  *max_private_blocks_out = max_private_blocks;
  pkv::clear_error();
  return PA_OK;
}
