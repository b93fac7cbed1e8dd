// Stress driver for the host block manager through its C ABI only.
// Seeded random operation streams (allocate / append_slot / append_slots /
// fork / free / export / queries) with the P06 invariants checked after
// every operation and the full dump compared across every failed operation
// (all-or-nothing).  Built by tests/test_bm_sanitizers.py with g++ and the
// address + undefined-behaviour sanitizers; exits non-zero on any failure.
#include <algorithm>
#include <map>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "pagedkv.h"

#define REQUIRE(c)                                                               \
  do {                                                                           \
    if (!(c)) {                                                                  \
      std::fprintf(stderr, "FAIL %s:%d %s (%s)\n", __FILE__, __LINE__, #c,       \
                   pa_last_error());                                             \
      std::exit(1);                                                              \
    }                                                                            \
  } while (0)

struct Dump {
  std::vector<int32_t> ref, fr, ev;
  std::vector<int8_t> has;
  int32_t nf = 0, ne = 0;
  bool operator==(const Dump& o) const {
    return ref == o.ref && has == o.has && nf == o.nf && ne == o.ne &&
           std::vector<int32_t>(fr.begin(), fr.begin() + nf) ==
               std::vector<int32_t>(o.fr.begin(), o.fr.begin() + o.nf) &&
           std::vector<int32_t>(ev.begin(), ev.begin() + ne) ==
               std::vector<int32_t>(o.ev.begin(), o.ev.begin() + o.ne);
  }
};

static Dump dump(pa_bm* bm, int nb) {
  Dump d;
  d.ref.resize(nb);
  d.has.resize(nb);
  d.fr.resize(nb);
  d.ev.resize(nb);
  REQUIRE(pa_bm_dump(bm, d.ref.data(), d.has.data(), d.fr.data(), &d.nf, d.ev.data(), &d.ne) == PA_OK);
  return d;
}

static void run(uint32_t seed, int nb, int bs, int prefix, int alphabet, int ops) {
  std::mt19937 rng(seed);
  pa_bm* bm = pa_bm_create(nb, bs, prefix);
  REQUIRE(bm);
  std::vector<int64_t> live, swapped;
  int64_t next = 1;
  long oob = 0, cow = 0, hits = 0, swap_hits = 0;
  for (int it = 0; it < ops; ++it) {
    const int r = rng() % 100;
    if (r < 25 || live.empty()) {
      int n = rng() % (4 * bs + 2);
      std::vector<int32_t> toks(n);
      for (auto& t : toks) t = rng() % alphabet;
      std::vector<int32_t> table((n + bs - 1) / bs + 1);
      int32_t nbk = -1;
      Dump before = dump(bm, nb);
      int st = pa_bm_allocate(bm, next, toks.data(), n, table.data(), (int32_t)table.size(), &nbk);
      if (st == PA_ERR_OUT_OF_BLOCKS) {
        ++oob;
        REQUIRE(dump(bm, nb) == before);
      } else {
        REQUIRE(st == PA_OK && nbk == (n + bs - 1) / bs);
        int32_t c = -1;
        REQUIRE(pa_bm_num_cached_tokens(bm, next, &c) == PA_OK);
        hits += c > 0;
        live.push_back(next++);
      }
    } else if (r < 50) {
      int64_t s = live[rng() % live.size()];
      int64_t slot = -2;
      int32_t src = -2, dst = -2, len0 = -1, len1 = -1;
      REQUIRE(pa_bm_seq_len(bm, s, &len0) == PA_OK);
      Dump before = dump(bm, nb);
      int st = pa_bm_append_slot(bm, s, (int32_t)(rng() % alphabet), &slot, &src, &dst);
      if (st == PA_ERR_OUT_OF_BLOCKS) {
        ++oob;
        REQUIRE(dump(bm, nb) == before);
        REQUIRE(pa_bm_seq_len(bm, s, &len1) == PA_OK && len1 == len0);
      } else {
        REQUIRE(st == PA_OK);
        int64_t again = -1;
        REQUIRE(pa_bm_slot(bm, s, len0, &again) == PA_OK && again == slot);
        cow += src >= 0;
        REQUIRE((src >= 0) == (dst >= 0));
      }
    } else if (r < 58) {
      // batched append over a few live sequences (distinct ids)
      std::vector<int64_t> ids;
      for (int k = 0; k < 3 && k < (int)live.size(); ++k) ids.push_back(live[(rng() % live.size())]);
      std::sort(ids.begin(), ids.end());
      ids.erase(std::unique(ids.begin(), ids.end()), ids.end());
      std::vector<int32_t> toks(ids.size(), 1);
      std::vector<int64_t> slots(ids.size());
      std::vector<int32_t> pairs(2 * ids.size());
      int32_t ncow = -1, ndone = -1;
      int st = pa_bm_append_slots(bm, ids.data(), toks.data(), (int32_t)ids.size(), slots.data(),
                                  pairs.data(), &ncow, &ndone);
      REQUIRE(st == PA_OK || st == PA_ERR_OUT_OF_BLOCKS);
      REQUIRE(ndone >= 0 && ndone <= (int32_t)ids.size() && ncow >= 0 && ncow <= ndone);
      if (st != PA_OK) ++oob;
    } else if (r < 65) {
      int64_t p = live[rng() % live.size()];
      if (rng() % 2) {
        REQUIRE(pa_bm_fork(bm, p, next) == PA_OK);
        REQUIRE(pa_bm_fork(bm, p, next) == PA_ERR_INVALID);   // child exists
        live.push_back(next++);
      } else {                                                 // batched, last one fails
        int64_t par[3] = {p, p, p}, kid[3] = {next, next + 1, next};
        int32_t done = -1;
        REQUIRE(pa_bm_fork_batch(bm, par, kid, 3, &done) == PA_ERR_INVALID && done == 2);
        live.push_back(next++);
        live.push_back(next++);
      }
    } else if (r < 71) {
      // preempt: swap out, with a too-small table first (must change nothing)
      size_t i = rng() % live.size();
      int64_t s = live[i];
      int32_t len = -1, n = -1;
      REQUIRE(pa_bm_seq_len(bm, s, &len) == PA_OK);
      const int32_t nbk = (len + bs - 1) / bs;
      std::vector<int32_t> table(nbk + 1, -7);
      if (nbk > 0) {
        Dump before = dump(bm, nb);
        REQUIRE(pa_bm_swap_out(bm, s, table.data(), nbk - 1, &n) == PA_ERR_INVALID);
        REQUIRE(dump(bm, nb) == before);
      }
      REQUIRE(pa_bm_swap_out(bm, s, table.data(), nbk, &n) == PA_OK && n == nbk);
      REQUIRE(table[nbk] == -7);
      REQUIRE(pa_bm_is_swapped(bm, s) == 1);
      REQUIRE(pa_bm_swap_out(bm, s, table.data(), nbk, &n) == PA_ERR_INVALID);
      live.erase(live.begin() + i);
      swapped.push_back(s);
    } else if (r < 77 && !swapped.empty()) {
      size_t i = rng() % swapped.size();
      int64_t s = swapped[i];
      int32_t cnt = -1;
      REQUIRE(pa_bm_swapped(bm, nullptr, nullptr, 0, &cnt) == PA_OK && cnt == (int32_t)swapped.size());
      std::vector<int64_t> ids(cnt);
      std::vector<int32_t> lens(cnt);
      REQUIRE(pa_bm_swapped(bm, ids.data(), lens.data(), cnt, &cnt) == PA_OK);
      int32_t len = -1;
      for (int32_t k = 0; k < cnt; ++k) if (ids[k] == s) len = lens[k];
      REQUIRE(len >= 0);
      const int32_t nbk = (len + bs - 1) / bs;
      std::vector<int32_t> table(nbk + 1, -7);
      int32_t n = -1, first = -1;
      Dump before = dump(bm, nb);
      int st = pa_bm_swap_in(bm, s, table.data(), nbk, &n, &first);
      if (st == PA_ERR_OUT_OF_BLOCKS) {
        ++oob;
        REQUIRE(dump(bm, nb) == before && pa_bm_is_swapped(bm, s) == 1);
      } else {
        REQUIRE(st == PA_OK && n == nbk && first >= 0 && first <= nbk && table[nbk] == -7);
        int32_t c = -1;
        REQUIRE(pa_bm_num_cached_tokens(bm, s, &c) == PA_OK && c == first * bs);
        swap_hits += first > 0;
        swapped.erase(swapped.begin() + i);
        live.push_back(s);
      }
    } else if (r < 92) {
      size_t i = rng() % live.size();
      if (rng() % 2) {
        REQUIRE(pa_bm_free(bm, live[i]) == PA_OK);
      } else {
        int64_t ids[2] = {live[i], -12345};
        REQUIRE(pa_bm_free_batch(bm, ids, 2) == PA_OK);
      }
      live.erase(live.begin() + i);
    } else {
      // export a random subset with a table width that may be too small
      std::vector<int64_t> ids(live.begin(), live.begin() + std::min<size_t>(live.size(), 4));
      int32_t width = rng() % 8;
      std::vector<int32_t> tabs(ids.size() * width + 1), lens(ids.size() + 1);
      int st = pa_bm_export_batch(bm, ids.data(), (int32_t)ids.size(), tabs.data(), width, -1,
                                  lens.data());
      REQUIRE(st == PA_OK || st == PA_ERR_INVALID);
      if (st == PA_OK)
        for (size_t k = 0; k < ids.size(); ++k) {
          int32_t n = -1;
          REQUIRE(pa_bm_seq_len(bm, ids[k], &n) == PA_OK && n == lens[k]);
        }
    }
    REQUIRE(pa_bm_check_invariants(bm) == PA_OK);
  }
  for (int64_t s : live) REQUIRE(pa_bm_free(bm, s) == PA_OK);
  for (int64_t s : swapped) REQUIRE(pa_bm_free(bm, s) == PA_OK && pa_bm_is_swapped(bm, s) == 0);
  REQUIRE(pa_bm_check_invariants(bm) == PA_OK);
  REQUIRE(pa_bm_num_free_blocks(bm) == nb);
  REQUIRE(pa_bm_num_seqs(bm) == 0);
  REQUIRE(oob > 0);
  if (prefix) REQUIRE(hits > 0 && swap_hits > 0);
  pa_bm_destroy(bm);
  std::printf("seed %u nb %d bs %d prefix %d: oob %ld cow %ld hits %ld swap hits %ld\n", seed, nb,
              bs, prefix, oob, cow, hits, swap_hits);
}

static void bad_arguments() {
  REQUIRE(pa_bm_create(0, 16, 1) == nullptr);
  REQUIRE(pa_bm_create(4, 0, 1) == nullptr);
  REQUIRE(pa_bm_allocate(nullptr, 1, nullptr, 0, nullptr, 0, nullptr) == PA_ERR_INVALID);
  pa_bm* bm = pa_bm_create(4, 2, 1);
  REQUIRE(bm);
  int32_t tab[4];
  REQUIRE(pa_bm_allocate(bm, 1, nullptr, 3, tab, 4, nullptr) == PA_ERR_INVALID);  // tokens NULL
  int32_t toks[3] = {1, 2, 3};
  REQUIRE(pa_bm_allocate(bm, 1, toks, -1, tab, 4, nullptr) == PA_ERR_INVALID);
  REQUIRE(pa_bm_allocate(bm, 1, toks, 3, tab, 1, nullptr) == PA_ERR_INVALID);  // cap too small
  REQUIRE(pa_bm_allocate(bm, 1, toks, 3, tab, 2, nullptr) == PA_OK);
  REQUIRE(pa_bm_allocate(bm, 1, toks, 3, tab, 2, nullptr) == PA_ERR_INVALID);  // exists
  REQUIRE(pa_bm_append_slot(bm, 99, 1, nullptr, nullptr, nullptr) == PA_ERR_INVALID);
  REQUIRE(pa_bm_free(bm, 99) == PA_OK);
  int64_t slot;
  REQUIRE(pa_bm_slot(bm, 1, 3, &slot) == PA_ERR_INVALID);
  REQUIRE(pa_bm_slot(bm, 1, -1, &slot) == PA_ERR_INVALID);
  int32_t n;
  REQUIRE(pa_bm_get_table(bm, 1, tab, 1, &n) == PA_ERR_INVALID);
  REQUIRE(pa_bm_can_allocate(bm, -1) == 0);
  REQUIRE(pa_bm_check_invariants(bm) == PA_OK);
  pa_bm_destroy(bm);
}

// Continuous-batching scheduler: seeded request streams with commits after
// every step; the manager's invariants and the host-record count must hold
// after every step, every request must finish with exactly its budget, and
// everything must drain back to an empty pool.
static void run_sched(uint32_t seed, int nb, int bs, int batch, int host, int prefix) {
  std::mt19937 rng(seed);
  pa_bm* bm = pa_bm_create(nb, bs, prefix);
  REQUIRE(bm);
  pa_sched* s = pa_sched_create(bm, batch, host);
  REQUIRE(s);
  const int cap_ids = batch, cap_pairs = std::max(host, 1), cap_pre = nb * bs;
  std::vector<int64_t> fin(cap_ids), res(cap_ids), adm(cap_ids), pre(cap_ids), rec(cap_ids),
      pslots(cap_pre), batch_ids(cap_ids), writes(cap_ids), slots(cap_ids);
  std::vector<int32_t> swin(2 * cap_pairs), swout(2 * cap_pairs), pcnt(cap_ids), cow(2 * cap_ids),
      cuts(3 * cap_ids);
  pa_sched_plan p{};
  p.ids_cap = cap_ids; p.pairs_cap = cap_pairs; p.prefill_cap = cap_pre;
  p.finished = fin.data(); p.resumed = res.data(); p.admitted = adm.data(); p.preempted = pre.data();
  p.recomputed = rec.data(); p.swap_in = swin.data(); p.swap_out = swout.data();
  p.prefill_slots = pslots.data(); p.prefill_counts = pcnt.data(); p.writes = writes.data();
  p.slots = slots.data(); p.cow_pairs = cow.data(); p.cuts = cuts.data(); p.batch = batch_ids.data();
  pa_sched_plan small = p;
  small.prefill_cap = cap_pre - 1;
  REQUIRE(pa_sched_step(s, &small) == PA_ERR_INVALID);          // refused before any change
  std::map<int64_t, int> budget, produced;
  int64_t next = 1;
  long preempted = 0, resumed = 0;
  const int n_req = 80;
  for (int step = 0; step < 20000; ++step) {
    while (next <= n_req && rng() % 10 < 3) {
      std::vector<int32_t> prompt(1 + rng() % (3 * bs));
      for (auto& t : prompt) t = rng() % 4;
      budget[next] = 1 + rng() % (4 * bs);
      REQUIRE(pa_sched_add_request(s, next, prompt.data(), (int32_t)prompt.size(), budget[next]) == PA_OK);
      ++next;
    }
    REQUIRE(pa_sched_step(s, &p) == PA_OK);
    for (int i = 0; i < p.n_finished; ++i) REQUIRE(produced[fin[i]] == budget[fin[i]]);
    preempted += p.n_preempted;
    resumed += p.n_resumed;
    REQUIRE(p.n_batch <= batch && p.n_writes <= batch && p.n_swap_in <= host && p.n_swap_out <= host);
    int32_t pw = 0, pc = 0, ps = 0;                               // cuts never go backwards
    for (int i = 0; i < p.n_preempted; ++i) {
      REQUIRE(cuts[3 * i] >= pw && cuts[3 * i + 1] >= pc && cuts[3 * i + 2] >= ps);
      pw = cuts[3 * i]; pc = cuts[3 * i + 1]; ps = cuts[3 * i + 2];
    }
    REQUIRE(pw <= p.n_writes && pc <= p.n_cow && ps == p.n_swap_out);
    std::vector<int64_t> ids(batch_ids.begin(), batch_ids.begin() + p.n_batch);
    for (int i = 0; i < p.n_admitted; ++i)                        // admitted and still running
      if (std::find(pre.begin(), pre.begin() + p.n_preempted, adm[i]) == pre.begin() + p.n_preempted)
        ids.push_back(adm[i]);
    if (!ids.empty()) {                                           // tokens owed: commit first
      pa_sched_plan again = p;
      REQUIRE(pa_sched_step(s, &again) == PA_ERR_INVALID);
    }
    std::vector<int32_t> toks(ids.size());
    for (auto& t : toks) t = rng() % 4;
    for (int64_t id : ids) ++produced[id];
    REQUIRE(pa_bm_check_invariants(bm) == PA_OK);
    int32_t nfree = -1, nswap = -1, nrun = -1, nwait = -1;
    REQUIRE(pa_sched_host_free(s, nullptr, 0, &nfree) == PA_OK);
    REQUIRE(pa_sched_swapped(s, nullptr, nullptr, 0, nullptr, 0, &nswap) == PA_OK);
    std::vector<int64_t> sid(nswap + 1);
    std::vector<int32_t> scnt(nswap + 1), srec(host + 1);
    REQUIRE(pa_sched_swapped(s, sid.data(), scnt.data(), nswap, srec.data(), host, &nswap) == PA_OK);
    int held = 0;
    for (int i = 0; i < nswap; ++i) held += scnt[i];
    REQUIRE(held + nfree == host);
    REQUIRE(pa_sched_running(s, nullptr, nullptr, 0, &nrun) == PA_OK && nrun <= batch);
    REQUIRE(pa_sched_waiting(s, nullptr, 0, &nwait) == PA_OK);
    REQUIRE(pa_sched_commit(s, ids.data(), toks.data(), (int32_t)ids.size()) == PA_OK);
    if (next > n_req && nrun == 0 && nwait == 0 && nswap == 0) break;
  }
  REQUIRE((int)produced.size() == n_req);
  for (auto& kv : budget) REQUIRE(produced[kv.first] == kv.second);
  REQUIRE(pa_bm_num_free_blocks(bm) == nb && pa_bm_num_seqs(bm) == 0);
  REQUIRE(preempted > 0);
  if (host > 0) REQUIRE(resumed > 0);
  pa_sched_destroy(s);
  pa_bm_destroy(bm);
  std::printf("sched seed %u: preempted %ld resumed %ld\n", seed, preempted, resumed);
}

int main() {
  bad_arguments();
  run_sched(11, 12, 4, 4, 16, 1);
  run_sched(12, 10, 2, 5, 6, 1);
  run_sched(13, 16, 4, 6, 0, 1);
  run_sched(14, 9, 3, 4, 40, 0);
  run(1, 8, 2, 1, 3, 20000);
  run(2, 12, 4, 1, 2, 20000);
  run(3, 24, 16, 1, 1, 5000);
  run(4, 10, 3, 0, 3, 20000);
  run(5, 6, 1, 1, 2, 20000);
  std::printf("bm_stress ok\n");
  return 0;
}
