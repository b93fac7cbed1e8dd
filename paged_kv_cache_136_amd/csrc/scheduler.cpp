// Continuous-batching scheduler over the host block manager.
//
// "qaqbuyan.com article 130", continuous-batching section: the step
// timeline (a finished request leaves and a waiting one joins at the next
// step) and the scheduler's step -- drop finished requests and free their
// blocks; admit waiting requests first come first served until the batch
// is full or blocks run short (the one that does not fit stays at the
// front); run the batch; append each request's new token, and when no
// block is left preempt the running request with the most generated
// tokens (_preempt_request), whose KV goes to host memory and whose blocks
// are freed.
//
// Where the page stops short:
//   * the step that admits a request runs its prompt and yields its first
//     token; every later step appends the previous token and decodes the
//     next; a request whose budget is met leaves at the next step;
//   * preempted requests resume (pa_bm_swap_in) before new admissions,
//     oldest preemption first;
//   * the appends walk the running list as it stood when they began,
//     skipping requests preempted meanwhile; the victim is the most
//     generated over every running request (the first such in running
//     order), and the failing request retries until it succeeds or is the
//     victim itself;
//   * nothing is undone: a victim that already appended keeps its token and
//     owes a decode, which it gets in the first step after it resumes,
//     without appending;
//   * host swap space is a FIFO pool of block records; a victim that does
//     not fit is recomputed instead: freed, and put back at the front of the
//     waiting queue with every token it has produced as its prompt.
//
// The scheduler only decides.  The caller performs the step's device work
// from the plan in decision order: swap-in copies, prompt K/V writes, then
// for each preemption the copy-on-write copies and writes of the appends
// before it followed by its swap-out copies (plan->cuts), then the rest of
// the copies and writes, then decode.
#include <algorithm>
#include <deque>
#include <memory>
#include <mutex>
#include <string>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "pagedkv.h"
#include "status.hpp"

namespace {

struct Req {
  int64_t id = 0;
  std::vector<int32_t> tokens;  // tokens the block manager holds
  int32_t max_new = 0;
  int32_t generated = 0;        // tokens produced (committed)
  bool has_pending = false;     // produced, not yet appended
  int32_t pending = 0;
  std::vector<int32_t> host;    // host records while swapped out
};

}  // namespace

struct pa_sched {
  pa_bm* bm = nullptr;
  int32_t max_batch = 0, host_total = 0, bs = 0, nb = 0;
  std::unordered_map<int64_t, std::unique_ptr<Req>> reqs;
  std::deque<Req*> waiting, swapped;
  std::vector<Req*> running;
  std::deque<int32_t> host_free;
  std::unordered_set<int64_t> to_commit;
  std::vector<int32_t> table;   // scratch
  std::mutex mu;
};

using pkv::fail;

namespace {

int32_t blocks_of(const pa_sched* s, size_t ntok) {
  return static_cast<int32_t>((ntok + s->bs - 1) / s->bs);
}

template <typename T>
bool push(T* arr, int32_t* n, int32_t cap, T v) {
  if (*n >= cap) return false;
  arr[(*n)++] = v;
  return true;
}

// Preempt `v` (already known to be running): swap to host records if they
// fit, else recompute.
int preempt(pa_sched* s, Req* v, pa_sched_plan* p) {
  int32_t len = 0;
  int st = pa_bm_seq_len(s->bm, v->id, &len);
  if (st != PA_OK) return st;
  const int32_t need = blocks_of(s, len);
  s->running.erase(std::find(s->running.begin(), s->running.end(), v));
  if (!push(p->preempted, &p->n_preempted, s->max_batch, v->id))
    return fail(PA_ERR_INVALID, "pa_sched_step: plan full");
  if (need <= static_cast<int32_t>(s->host_free.size())) {
    s->table.resize(std::max(need, 1));
    int32_t n = 0;
    st = pa_bm_swap_out(s->bm, v->id, s->table.data(), need, &n);
    if (st != PA_OK) return st;
    v->host.clear();
    for (int32_t i = 0; i < n; ++i) {
      const int32_t r = s->host_free.front();
      s->host_free.pop_front();
      v->host.push_back(r);
      if (p->n_swap_out >= s->host_total) return fail(PA_ERR_INVALID, "pa_sched_step: plan full");
      p->swap_out[2 * p->n_swap_out] = s->table[i];
      p->swap_out[2 * p->n_swap_out + 1] = r;
      ++p->n_swap_out;
    }
    s->swapped.push_back(v);
  } else {
    st = pa_bm_free(s->bm, v->id);
    if (st != PA_OK) return st;
    if (v->has_pending) {       // its K/V was never computed: part of the new prompt
      v->tokens.push_back(v->pending);
      v->has_pending = false;
    }
    s->waiting.push_front(v);
    if (!push(p->recomputed, &p->n_recomputed, s->max_batch, v->id))
      return fail(PA_ERR_INVALID, "pa_sched_step: plan full");
  }
  int32_t* cut = p->cuts + 3 * (p->n_preempted - 1);
  cut[0] = p->n_writes;
  cut[1] = p->n_cow;
  cut[2] = p->n_swap_out;
  return PA_OK;
}

int step_locked(pa_sched* s, pa_sched_plan* p) {
  const int32_t mb = s->max_batch;
  // 1. finished requests leave; their blocks are freed.
  for (size_t i = 0; i < s->running.size();) {
    Req* r = s->running[i];
    if (r->generated >= r->max_new) {
      int st = pa_bm_free(s->bm, r->id);
      if (st != PA_OK) return st;
      push(p->finished, &p->n_finished, mb, r->id);
      s->running.erase(s->running.begin() + i);
      s->reqs.erase(r->id);
    } else {
      ++i;
    }
  }
  // 2. preempted requests resume first, oldest first.
  while (!s->swapped.empty() && static_cast<int32_t>(s->running.size()) < mb) {
    Req* r = s->swapped.front();
    const int32_t need = blocks_of(s, r->tokens.size());
    s->table.resize(std::max(need, 1));
    int32_t n = 0, first = 0;
    int st = pa_bm_swap_in(s->bm, r->id, s->table.data(), need, &n, &first);
    if (st == PA_ERR_OUT_OF_BLOCKS) break;
    if (st != PA_OK) return st;
    s->swapped.pop_front();
    for (int32_t i = first; i < n; ++i) {
      if (p->n_swap_in >= s->host_total) return fail(PA_ERR_INVALID, "pa_sched_step: plan full");
      p->swap_in[2 * p->n_swap_in] = r->host[i];
      p->swap_in[2 * p->n_swap_in + 1] = s->table[i];
      ++p->n_swap_in;
    }
    for (int32_t h : r->host) s->host_free.push_back(h);
    r->host.clear();
    s->running.push_back(r);
    push(p->resumed, &p->n_resumed, mb, r->id);
  }
  // 3. admit waiting requests, first come first served.
  std::unordered_set<int64_t> admitted;
  while (!s->waiting.empty() && static_cast<int32_t>(s->running.size()) < mb) {
    Req* r = s->waiting.front();
    const int32_t ntok = static_cast<int32_t>(r->tokens.size());
    const int32_t need = blocks_of(s, ntok);
    s->table.resize(std::max(need, 1));
    int32_t nbk = 0;
    int st = pa_bm_allocate(s->bm, r->id, r->tokens.data(), ntok, s->table.data(), need, &nbk);
    if (st == PA_ERR_OUT_OF_BLOCKS) break;
    if (st != PA_OK) return st;
    s->waiting.pop_front();
    int32_t cached = 0;
    st = pa_bm_num_cached_tokens(s->bm, r->id, &cached);
    if (st != PA_OK) return st;
    if (p->n_prefill_slots + (ntok - cached) > p->prefill_cap)
      return fail(PA_ERR_INVALID, "pa_sched_step: prefill_slots too small");
    for (int32_t pos = cached; pos < ntok; ++pos)
      p->prefill_slots[p->n_prefill_slots++] =
          static_cast<int64_t>(s->table[pos / s->bs]) * s->bs + pos % s->bs;
    p->prefill_counts[p->n_admitted] = ntok - cached;
    push(p->admitted, &p->n_admitted, mb, r->id);
    s->running.push_back(r);
    admitted.insert(r->id);
  }
  // 4. append each running request's pending token, preempting the most
  //    generated running request whenever no block is left.
  const std::vector<Req*> order = s->running;
  for (Req* r : order) {
    if (admitted.count(r->id) || !r->has_pending) continue;
    if (std::find(s->running.begin(), s->running.end(), r) == s->running.end()) continue;
    for (;;) {
      int64_t slot = -1;
      int32_t src = -1, dst = -1;
      int st = pa_bm_append_slot(s->bm, r->id, r->pending, &slot, &src, &dst);
      if (st == PA_ERR_OUT_OF_BLOCKS) {
        Req* victim = nullptr;   // most generated; the first such in running order
        for (Req* x : s->running)
          if (!victim || x->generated > victim->generated) victim = x;
        st = preempt(s, victim, p);
        if (st != PA_OK) return st;
        if (victim == r) break;
        continue;
      }
      if (st != PA_OK) return st;
      r->tokens.push_back(r->pending);
      r->has_pending = false;
      p->writes[p->n_writes] = r->id;
      p->slots[p->n_writes] = slot;
      ++p->n_writes;
      if (src >= 0) {
        p->cow_pairs[2 * p->n_cow] = src;
        p->cow_pairs[2 * p->n_cow + 1] = dst;
        ++p->n_cow;
      }
      break;
    }
  }
  // The decode batch: every running request not admitted in this step; each
  // has its last token in the cache (appended now, or before a preemption).
  s->to_commit.clear();
  for (Req* r : s->running) {
    s->to_commit.insert(r->id);
    if (!admitted.count(r->id)) p->batch[p->n_batch++] = r->id;
  }
  return PA_OK;
}

}  // namespace

extern "C" {

pa_sched* pa_sched_create(pa_bm* bm, int32_t max_batch, int32_t host_slots) {
  if (!bm || max_batch <= 0 || host_slots < 0) {
    fail(PA_ERR_INVALID, "pa_sched_create: need a manager, max_batch > 0 and host_slots >= 0");
    return nullptr;
  }
  pa_sched* s = new pa_sched;
  s->bm = bm;
  s->max_batch = max_batch;
  s->host_total = host_slots;
  s->bs = pa_bm_block_size(bm);
  s->nb = pa_bm_num_blocks(bm);
  for (int32_t i = 0; i < host_slots; ++i) s->host_free.push_back(i);
  pkv::clear_error();
  return s;
}

void pa_sched_destroy(pa_sched* s) { delete s; }

int pa_sched_add_request(pa_sched* s, int64_t id, const int32_t* prompt, int32_t n,
                         int32_t max_new_tokens) {
  if (!s) return fail(PA_ERR_INVALID, "pa_sched_add_request: null scheduler");
  std::lock_guard<std::mutex> lock(s->mu);
  if (n <= 0 || !prompt || max_new_tokens < 1)
    return fail(PA_ERR_INVALID, "pa_sched_add_request: need a prompt and max_new_tokens >= 1");
  int32_t live_len = 0;
  if (s->reqs.count(id) || pa_bm_seq_len(s->bm, id, &live_len) == PA_OK ||
      pa_bm_is_swapped(s->bm, id) == 1)
    return fail(PA_ERR_INVALID, "pa_sched_add_request: id in use");
  auto r = std::make_unique<Req>();
  r->id = id;
  r->tokens.assign(prompt, prompt + n);
  r->max_new = max_new_tokens;
  s->waiting.push_back(r.get());
  s->reqs.emplace(id, std::move(r));
  pkv::clear_error();
  return PA_OK;
}

int pa_sched_step(pa_sched* s, pa_sched_plan* p) {
  if (!s || !p) return fail(PA_ERR_INVALID, "pa_sched_step: null argument");
  std::lock_guard<std::mutex> lock(s->mu);
  if (!s->to_commit.empty()) return fail(PA_ERR_INVALID, "pa_sched_step: commit the previous step first");
  if (!p->finished || !p->resumed || !p->admitted || !p->preempted || !p->recomputed ||
      !p->prefill_counts || !p->writes || !p->slots || !p->cow_pairs || !p->cuts || !p->batch ||
      (s->host_total > 0 && (!p->swap_in || !p->swap_out)) || (p->prefill_cap > 0 && !p->prefill_slots) ||
      p->prefill_cap < 0)
    return fail(PA_ERR_INVALID, "pa_sched_step: plan arrays missing");
  // With these capacities no array can fill up mid-step (uncached prompt
  // tokens only occupy blocks taken in this step), so a step never stops
  // half done.
  if (p->ids_cap < s->max_batch || p->pairs_cap < s->host_total ||
      p->prefill_cap < static_cast<int64_t>(s->nb) * s->bs)
    return fail(PA_ERR_INVALID, "pa_sched_step: plan arrays need max_batch ids, host_slots pairs "
                                "and num_blocks * block_size prefill slots");
  p->n_finished = p->n_resumed = p->n_admitted = p->n_preempted = p->n_recomputed = 0;
  p->n_swap_in = p->n_swap_out = p->n_prefill_slots = p->n_writes = p->n_cow = p->n_batch = 0;
  int st = step_locked(s, p);
  if (st == PA_OK) pkv::clear_error();
  return st;
}

int pa_sched_commit(pa_sched* s, const int64_t* ids, const int32_t* tokens, int32_t n) {
  if (!s || n < 0 || (n > 0 && (!ids || !tokens))) return fail(PA_ERR_INVALID, "pa_sched_commit: bad arguments");
  std::lock_guard<std::mutex> lock(s->mu);
  std::unordered_set<int64_t> seen;
  for (int32_t i = 0; i < n; ++i)
    if (!s->to_commit.count(ids[i]) || !seen.insert(ids[i]).second)
      return fail(PA_ERR_INVALID, "pa_sched_commit: id not owed a token, or repeated");
  if (seen.size() != s->to_commit.size())
    return fail(PA_ERR_INVALID, "pa_sched_commit: every request of the step needs its token");
  for (int32_t i = 0; i < n; ++i) {
    Req* r = s->reqs.at(ids[i]).get();
    r->pending = tokens[i];
    r->has_pending = true;
    ++r->generated;
  }
  s->to_commit.clear();
  pkv::clear_error();
  return PA_OK;
}

int pa_sched_running(pa_sched* s, int64_t* ids, int32_t* generated, int32_t cap, int32_t* n_out) {
  if (!s || !n_out) return fail(PA_ERR_INVALID, "pa_sched_running: null argument");
  std::lock_guard<std::mutex> lock(s->mu);
  const int32_t n = static_cast<int32_t>(s->running.size());
  *n_out = n;
  if (!ids && !generated) return PA_OK;
  if (n > cap || !ids || !generated) return fail(PA_ERR_INVALID, "pa_sched_running: output too small");
  for (int32_t i = 0; i < n; ++i) {
    ids[i] = s->running[i]->id;
    generated[i] = s->running[i]->generated;
  }
  return PA_OK;
}

int pa_sched_waiting(pa_sched* s, int64_t* ids, int32_t cap, int32_t* n_out) {
  if (!s || !n_out) return fail(PA_ERR_INVALID, "pa_sched_waiting: null argument");
  std::lock_guard<std::mutex> lock(s->mu);
  const int32_t n = static_cast<int32_t>(s->waiting.size());
  *n_out = n;
  if (!ids) return PA_OK;
  if (n > cap) return fail(PA_ERR_INVALID, "pa_sched_waiting: output too small");
  for (int32_t i = 0; i < n; ++i) ids[i] = s->waiting[i]->id;
  return PA_OK;
}

int pa_sched_swapped(pa_sched* s, int64_t* ids, int32_t* num_records, int32_t cap,
                     int32_t* records, int32_t records_cap, int32_t* n_out) {
  if (!s || !n_out) return fail(PA_ERR_INVALID, "pa_sched_swapped: null argument");
  std::lock_guard<std::mutex> lock(s->mu);
  const int32_t n = static_cast<int32_t>(s->swapped.size());
  *n_out = n;
  if (!ids && !num_records && !records) return PA_OK;
  int32_t total = 0;
  for (Req* r : s->swapped) total += static_cast<int32_t>(r->host.size());
  if (n > cap || total > records_cap || !ids || !num_records || (total > 0 && !records))
    return fail(PA_ERR_INVALID, "pa_sched_swapped: output too small");
  int32_t k = 0;
  for (int32_t i = 0; i < n; ++i) {
    const Req* r = s->swapped[i];
    ids[i] = r->id;
    num_records[i] = static_cast<int32_t>(r->host.size());
    for (int32_t h : r->host) records[k++] = h;
  }
  return PA_OK;
}

int pa_sched_host_free(pa_sched* s, int32_t* records, int32_t cap, int32_t* n_out) {
  if (!s || !n_out) return fail(PA_ERR_INVALID, "pa_sched_host_free: null argument");
  std::lock_guard<std::mutex> lock(s->mu);
  const int32_t n = static_cast<int32_t>(s->host_free.size());
  *n_out = n;
  if (!records) return PA_OK;
  if (n > cap) return fail(PA_ERR_INVALID, "pa_sched_host_free: output too small");
  for (int32_t i = 0; i < n; ++i) records[i] = s->host_free[i];
  return PA_OK;
}

}  // extern "C"
