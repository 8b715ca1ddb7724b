// Host step builder: the scheduler that turns requests into the flat ragged steps the device
// path consumes (cu_seqlens_q, ctx_lens, block tables, slots, block copies).
//
// "P3: native paged-KV continuous-batching sampler", section "Design > engine.py": a sequence
// is a token count plus num_computed; each scheduled sequence gets
// n_new = min(remaining, chunk_size, budget) rows; decodes are scheduled first and share the
// step with prefill chunks; admission is FIFO when the whole token list fits; on block
// exhaustion the youngest unscheduled running sequence is preempted by recompute; prefix
// sharing adopts the leading full blocks of a running sequence of the same prompt and always
// recomputes the last prompt token. "Optional paged KV cache (vLLM-style) — v1 design",
// sections "Design" (trim frees the now-unoccupied tail blocks) and "Follow-ups" (block-level
// copy-on-write: refcounted tables, fork on a divergent write).
//
// Where the pages leave a step open, the same readings as the oracle twin are taken: running
// sequences in admission order (forks admitted when made, preempted ones stay running with
// no blocks); admission promises each admitted sequence its whole token list within one
// step's admission round, nothing for the residents' growth; the victim is the youngest
// running sequence holding blocks and not yet scheduled (possibly the asker, which then waits);
// a sequence preempted while the step is built waits for a later step; adoption takes
// (prompt_len - 1) / block_size blocks of the oldest running sequence of the same group and
// prompt length once it has computed them; a chunk's blocks are one copy-on-write target (if
// it writes into a shared block) then the missing tail, in one all-or-nothing allocation;
// trim(n) keeps n tokens and feeds the last one again.
#include <algorithm>
#include <deque>
#include <new>
#include <string>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "common.h"

namespace {

enum { kWaiting = 0, kRunning = 1, kFinished = 2 };

struct Seq {
  int32_t sid = 0, prompt_len = 0, group = -1, n_tokens = 0, num_computed = 0;
  std::vector<int32_t> blocks;
  int32_t state = kWaiting;
  int64_t order = -1;  // admission counter; larger = younger
};

struct Plan {
  std::vector<int32_t> seq_ids, n_new, ctx_lens, cu_seqlens, slots, copies, preempted;
  std::vector<std::vector<int32_t>> tables;
  bool pending = false;
};

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

struct pkv_sched {
  int32_t bs = 0, chunk = 0, budget = 0, max_seqs = 0, max_blocks = 0;
  bool sharing = false;
  pkv_alloc* alloc = nullptr;
  std::unordered_map<int32_t, Seq> seqs;
  std::deque<int32_t> waiting;
  std::vector<int32_t> running;  // admission order
  int64_t counter = 0, preemptions = 0, shared_tokens = 0;
  Plan plan;
};

using pkv::fail;
using pkv::ok;

namespace {

void admit(pkv_sched* s, Seq& q, const std::vector<int32_t>& adopted) {
  if (!adopted.empty()) {
    pkv_alloc_incref(s->alloc, static_cast<int32_t>(adopted.size()), adopted.data());
    s->shared_tokens += static_cast<int64_t>(adopted.size()) * s->bs;
  }
  q.blocks = adopted;
  q.num_computed = static_cast<int32_t>(adopted.size()) * s->bs;
  q.state = kRunning;
  q.order = s->counter++;
  s->running.push_back(q.sid);
}

const Seq* leader_of(const pkv_sched* s, const Seq& q) {
  for (int32_t rid : s->running) {
    const Seq& r = s->seqs.at(rid);
    if (r.group == q.group && r.prompt_len == q.prompt_len) return &r;
  }
  return nullptr;
}

void admission(pkv_sched* s) {
  int64_t room = pkv_alloc_num_free(s->alloc);
  while (!s->waiting.empty() && static_cast<int32_t>(s->running.size()) < s->max_seqs) {
    Seq& q = s->seqs.at(s->waiting.front());
    std::vector<int32_t> adopted;
    if (s->sharing && q.group >= 0) {
      const Seq* lead = leader_of(s, q);
      const int32_t target = (q.prompt_len - 1) / s->bs;
      if (lead != nullptr && target > 0) {
        if (lead->num_computed < target * s->bs) return;  // defer: still being computed
        adopted.assign(lead->blocks.begin(), lead->blocks.begin() + target);
      }
    }
    const int64_t need = ceil_div(q.n_tokens, s->bs) - static_cast<int64_t>(adopted.size());
    if (need > room) return;
    room -= need;
    s->waiting.pop_front();
    admit(s, q, adopted);
  }
}

void free_blocks(pkv_sched* s, Seq& q) {
  if (!q.blocks.empty())
    pkv_alloc_free(s->alloc, static_cast<int32_t>(q.blocks.size()), q.blocks.data());
  q.blocks.clear();
}

Seq* victim_of(pkv_sched* s, const std::unordered_set<int32_t>& scheduled) {
  Seq* best = nullptr;
  for (int32_t rid : s->running) {
    Seq& r = s->seqs.at(rid);
    if (scheduled.count(rid) || r.blocks.empty()) continue;
    if (best == nullptr || r.order > best->order) best = &r;
  }
  return best;
}

// Blocks for q's next chunk of n_new rows, preempting as needed; false if q does not run now.
bool reserve(pkv_sched* s, Seq& q, int32_t n_new, const std::unordered_set<int32_t>& scheduled) {
  for (;;) {
    const int32_t j = q.num_computed / s->bs;
    const bool cow = j < static_cast<int32_t>(q.blocks.size()) &&
                     pkv_alloc_refcount(s->alloc, q.blocks[j]) > 1;
    const int64_t grow = std::max<int64_t>(
        0, ceil_div(static_cast<int64_t>(q.num_computed) + n_new, s->bs) -
               static_cast<int64_t>(q.blocks.size()));
    const int32_t need = static_cast<int32_t>(grow) + (cow ? 1 : 0);
    std::vector<int32_t> ids(need);
    if (pkv_alloc_allocate(s->alloc, need, ids.data()) != PKV_OK) {
      Seq* v = victim_of(s, scheduled);
      if (v == nullptr) return false;
      free_blocks(s, *v);
      v->num_computed = 0;
      ++s->preemptions;
      s->plan.preempted.push_back(v->sid);
      if (v == &q) return false;
      continue;
    }
    size_t first = 0;
    if (cow) {
      const int32_t src = q.blocks[j];
      s->plan.copies.push_back(src);
      s->plan.copies.push_back(ids[0]);
      pkv_alloc_free(s->alloc, 1, &src);
      q.blocks[j] = ids[0];
      first = 1;
    }
    q.blocks.insert(q.blocks.end(), ids.begin() + first, ids.end());
    return true;
  }
}

}  // namespace

extern "C" int32_t pkv_sched_create(int32_t num_blocks, int32_t block_size, int32_t chunk_size,
                                    int32_t token_budget, int32_t max_num_seqs,
                                    int32_t max_blocks_per_seq, int32_t prefix_sharing,
                                    pkv_sched** out) {
  if (out == nullptr) return fail(PKV_ERR_INVALID, "sched_create: out is NULL");
  *out = nullptr;
  if (num_blocks < 0 || block_size < 1 || chunk_size < 1 || token_budget < 1 ||
      max_num_seqs < 1 || max_blocks_per_seq < 1)
    return fail(PKV_ERR_INVALID, "sched_create: sizes must be >= 1 (num_blocks >= 0)");
  if (static_cast<int64_t>(max_blocks_per_seq) * block_size > INT32_MAX)
    return fail(PKV_ERR_INVALID, "sched_create: max_blocks_per_seq * block_size overflows");
  pkv_sched* s = new (std::nothrow) pkv_sched();
  if (s == nullptr) return fail(PKV_ERR_INVALID, "sched_create: out of host memory");
  if (pkv_alloc_create(num_blocks, &s->alloc) != PKV_OK) {
    delete s;
    return fail(PKV_ERR_INVALID, "sched_create: allocator");
  }
  s->bs = block_size;
  s->chunk = chunk_size;
  s->budget = token_budget;
  s->max_seqs = max_num_seqs;
  s->max_blocks = max_blocks_per_seq;
  s->sharing = prefix_sharing != 0;
  *out = s;
  return ok();
}

extern "C" void pkv_sched_destroy(pkv_sched* s) {
  if (s == nullptr) return;
  pkv_alloc_destroy(s->alloc);
  delete s;
}

extern "C" pkv_alloc* pkv_sched_allocator(pkv_sched* s) { return s ? s->alloc : nullptr; }

extern "C" int32_t pkv_sched_add(pkv_sched* s, int32_t seq_id, int32_t prompt_len,
                                 int32_t group) {
  if (s == nullptr) return fail(PKV_ERR_INVALID, "sched_add: NULL handle");
  if (s->seqs.count(seq_id)) return fail(PKV_ERR_INVALID, "sched_add: sequence id exists");
  if (prompt_len < 1 || static_cast<int64_t>(prompt_len) > static_cast<int64_t>(s->max_blocks) * s->bs)
    return fail(PKV_ERR_INVALID, "sched_add: prompt length outside [1, max_blocks_per_seq * "
                                 "block_size]");
  Seq q;
  q.sid = seq_id;
  q.prompt_len = prompt_len;
  q.group = group;
  q.n_tokens = prompt_len;
  s->seqs.emplace(seq_id, std::move(q));
  s->waiting.push_back(seq_id);
  return ok();
}

extern "C" int32_t pkv_sched_step(pkv_sched* s, int32_t* B, int32_t* T, int32_t* n_copies,
                                  int32_t* n_preempted) {
  if (s == nullptr) return fail(PKV_ERR_INVALID, "sched_step: NULL handle");
  if (s->plan.pending) return fail(PKV_ERR_INVALID, "sched_step: previous step not completed");
  s->plan = Plan();
  admission(s);
  int32_t budget = s->budget;
  std::unordered_set<int32_t> scheduled;
  std::vector<std::pair<int32_t, int32_t>> order;
  for (int pass = 0; pass < 2; ++pass) {
    const bool decode_pass = pass == 0;
    const std::vector<int32_t> run = s->running;
    for (int32_t rid : run) {
      if (budget == 0) break;
      Seq& q = s->seqs.at(rid);
      const int32_t rem = q.n_tokens - q.num_computed;
      if (rem <= 0 || scheduled.count(rid) ||
          std::find(s->plan.preempted.begin(), s->plan.preempted.end(), rid) !=
              s->plan.preempted.end() ||
          (rem == 1) != decode_pass)
        continue;
      const int32_t n_new = std::min(std::min(rem, s->chunk), budget);
      if (reserve(s, q, n_new, scheduled)) {
        scheduled.insert(rid);
        order.emplace_back(rid, n_new);
        budget -= n_new;
      }
    }
  }
  Plan& p = s->plan;
  p.cu_seqlens.push_back(0);
  for (const auto& e : order) {
    const Seq& q = s->seqs.at(e.first);
    p.seq_ids.push_back(e.first);
    p.n_new.push_back(e.second);
    p.ctx_lens.push_back(q.num_computed + e.second);
    p.cu_seqlens.push_back(p.cu_seqlens.back() + e.second);
    p.tables.push_back(q.blocks);
    for (int32_t pos = q.num_computed; pos < q.num_computed + e.second; ++pos)
      p.slots.push_back(q.blocks[pos / s->bs] * s->bs + pos % s->bs);
  }
  p.pending = true;
  if (B) *B = static_cast<int32_t>(p.seq_ids.size());
  if (T) *T = p.cu_seqlens.back();
  if (n_copies) *n_copies = static_cast<int32_t>(p.copies.size() / 2);
  if (n_preempted) *n_preempted = static_cast<int32_t>(p.preempted.size());
  return ok();
}

extern "C" int32_t pkv_sched_plan(const pkv_sched* s, int32_t* seq_ids, int32_t* n_new,
                                  int32_t* ctx_lens, int32_t* cu_seqlens_q, int32_t* block_tables,
                                  int32_t* slots, int32_t* copies, int32_t* preempted) {
  if (s == nullptr) return fail(PKV_ERR_INVALID, "sched_plan: NULL handle");
  if (!s->plan.pending) return fail(PKV_ERR_INVALID, "sched_plan: no step pending");
  const Plan& p = s->plan;
  const size_t B = p.seq_ids.size();
  if (seq_ids) std::copy(p.seq_ids.begin(), p.seq_ids.end(), seq_ids);
  if (n_new) std::copy(p.n_new.begin(), p.n_new.end(), n_new);
  if (ctx_lens) std::copy(p.ctx_lens.begin(), p.ctx_lens.end(), ctx_lens);
  if (cu_seqlens_q) std::copy(p.cu_seqlens.begin(), p.cu_seqlens.end(), cu_seqlens_q);
  if (block_tables) {
    for (size_t b = 0; b < B; ++b) {
      int32_t* row = block_tables + b * s->max_blocks;
      std::fill(row, row + s->max_blocks, -1);
      std::copy(p.tables[b].begin(), p.tables[b].end(), row);
    }
  }
  if (slots) std::copy(p.slots.begin(), p.slots.end(), slots);
  if (copies) std::copy(p.copies.begin(), p.copies.end(), copies);
  if (preempted) std::copy(p.preempted.begin(), p.preempted.end(), preempted);
  return ok();
}

extern "C" int32_t pkv_sched_complete(pkv_sched* s, const int32_t* finished, int32_t n_finished,
                                      int32_t* sampled, int32_t* n_sampled) {
  if (s == nullptr) return fail(PKV_ERR_INVALID, "sched_complete: NULL handle");
  if (!s->plan.pending) return fail(PKV_ERR_INVALID, "sched_complete: no step pending");
  if (n_finished < 0 || (n_finished > 0 && finished == nullptr))
    return fail(PKV_ERR_INVALID, "sched_complete: bad finished list");
  std::unordered_set<int32_t> fin(finished, finished + n_finished);
  const int64_t cap = static_cast<int64_t>(s->max_blocks) * s->bs;
  int32_t ns = 0;
  Plan& p = s->plan;
  for (size_t b = 0; b < p.seq_ids.size(); ++b) {
    Seq& q = s->seqs.at(p.seq_ids[b]);
    q.num_computed += p.n_new[b];
    if (q.num_computed == q.n_tokens) {
      if (sampled) sampled[ns] = q.sid;
      ++ns;
      if (fin.count(q.sid) || q.n_tokens >= cap) {
        free_blocks(s, q);
        q.state = kFinished;
        s->running.erase(std::find(s->running.begin(), s->running.end(), q.sid));
      } else {
        ++q.n_tokens;
      }
    }
  }
  p.pending = false;
  if (n_sampled) *n_sampled = ns;
  return ok();
}

extern "C" int32_t pkv_sched_trim(pkv_sched* s, int32_t seq_id, int32_t n_tokens) {
  if (s == nullptr) return fail(PKV_ERR_INVALID, "sched_trim: NULL handle");
  if (s->plan.pending) return fail(PKV_ERR_INVALID, "sched_trim: a step awaits completion");
  auto it = s->seqs.find(seq_id);
  if (it == s->seqs.end() || it->second.state != kRunning || n_tokens < 1 ||
      n_tokens > it->second.n_tokens)
    return fail(PKV_ERR_INVALID, "sched_trim: not a running sequence, or past its tokens");
  Seq& q = it->second;
  q.n_tokens = n_tokens;
  q.num_computed = std::min(q.num_computed, n_tokens - 1);
  const size_t keep = static_cast<size_t>(ceil_div(q.num_computed, s->bs));
  if (q.blocks.size() > keep) {
    pkv_alloc_free(s->alloc, static_cast<int32_t>(q.blocks.size() - keep), q.blocks.data() + keep);
    q.blocks.resize(keep);
  }
  return ok();
}

extern "C" int32_t pkv_sched_fork(pkv_sched* s, int32_t src_id, int32_t new_id) {
  if (s == nullptr) return fail(PKV_ERR_INVALID, "sched_fork: NULL handle");
  if (s->plan.pending) return fail(PKV_ERR_INVALID, "sched_fork: a step awaits completion");
  auto it = s->seqs.find(src_id);
  if (it == s->seqs.end() || it->second.state != kRunning)
    return fail(PKV_ERR_INVALID, "sched_fork: not a running sequence");
  if (s->seqs.count(new_id)) return fail(PKV_ERR_INVALID, "sched_fork: new id exists");
  if (static_cast<int32_t>(s->running.size()) >= s->max_seqs)
    return fail(PKV_ERR_INVALID, "sched_fork: max_num_seqs reached");
  Seq f = it->second;
  f.sid = new_id;
  if (!f.blocks.empty())
    pkv_alloc_incref(s->alloc, static_cast<int32_t>(f.blocks.size()), f.blocks.data());
  f.state = kRunning;
  f.order = s->counter++;
  s->seqs.emplace(new_id, std::move(f));
  s->running.push_back(new_id);
  return ok();
}

extern "C" int32_t pkv_sched_seq_info(const pkv_sched* s, int32_t seq_id, int32_t* state,
                                      int32_t* n_tokens, int32_t* num_computed,
                                      int32_t* n_blocks) {
  if (s == nullptr) return fail(PKV_ERR_INVALID, "sched_seq_info: NULL handle");
  auto it = s->seqs.find(seq_id);
  if (it == s->seqs.end()) return fail(PKV_ERR_INVALID, "sched_seq_info: unknown sequence");
  if (state) *state = it->second.state;
  if (n_tokens) *n_tokens = it->second.n_tokens;
  if (num_computed) *num_computed = it->second.num_computed;
  if (n_blocks) *n_blocks = static_cast<int32_t>(it->second.blocks.size());
  return ok();
}

extern "C" int32_t pkv_sched_seq_blocks(const pkv_sched* s, int32_t seq_id, int32_t* blocks) {
  if (s == nullptr || blocks == nullptr) return fail(PKV_ERR_INVALID, "sched_seq_blocks: NULL");
  auto it = s->seqs.find(seq_id);
  if (it == s->seqs.end()) return fail(PKV_ERR_INVALID, "sched_seq_blocks: unknown sequence");
  std::copy(it->second.blocks.begin(), it->second.blocks.end(), blocks);
  return ok();
}

extern "C" int32_t pkv_sched_stats(const pkv_sched* s, int64_t* preemptions,
                                   int64_t* shared_tokens, int32_t* n_running,
                                   int32_t* n_waiting) {
  if (s == nullptr) return fail(PKV_ERR_INVALID, "sched_stats: NULL handle");
  if (preemptions) *preemptions = s->preemptions;
  if (shared_tokens) *shared_tokens = s->shared_tokens;
  if (n_running) *n_running = static_cast<int32_t>(s->running.size());
  if (n_waiting) *n_waiting = static_cast<int32_t>(s->waiting.size());
  return ok();
}

extern "C" int32_t pkv_sched_check(const pkv_sched* s) {
  if (s == nullptr) return fail(PKV_ERR_INVALID, "sched_check: NULL handle");
  if (pkv_alloc_check_consistent(s->alloc) != PKV_OK)
    return fail(PKV_ERR_INCONSISTENT, "sched_check: allocator inconsistent");
  std::vector<int32_t> ref(pkv_alloc_num_blocks(s->alloc), 0);
  for (const auto& kv : s->seqs) {
    const Seq& q = kv.second;
    if (q.state != kRunning) {
      if (!q.blocks.empty())
        return fail(PKV_ERR_INCONSISTENT, "sched_check: a non-running sequence holds blocks");
      continue;
    }
    for (int32_t b : q.blocks) ++ref[b];
    if (static_cast<int64_t>(q.blocks.size()) < ceil_div(q.num_computed, s->bs))
      return fail(PKV_ERR_INCONSISTENT, "sched_check: computed past the blocks held");
  }
  for (size_t b = 0; b < ref.size(); ++b)
    if (ref[b] != pkv_alloc_refcount(s->alloc, static_cast<int32_t>(b)))
      return fail(PKV_ERR_INCONSISTENT, "sched_check: refcounts differ from the live tables");
  return ok();
}
