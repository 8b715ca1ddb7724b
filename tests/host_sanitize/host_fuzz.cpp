// Randomised exercise of the library's host C++ (block allocator, slot mapping, slot checks,
// step builder and work planner), built with g++ under AddressSanitizer and
// UndefinedBehaviorSanitizer together with allocator.cpp, scheduler.cpp and planner.cpp only
// (no HIP): any out-of-bounds access, use after free, leak, signed overflow or misaligned
// access fails the run. Beside the sanitizers it checks the invariants the host code promises:
//   - allocator books after every event: pkv_alloc_check_consistent, and refcounts equal to
//     the references held by a model of the live block tables ("P3: native paged-KV
//     continuous-batching sampler", section "Design > paged.py": check_consistent);
//   - the step builder's own check (pkv_sched_check) after every event;
//   - the work planner: lists fill their layout exactly, every decode row's splits appear
//     once with the merge and partial slots it needs, every tile-path row is covered once per
//     split, partial slots are disjoint and inside the layout, lists are longest first.
// Usage: host_fuzz <seed> <rounds>. Prints one summary line; exits non-zero on a failed check.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <random>
#include <set>
#include <vector>

#include "pkv.h"
#include "planner.h"

namespace {

int g_fail = 0;
#define CHECK(c)                                                                    \
  do {                                                                              \
    if (!(c)) {                                                                     \
      std::fprintf(stderr, "check failed at %s:%d: %s\n", __FILE__, __LINE__, #c); \
      ++g_fail;                                                                     \
      return;                                                                       \
    }                                                                               \
  } while (0)

using Rng = std::mt19937_64;
int uni(Rng& r, int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(r); }
double unif(Rng& r) { return std::uniform_real_distribution<double>(0.0, 1.0)(r); }

// ---- allocator: admissions with optional prefix sharing, growth, finishes --------------
void fuzz_allocator(Rng& rng, int events, long* counters) {
  const int nb = uni(rng, 1, 96);
  const int bs = uni(rng, 1, 8);
  pkv_alloc* a = nullptr;
  CHECK(pkv_alloc_create(nb, &a) == PKV_OK);
  std::vector<std::vector<int32_t>> tables;   // live sequences' blocks
  std::vector<int> full;                      // blocks of each table that are full (shareable)
  for (int e = 0; e < events; ++e) {
    const double ev = unif(rng);
    if (ev < 0.35 || tables.empty()) {        // admit, maybe adopting a prefix
      std::vector<int32_t> t;
      if (!tables.empty() && unif(rng) < 0.4) {
        const int src = uni(rng, 0, static_cast<int>(tables.size()) - 1);
        const int n = uni(rng, 0, full[src]);
        if (n > 0) {
          CHECK(pkv_alloc_incref(a, n, tables[src].data()) == PKV_OK);
          t.assign(tables[src].begin(), tables[src].begin() + n);
          counters[1] += 1;
        }
      }
      const int fresh = uni(rng, 1, 6);
      std::vector<int32_t> ids(fresh);
      const int free_before = pkv_alloc_num_free(a);
      const int32_t st = pkv_alloc_allocate(a, fresh, ids.data());
      if (st == PKV_ERR_POOL_EXHAUSTED) {
        CHECK(fresh > free_before && pkv_alloc_num_free(a) == free_before);
        counters[0] += 1;
        if (!t.empty()) CHECK(pkv_alloc_free(a, static_cast<int32_t>(t.size()), t.data()) == PKV_OK);
      } else {
        CHECK(st == PKV_OK);
        t.insert(t.end(), ids.begin(), ids.end());
        const int shared = static_cast<int>(t.size()) - fresh;
        tables.push_back(t);
        full.push_back(shared + uni(rng, 0, fresh - 1));
      }
    } else if (ev < 0.6) {                     // finish a sequence
      const int i = uni(rng, 0, static_cast<int>(tables.size()) - 1);
      CHECK(pkv_alloc_free(a, static_cast<int32_t>(tables[i].size()), tables[i].data()) == PKV_OK);
      tables.erase(tables.begin() + i);
      full.erase(full.begin() + i);
    } else if (ev < 0.8) {                     // slot mapping over a sequence's own blocks
      const int i = uni(rng, 0, static_cast<int>(tables.size()) - 1);
      const auto& t = tables[i];
      const int n_tok = static_cast<int>(t.size()) * bs;
      const int start = uni(rng, 0, n_tok - 1);
      const int n_new = uni(rng, 1, n_tok - start);
      std::vector<int32_t> slots(n_new, -9);
      const int32_t st = pkv_slot_mapping(a, t.data(), static_cast<int32_t>(t.size()), bs, start,
                                          n_new, slots.data());
      bool any_shared = false;
      for (int p = start; p < start + n_new; ++p)
        any_shared |= pkv_alloc_refcount(a, t[p / bs]) > 1;
      if (any_shared) {
        CHECK(st == PKV_ERR_SHARED_WRITE);
      } else {
        CHECK(st == PKV_OK);
        for (int k = 0; k < n_new; ++k) {
          const int p = start + k;
          CHECK(slots[k] == t[p / bs] * bs + p % bs);
        }
        CHECK(pkv_validate_slots(slots.data(), n_new, static_cast<int64_t>(nb) * bs) == PKV_OK);
      }
    } else if (ev < 0.9) {                     // refusals change nothing
      std::vector<int32_t> rc0(nb), rc1(nb), st0(nb + 1), st1(nb + 1);
      CHECK(pkv_alloc_snapshot(a, st0.data(), rc0.data()) == PKV_OK);
      int32_t dead = -1;
      for (int b = 0; b < nb; ++b)
        if (rc0[b] == 0) dead = b;
      if (dead >= 0) {
        CHECK(pkv_alloc_free(a, 1, &dead) == PKV_ERR_DOUBLE_FREE);
        CHECK(pkv_alloc_incref(a, 1, &dead) == PKV_ERR_INVALID);
        counters[2] += 1;
      }
      const int32_t out_of_pool = nb + uni(rng, 0, 3);
      CHECK(pkv_alloc_free(a, 1, &out_of_pool) == PKV_ERR_INVALID);
      CHECK(pkv_alloc_snapshot(a, st1.data(), rc1.data()) == PKV_OK);
      CHECK(rc0 == rc1 && st0 == st1);
    } else {                                   // slot array checks (both code paths)
      const int n = uni(rng, 0, 40);
      const int64_t ns = static_cast<int64_t>(uni(rng, 1, 1 << 20));
      std::vector<int32_t> s(n);
      std::set<int32_t> seen;
      bool dup = false, out = false;
      for (int k = 0; k < n; ++k) {
        const double c = unif(rng);
        s[k] = c < 0.1 ? -1 - uni(rng, 0, 5)
                       : (c < 0.15 ? static_cast<int32_t>(ns + uni(rng, 0, 9))
                                   : static_cast<int32_t>(uni(rng, 0, static_cast<int>(std::min<int64_t>(ns - 1, 200)))));
        if (s[k] >= ns) out = true;
        if (s[k] >= 0 && s[k] < ns && !seen.insert(s[k]).second) dup = true;
        if (unif(rng) < 0.5 && s[k] >= 0 && s[k] < ns)
          s[k] = static_cast<int32_t>(std::min<int64_t>(ns - 1, static_cast<int64_t>(s[k]) * 997));
      }
      // recompute the expectation after the spread (ranges far apart take the sorted path)
      seen.clear();
      dup = false;
      out = false;
      for (int k = 0; k < n; ++k) {
        if (s[k] >= ns) out = true;
        else if (s[k] >= 0 && !seen.insert(s[k]).second) dup = true;
      }
      const int32_t st = pkv_validate_slots(s.data(), n, ns);
      CHECK((st == PKV_OK) == !(dup || out));
    }
    // books after every event
    CHECK(pkv_alloc_check_consistent(a) == PKV_OK);
    std::vector<int32_t> rc(nb), model(nb, 0);
    CHECK(pkv_alloc_snapshot(a, nullptr, rc.data()) == PKV_OK);
    for (const auto& t : tables)
      for (int32_t b : t) model[b] += 1;
    CHECK(rc == model);
  }
  pkv_alloc_destroy(a);
}

// ---- step builder ----------------------------------------------------------------------
void fuzz_scheduler(Rng& rng, int events, long* counters) {
  const int bs = uni(rng, 1, 16);
  const int max_blocks = uni(rng, 2, 12);
  pkv_sched* s = nullptr;
  CHECK(pkv_sched_create(uni(rng, 4, 48), bs, uni(rng, 1, 12), uni(rng, 1, 24), uni(rng, 1, 8),
                         max_blocks, unif(rng) < 0.7 ? 1 : 0, &s) == PKV_OK);
  int next_id = 0;
  std::vector<int> ids;
  for (int e = 0; e < events; ++e) {
    const double ev = unif(rng);
    if (ev < 0.3) {
      const int plen = uni(rng, 1, max_blocks * bs);
      const int grp = unif(rng) < 0.6 ? uni(rng, 0, 2) : -1;
      if (pkv_sched_add(s, next_id, plen, grp) == PKV_OK) ids.push_back(next_id++);
    } else if (ev < 0.36 && !ids.empty()) {
      const int sid = ids[uni(rng, 0, static_cast<int>(ids.size()) - 1)];
      int32_t st = 0, nt = 0;
      CHECK(pkv_sched_seq_info(s, sid, &st, &nt, nullptr, nullptr) == PKV_OK);
      (void)pkv_sched_trim(s, sid, uni(rng, 0, nt + 1));
    } else if (ev < 0.42 && !ids.empty()) {
      const int sid = ids[uni(rng, 0, static_cast<int>(ids.size()) - 1)];
      if (pkv_sched_fork(s, sid, next_id) == PKV_OK) ids.push_back(next_id++);
    }
    CHECK(pkv_sched_check(s) == PKV_OK);
    int32_t B = 0, T = 0, nc = 0, np = 0;
    CHECK(pkv_sched_step(s, &B, &T, &nc, &np) == PKV_OK);
    std::vector<int32_t> sid(B + 1), nn(B + 1), ctx(B + 1), cu(B + 1), bt((B + 1) * max_blocks),
        slots(T + 1), cp(2 * nc + 1), pre(np + 1);
    CHECK(pkv_sched_plan(s, sid.data(), nn.data(), ctx.data(), cu.data(), bt.data(), slots.data(),
                         cp.data(), pre.data()) == PKV_OK);
    counters[3] += T;
    counters[4] += np;
    counters[5] += nc;
    CHECK(cu[0] == 0 && cu[B] == T);
    for (int b = 0; b < B; ++b) CHECK(cu[b + 1] - cu[b] == nn[b] && nn[b] <= ctx[b]);
    CHECK(pkv_validate_slots(slots.data(), T, 1LL << 30) == PKV_OK);
    int32_t d0 = 0, d1 = 0, d2 = 0, d3 = 0;
    CHECK(pkv_sched_step(s, &d0, &d1, &d2, &d3) == PKV_ERR_INVALID);   // pending
    std::vector<int32_t> fin;
    for (int b = 0; b < B; ++b)
      if (unif(rng) < 0.15) fin.push_back(sid[b]);
    std::vector<int32_t> sampled(B + 1);
    int32_t ns = 0;
    CHECK(pkv_sched_complete(s, fin.data(), static_cast<int32_t>(fin.size()), sampled.data(), &ns) == PKV_OK);
    CHECK(pkv_sched_check(s) == PKV_OK);
  }
  pkv_sched_destroy(s);
}

// ---- work planner --------------------------------------------------------------------------
void fuzz_planner(Rng& rng, long* counters) {
  const int B = uni(rng, 0, 40);
  const int group = 1 << uni(rng, 0, 3);
  const int hkv = uni(rng, 1, 4);
  const int hq = group * hkv;
  const int head_dim = unif(rng) < 0.5 ? 64 : 128;
  const bool consistent = unif(rng) < 0.4;
  const int kv_split = 64 * uni(rng, 1, consistent ? 64 : 32);
  std::vector<int32_t> ctx(B), cu(B + 1, 0);
  for (int b = 0; b < B; ++b) {
    const double c = unif(rng);
    const int ql = c < 0.5 ? 1 : (c < 0.6 ? 0 : uni(rng, 2, 300));
    ctx[b] = ql + (unif(rng) < 0.2 ? 0 : uni(rng, 0, 6000));
    cu[b + 1] = cu[b] + ql;
  }
  const int T = cu[B];
  CHECK(pkv::check_step(ctx.data(), cu.data(), B, T, -1) == PKV_OK);
  pkv::StepShape s;
  s.ctx = ctx.data();
  s.cu = cu.data();
  s.B = B;
  s.kv_split = kv_split;
  s.prefill_on_mfma = unif(rng) < 0.9;
  s.all_mfma = consistent;
  s.prefill_rows_per_item = 128 / group;
  s.tile_split = consistent ? kv_split : 0;
  // host tables for shared reads: some rows copy a prefix of an earlier row's blocks
  const int bs = 1 << uni(rng, 0, 6);
  int max_blocks = 1;
  for (int b = 0; b < B; ++b) max_blocks = std::max(max_blocks, (ctx[b] + bs - 1) / bs);
  std::vector<int32_t> tables(static_cast<size_t>(std::max(B, 1)) * max_blocks, -1);
  int next_block = 0;
  for (int b = 0; b < B; ++b) {
    const int nb = (ctx[b] + bs - 1) / bs;
    const int src = b > 0 && unif(rng) < 0.6 ? uni(rng, 0, b - 1) : -1;
    const int nsrc = src >= 0 ? (ctx[src] + bs - 1) / bs : 0;
    const int shared = src >= 0 ? uni(rng, 0, std::min(nb, nsrc)) : 0;
    for (int j = 0; j < nb; ++j)
      tables[static_cast<size_t>(b) * max_blocks + j] =
          j < shared ? tables[static_cast<size_t>(src) * max_blocks + j] : next_block++;
  }
  const int gr = std::vector<int>{0, 2, 4}[uni(rng, 0, 2)];
  if (gr > 0) {
    s.bt_host = tables.data();
    s.bt_stride = max_blocks;
    s.block_size = bs;
    s.group_rows = gr;
  }
  const int n_write = uni(rng, 0, 50);
  const pkv::WorkspaceLayout L = pkv::layout_for(s, hq, head_dim, n_write);
  // the lists exactly as large as the layout says: ASan reports a write past them
  std::vector<char> host(L.list_bytes);
  pkv::build_lists(s, L, host.data());
  CHECK(L.decode_off + L.n_decode * sizeof(pkv::DecodeItem) <= L.group_off);
  CHECK(L.group_off + L.n_group * sizeof(pkv::DecodeGroupItem) <= L.merge_off);
  CHECK(gr > 0 || L.n_group == 0);
  CHECK(L.merge_off + L.n_merge * sizeof(pkv::MergeItem) <= L.prefill_off);
  CHECK(L.prefill_off + L.n_prefill * sizeof(pkv::PrefillItem) <= L.slots_off);
  CHECK(L.slots_off + n_write * sizeof(int32_t) <= L.list_bytes);
  CHECK(L.part_acc_off + static_cast<size_t>(L.n_part) * hq * head_dim * sizeof(float) <= L.total);
  const auto* dec = reinterpret_cast<const pkv::DecodeItem*>(host.data() + L.decode_off);
  const auto* mer = reinterpret_cast<const pkv::MergeItem*>(host.data() + L.merge_off);
  const auto* pre = reinterpret_cast<const pkv::PrefillItem*>(host.data() + L.prefill_off);
  counters[6] += L.n_decode + L.n_prefill;

  std::vector<int> part_use(static_cast<size_t>(L.n_part), 0);
  // decode rows: splits 0..ns-1 once each; a merge and ns partial slots iff ns > 1
  std::map<int, std::vector<int>> splits_of_row;
  std::map<int, int> part_of_row;           // a row's partial base, as its items carry it
  std::map<int, int> keys_of_row;
  for (int64_t i = 0; i < L.n_decode; ++i) {
    splits_of_row[dec[i].row].push_back(dec[i].split);
    part_of_row[dec[i].row] = dec[i].part;
    keys_of_row[dec[i].row] = dec[i].n_keys;
    CHECK(dec[i].seq >= 0 && dec[i].seq < B);
    if (dec[i].part >= 0) {
      const int64_t p = static_cast<int64_t>(dec[i].part) + dec[i].split;
      CHECK(p >= 0 && p < L.n_part);
      part_use[p] += 1;
    }
  }
  // group items: 2 .. group_rows rows, a whole split of each, the same blocks over it
  const auto* grpi = reinterpret_cast<const pkv::DecodeGroupItem*>(host.data() + L.group_off);
  std::map<int, int> seq_of_row;
  for (int b = 0; b < B; ++b)
    for (int r = cu[b]; r < cu[b + 1]; ++r) seq_of_row[r] = b;
  for (int64_t i = 0; i < L.n_group; ++i) {
    const pkv::DecodeGroupItem& gi = grpi[i];
    counters[7] += 1;
    CHECK(gi.n_rows >= 2 && gi.n_rows <= gr && gi.n_rows <= pkv::kGroupRows);
    const int64_t k1 = static_cast<int64_t>(gi.split + 1) * kv_split;
    CHECK(gi.n_keys >= k1);
    const int j0 = gi.split * kv_split / bs;
    const int j1 = static_cast<int>((k1 - 1) / bs);
    for (int r = 0; r < gi.n_rows; ++r) {
      const int row = gi.row[r];
      CHECK(seq_of_row.count(row) == 1 && seq_of_row[row] == gi.seq[r]);
      const int b = gi.seq[r];
      const int ql = cu[b + 1] - cu[b];
      const int n_keys = ctx[b] - ql + (row - cu[b]) + 1;
      CHECK(n_keys >= k1);
      for (int j = j0; j <= j1; ++j)
        CHECK(tables[static_cast<size_t>(b) * max_blocks + j] ==
              tables[static_cast<size_t>(gi.seq[0]) * max_blocks + j]);
      splits_of_row[row].push_back(gi.split);
      if (part_of_row.count(row)) CHECK(part_of_row[row] == gi.part[r]);
      part_of_row[row] = gi.part[r];
      keys_of_row[row] = n_keys;
      if (gi.part[r] >= 0) {
        const int64_t p = static_cast<int64_t>(gi.part[r]) + gi.split;
        CHECK(p >= 0 && p < L.n_part);
        part_use[p] += 1;
      }
    }
  }
  std::map<int, const pkv::MergeItem*> merge_of_row;
  for (int64_t i = 0; i < L.n_merge; ++i) {
    CHECK(merge_of_row.count(mer[i].row) == 0);
    merge_of_row[mer[i].row] = &mer[i];
    CHECK(mer[i].part >= 0 && mer[i].part + mer[i].n_splits <= L.n_part && mer[i].n_splits >= 2);
  }
  int tile_rows = 0;
  for (int b = 0; b < B; ++b) {
    const int ql = cu[b + 1] - cu[b];
    if (ql == 0) continue;
    if (pkv::on_tiles(s, ql)) {
      tile_rows += ql;
      continue;
    }
    for (int i = 0; i < ql; ++i) {
      const int row = cu[b] + i;
      const int n_keys = ctx[b] - ql + i + 1;
      const int ns = (n_keys + kv_split - 1) / kv_split;
      auto sp = splits_of_row[row];
      std::sort(sp.begin(), sp.end());
      CHECK(static_cast<int>(sp.size()) == ns);
      for (int k = 0; k < ns; ++k) CHECK(sp[k] == k);
      CHECK(keys_of_row[row] == n_keys);
      CHECK((ns > 1) == (merge_of_row.count(row) == 1));
      if (ns > 1) CHECK(merge_of_row[row]->n_splits == ns && merge_of_row[row]->part == part_of_row[row]);
      else CHECK(part_of_row[row] < 0);
    }
  }
  // tile-path rows: each row once per split its last key reaches (once without splits)
  std::map<std::pair<int, int>, int> covered;   // (row, split) -> count
  for (int64_t i = 0; i < L.n_prefill; ++i) {
    const pkv::PrefillItem& p = pre[i];
    CHECK(p.seq >= 0 && p.seq < B && p.n_rows >= 1 && p.n_rows <= s.prefill_rows_per_item);
    const int ql = cu[p.seq + 1] - cu[p.seq];
    const int prior = ctx[p.seq] - ql;
    CHECK(p.row0 >= cu[p.seq] && p.row0 + p.n_rows <= cu[p.seq + 1]);
    CHECK(p.pos0 == prior + (p.row0 - cu[p.seq]));
    for (int r = 0; r < p.n_rows; ++r) {
      covered[{p.row0 + r, p.split}] += 1;
      if (p.part >= 0) {
        const int64_t slot = static_cast<int64_t>(p.part) + static_cast<int64_t>(r) * p.pstride + p.split;
        CHECK(slot >= 0 && slot < L.n_part);
        const int pos = p.pos0 + r;
        if (s.tile_split > 0 && pos >= p.split * s.tile_split) part_use[slot] += 1;
      }
    }
  }
  int covered_rows = 0;
  for (const auto& kv : covered) {
    CHECK(kv.second == 1);
    if (kv.first.second == 0) covered_rows += 1;
  }
  CHECK(covered_rows == tile_rows);
  for (int64_t p = 0; p < L.n_part; ++p) CHECK(part_use[p] <= 1);
  // longest first
  for (int64_t i = 1; i < L.n_decode; ++i) {
    auto keys = [&](const pkv::DecodeItem& x) {
      return std::min(x.n_keys - x.split * kv_split, kv_split);
    };
    CHECK(keys(dec[i - 1]) >= keys(dec[i]));
  }
}

}  // namespace

int main(int argc, char** argv) {
  const unsigned long seed = argc > 1 ? std::strtoul(argv[1], nullptr, 10) : 1;
  const int rounds = argc > 2 ? std::atoi(argv[2]) : 20;
  Rng rng(seed);
  long counters[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int r = 0; r < rounds && g_fail == 0; ++r) {
    fuzz_allocator(rng, 2000, counters);
    fuzz_scheduler(rng, 300, counters);
    for (int k = 0; k < 50 && g_fail == 0; ++k) fuzz_planner(rng, counters);
  }
  std::printf("host_fuzz seed=%lu rounds=%d exhaustions=%ld shared_admits=%ld refusals=%ld "
              "sched_rows=%ld preemptions=%ld copies=%ld planned_items=%ld group_items=%ld "
              "failures=%d\n",
              seed, rounds, counters[0], counters[1], counters[2], counters[3], counters[4],
              counters[5], counters[6], counters[7], g_fail);
  return g_fail == 0 ? 0 : 1;
}
