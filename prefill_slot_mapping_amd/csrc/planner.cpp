// Host work planner (declarations and the rules it follows in planner.h).
#include "planner.h"

#include <algorithm>
#include <climits>
#include <map>
#include <set>
#include <string>
#include <vector>

#include "common.h"

namespace pkv {

namespace {
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

bool SharedSplits::contains(int32_t row, int32_t split) const {
  return std::binary_search(taken.begin(), taken.end(), std::make_pair(row, split));
}

SharedSplits find_shared_splits(const StepShape& s) {
  SharedSplits out;
  if (s.bt_host == nullptr || s.group_rows < 2 || s.block_size <= 0) return out;
  // one record per whole split of a decode row, keyed by a hash of the split index and the
  // block ids covering it (no allocation per split); equal keys are compared id by id below
  struct Rec {
    uint64_t h;
    int32_t split, row, seq, n_keys, part;
    int64_t j0, j1;
  };
  std::vector<Rec> recs;
  int64_t part = 0;
  for (int32_t b = 0; b < s.B; ++b) {
    const int32_t ql = s.cu[b + 1] - s.cu[b];
    if (ql == 0) continue;
    if (on_tiles(s, ql)) {
      if (s.tile_split > 0) {
        const int64_t ns_max = ceil_div(s.ctx[b], s.tile_split);
        if (ns_max > 1) part += static_cast<int64_t>(ql) * ns_max;
      }
      continue;
    }
    const int32_t* tb = s.bt_host + static_cast<int64_t>(b) * s.bt_stride;
    for (int32_t i = 0; i < ql; ++i) {
      const int32_t row = s.cu[b] + i;
      const int32_t n_keys = s.ctx[b] - ql + i + 1;
      const int32_t ns = static_cast<int32_t>(ceil_div(n_keys, s.kv_split));
      const int32_t pbase = ns > 1 ? static_cast<int32_t>(part) : -1;
      if (ns > 1) part += ns;
      for (int32_t sp = 0; sp < ns; ++sp) {
        const int64_t k1 = static_cast<int64_t>(sp + 1) * s.kv_split;   // the split's end
        if (k1 > n_keys) continue;                                       // not a whole split
        const int64_t j0 = static_cast<int64_t>(sp) * s.kv_split / s.block_size;
        const int64_t j1 = (k1 - 1) / s.block_size;
        uint64_t h = 1469598103934665603ull ^ static_cast<uint64_t>(sp);
        for (int64_t j = j0; j <= j1; ++j) {
          h ^= static_cast<uint32_t>(tb[j]);
          h *= 1099511628211ull;
        }
        recs.push_back(Rec{h, sp, row, b, n_keys, pbase, j0, j1});
      }
    }
  }
  // equal keys together, in step order within a key
  std::stable_sort(recs.begin(), recs.end(), [](const Rec& x, const Rec& y) {
    return x.h != y.h ? x.h < y.h : x.split < y.split;
  });
  const auto same_blocks = [&](const Rec& x, const Rec& y) {
    if (x.split != y.split) return false;
    const int32_t* tx = s.bt_host + static_cast<int64_t>(x.seq) * s.bt_stride;
    const int32_t* ty = s.bt_host + static_cast<int64_t>(y.seq) * s.bt_stride;
    return std::equal(tx + x.j0, tx + x.j1 + 1, ty + y.j0);
  };
  std::vector<std::vector<DecodeGroupItem>> runs;   // the group items of each shared split
  for (size_t i0 = 0; i0 < recs.size();) {
    size_t i1 = i0 + 1;
    while (i1 < recs.size() && recs[i1].h == recs[i0].h && recs[i1].split == recs[i0].split) ++i1;
    // members that name exactly the first one's blocks (a hash collision leaves the others
    // as per-row items)
    std::vector<size_t> mem;
    for (size_t k = i0; k < i1; ++k)
      if (k == i0 || same_blocks(recs[i0], recs[k])) mem.push_back(k);
    for (size_t m0 = 0; m0 < mem.size(); m0 += s.group_rows) {
      const size_t n = std::min(mem.size() - m0, static_cast<size_t>(s.group_rows));
      if (n < 2) break;
      DecodeGroupItem gi{};
      gi.split = recs[mem[m0]].split;
      gi.n_rows = static_cast<int32_t>(n);
      gi.n_keys = INT32_MAX;
      for (int r = 0; r < kGroupRows; ++r) {
        gi.row[r] = gi.seq[r] = 0;
        gi.part[r] = -1;
      }
      for (size_t r = 0; r < n; ++r) {
        const Rec& m = recs[mem[m0 + r]];
        gi.row[r] = m.row;
        gi.seq[r] = m.seq;
        gi.part[r] = m.part;
        gi.n_keys = std::min(gi.n_keys, m.n_keys);
        out.taken.push_back({m.row, gi.split});
      }
      if (m0 == 0) runs.emplace_back();
      runs.back().push_back(gi);
    }
    i0 = i1;
  }
  // The launch deals consecutive workgroups (item i, kv head g at index i hkv + g) to the 8
  // XCDs in turn, so items d = 8 / gcd(hkv, 8) apart run on one XCD at about the same time:
  // the items of one shared split are listed d apart (runs taken d at a time, round robin),
  // so that they read the split through one L2. Measured on the prefix-shared step (4 kv
  // heads, 2 items per prompt split): decode pass 121.6 -> 116.2 us. Item order changes no
  // row's bits.
  int d = 8;
  for (int h = s.hkv; h % 2 == 0 && d > 1; h /= 2) d /= 2;
  for (size_t r0 = 0; r0 < runs.size(); r0 += d) {
    const size_t r1 = std::min(runs.size(), r0 + d);
    size_t len = 0;
    for (size_t r = r0; r < r1; ++r) len = std::max(len, runs[r].size());
    for (size_t j = 0; j < len; ++j)
      for (size_t r = r0; r < r1; ++r)
        if (j < runs[r].size()) out.groups.push_back(runs[r][j]);
  }
  std::sort(out.taken.begin(), out.taken.end());
  return out;
}

bool on_tiles(const StepShape& s, int32_t ql) { return s.all_mfma || (ql > 1 && s.prefill_on_mfma); }


WorkspaceLayout layout_for(const StepShape& s, int32_t hq, int32_t head_dim,
                           int32_t n_write_rows) {
  WorkspaceLayout L;
  for (int32_t b = 0; b < s.B; ++b) {
    const int32_t ql = s.cu[b + 1] - s.cu[b];
    if (ql == 0) continue;
    if (on_tiles(s, ql)) {
      const int32_t prior = s.ctx[b] - ql;
      if (s.tile_split == 0) {
        L.n_prefill += ceil_div(ql, s.prefill_rows_per_item);
        continue;
      }
      // an item per row chunk and split reached by its last row; split partials for every row
      // of a segment whose context reaches past split 0, and a merge per such row
      for (int32_t r0 = 0; r0 < ql; r0 += s.prefill_rows_per_item) {
        const int32_t last = prior + std::min(r0 + s.prefill_rows_per_item, ql) - 1;
        L.n_prefill += last / s.tile_split + 1;
      }
      const int64_t ns_max = ceil_div(s.ctx[b], s.tile_split);
      if (ns_max > 1) {
        L.n_part += static_cast<int64_t>(ql) * ns_max;
        L.n_merge += prior + ql - std::max(prior, s.tile_split);
      }
      continue;
    }
    for (int32_t i = 0; i < ql; ++i) {
      const int64_t n_keys = static_cast<int64_t>(s.ctx[b]) - ql + i + 1;
      const int64_t ns = ceil_div(n_keys, s.kv_split);
      L.n_decode += ns;
      if (ns > 1) {
        L.n_merge += 1;
        L.n_part += ns;
      }
    }
  }
  if (s.bt_host != nullptr && s.group_rows > 1) {
    SharedSplits local;
    const SharedSplits& sh = s.shared != nullptr ? *s.shared : (local = find_shared_splits(s));
    L.n_group = static_cast<int64_t>(sh.groups.size());
    L.n_decode -= static_cast<int64_t>(sh.taken.size());
  }
  size_t off = 0;
  L.decode_off = off;
  off = align_up(off + L.n_decode * sizeof(DecodeItem));
  L.group_off = off;
  off = align_up(off + L.n_group * sizeof(DecodeGroupItem));
  L.merge_off = off;
  off = align_up(off + L.n_merge * sizeof(MergeItem));
  L.prefill_off = off;
  off = align_up(off + L.n_prefill * sizeof(PrefillItem));
  L.slots_off = off;
  off = align_up(off + static_cast<size_t>(n_write_rows) * sizeof(int32_t));
  L.list_bytes = off;
  L.part_m_off = off;
  off = align_up(off + L.n_part * hq * sizeof(float));
  L.part_l_off = off;
  off = align_up(off + L.n_part * hq * sizeof(float));
  L.part_acc_off = off;
  off = align_up(off + L.n_part * hq * head_dim * sizeof(float));
  L.total = off;
  return L;
}

void build_lists(const StepShape& s, const WorkspaceLayout& L, char* host) {
  SharedSplits local;
  const SharedSplits& sh = L.n_group == 0 ? local
                           : s.shared != nullptr ? *s.shared : (local = find_shared_splits(s));
  std::copy(sh.groups.begin(), sh.groups.end(),
            reinterpret_cast<DecodeGroupItem*>(host + L.group_off));
  auto* dec = reinterpret_cast<DecodeItem*>(host + L.decode_off);
  auto* mer = reinterpret_cast<MergeItem*>(host + L.merge_off);
  auto* pre = reinterpret_cast<PrefillItem*>(host + L.prefill_off);
  int64_t nd = 0, nm = 0, np = 0, part = 0;
  for (int32_t b = 0; b < s.B; ++b) {
    const int32_t ql = s.cu[b + 1] - s.cu[b];
    if (ql == 0) continue;
    if (on_tiles(s, ql)) {
      const int32_t prior = s.ctx[b] - ql;
      const int32_t S = s.tile_split;
      const int32_t ns_max = S > 0 ? static_cast<int32_t>(ceil_div(s.ctx[b], S)) : 1;
      const int32_t pbase = ns_max > 1 ? static_cast<int32_t>(part) : -1;
      if (ns_max > 1) {
        part += static_cast<int64_t>(ql) * ns_max;
        for (int32_t i = std::max(0, S - prior); i < ql; ++i)   // rows at positions >= S
          mer[nm++] = MergeItem{s.cu[b] + i, (prior + i) / S + 1, pbase + i * ns_max, 0};
      }
      for (int32_t r0 = 0; r0 < ql; r0 += s.prefill_rows_per_item) {
        const int32_t n = std::min(s.prefill_rows_per_item, ql - r0);
        const int32_t n_splits = S > 0 ? (prior + r0 + n - 1) / S + 1 : 1;
        for (int32_t sp = 0; sp < n_splits; ++sp) {
          PrefillItem& p = pre[np++];
          p.seq = b;
          p.row0 = s.cu[b] + r0;
          p.n_rows = n;
          p.pos0 = prior + r0;
          p.split = sp;
          p.part = pbase < 0 ? -1 : pbase + r0 * ns_max;
          p.pstride = ns_max;
          p.pad = 0;
        }
      }
      continue;
    }
    for (int32_t i = 0; i < ql; ++i) {
      const int32_t row = s.cu[b] + i;
      const int32_t n_keys = s.ctx[b] - ql + i + 1;
      const int32_t ns = static_cast<int32_t>(ceil_div(n_keys, s.kv_split));
      int32_t pbase = -1;
      if (ns > 1) {
        pbase = static_cast<int32_t>(part);
        mer[nm++] = MergeItem{row, ns, pbase, 0};
        part += ns;
      }
      for (int32_t sp = 0; sp < ns; ++sp)
        if (sh.taken.empty() || !sh.contains(row, sp))
          dec[nd++] = DecodeItem{row, b, n_keys, sp, pbase, 0, 0, 0};
    }
  }
  // longest work first: short tail items then fill the gaps at the end of each launch (item
  // order never affects any row's bits). A prefill item's work grows with its last key.
  const auto pre_keys = [&](const PrefillItem& x) -> int64_t {
    const int64_t end = x.pos0 + x.n_rows;
    if (s.tile_split == 0) return end;
    const int64_t k0 = static_cast<int64_t>(x.split) * s.tile_split;
    return std::min<int64_t>(end, k0 + s.tile_split) - k0;
  };
  std::stable_sort(pre, pre + np, [&](const PrefillItem& x, const PrefillItem& y) {
    return pre_keys(x) > pre_keys(y);
  });
  std::stable_sort(dec, dec + nd, [&](const DecodeItem& x, const DecodeItem& y) {
    const int64_t kx = std::min<int64_t>(x.n_keys - static_cast<int64_t>(x.split) * s.kv_split, s.kv_split);
    const int64_t ky = std::min<int64_t>(y.n_keys - static_cast<int64_t>(y.split) * s.kv_split, s.kv_split);
    return kx > ky;
  });
}


int32_t check_step(const int32_t* ctx, const int32_t* cu, int32_t B, int32_t T,
                   int64_t max_keys) {
  if (B < 0 || T < 0) return fail(PKV_ERR_INVALID, "B and T must be >= 0");
  if (B > 0 && (ctx == nullptr || cu == nullptr))
    return fail(PKV_ERR_INVALID, "ctx_lens_host / cu_seqlens_q_host is NULL");
  if (B == 0) {
    if (T != 0) return fail(PKV_ERR_INVALID, "T must be 0 when B is 0");
    return PKV_OK;
  }
  if (cu[0] != 0) return fail(PKV_ERR_INVALID, "cu_seqlens_q[0] must be 0");
  for (int32_t b = 0; b < B; ++b) {
    const int32_t ql = cu[b + 1] - cu[b];
    if (cu[b + 1] < cu[b]) return fail(PKV_ERR_INVALID, "cu_seqlens_q must be non-decreasing");
    if (ctx[b] < 0) return fail(PKV_ERR_INVALID, "ctx_lens must be >= 0");
    if (ql > ctx[b])
      return fail(PKV_ERR_INVALID, "sequence " + std::to_string(b) + ": q_len " +
                                       std::to_string(ql) + " > ctx_len " + std::to_string(ctx[b]));
    if (max_keys >= 0 && ctx[b] > max_keys)
      return fail(PKV_ERR_INVALID, "sequence " + std::to_string(b) +
                                       ": ctx_len exceeds max_blocks * block_size");
  }
  if (cu[B] != T) return fail(PKV_ERR_INVALID, "cu_seqlens_q[B] must equal T");
  return PKV_OK;
}

}  // namespace pkv
