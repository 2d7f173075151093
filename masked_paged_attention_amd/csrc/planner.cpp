// Host-side launch planning (see planner.h).
#include "planner.h"

#include <algorithm>
#include <numeric>

namespace mpa {

namespace {

int gcd_int(int a, int b) {
  while (b) {
    int t = a % b;
    a = b;
    b = t;
  }
  return a;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

PrefillPlan plan_prefill(const int32_t* seq_len, const int32_t* kv_len, int batch, bool causal,
                         int head_num, int kv_head_num) {
  PrefillPlan plan;
  const int group = head_num / kv_head_num;
  // Heads of one KV group share a workgroup (and so every K/V tile it loads);
  // the rest of the four waves cover more rows of the same heads.
  plan.heads_per_item = gcd_int(group, kPrefillWaves);
  plan.rows_per_item = kRowsPerWave * (kPrefillWaves / plan.heads_per_item);

  struct Group {
    int64_t work = 0;
    std::vector<PrefillItem> items;
  };
  std::vector<Group> groups;
  for (int b = 0; b < batch; ++b) {
    const int L = seq_len[b];
    const int kv = kv_len[b];
    if (L <= 0) continue;
    const int prefix = kv - L;
    for (int kvh = 0; kvh < kv_head_num; ++kvh) {
      Group g;
      for (int h0 = kvh * group; h0 < (kvh + 1) * group; h0 += plan.heads_per_item) {
        for (int r0 = 0; r0 < L; r0 += plan.rows_per_item) {
          const int r_end = std::min(L, r0 + plan.rows_per_item);
          const int64_t keys = causal ? std::min<int64_t>(kv, (int64_t)prefix + r_end) : kv;
          const int n_tiles = (int)ceil_div(keys, kKeysPerTile);
          g.items.push_back({b, h0, r0, n_tiles});
          g.work += n_tiles;
        }
      }
      std::stable_sort(g.items.begin(), g.items.end(),
                       [](const PrefillItem& x, const PrefillItem& y) { return x.n_tiles > y.n_tiles; });
      groups.push_back(std::move(g));
    }
  }
  // Greedy: biggest groups first, each to the least loaded XCD.
  std::vector<int> order(groups.size());
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(),
                   [&](int x, int y) { return groups[x].work > groups[y].work; });
  std::vector<int64_t> load(kNumXcd, 0);
  std::vector<std::vector<PrefillItem>> lists(kNumXcd);
  for (int gi : order) {
    int x = (int)(std::min_element(load.begin(), load.end()) - load.begin());
    load[x] += groups[gi].work;
    lists[x].insert(lists[x].end(), groups[gi].items.begin(), groups[gi].items.end());
  }
  size_t longest = 0;
  for (auto& l : lists) longest = std::max(longest, l.size());
  plan.items.reserve(longest * kNumXcd);
  for (size_t k = 0; k < longest; ++k) {
    for (int x = 0; x < kNumXcd; ++x) {
      if (k < lists[x].size()) {
        plan.items.push_back(lists[x][k]);
        ++plan.real_items;
      } else {
        plan.items.push_back({-1, 0, 0, 0});
      }
    }
  }
  // Trailing empty slots launch nothing useful: drop them.
  while (!plan.items.empty() && plan.items.back().b < 0) plan.items.pop_back();
  return plan;
}

MlaPlan plan_mla(const int32_t* ctx, const int32_t* q_len, int batch, int head_num, int slots,
                 int key_tile, int rows_per_group, int split_overhead_keys) {
  MlaPlan plan;
  plan.rows_per_group = rows_per_group;
  int64_t total_keys = 0;
  int max_rows = 0;
  for (int b = 0; b < batch; ++b) {
    total_keys += ctx[b];
    max_rows = std::max(max_rows, q_len[b] * head_num);
  }
  plan.row_groups = (int)ceil_div(max_rows, plan.rows_per_group);
  // Chunk of keys per split (a multiple of the key tile).  Cost model, in keys:
  // the work of all splits spread over `slots` concurrent workgroups, plus the
  // longest split (the tail), where every split also pays a fixed overhead
  // (loading its queries, writing and re-reading its fp32 partial rows).
  const int64_t overhead = split_overhead_keys;
  int64_t max_ctx = 1;
  for (int b = 0; b < batch; ++b) max_ctx = std::max<int64_t>(max_ctx, ctx[b]);
  int64_t chunk = ceil_div(max_ctx, key_tile) * key_tile;
  double best = -1.0;
  for (int64_t c = key_tile; c <= ceil_div(max_ctx, key_tile) * key_tile; c += key_tile) {
    int64_t splits = 0, longest = 0;
    for (int b = 0; b < batch; ++b) {
      const int64_t n = std::max<int64_t>(1, ceil_div(ctx[b], c));
      splits += n;
      longest = std::max<int64_t>(longest, ceil_div(ceil_div(ctx[b], n), key_tile) * key_tile);
    }
    const double cost = (double)(total_keys + splits * overhead) * plan.row_groups / std::max(1, slots) +
                        (double)(longest + overhead);
    if (best < 0 || cost < best) {
      best = cost;
      chunk = c;
    }
  }

  plan.seqs.resize(batch);
  int64_t part_row = 0, tok = 0;
  for (int b = 0; b < batch; ++b) {
    MlaSeq s{};
    s.ctx = ctx[b];
    s.q_len = q_len[b];
    s.tok0 = (int32_t)tok;
    tok += q_len[b];
    // Spread the keys evenly over the splits instead of leaving a short tail.
    const int n = (int)std::max<int64_t>(1, ceil_div(ctx[b], chunk));
    int64_t per = ceil_div(ceil_div(ctx[b], n), key_tile) * key_tile;
    s.n_splits = 0;
    s.split0 = -1;
    s.part_row0 = (int32_t)part_row;
    for (int64_t k0 = 0; k0 < ctx[b]; k0 += per) {
      const int64_t k1 = std::min<int64_t>(ctx[b], k0 + per);
      plan.splits.push_back({b, (int32_t)k0, (int32_t)k1, (int32_t)part_row});
      part_row += (int64_t)q_len[b] * head_num;
      ++s.n_splits;
    }
    plan.seqs[b] = s;
  }
  plan.tokens = tok;
  plan.part_rows = part_row;
  // Longest splits first (all are near the chunk size; short ones go last).
  std::vector<MlaSplit> sorted = plan.splits;
  std::stable_sort(sorted.begin(), sorted.end(), [](const MlaSplit& x, const MlaSplit& y) {
    return (x.k1 - x.k0) > (y.k1 - y.k0);
  });
  plan.splits = sorted;
  // Per sequence, the list of its splits' partial rows lives in seq_splits.
  plan.seq_splits.clear();
  for (int b = 0; b < batch; ++b) {
    plan.seqs[b].split0 = (int32_t)plan.seq_splits.size();
    int cnt = 0;
    for (size_t i = 0; i < plan.splits.size(); ++i)
      if (plan.splits[i].b == b) {
        plan.seq_splits.push_back((int32_t)i);
        ++cnt;
      }
    plan.seqs[b].n_splits = cnt;
  }
  while (plan.splits.size() % kNumXcd) plan.splits.push_back({-1, 0, 0, 0});
  return plan;
}

}  // namespace mpa
