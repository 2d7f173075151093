// Host-side launch planning (see planner.h).
#include "planner.h"

#include <algorithm>
#include <functional>
#include <numeric>
#include <queue>

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

// Modelled finish time (in key tiles) of one XCD's prefill items started in list
// order on its workgroup slots (32 compute units x 2 resident workgroups), each
// item costing its key tiles plus 1.5 tiles of prologue and epilogue.
template <typename Work>
double list_makespan(const std::vector<PrefillItem>& items, Work work) {
  constexpr int kSlotsPerXcd = 64;
  std::priority_queue<double, std::vector<double>, std::greater<double>> free_at;
  for (int i = 0; i < kSlotsPerXcd; ++i) free_at.push(0.0);
  double end = 0.0;
  for (const auto& it : items) {
    const double t = free_at.top() + work(it) + 1.5;
    free_at.pop();
    free_at.push(t);
    end = std::max(end, t);
  }
  return end;
}

}  // namespace

PrefillPlan plan_prefill(const int32_t* seq_len, const int32_t* kv_len, int batch, bool causal,
                         int head_num, int kv_head_num, int chunk) {
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
  // Key tiles an item computes: from its chunk's first tile (chunked mask) to
  // its last visible tile.
  auto item_work = [&](const PrefillItem& it) -> int {
    if (chunk <= 0) return it.n_tiles;
    const int64_t prefix = (int64_t)kv_len[it.b] - seq_len[it.b];
    return it.n_tiles - (int)(((prefix + it.row0) / chunk) * chunk / kKeysPerTile);
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
          g.work += item_work(g.items.back());
        }
      }
      std::stable_sort(g.items.begin(), g.items.end(), [&](const PrefillItem& x, const PrefillItem& y) {
        return item_work(x) > item_work(y);
      });
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
  // Inside an XCD the items run group after group, so the workgroups running
  // together share their K/V through the XCD's L2.  When that order leaves a
  // long tail -- long items of a late group starting last -- the items run
  // longest first instead: chosen when list scheduling of the XCD's items on its
  // workgroup slots finishes more than 3% earlier that way.
  for (auto& l : lists) {
    std::vector<PrefillItem> lpt = l;
    std::stable_sort(lpt.begin(), lpt.end(), [&](const PrefillItem& x, const PrefillItem& y) {
      return item_work(x) > item_work(y);
    });
    if (list_makespan(lpt, item_work) < 0.97 * list_makespan(l, item_work)) l.swap(lpt);
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

MlaPlan plan_mla(const int32_t* ctx, const int32_t* q_len, int batch, int head_num, int slots) {
  MlaPlan plan;
  std::vector<int64_t> tile0(batch + 1, 0);  // first flattened tile of each sequence
  for (int b = 0; b < batch; ++b) {
    tile0[b + 1] = tile0[b] + ceil_div(ctx[b], kMlaKeyTile);
    plan.max_rows = std::max(plan.max_rows, q_len[b] * head_num);
  }
  plan.row_groups = (int)ceil_div(plan.max_rows, kMlaRowsPerGroup);

  plan.seqs.resize(batch);
  {
    int64_t tok = 0;
    for (int b = 0; b < batch; ++b) {
      MlaSeq& s = plan.seqs[b];
      s.ctx = ctx[b];
      s.q_len = q_len[b];
      s.tok0 = (int32_t)tok;
      s.rows = q_len[b] * head_num;
      tok += q_len[b];
    }
    plan.tokens = tok;
  }

  // Whole sequences, when a longest-first schedule of the (sequence, row group)
  // pairs (key tiles + 1.5 per workgroup) ends within 10% of a perfect balance.
  {
    std::vector<int> order(batch);
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return ctx[x] > ctx[y]; });
    std::priority_queue<double, std::vector<double>, std::greater<double>> free_at;
    for (int i = 0; i < std::max(1, slots); ++i) free_at.push(0.0);
    double end = 0.0, sum = 0.0;
    int64_t pairs = 0;
    for (int b : order) {
      const double w = (double)ceil_div(ctx[b], kMlaKeyTile) + 1.5;
      pairs += ceil_div(plan.seqs[b].rows, kMlaRowsPerGroup);
      for (int64_t r = 0; r < ceil_div(plan.seqs[b].rows, kMlaRowsPerGroup); ++r) {
        const double t = free_at.top() + w;
        free_at.pop();
        free_at.push(t);
        end = std::max(end, t);
        sum += w;
      }
    }
    // (the grid holds batch x row_groups workgroups, those past a sequence's
    // rows exiting at once: at most three in four of them may be such)
    const int64_t grid = (int64_t)batch * plan.row_groups;
    if (end <= 1.1 * sum / std::max(1, slots) && grid <= 4 * pairs && grid < ((int64_t)1 << 30)) {
      plan.whole = true;
      plan.pieces_per_xcd = 1;
      for (int b : order) {
        plan.piece_seg.push_back((int32_t)plan.segs.size());
        MlaSegment sg;
        sg.b = b;
        sg.k0 = 0;
        sg.k1 = ctx[b];
        sg.part = -1;
        plan.segs.push_back(sg);
      }
      plan.piece_seg.push_back((int32_t)plan.segs.size());
      plan.grid = (int)(batch * (int64_t)plan.row_groups);
      for (MlaSeq& s : plan.seqs) {
        s.n_parts = 0;
        s.part_row0 = 0;
      }
      plan.part_rows = 0;
      return plan;
    }
  }

  plan.pieces_per_xcd = std::max(1, slots / (kNumXcd * plan.row_groups));
  const int64_t total = tile0[batch];
  // Small problems: no piece shorter than kMinTiles tiles (the rest stay empty).
  constexpr int64_t kMinTiles = 4;
  const int64_t n_pieces = (int64_t)kNumXcd * plan.pieces_per_xcd;
  const int64_t used = std::max<int64_t>(1, std::min<int64_t>(n_pieces, ceil_div(total, kMinTiles)));
  plan.grid = (int)(n_pieces * plan.row_groups);

  // Piece p covers flattened tiles [p * total / used, (p + 1) * total / used).
  std::vector<int32_t> n_seg(batch, 0);
  plan.piece_seg.assign(n_pieces + 1, 0);
  int b = 0;
  for (int64_t p = 0; p < n_pieces; ++p) {
    plan.piece_seg[p] = (int32_t)plan.segs.size();
    if (p >= used) continue;
    const int64_t a = p * total / used, e = (p + 1) * total / used;
    while (b < batch && tile0[b + 1] <= a) ++b;
    for (int bb = b; bb < batch && tile0[bb] < e; ++bb) {
      const int64_t t0 = std::max(a, tile0[bb]) - tile0[bb];
      const int64_t t1 = std::min(e, tile0[bb + 1]) - tile0[bb];
      if (t1 <= t0) continue;
      MlaSegment sg;
      sg.b = bb;
      sg.k0 = (int32_t)(t0 * kMlaKeyTile);
      sg.k1 = (int32_t)std::min<int64_t>(ctx[bb], t1 * kMlaKeyTile);
      sg.part = n_seg[bb]++;
      plan.segs.push_back(sg);
    }
  }
  plan.piece_seg[n_pieces] = (int32_t)plan.segs.size();
  // Sequences covered by one segment write their output directly.
  int64_t part_row = 0;
  for (int bb = 0; bb < batch; ++bb) {
    MlaSeq& s = plan.seqs[bb];
    s.n_parts = n_seg[bb] > 1 ? n_seg[bb] : 0;
    s.part_row0 = (int32_t)part_row;
    part_row += (int64_t)s.n_parts * s.rows;
  }
  for (MlaSegment& sg : plan.segs)
    if (n_seg[sg.b] == 1) sg.part = -1;
  plan.part_rows = part_row;
  return plan;
}

}  // namespace mpa
