// Host-side launch planning for the prefill and MLA kernels.  Pure C++: no HIP
// call, so the plans can be built and inspected without a GPU.
#pragma once

#include <cstdint>
#include <vector>

namespace mpa {

// Geometry of one prefill workgroup: 4 waves, each owning 32 query rows of one
// head, sharing every K/V tile of KEYS_PER_TILE keys staged in LDS.
constexpr int kPrefillWaves = 4;
constexpr int kRowsPerWave = 32;
constexpr int kKeysPerTile = 64;
// Workgroups are spread round-robin over the XCDs by workgroup id.
constexpr int kNumXcd = 8;

struct PrefillItem {
  int32_t b;        // sequence, or -1 for an empty slot (exits at once)
  int32_t head0;    // first query head of the workgroup
  int32_t row0;     // first query row (within the sequence)
  int32_t n_tiles;  // key tiles the workgroup visits
};

struct PrefillPlan {
  int heads_per_item = 1;   // query heads sharing one workgroup (same KV head)
  int rows_per_item = 128;  // query rows per head in one workgroup
  std::vector<PrefillItem> items;  // launch order (grid = items.size())
  int64_t real_items = 0;          // items with b >= 0
};

// Plans the prefill launch.  For each sequence with seqLen > 0, each group of
// heads_per_item heads and each block of rows_per_item rows it emits one item
// whose key range ends at the last key any of its rows can see.  Items of one
// (sequence, KV head) go to one XCD (so its L2 serves their shared K/V);
// (sequence, KV head) groups are spread over XCDs greedily by work; inside an
// XCD groups run one after another and each group's items longest first.
// Slots left over by uneven XCD loads are filled with empty items.
PrefillPlan plan_prefill(const int32_t* seq_len, const int32_t* kv_len, int batch, bool causal,
                         int head_num, int kv_head_num);

struct MlaSplit {
  int32_t b;        // sequence, or -1 for an empty slot
  int32_t k0, k1;   // key range [k0, k1)
  int32_t part_row; // first row of this split's partial results in the workspace
};

struct MlaSeq {
  int32_t ctx;         // keys
  int32_t q_len;       // query tokens
  int32_t tok0;        // first token row
  int32_t n_splits;    // splits of this sequence
  int32_t split0;      // index (in split order) of its first split
  int32_t part_row0;   // partial-result row of its first split
  int32_t pad0, pad1;
};

struct MlaPlan {
  std::vector<MlaSplit> splits;  // padded to a multiple of kNumXcd
  std::vector<MlaSeq> seqs;
  std::vector<int32_t> seq_splits;  // for each sequence, its split indices (n_splits each, from split0 into this list)
  int rows_per_group = 64;          // query rows (token, head) per workgroup
  int row_groups = 1;               // workgroups per split along the rows
  int64_t part_rows = 0;            // rows of fp32 partial output in the workspace
  int64_t tokens = 0;
};

// Splits every sequence's keys into equal chunks (multiples of the kernel's key
// tile) whose size minimises a makespan estimate for `slots` workgroups running
// at once, each split costing its keys plus `split_overhead_keys`.  Split s of
// sequence b writes q_len[b] * head_num partial rows; its rows are processed by
// row groups of `rows_per_group`.
MlaPlan plan_mla(const int32_t* ctx, const int32_t* q_len, int batch, int head_num, int slots,
                 int key_tile, int rows_per_group, int split_overhead_keys);

}  // namespace mpa
