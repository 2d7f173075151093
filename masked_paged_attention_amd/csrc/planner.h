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
  int32_t n_tiles;  // key tiles up to the last one the workgroup visits
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
// chunk > 0: chunked local causal mask, an item's work starts at the tile of its
// first row's chunk.
PrefillPlan plan_prefill(const int32_t* seq_len, const int32_t* kv_len, int batch, bool causal,
                         int head_num, int kv_head_num, int chunk = 0);

// MLA decode geometry: one workgroup (8 waves) covers 128 query rows -- the
// (token, head) pairs of a sequence, token-major -- and walks key tiles of 32.
constexpr int kMlaKeyTile = 32;
constexpr int kMlaRowsPerGroup = 128;

struct MlaSegment {
  int32_t b;        // sequence
  int32_t k0, k1;   // key range [k0, k1); k0 is a multiple of the key tile
  int32_t part;     // index among the sequence's segments, or -1 when the segment
                    // covers every key of the sequence (final output written directly)
};

struct MlaSeq {
  int32_t ctx;         // keys
  int32_t q_len;       // query tokens
  int32_t tok0;        // first token row
  int32_t n_parts;     // segments of this sequence when it has more than one, else 0
  int32_t part_row0;   // first partial-result row of its segments
  int32_t rows;        // q_len * head_num
  int32_t pad0, pad1;
};

struct MlaPlan {
  // Pieces: contiguous runs of the key tiles of all sequences (sequence after
  // sequence), of near-equal length; piece p holds segments
  // [piece_seg[p], piece_seg[p + 1]) of `segs`.
  std::vector<MlaSegment> segs;
  std::vector<int32_t> piece_seg;
  std::vector<MlaSeq> seqs;
  int row_groups = 1;          // workgroups per piece (row groups of the largest sequence)
  int pieces_per_xcd = 1;      // pieces handled by the workgroups of one XCD
  int grid = 8;                // workgroups: 8 * pieces_per_xcd * row_groups
  int64_t part_rows = 0;       // partial-result rows in the workspace
  int64_t tokens = 0;
  int max_rows = 0;            // largest q_len * head_num
  // Whole sequences: every piece is one sequence (one segment, no partial
  // results); workgroup i handles piece i / row_groups, row group i % row_groups,
  // so a sequence's row groups spread over all XCDs.
  bool whole = false;
};

// Plans the split-KV MLA launch for `slots` workgroups resident at once (one per
// compute unit).  When the (sequence, row group) pairs are many -- a prefill of
// long prompts at 128 heads -- and a longest-first schedule of them on the slots
// ends within 10% of a perfect balance, the plan takes whole sequences instead
// (MlaPlan::whole: no key split, no partial results, sequences longest first).
// Otherwise:  The key tiles of all sequences are laid end to end and cut
// into 8 * pieces_per_xcd pieces of near-equal tile counts; every piece is
// processed by row_groups workgroups (one per 128-row group) that sit on one XCD,
// and consecutive pieces go to the same XCD, so the segments of one sequence
// mostly share an L2.  Workgroup i runs on XCD i % 8 and handles piece
// (i % 8) * pieces_per_xcd + (i / 8) / row_groups, row group (i / 8) % row_groups.
MlaPlan plan_mla(const int32_t* ctx, const int32_t* q_len, int batch, int head_num, int slots);

}  // namespace mpa
