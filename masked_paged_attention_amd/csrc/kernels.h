// Kernel parameter blocks and host launchers shared by api.cpp and the .hip
// kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mpa {

struct PrefillParams {
  const void* q;               // [nTokens, headNum, D]
  const void* k;               // [numBlocks, blockSize, kvHeadNum, D]
  const void* v;
  void* out;                   // [nTokens, headNum, D]
  float* lse;                  // [nTokens, headNum] or null
  const int32_t* block_tables; // [batch, maxBlocks]
  const float* slopes;         // [headNum] or null
  const int4* items;           // launch plan: {b, head0, row0, n_tiles}
  const int4* seqs;            // per sequence: {seqLen, kvSeqLen, qStart lo, qStart hi}
  int head_num;
  int kv_head_num;
  int block_size;
  int bs_shift;                // log2(blockSize) when a power of two, else -1
  int max_blocks;
  int heads_per_item;
  int chunk;                   // chunk size of the chunked local mask (mask 10), else 0
  const void* mask;            // compressed mask tile (mask_type | kMaskTileFlag), else null
  int mask_stride;             // elements per tile row (128 or 256)
  float* mask_f32;             // workspace copy of the tile in fp32 where
                               // prefill_tile_f32_bytes() > 0, filled by each execution
  float scale2;                // qkScale * log2(e)
};

// Kernel mask type of a compressed mask tile read from memory: maskType (3, 4, 5, 9)
// | kMaskTileFlag; the tile grid is kMaskTile absolute positions.
constexpr int kMaskTileFlag = 16;
constexpr int kMaskTile = 128;

// Workspace bytes of the fp32 copy of an ALiBi tile (right, sqrt, left) that the
// direct-load kernel (headSize 128, power-of-two blockSize >= 16) reads in place
// of the caller's fp16/bf16 tile: one conversion per entry and execution instead
// of one per score.  0 where the kernel reads the tile as given.
inline size_t prefill_tile_f32_bytes(int head_size, int bs_shift, int mask_type, int mask_stride) {
  const bool dma = head_size == 128 && bs_shift >= 4;
  const bool alibi_tile = mask_type == (kMaskTileFlag | 3) || mask_type == (kMaskTileFlag | 4) || mask_type == (kMaskTileFlag | 5);
  return dma && alibi_tile ? (size_t)mask_stride * (size_t)mask_stride * sizeof(float) : 0;
}

// Events a call records on its own kernels' dispatch packets (hipExtLaunchKernel):
// start when its first kernel starts, stop when its last kernel ends; null = none.
struct LaunchEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

// dtype: 0 fp16, 1 bf16; head_size 64/128; mask_type 0/3/4/5/9, 10 (chunked local
// causal), or 3/4/5/9 | kMaskTileFlag (compressed tile in p.mask).
hipError_t launch_prefill(const PrefillParams& p, int dtype, int head_size, int mask_type,
                          int grid, hipStream_t stream, const LaunchEvents& ev = {});

struct MlaParams {
  const void* q_nope;          // [T, H, 512]
  const void* q_rope;          // [T, H, 64]
  const void* ckv;             // [NB, BS, 1, ckv_stride] (512 or 576 wide)
  const void* krope;           // [NB, BS, 1, 64], or null when the rope part sits in ckv
  const int32_t* block_tables; // [batch, maxBlocks]
  const int4* segs;            // {b, k0, k1, part (-1: whole sequence)}
  const int32_t* piece_seg;    // piece p: segments [piece_seg[p], piece_seg[p + 1])
  const int4* seqs;            // per sequence: {ctx, q_len, tok0, n_parts}
  const int4* seqs2;           // per sequence: {part_row0, rows (q_len * H), 0, 0}
  void* part_o;                // [part_rows, 512] fp32 partial outputs in the workspace
  float* part_lse;             // [part_rows] fp32 log2-domain LSE in the workspace
  void* out;                   // [T, H, 512]
  float* lse;                  // [T, H] or null
  int head_num;
  int block_size;
  int bs_shift;                // log2(blockSize) when a power of two, else -1
  int max_blocks;
  int ckv_stride;              // elements per cache row of ckv (512 or 576)
  int spec_mask;               // 1: token t sees keys <= ctx - q_len + t
  int grid;                    // split-kernel workgroups
  int row_groups;              // workgroups per piece
  int pieces_per_xcd;
  int batch;
  int max_rows;                // largest q_len * H (combine grid)
  int any_parts;               // some sequence has partial results to merge
  int whole;                   // whole-sequence plan: workgroup i = piece i / row_groups, row group i % row_groups
  float scale2;                // qkScale * log2(e)
  int quant;                   // 1: int8 qNope / ctKV with per-head descales
  const float* qk_descale;     // [H] (quant only)
  const float* pv_descale;     // [H] (quant only)
};

hipError_t launch_mla(const MlaParams& p, int dtype, hipStream_t stream, const LaunchEvents& ev = {});

struct LseMergeParams {
  const void* o_parts;         // [n_parts, rows, head_dim] partial outputs
  const float* lse_parts;      // [n_parts, rows] natural-log LSE of each part
  void* out;                   // [rows, head_dim]
  float* lse_out;              // [rows] or null
  long long rows;
  int n_parts;
  int head_dim;                // multiple of 8
};

hipError_t launch_lse_merge(const LseMergeParams& p, int dtype, hipStream_t stream);

// Bytes of the library-owned device buffer behind mpaMLAStaticScratch (per GPU).
constexpr size_t kStaticScratchBytes = size_t(128) << 20;

// Device address (on the current device) and size of that buffer; looked up
// once per device.
hipError_t static_scratch(void** ptr, size_t* bytes);

}  // namespace mpa
