// Fused masked attention over a paged KV cache (prefill / prefix encoder) for
// gfx950.
//
// What it computes (Ascend ATB page "PrefixEncoder", parameter table; masks of
// the ATB page "压缩mask", sections 开启方式 and 约束说明; the formula
// softmax(QK^T * scale + M) V of the nalar.dev padding-mask article, section
// "Masking mengubah kelayakan relasi attention"): for each sequence b, query
// head h and new row i (absolute position a = kvSeqLen - seqLen + i)
//   s_j = qkScale * q.k_j + bias(a, j) over visible keys j,  o = softmax(s) V,
//   lse = ln sum_j exp(s_j).
// Visibility and bias are generated in registers from (maskType, slopes,
// seqLen, kvSeqLen), or read from an explicit compressed mask tile (ATB page
// "压缩mask", section 约束说明) by either kernel.
//
// Shape of one workgroup (256 threads = 4 waves of 64):
//   * each wave owns 32 query rows of one head; the heads of one KV group share
//     the workgroup when the group is larger than one head, so every K/V tile
//     staged in LDS serves all of them;
//   * keys stream in tiles of 64: K and V rows are gathered through blockTables
//     with 16-byte coalesced loads (one 256-byte row segment per 16 lanes),
//     double-buffered in LDS; the loads of tile t+1 are in flight while tile t
//     is computed;
//   * scores are formed transposed, S^T = K Q^T, with the 32x32x16 MFMA: K rows
//     come from LDS, Q^T stays in registers for the whole loop.  The fp32 S^T
//     accumulator of a lane holds 32 keys of one query row -- exactly the
//     B-operand layout of the next MFMA, O^T += V^T P^T, so P never leaves
//     registers; V^T comes from the row-major V tile through the LDS transpose
//     read;
//   * per tile a wave-uniform test decides whether a tile is fully visible for
//     all 32 rows (no predicate), partly visible (per-element predicate) or not
//     visible (skipped); the ALiBi bias is one or two FMAs per score; the row
//     max and sum need one cross-half permlane swap per row;
//   * softmax runs in the log2 domain (scale and slopes pre-multiplied by
//     log2 e) with fp32 running max / sum, scores formed directly relative to
//     a reference max that only moves when a row's max grows by more than 2^10
//     (so the output is rarely rescaled); P is rounded to the input type for
//     the PV MFMA.

#include <type_traits>

#include <hip/hip_ext.h>

#include "device.h"
#include "kernels.h"

namespace mpa {

namespace {

constexpr int kWaves = 4;
constexpr int kRowsPerWave = 32;
constexpr int kBN = 64;  // keys per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 10.0f;  // log2 units of growth tolerated before rescaling
constexpr int kSqrtFar = 384;  // sqrt ALiBi: distance from which a tile's bias is expanded

template <typename T, int D, int MASK>
__global__ void __launch_bounds__(256, 2) prefill_fwd_kernel(PrefillParams p) {
  using V8 = typename Vec<T>::x8;
  using V4 = typename Vec<T>::x4;
  constexpr int KSTR = D + 8;   // K tile row stride (elements): conflict-free 16-byte row reads
  constexpr int VSTR = D + 32;  // V tile row stride: conflict-free transpose reads
  constexpr int kType = MASK & 15;          // maskType (0, 3, 4, 5, 9) or 10 (chunked)
  constexpr bool kTile = (MASK & kMaskTileFlag) != 0;  // bias read from a compressed tile
  constexpr bool kCausal = kType != 0;
  constexpr bool kAlibiLinear = kType == 3 || kType == 5;
  constexpr bool kAlibiSqrt = kType == 4;
  constexpr bool kChunked = kType == 10;    // causal inside chunks of p.chunk keys
  constexpr int NC = D / 16;                // 16-wide contraction chunks of QK^T
  constexpr int NDT = D / 32;               // 32-row tiles of O^T
  constexpr int CPR = D / 8;                // 16-byte chunks per K/V row
  constexpr int CPT = kBN * CPR / 256;      // chunks per thread per tile

  __shared__ __attribute__((aligned(16))) T k_lds[2][kBN * KSTR];
  __shared__ __attribute__((aligned(16))) T v_lds[2][kBN * VSTR];

  const int4 item = p.items[blockIdx.x];
  const int b = item.x;
  if (b < 0) return;
  const int head0 = item.y;
  const int row0 = item.z;
  const int4 sq = p.seqs[b];
  const int L = sq.x;
  const int kv = sq.y;
  const long long qs = (long long)(unsigned)sq.z | ((long long)sq.w << 32);
  const int prefix = kv - L;

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int l = tid & 63;
  const int g = l >> 5;   // which half of the wave
  const int lq = l & 31;  // query column of this lane
  const int hpw = p.heads_per_item;
  const int head = head0 + (w % hpw);
  const int wrow0 = row0 + (w / hpw) * kRowsPerWave;
  const int rows_per_item = kRowsPerWave * kWaves / hpw;
  const int kvh = head0 / (p.head_num / p.kv_head_num);
  const long long q_row_stride = (long long)p.head_num * D;
  const long long kv_slot_stride = (long long)p.kv_head_num * D;

  // Keys the workgroup visits, keys this wave needs, and keys every row of the
  // wave sees (tiles below that need no predicate).
  // With a compressed tile the diagonal 128-block of a row is read whole (the
  // tile decides which of its keys are visible), so the keys run to the end of
  // the last row's block; every tile then takes the per-element predicate.
  auto keys_to = [&](int rows_end) {
    if constexpr (!kCausal) return kv;
    const int a_last = prefix + rows_end - 1;
    return kTile ? min(kv, (a_last / kMaskTile + 1) * kMaskTile) : min(kv, a_last + 1);
  };
  const int item_rows_end = min(L, row0 + rows_per_item);
  const int wg_keys = keys_to(item_rows_end);
  const int n_tiles = (wg_keys + kBN - 1) / kBN;
  const bool w_active = wrow0 < L;
  const int w_rows_end = min(L, wrow0 + kRowsPerWave);
  const int w_keys = keys_to(w_rows_end);
  // (norm tile: keys in 128-blocks before the first row's block have bias 0 for
  // every row; the ALiBi tiles are read for every key)
  const int w_full_keys = kTile ? (kType == 9 ? min(kv, (prefix + wrow0) / kMaskTile * kMaskTile) : 0)
                                : kCausal ? min(kv, prefix + wrow0 + 1) : kv;
  // Chunked mask: row a sees keys from lo(a) = chunk * floor(a / chunk) on; the
  // item starts at the tile of its first row's lo, a wave skips the tiles below
  // its first row's lo, and a tile below its last row's lo needs the predicate.
  auto chunk_lo = [&](int a) { return kChunked ? (a / p.chunk) * p.chunk : 0; };
  const int t_lo = chunk_lo(prefix + row0) / kBN;
  const int w_lo = chunk_lo(prefix + wrow0);
  const int w_lo_last = chunk_lo(prefix + max(wrow0, w_rows_end - 1));

  // Q^T operand: lane l holds query row wrow0 + lq, dims 16c + 8g .. +8.
  V8 qreg[NC];
  {
    const int qi = wrow0 + lq;
    const T* qrow = (const T*)p.q + (qs + qi) * q_row_stride + (long long)head * D + 8 * g;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (qi < L) {
        qreg[c] = *(const V8*)(qrow + 16 * c);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qreg[c][e] = (T)0.0f;
      }
    }
  }

  const T* kbase = (const T*)p.k + (long long)kvh * D;
  const T* vbase = (const T*)p.v + (long long)kvh * D;
  const int32_t* btab = p.block_tables + (long long)b * p.max_blocks;
  // A 64-key tile lies inside one cache block when the block size is a power of
  // two >= 64: its block id is then one wave-uniform (scalar) load, fetched two
  // tiles ahead.  Otherwise every row looks its block up, all lookups first.
  const bool one_block = p.bs_shift >= 6;
  uint4 kr[CPT], vr[CPT];

  auto load_tile = [&](int j0, int blk) {
    if (one_block) {
      const long long base = ((long long)blk * p.block_size + (j0 & (p.block_size - 1))) * kv_slot_stride;
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const int x = tid + 256 * i;
        const int row = x / CPR;
        const int c = x % CPR;
        if (j0 + row < kv) {
          const long long off = base + row * kv_slot_stride + 8 * c;
          kr[i] = *(const uint4*)(kbase + off);
          vr[i] = *(const uint4*)(vbase + off);
        } else {
          kr[i] = make_uint4(0, 0, 0, 0);
          vr[i] = make_uint4(0, 0, 0, 0);
        }
      }
    } else {
      int bid[CPT];
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const int j = j0 + (tid + 256 * i) / CPR;
        bid[i] = j < kv ? btab[j / p.block_size] : 0;
      }
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const int x = tid + 256 * i;
        const int row = x / CPR;
        const int c = x % CPR;
        const int j = j0 + row;
        if (j < kv) {
          const int slot = j - (j / p.block_size) * p.block_size;
          const long long off = ((long long)bid[i] * p.block_size + slot) * kv_slot_stride + 8 * c;
          kr[i] = *(const uint4*)(kbase + off);
          vr[i] = *(const uint4*)(vbase + off);
        } else {
          kr[i] = make_uint4(0, 0, 0, 0);
          vr[i] = make_uint4(0, 0, 0, 0);
        }
      }
    }
  };
  auto tile_block = [&](int t) -> int {
    return one_block ? btab[(t * kBN) >> p.bs_shift] : 0;
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int x = tid + 256 * i;
      const int row = x / CPR;
      const int c = x % CPR;
      *(uint4*)&k_lds[buf][row * KSTR + 8 * c] = kr[i];
      *(uint4*)&v_lds[buf][row * VSTR + 8 * c] = vr[i];
    }
  };

  f32x16 o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) o[dt] = f32x16{};
  float m_run = -INFINITY;  // running max (log2 domain) of this lane's query row
  float l_run = 0.0f;       // running sum of this lane's half of the keys
  const int a_lane = prefix + wrow0 + lq;  // absolute position of the query row
  float slope2 = 0.0f;
  if constexpr (kAlibiLinear || kAlibiSqrt) slope2 = p.slopes[head] * kLog2e;
  const float scale2 = p.scale2;

  int blk_next = t_lo + 1 < n_tiles ? tile_block(t_lo + 1) : 0;
  load_tile(t_lo * kBN, tile_block(t_lo));
  store_tile(0);
  __syncthreads();

  // Compressed tile (row-major, p.mask_stride elements per row) on a grid of
  // kMaskTile absolute positions: query block bq = a / 128, in-block row r; key
  // block bk, in-block column c; dk = bq - bk.  Keys of later blocks (dk < 0) are
  // hidden.  Norm tile [128,128]: a key dk >= 1 blocks behind gets 0, one in the
  // diagonal block tile[r][c].  ALiBi tiles [256,256]: the diagonal block reads
  // row r, a key dk >= 1 blocks behind row 128 + r; the right-aligned bias
  // (linear and sqrt) then moves by -128 per block beyond the first, the
  // left-aligned one adds the key block origin 128 bk, applied here relative to
  // the query block origin (-128 dk) with 128 bq slope moved into the LSE.  A -inf
  // entry hides its key.
  const int a_bq = a_lane / kMaskTile;
  const T* mrow_diag = nullptr;
  const T* mrow_back = nullptr;
  if constexpr (kTile) {
    const int r = a_lane - a_bq * kMaskTile;
    mrow_diag = (const T*)p.mask + (long long)r * p.mask_stride + 4 * g;
    mrow_back = kType == 9 ? mrow_diag : mrow_diag + (long long)kMaskTile * p.mask_stride;
  }

  for (int t = t_lo; t < n_tiles; ++t) {
    const int buf = (t - t_lo) & 1;
    const int j0 = t * kBN;
    // Tile entries of this lane's 32 keys: 8 runs of 4 (issued before the next
    // K/V tile so that waiting on them leaves those loads in flight).
    V4 mv[8];
    int dk = 0;
    if constexpr (kTile) {
      dk = a_bq - j0 / kMaskTile;
      if (j0 + kBN > w_full_keys) {  // tiles every row sees with bias 0 read nothing
        const T* src = (dk == 0 ? mrow_diag : mrow_back) + (j0 & (kMaskTile - 1));
#pragma unroll
        for (int u = 0; u < 8; ++u) mv[u] = *(const V4*)(src + 8 * u);
      }
    }
    if (t + 1 < n_tiles) {
      load_tile(j0 + kBN, blk_next);
      if (t + 2 < n_tiles) blk_next = tile_block(t + 2);
    }

    if (w_active && j0 < w_keys && j0 + kBN > w_lo) {
      // S^T = K Q^T for keys j0 .. j0+63 (two 32-key blocks).
      f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const V8 a = *(const V8*)&k_lds[buf][(32 * kb + lq) * KSTR + 16 * c + 8 * g];
          s[kb] = mfma32(a, qreg[c], s[kb]);
        }
      }
      // Element (kb, r) is key j0 + 4g + C with C = 32kb + 8(r/4) + r%4.  Scores
      // are formed relative to the running reference max m_ref of the row (log2
      // domain), so that the exponent needs no further subtraction.
      const int dbase = a_lane - j0 - 4 * g;  // a - key at C = 0
      const int klim = kv - j0 - 4 * g;       // key < kv  <=>  C < klim
      const int vlim = kCausal && !kTile ? min(klim, dbase + 1) : klim;
      const int llim = chunk_lo(a_lane) - j0 - 4 * g;  // chunked: key >= lo(a)  <=>  C >= llim
      const bool partial = j0 + kBN > w_full_keys || (kChunked && j0 < w_lo_last);
      const float m_ref = (m_run == -INFINITY) ? 0.0f : m_run;
      const float dbf = (float)dbase;
      const float nbm = -slope2 * dbf - m_ref;  // linear ALiBi: slope2 * (C - dbase) - m_ref
      // Scores of the tile; tiles every row sees entirely take the branch without
      // the per-element predicate (a real, wave-uniform branch).
      auto form_scores = [&](auto with_mask) __attribute__((always_inline)) -> float {
        float m = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int C = 32 * kb + 8 * (r >> 2) + (r & 3);
            float x;
            if constexpr (kTile && !decltype(with_mask)::value) {
              // a tile every row sees with bias 0 (norm tile only)
              x = __builtin_fmaf(s[kb][r], scale2, -m_ref);
            } else if constexpr (kTile) {
              const float mval = (float)mv[4 * kb + (r >> 2)][r & 3];
              bool hide = dk < 0 || mval == -INFINITY;
              float bias2;  // bias in log2 units
              if constexpr (kType == 9) {
                bias2 = dk > 0 ? 0.0f : mval * kLog2e;
                hide = dk < 0 || (dk == 0 && mval == -INFINITY);
              } else if constexpr (kType == 5) {
                bias2 = slope2 * (mval - (float)(kMaskTile * dk));
              } else {
                const float y = dk > 0 ? mval - (float)(kMaskTile * (dk - 1)) : mval;
                bias2 = kAlibiSqrt ? -slope2 * fast_sqrt(-y) : slope2 * y;
              }
              x = __builtin_fmaf(s[kb][r], scale2, bias2 - m_ref);
              x = hide ? -INFINITY : x;
            } else if constexpr (kAlibiLinear) {
              x = __builtin_fmaf(s[kb][r], scale2, __builtin_fmaf(slope2, (float)C, nbm));
            } else if constexpr (kAlibiSqrt) {
              x = __builtin_fmaf(-slope2, fast_sqrt(dbf - (float)C), __builtin_fmaf(s[kb][r], scale2, -m_ref));
            } else {
              x = __builtin_fmaf(s[kb][r], scale2, -m_ref);
            }
            if constexpr (decltype(with_mask)::value)
              x = (C < vlim && (!kChunked || C >= llim)) ? x : -INFINITY;
            s[kb][r] = x;
            m = fmaxf(m, x);
          }
        }
        return m;
      };
      float mx;
      if (partial) {
        mx = form_scores(std::true_type{});
      } else {
        mx = form_scores(std::false_type{});
      }
      mx = max_with_other_half(mx);  // tile max of the row, relative to m_ref
      // Move the reference only when a row's max grows by more than 2^10 (or on the
      // row's first visible key): P stays <= 2^10 and the final normalisation uses
      // the same reference, so the result is exact; the rescale of O is rare.
      const bool need = (m_run == -INFINITY) ? (mx > -INFINITY) : (mx > kRescaleSlack);
      if (__builtin_amdgcn_ballot_w64(need) != 0) {
        const float m_new = fmaxf(m_run, m_ref + mx);
        const float delta = (m_new == -INFINITY) ? 0.0f : m_new - m_ref;
        const float alpha = (m_new == -INFINITY) ? 1.0f : fast_exp2(m_run - m_new);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) s[kb] -= delta;
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[dt] *= alpha;
        m_run = m_new;
      }
      float psum = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = fast_exp2(s[kb][r]);
          s[kb][r] = e;
          psum += e;
        }
      }
      l_run += psum;

      // O^T += V^T P^T, 16 keys per MFMA.  P^T operand of key chunk kc: registers
      // 8(kc%2) .. +8 of S^T block kc/2, i.e. keys 16kc + {4g..4g+3, 8+4g..8+4g+3}.
      V8 pk[4];
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
#pragma unroll
        for (int e = 0; e < 8; ++e) pk[kc][e] = (T)s[kc >> 1][8 * (kc & 1) + e];
      }
      const int tr_row = 4 * g + ((l & 15) >> 2);
      const int tr_col = 16 * ((l >> 4) & 1) + 4 * (l & 3);
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const T* src = &v_lds[buf][(16 * kc + tr_row) * VSTR + 32 * dt + tr_col];
          const s16x4 lo = lds_read_tr16(src);
          const s16x4 hi = lds_read_tr16(src + 8 * VSTR);
          const s16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          o[dt] = mfma32(__builtin_bit_cast(V8, both), pk[kc], o[dt]);
        }
      }
    }

    if (t + 1 < n_tiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  if (!w_active) return;
  const float l_tot = sum_with_other_half(l_run);
  const int i = wrow0 + lq;
  if (i >= L) return;
  // A row whose tile hides every key gets O = 0 (and LSE = -inf).
  const float inv = kTile && l_tot == 0.0f ? 0.0f : 1.0f / l_tot;
  T* orow = (T*)p.out + (qs + i) * q_row_stride + (long long)head * D + 4 * g;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      V4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (T)(o[dt][4 * rg + e] * inv);
      *(V4*)(orow + 32 * dt + 8 * rg) = v;
    }
  }
  if (p.lse != nullptr && g == 0) {
    float lse = (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2;
    if constexpr (kType == 5) lse += p.slopes[head] * (float)(kTile ? a_bq * kMaskTile : a_lane);
    p.lse[(qs + i) * p.head_num + head] = lse;
  }
}

// headSize 128 with a power-of-two blockSize >= 16 (each wave's 16 rows of a
// 64-key tile inside one cache block): the same computation, with K and V
// tiles brought into LDS by direct global->LDS loads (no register staging).  LDS layout of a tile: 16
// blocks of 4 rows (1 KB, one load instruction each) plus 16 bytes of padding;
// inside a block the 16-byte chunks of row m are XOR-swizzled by 4m.  Both read
// patterns -- 32 rows at one 16-byte column (QK operand) and 4 rows x 64 bytes
// (V^T transpose read) -- then hit distinct bank groups, and each lane needs 4
// base addresses per pattern (the rest are immediate offsets).
//
// With an ALiBi mask the two key tiles nearest the diagonal come first (the
// last one, then the one before: between them they hold every wave's diagonal
// when the workgroup has 128 rows), then the rest in key order from the
// first.  The largest biases sit next to the diagonal, so the running max is
// set by the first tiles and rarely moves, and a tile that every row sees
// needs no max at all -- P = exp2(score - m_run) is formed at once, and a
// lane's partial row sum above 2^10 (the only way some P can exceed 2^10) sends
// the tile through the full path, which finds the tile max and moves the
// reference.  The result is the same either way: only the reference of the
// exponent differs.  After the diagonal tiles, the workgroups of one head
// that run side by side read the same key tiles at about the same time, so
// they share them in L2 (visiting every tile from the diagonal down, they
// would read each tile two steps apart, a reuse distance that fills the L2 of
// a die).  Other masks visit the tiles in key order and take the same fast
// path after their first tile (whose max sets the reference) on every tile
// that all rows see whole.
template <typename T, int MASK>
__global__ void __launch_bounds__(256, 2) prefill_dma_kernel(PrefillParams p,
                                                             const int32_t* __restrict__ block_tables) {
  using V8 = typename Vec<T>::x8;
  using V4 = typename Vec<T>::x4;
  constexpr int D = 128;
  constexpr int kType = MASK & 15;        // maskType (0, 3, 4, 5, 9) or 10 (chunked)
  constexpr bool kTile = (MASK & kMaskTileFlag) != 0;  // bias read from a compressed tile (p.mask)
  constexpr bool kCausal = kType != 0;
  constexpr bool kAlibiLinear = !kTile && (kType == 3 || kType == 5);  // generated ALiBi bias
  constexpr bool kAlibiSqrt = !kTile && kType == 4;
  constexpr bool kTileAlibi = kTile && (kType == 3 || kType == 4 || kType == 5);
  // ALiBi tiles come as the execution's fp32 copy of the caller's tile (p.mask
  // points at it); the norm tile in the input type
  constexpr bool kTileF32 = kTile && (kType == 3 || kType == 4 || kType == 5);
  using MT = std::conditional_t<kTileF32, float, T>;
  using MV4 = MT __attribute__((ext_vector_type(4)));
  constexpr bool kReverse = kType == 3 || kType == 4 || kType == 5;
  constexpr bool kChunked = kType == 10;  // causal inside chunks of p.chunk keys
  constexpr int NC = D / 16;              // 16-wide contraction chunks of QK^T
  constexpr int NDT = D / 32;             // 32-row tiles of O^T
  constexpr int kRowBytes = D * (int)sizeof(T);   // 256
  constexpr int kBlkBytes = 4 * kRowBytes + 16;   // 1040
  constexpr int kTileBytes = 16 * kBlkBytes;      // 64 rows
  constexpr int kBufBytes = 2 * kTileBytes;       // K tile, then V tile
  constexpr float kSumLimit = 1024.0f;            // 2^kRescaleSlack

  __shared__ __attribute__((aligned(1024))) char lds[2 * kBufBytes];

  const int4 item = p.items[blockIdx.x];
  const int b = item.x;
  if (b < 0) return;
  const int head0 = item.y;
  const int row0 = item.z;
  const int4 sq = p.seqs[b];
  const int L = sq.x;
  const int kv = sq.y;
  const long long qs = (long long)(unsigned)sq.z | ((long long)sq.w << 32);
  const int prefix = kv - L;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63;
  const int g = l >> 5;   // which half of the wave
  const int lq = l & 31;  // query column of this lane
  const int hpw = p.heads_per_item;
  const int head = head0 + (w % hpw);
  const int wrow0 = row0 + (w / hpw) * kRowsPerWave;
  const int rows_per_item = kRowsPerWave * kWaves / hpw;
  const int kvh = head0 / (p.head_num / p.kv_head_num);
  const long long q_row_stride = (long long)p.head_num * D;
  const unsigned kv_row_bytes = (unsigned)p.kv_head_num * (unsigned)kRowBytes;

  const int item_rows_end = min(L, row0 + rows_per_item);
  // Compressed tile: keys run to the end of the last row's 128-block (the tile
  // decides inside the diagonal block).
  auto keys_to = [&](int rows_end) {
    const int a_last = prefix + rows_end - 1;
    return kTile ? min(kv, (a_last / kMaskTile + 1) * kMaskTile) : kCausal ? min(kv, a_last + 1) : kv;
  };
  const int wg_keys = keys_to(item_rows_end);
  const int n_end = (wg_keys + kBN - 1) / kBN;
  // Chunked mask: row a sees keys from lo(a) = chunk * floor(a / chunk) on; the
  // item starts at the tile of its first row's lo.
  auto chunk_lo = [&](int a) { return kChunked ? (a / p.chunk) * p.chunk : 0; };
  const int t_lo = chunk_lo(prefix + row0) / kBN;
  const int n_tiles = n_end - t_lo;  // iterations
  const bool w_active = wrow0 < L;
  const int w_rows_end = min(L, wrow0 + kRowsPerWave);
  const int w_keys = keys_to(w_rows_end);
  const int w_tiles = w_active ? (w_keys + kBN - 1) / kBN : 0;  // tiles 0 .. w_tiles-1 matter here
  // (compressed tiles: keys in 128-blocks before the first row's block are
  // behind every row's diagonal block)
  const int w_full_keys = kTile ? min(kv, (prefix + wrow0) / kMaskTile * kMaskTile)
                                : kCausal ? min(kv, prefix + wrow0 + 1) : kv;
  const int w_t_lo = chunk_lo(prefix + wrow0) / kBN;                       // first tile the wave sees
  const int w_lo_last = chunk_lo(prefix + max(wrow0, w_rows_end - 1));   // below it: predicate

  // Q^T operand: lane l holds query row wrow0 + lq, dims 16c + 8g .. +8.
  V8 qreg[NC];
  {
    const int qi = wrow0 + lq;
    const T* qrow = (const T*)p.q + (qs + qi) * q_row_stride + (long long)head * D + 8 * g;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (qi < L) {
        qreg[c] = *(const V8*)(qrow + 16 * c);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qreg[c][e] = (T)0.0f;
      }
    }
  }

  // ---- tile loads: wave w issues the 4-row blocks 4w .. 4w+3 of K and of V ----
  // Lane l of a block load carries row 4i + l/16 (clamped to the last key),
  // physical chunk l % 16 = logical chunk (l % 16) ^ 4(l / 16).  Iteration u
  // handles tile tile_of(u).
  const int32_t* __restrict__ btab = block_tables + (long long)b * p.max_blocks;
  const int lrow = l >> 4;
  const unsigned lchunk16 = 16u * (unsigned)((l & 15) ^ (4 * lrow));
  const unsigned lds_base = (unsigned)(unsigned long)(const __attribute__((address_space(3))) void*)lds;
  auto tile_of = [&](int u) { return kReverse ? (u < 2 ? n_tiles - 1 - u : u - 2) : t_lo + u; };
  // The wave's 16 rows of a tile lie in one cache block (blockSize >= 16, a
  // power of two, and tiles start at multiples of 64): its loads take one
  // wave-uniform base, at the first row of its 16-row group -- clamped to the
  // group of the tile's last key when the wave's rows are all past it, so that
  // no block-table entry past the sequence's keys is read.
  auto wave_row0 = [&](int last) { return min(16 * w, last & ~15); };
  auto tile_last = [&](int u) { return min(kBN, kv - tile_of(u) * kBN) - 1; };
  auto block_of = [&](int u) -> int {
    return (u < n_tiles) ? btab[(tile_of(u) * kBN + wave_row0(tile_last(u))) >> p.bs_shift] : 0;
  };
  struct TileSrc {
    const char* k;  // the wave's first row (wave_row0) of the tile, K and V
    const char* v;
    int last;       // the tile's last key, counted from that row
    int d0;         // the wave's own first row, counted from that row
    bool full;      // a tile of kBN keys
  };
  auto tile_src = [&](int u, int blk) -> TileSrc {
    const int j0 = tile_of(u) * kBN;
    const int last = min(kBN, kv - j0) - 1;
    const int r0 = wave_row0(last);
    const long long row = (long long)blk * p.block_size + ((j0 + r0) & (p.block_size - 1));
    const long long off = (row * p.kv_head_num + kvh) * D;
    return {(const char*)((const T*)p.k + off), (const char*)((const T*)p.v + off), last - r0, 16 * w - r0,
            last == kBN - 1};
  };
  // Byte offsets of this lane's rows in the wave's 4 blocks of a full tile
  // (no clamp), computed once.
  unsigned off_full[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) off_full[i] = (unsigned)(4 * i + lrow) * kv_row_bytes + lchunk16;
  // Block 4w + i of tile `ts` (FULL: a tile of kBN keys, known at compile time:
  // the precomputed offsets; else rows clamped to the last key).
  auto issue_block = [&](int kind, int i, const TileSrc& ts, int buf, auto FULL) __attribute__((always_inline)) {
    unsigned off;
    if constexpr (decltype(FULL)::value) {
      off = off_full[i];
    } else {
      // (the row is rebuilt at each use rather than kept per block: registers)
      int rr = ts.d0 + lrow;
      asm volatile("" : "+v"(rr));
      off = (unsigned)min(rr + 4 * i, ts.last) * kv_row_bytes + lchunk16;
    }
    i += 4 * w;
    dma16s_m0_nomem(kind ? ts.v : ts.k, off,
                    lds_base + (unsigned)(buf * kBufBytes + kind * kTileBytes + i * kBlkBytes));
  };

  // ---- LDS read addresses (bytes, without the buffer offset) ----
  // QK operand of key row 32kb + lq, logical chunk q16 = 2c + g:
  //   (8kb + lq/4) * 1040 + m * 256 + 16 * (q16 ^ 4m), m = lq % 4
  //   = qa[(c / 2) ^ m] + 8320 kb + 32 (c % 2),  qa[x] = (lq/4) * 1040 + m * 256 + 64 x + 16 g.
  const int mq = lq & 3;
  unsigned qa[4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
    qa[x] = (unsigned)((lq >> 2) * kBlkBytes + mq * kRowBytes + 64 * (x ^ mq) + 16 * g);
  // V^T operand, keys 16kc + 4g + s/4 (s = l % 16), dims 32dt + 16h + 4(s % 4):
  //   (4kc + g) * 1040 + mv * 256 + 16 * ((4dt + 2h + (s%4)/2) ^ 4mv) + 8 (s % 2)
  //   = va[dt] + 4160 kc;  the keys + 8 are 2 blocks (2080 bytes) further.
  const int sl = l & 15;
  const int mv = sl >> 2;
  const int hh = (l >> 4) & 1;
  unsigned va[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
    va[dt] = (unsigned)(g * kBlkBytes + kTileBytes + mv * kRowBytes + 64 * (dt ^ mv) + 32 * hh +
                        16 * ((sl & 3) >> 1) + 8 * (sl & 1));

  f32x16 o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) o[dt] = f32x16{};
  f32x16 s[2];
  V8 pk[4];
  float m_run = -INFINITY;
  float l_run = 0.0f;
  const int a_lane = prefix + wrow0 + lq;
  const int a_lane0 = prefix + wrow0;  // the wave's first row
  float slope2 = 0.0f;
  if constexpr (kAlibiLinear || kAlibiSqrt || kTileAlibi) slope2 = p.slopes[head] * kLog2e;
  float scale2 = p.scale2;
  // Linear ALiBi: the S^T accumulator of every key tile starts at slope2 C /
  // scale2 for its key C (the same for every lane and tile), so that the score
  // S^T scale2 + (-slope2 dbase - m) is one FMA.  Below |scale2| = 2^-100, where
  // slope2 / scale2 could overflow, the q.k part (at most 2^-100 |q.k|, under
  // 2^-60 for fp16 inputs and for bf16 inputs below 2^16) is dropped: Q is zeroed
  // and the scale taken as 1.
  f32x16 binit[2];
  if constexpr (kAlibiLinear) {
    if (!(__builtin_fabsf(scale2) >= 0x1p-100f)) {
#pragma unroll
      for (int c = 0; c < NC; ++c) qreg[c] = V8{};
      scale2 = 1.0f;
    }
    const float c2 = slope2 / scale2;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) binit[kb][r] = c2 * (float)(32 * kb + 8 * (r >> 2) + (r & 3));
    }
  }

  // Compressed tile entries of this lane's query row for a key tile that needs
  // them: 8 runs of 4 (the tile's 64 columns) from row r = a mod 128 (the key in
  // the row's own 128-block) or 128 + r (a key dk >= 1 blocks behind: ALiBi
  // tiles); dk = the row's 128-block minus the key's.  The norm tile is read
  // for the few tiles from the first row's block on, at the start of their
  // iteration; the ALiBi tiles for every tile, one iteration ahead, so that the
  // wait that ends an iteration has them in place and none is needed before
  // the softmax (it would drain the next tile's direct loads).
  MV4 mtv[8];
  int mdk = 0;
  // ALiBi tiles: the block shift of this tile's entries (times slope2 for the
  // linear types)
  float mshift = 0.0f;
  const int a_bq = a_lane / kMaskTile;
  // (byte offsets from the tile's base: a 32-bit lane offset of the row in the
  // diagonal block, and the wave-uniform distance to its row behind it)
  unsigned mrow_off = 0;
  unsigned mback_off = 0;
  if constexpr (kTile) {
    mrow_off = ((unsigned)(a_lane - a_bq * kMaskTile) * (unsigned)p.mask_stride + 4u * g) * (unsigned)sizeof(MT);
    mback_off = kType == 9 ? 0u : (unsigned)kMaskTile * (unsigned)p.mask_stride * (unsigned)sizeof(MT);
  }
  auto needs_tile_mask = [&](int t) { return kTileAlibi || (kTile && t * kBN + kBN > w_full_keys); };
  auto load_tile_mask = [&](int t) __attribute__((always_inline)) {
    const int j0 = t * kBN;
    mdk = a_bq - j0 / kMaskTile;
    // right ALiBi: y - 128 (dk - 1) behind the diagonal block; left ALiBi:
    // y - 128 dk (relative to the row's block origin)
    if constexpr (kType == 5) {
      mshift = -slope2 * (float)(kMaskTile * mdk);
    } else if constexpr (kTileAlibi) {
      mshift = mdk > 0 ? -(float)(kMaskTile * (mdk - 1)) : 0.0f;
      if constexpr (kType == 3) mshift *= slope2;
    }
    const unsigned off = mrow_off + (mdk == 0 ? 0u : mback_off) + (unsigned)(j0 & (kMaskTile - 1)) * (unsigned)sizeof(MT);
    const char* base = (const char*)p.mask;
#pragma unroll
    for (int u = 0; u < 8; ++u) mtv[u] = *(const MV4*)(base + off + 8 * (int)sizeof(MT) * u);
  };

  // P of tile t from S^T (in s): running max and sum (see the comment above).
  auto softmax = [&](int t) __attribute__((always_inline)) {
    const int j0 = t * kBN;
    const int dbase = a_lane - j0 - 4 * g;
    const int klim = kv - j0 - 4 * g;
    const int vlim = kCausal && !kTile ? min(klim, dbase + 1) : klim;
    const int llim = chunk_lo(a_lane) - j0 - 4 * g;  // chunked: key >= lo(a)  <=>  C >= llim
    const bool partial = j0 + kBN > w_full_keys || (kChunked && j0 < w_lo_last);
    const float dbf = (float)dbase;
    float x[2][16];
    float psum;
    // (checked: ALiBi tiles select -inf for a -inf entry; the unchecked form,
    // used by the fast path, gets -inf from it for a positive slope, and NaN or
    // +inf otherwise, which fail that path's sum test and send the tile to the
    // checked path)
    auto score = [&](int kb, int r, float m_ref, float nbm, bool checked) __attribute__((always_inline)) -> float {
      const int C = 32 * kb + 8 * (r >> 2) + (r & 3);
      if constexpr (kAlibiLinear) {
        (void)C;
        return __builtin_fmaf(s[kb][r], scale2, nbm);  // slope2 C is in S^T (binit)
      } else if constexpr (kAlibiSqrt) {
        return __builtin_fmaf(-slope2, fast_sqrt(dbf - (float)C), __builtin_fmaf(s[kb][r], scale2, -m_ref));
      } else if constexpr (kTileAlibi) {
        // the tile's entry y (+ block shift) as slope y, or -slope sqrt(-y);
        // a -inf entry hides the key
        const float mval = (float)mtv[4 * kb + (r >> 2)][r & 3];
        float v;
        if constexpr (kType == 4) {
          v = __builtin_fmaf(-slope2, fast_sqrt(-mval - mshift), __builtin_fmaf(s[kb][r], scale2, -m_ref));
        } else {
          v = __builtin_fmaf(s[kb][r], scale2, __builtin_fmaf(slope2, mval, mshift - m_ref));
        }
        return checked && mval == -INFINITY ? -INFINITY : v;
      } else {
        return __builtin_fmaf(s[kb][r], scale2, -m_ref);
      }
    };
    bool done = false;
    // (every mask: after the first tile the running max is set, and later tiles
    // exceed it by far less than the slack unless a score spikes, which the sum
    // test catches; a tile every row sees carries no tile entries)
    if (!partial && __builtin_amdgcn_ballot_w64(m_run == -INFINITY) == 0) {
      const float nbm = -slope2 * dbf - m_run;
      float ps[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      // Sqrt ALiBi on a tile whose every distance is >= kSqrtFar: the bias of
      // each 32-key half from a quadratic expansion of -slope2 sqrt(d) around
      // the half's centre (a lane's keys C = 32kb + 0..27, centre 32kb + 13.5):
      // one square root per half instead of one per score; |error| <=
      // 13.5^3 / (16 kSqrtFar^2.5) = 5.3e-5 in units of sqrt(d), times slope2.
      auto fast = [&](auto FAR) __attribute__((always_inline)) {
        float b0[2], b1[2], b2[2];
        if constexpr (decltype(FAR)::value) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            const float d0 = dbf - (32.0f * kb + 13.5f);
            const float rs = __builtin_amdgcn_rsqf(d0);
            b0[kb] = -slope2 * d0 * rs - m_run;  // -slope2 sqrt(d0), relative to m_run
            b1[kb] = 0.5f * slope2 * rs;         // first-order term (d falls as C grows)
            b2[kb] = 0.25f * b1[kb] * rs * rs;   // second-order term, slope2 / (8 d0^1.5)
          }
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float sc;
            if constexpr (decltype(FAR)::value) {
              const float dl = (float)(8 * (r >> 2) + (r & 3)) - 13.5f;
              sc = __builtin_fmaf(s[kb][r], scale2, __builtin_fmaf(__builtin_fmaf(b2[kb], dl, b1[kb]), dl, b0[kb]));
            } else {
              sc = score(kb, r, m_run, nbm, false);
            }
            const float e = fast_exp2(sc);
            x[kb][r] = e;
            ps[r & 3] += e;
          }
        }
      };
      if (kAlibiSqrt && a_lane0 - t * kBN - (kBN - 1) >= kSqrtFar) {
        fast(std::true_type{});
      } else {
        fast(std::false_type{});
      }
      psum = (ps[0] + ps[1]) + (ps[2] + ps[3]);
      done = __builtin_amdgcn_ballot_w64(!(psum <= kSumLimit)) == 0;
    }
    if (!done) {
      // Full path: tile max; the reference moves when a row's max grows by
      // more than 2^10 (or on the row's first visible key).
      const float m_ref = (m_run == -INFINITY) ? 0.0f : m_run;
      const float nbm = -slope2 * dbf - m_ref;
      // scores and the lane max, with or without the per-element predicate
      // (a wave-uniform branch between two straight-line versions)
      auto form = [&](auto with_mask) __attribute__((always_inline)) -> float {
        float m = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int C = 32 * kb + 8 * (r >> 2) + (r & 3);
            float v = score(kb, r, m_ref, nbm, true);
            if constexpr (kType == 9 && kTile && decltype(with_mask)::value) {
              // norm tile: the entry in the diagonal block (-inf hides the
              // key), 0 behind it, later blocks hidden
              const float mval = (float)mtv[4 * kb + (r >> 2)][r & 3];
              const bool hide = mdk < 0 || (mdk == 0 && mval == -INFINITY);
              v = mdk == 0 ? v + mval * kLog2e : v;
              v = hide ? -INFINITY : v;
            }
            if constexpr (kTileAlibi && decltype(with_mask)::value) v = mdk < 0 ? -INFINITY : v;
            if constexpr (decltype(with_mask)::value)
              v = (C < vlim && (!kChunked || C >= llim)) ? v : -INFINITY;
            x[kb][r] = v;
            m = fmaxf(m, v);
            // (sqrt tile: one group of four entries at a time, which keeps
            // the converted entries' registers few)
            if constexpr (kTileAlibi && kType == 4) {
              if ((r & 3) == 3) __builtin_amdgcn_sched_barrier(0);
            }
          }
        }
        return m;
      };
      float m;
      if (partial) {
        m = form(std::true_type{});
      } else {
        m = form(std::false_type{});
      }
      const float mx = max_with_other_half(m);
      const bool need = (m_run == -INFINITY) ? (mx > -INFINITY) : (mx > kRescaleSlack);
      if (__builtin_amdgcn_ballot_w64(need) != 0) {
        const float m_new = fmaxf(m_run, m_ref + mx);
        const float delta = (m_new == -INFINITY) ? 0.0f : m_new - m_ref;
        const float alpha = (m_new == -INFINITY) ? 1.0f : fast_exp2(m_run - m_new);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) x[kb][r] -= delta;
        }
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[dt] *= alpha;
        m_run = m_new;
      }
      float ps[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = fast_exp2(x[kb][r]);
          x[kb][r] = e;
          ps[r & 3] += e;
        }
      }
      psum = (ps[0] + ps[1]) + (ps[2] + ps[3]);
    }
    l_run += psum;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
#pragma unroll
      for (int e = 0; e < 8; ++e) pk[kc][e] = (T)x[kc >> 1][8 * (kc & 1) + e];
    }
  };

  // prologue: tile of iteration 0, then a full wait the compiler sees (Q has
  // landed too, so no wait for Q is left for it to place inside the loop,
  // where it would also drain the tile loads in flight).
  int blk_next = block_of(1);  // block id of the next iteration's tile
  // (the tile entries are read by every wave and iteration, unconditionally:
  // any lane's row offset lies inside the tile, and a branch around the loads
  // would keep two copies of the entries live)
  if constexpr (kTileAlibi) load_tile_mask(tile_of(0));
  {
    const TileSrc ts = tile_src(0, block_of(0));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      issue_block(0, i, ts, 0, std::false_type{});
      issue_block(1, i, ts, 0, std::false_type{});
    }
  }
  __builtin_amdgcn_s_waitcnt(0xF70);
  asm volatile("s_barrier" ::: "memory");

  auto iteration = [&](int u, auto BUF) __attribute__((always_inline)) {
    constexpr int buf = decltype(BUF)::value;
    constexpr unsigned kB = (unsigned)(buf * kBufBytes);
    const int t = tile_of(u);
    const bool load_next = u + 1 < n_tiles;
    TileSrc nx{};
    if (load_next) nx = tile_src(u + 1, blk_next);
    // Loads of the next iteration's tile (into the other buffer), spread between
    // the QK MFMAs.
    auto issue_next = [&](int k) __attribute__((always_inline)) {
      if (load_next) issue_block(k & 1, k >> 1, nx, buf ^ 1, std::false_type{});
    };
    if (t < w_tiles && (!kChunked || t >= w_t_lo)) {
      if constexpr (kType == 9 && kTile) {
        // (their wait before the softmax also covers the next tile's loads
        // issued below: only the tiles from the first row's block on)
        if (needs_tile_mask(t)) load_tile_mask(t);
      }
      if constexpr (kAlibiLinear) {
        s[0] = binit[0];
        s[1] = binit[1];
      } else {
        s[0] = f32x16{};
        s[1] = f32x16{};
      }
      // K operand reads run kQkDepth MFMAs ahead; the next tile's loads sit
      // between the MFMAs in straight-line versions (no branch between them):
      // LOAD 2 for a full next tile, 1 for a partial one (rows clamped to its
      // last key), 0 for none (last iteration).
      auto qk = [&](auto LOAD) __attribute__((always_inline)) {
        auto rd = [&](int i) -> V8 {
          const int c = i >> 1, kb = i & 1;
          return *(const V8*)(lds + kB + qa[c >> 1] + 8320 * kb + 32 * (c & 1));
        };
        constexpr int kQkDepth = 4;
        V8 ring[kQkDepth];
#pragma unroll
        for (int i = 0; i < kQkDepth; ++i) ring[i] = rd(i);
#pragma unroll
        for (int i = 0; i < 2 * NC; ++i) {
          const V8 a = ring[i % kQkDepth];
          if (i + kQkDepth < 2 * NC) ring[i % kQkDepth] = rd(i + kQkDepth);
          s[i & 1] = mfma32(a, qreg[i >> 1], s[i & 1]);
          if constexpr (decltype(LOAD)::value > 0) {
            if (i & 1)
              issue_block((i >> 1) & 1, i >> 2, nx, buf ^ 1, std::bool_constant<decltype(LOAD)::value == 2>{});
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      // Wave priorities 3 for QK, 1 for PV, 0 for the softmax: of the two
      // waves sharing a SIMD, one in its softmax yields issue slots to one
      // feeding the matrix cores, and one starting a tile's QK goes ahead of
      // one finishing a PV, which spreads the two waves' phases apart.
      __builtin_amdgcn_s_setprio(3);
      if (!load_next) {
        qk(std::integral_constant<int, 0>{});
      } else if (!kTile && nx.full) {  // (the tile variants keep their registers)
        qk(std::integral_constant<int, 2>{});
      } else {
        qk(std::integral_constant<int, 1>{});
      }
      // block id two iterations ahead, read while the softmax runs
      blk_next = block_of(u + 2);
      __builtin_amdgcn_s_setprio(0);
      softmax(t);
      __builtin_amdgcn_s_setprio(1);
      // the next key tile's ALiBi tile entries (this tile's are consumed)
      if constexpr (kTileAlibi) load_tile_mask(tile_of(min(u + 1, n_tiles - 1)));
      {
        auto rv = [&](int i) -> V8 {
          const int kc = i / NDT, dt = i % NDT;
          const char* src = lds + kB + va[dt] + 4160 * kc;
          const s16x4 lo = lds_read_tr16((const T*)src);
          const s16x4 hi = lds_read_tr16((const T*)(src + 2080));
          return __builtin_bit_cast(V8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        };
        constexpr int kPvDepth = 3;
        V8 vring[kPvDepth];
#pragma unroll
        for (int i = 0; i < kPvDepth; ++i) vring[i] = rv(i);
#pragma unroll
        for (int i = 0; i < 4 * NDT; ++i) {
          const V8 a = vring[i % kPvDepth];
          if (i + kPvDepth < 4 * NDT) vring[i % kPvDepth] = rv(i + kPvDepth);
          o[i % NDT] = mfma32(a, pk[i / NDT], o[i % NDT]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) issue_next(k);
      blk_next = block_of(u + 2);
      if constexpr (kTileAlibi) load_tile_mask(tile_of(min(u + 1, n_tiles - 1)));
    }
    // The next tile has landed (each wave waits for its own loads; the barrier
    // publishes them and ends every read of this buffer).
    __builtin_amdgcn_s_waitcnt(0xF70);
    asm volatile("s_barrier" ::: "memory");
  };
  for (int u = 0; u < n_tiles; u += 2) {
    iteration(u, std::integral_constant<int, 0>{});
    if (u + 1 < n_tiles) iteration(u + 1, std::integral_constant<int, 1>{});
  }

  if (!w_active) return;
  const float l_tot = sum_with_other_half(l_run);
  const int i = wrow0 + lq;
  // A row whose tile hides every key gets O = 0 (and LSE = -inf).
  const float inv = kTile && l_tot == 0.0f ? 0.0f : 1.0f / l_tot;
  // The wave's 32 x 128 output block is staged in LDS (the tile buffers are
  // free after the loop's last barrier, and no direct load is in flight; each
  // wave uses 8.7 KB of its own), so that every global store writes whole
  // 256-byte rows: lane l of pass k stores 16 bytes of row 4k + l / 16.
  constexpr int kOutRow = kRowBytes + 16;  // staged row, padded against bank conflicts
  char* ostage = lds + w * (kRowsPerWave * kOutRow);
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      V4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (T)(o[dt][4 * rg + e] * inv);
      *(V4*)(ostage + lq * kOutRow + (int)sizeof(T) * (32 * dt + 8 * rg + 4 * g)) = v;
    }
  }
  // (the wave's LDS writes complete before its reads below; the clobber keeps
  // the compiler from moving them across)
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  {
    const int rr = l >> 4, ch = l & 15;
    T* obase = (T*)p.out + (qs + wrow0) * q_row_stride + (long long)head * D + 8 * ch;
#pragma unroll
    for (int k = 0; k < kRowsPerWave / 4; ++k) {
      const int r = 4 * k + rr;
      const V8 v = *(const V8*)(ostage + r * kOutRow + 16 * ch);
      if (wrow0 + r < L) *(V8*)(obase + (long long)r * q_row_stride) = v;
    }
  }
  if (i >= L) return;
  if (p.lse != nullptr && g == 0) {
    float lse = (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2;
    if constexpr (kType == 5) lse += p.slopes[head] * (float)(kTile ? a_bq * kMaskTile : a_lane);
    p.lse[(qs + i) * p.head_num + head] = lse;
  }
}

// fp32 copy of a compressed tile: entry i of src to dst[i], 4 per lane (n4 groups).
template <typename T>
__global__ void __launch_bounds__(256) tile_to_f32_kernel(const T* __restrict__ src, float* __restrict__ dst,
                                                          int n4) {
  using V4 = typename Vec<T>::x4;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const V4 v = ((const V4*)src)[i];
  float4 f;
  f.x = (float)v[0];
  f.y = (float)v[1];
  f.z = (float)v[2];
  f.w = (float)v[3];
  ((float4*)dst)[i] = f;
}

// The direct-load kernel over an ALiBi tile (right, sqrt, left): the tile's
// fp32 copy into p.mask_f32, then the attention reading it.  The call's start
// event goes on the copy, its stop event on the attention.
template <typename T, int MASK>
hipError_t launch_f32_tile(const PrefillParams& p, dim3 g, hipStream_t s, const LaunchEvents& ev) {
  if (p.mask_f32 == nullptr || p.mask == nullptr) return hipErrorInvalidValue;
  const int n4 = p.mask_stride * p.mask_stride / 4;
  hipExtLaunchKernelGGL(tile_to_f32_kernel<T>, dim3((n4 + 255) / 256), dim3(256), 0, s, ev.start, nullptr, 0,
                        (const T*)p.mask, p.mask_f32, n4);
  PrefillParams q = p;
  q.mask = p.mask_f32;
  hipExtLaunchKernelGGL((prefill_dma_kernel<T, MASK>), g, dim3(256), 0, s, nullptr, ev.stop, 0, q, p.block_tables);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_mask(const PrefillParams& p, int mask_type, int grid, hipStream_t s, const LaunchEvents& ev) {
  const dim3 g(grid), blk(256);
  if (D == 128 && p.bs_shift >= 4) {
    switch (mask_type) {
      case kMaskTileFlag | 3:
        return launch_f32_tile<T, kMaskTileFlag | 3>(p, g, s, ev);
      case kMaskTileFlag | 4:
        return launch_f32_tile<T, kMaskTileFlag | 4>(p, g, s, ev);
      case kMaskTileFlag | 5:
        return launch_f32_tile<T, kMaskTileFlag | 5>(p, g, s, ev);
      case kMaskTileFlag | 9:
        hipExtLaunchKernelGGL((prefill_dma_kernel<T, kMaskTileFlag | 9>), g, blk, 0, s, ev.start, ev.stop, 0, p, p.block_tables);
        break;
      case 0: hipExtLaunchKernelGGL((prefill_dma_kernel<T, 0>), g, blk, 0, s, ev.start, ev.stop, 0, p, p.block_tables); break;
      case 3: hipExtLaunchKernelGGL((prefill_dma_kernel<T, 3>), g, blk, 0, s, ev.start, ev.stop, 0, p, p.block_tables); break;
      case 4: hipExtLaunchKernelGGL((prefill_dma_kernel<T, 4>), g, blk, 0, s, ev.start, ev.stop, 0, p, p.block_tables); break;
      case 5: hipExtLaunchKernelGGL((prefill_dma_kernel<T, 5>), g, blk, 0, s, ev.start, ev.stop, 0, p, p.block_tables); break;
      case 9: hipExtLaunchKernelGGL((prefill_dma_kernel<T, 9>), g, blk, 0, s, ev.start, ev.stop, 0, p, p.block_tables); break;
      case 10: hipExtLaunchKernelGGL((prefill_dma_kernel<T, 10>), g, blk, 0, s, ev.start, ev.stop, 0, p, p.block_tables); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  switch (mask_type) {
    case 0: hipExtLaunchKernelGGL((prefill_fwd_kernel<T, D, 0>), g, blk, 0, s, ev.start, ev.stop, 0, p); break;
    case 3: hipExtLaunchKernelGGL((prefill_fwd_kernel<T, D, 3>), g, blk, 0, s, ev.start, ev.stop, 0, p); break;
    case 4: hipExtLaunchKernelGGL((prefill_fwd_kernel<T, D, 4>), g, blk, 0, s, ev.start, ev.stop, 0, p); break;
    case 5: hipExtLaunchKernelGGL((prefill_fwd_kernel<T, D, 5>), g, blk, 0, s, ev.start, ev.stop, 0, p); break;
    case 9: hipExtLaunchKernelGGL((prefill_fwd_kernel<T, D, 9>), g, blk, 0, s, ev.start, ev.stop, 0, p); break;
    case 10: hipExtLaunchKernelGGL((prefill_fwd_kernel<T, D, 10>), g, blk, 0, s, ev.start, ev.stop, 0, p); break;
    case kMaskTileFlag | 3: hipExtLaunchKernelGGL((prefill_fwd_kernel<T, D, kMaskTileFlag | 3>), g, blk, 0, s, ev.start, ev.stop, 0, p); break;
    case kMaskTileFlag | 4: hipExtLaunchKernelGGL((prefill_fwd_kernel<T, D, kMaskTileFlag | 4>), g, blk, 0, s, ev.start, ev.stop, 0, p); break;
    case kMaskTileFlag | 5: hipExtLaunchKernelGGL((prefill_fwd_kernel<T, D, kMaskTileFlag | 5>), g, blk, 0, s, ev.start, ev.stop, 0, p); break;
    case kMaskTileFlag | 9: hipExtLaunchKernelGGL((prefill_fwd_kernel<T, D, kMaskTileFlag | 9>), g, blk, 0, s, ev.start, ev.stop, 0, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, int dtype, int head_size, int mask_type,
                          int grid, hipStream_t stream, const LaunchEvents& ev) {
  if (grid <= 0) return hipSuccess;
  if (dtype == 0) {
    return head_size == 64 ? launch_mask<_Float16, 64>(p, mask_type, grid, stream, ev)
                           : launch_mask<_Float16, 128>(p, mask_type, grid, stream, ev);
  }
  return head_size == 64 ? launch_mask<__bf16, 64>(p, mask_type, grid, stream, ev)
                         : launch_mask<__bf16, 128>(p, mask_type, grid, stream, ev);
}

}  // namespace mpa
