// Split-KV decode of multi-head latent attention (MLA) for gfx950.
//
// What it computes (Ascend ATB page "MLA", parameter table): query token t,
// head h: q = [qNope 512 | qRope 64]; key j = [ctKV_j 512 | kRope_j 64] of the
// single latent KV head; value j = ctKV_j (512);
//   s_j = qkScale * q.k_j over keys j < contextLens (maskType SPEC: j <=
//   contextLens - q_len + t), out = softmax(s) V, lse = ln sum_j exp(s_j).
//
// Kernel 1 (split): one workgroup of 8 waves per (piece, 128-row group), one
// workgroup per compute unit.  The key tiles (32 keys) of all sequences, laid
// end to end, are cut into pieces of near-equal length; a piece's part of one
// sequence is a segment.  The rows of a sequence are its (token, head) pairs;
// the 8 waves form 4 pairs of 32 rows: one wave of a pair contracts the first
// half of the 576 query/key dims and accumulates output dims 0..255, the other
// the rest; the two partial score tiles are summed through LDS.  Waves 0..3
// gather each tile's latent rows through blockTables into LDS (direct
// global->LDS loads, three buffers, two tiles ahead); each wave forms S^T = K
// Q^T with the 32x32x16 MFMA (the nope part of Q^T stays in registers, the
// rope part in LDS), runs the online softmax in the log2 domain and
// accumulates O^T += V^T P^T, reading V^T -- the first 512 columns of the same
// LDS rows -- with the LDS transpose read: every latent row is loaded from HBM
// once and serves as key and as value.  Waves 0..3 and 4..7 run half a tile
// apart so that one wave's MFMA work overlaps the other's.  The running output
// is rescaled only when a row's max grows by more than 2^8 (exact: the final
// normalisation uses the same reference max).  A segment that covers its whole
// sequence writes the final output; the others write a normalised partial
// output and a log2-domain LSE, both fp32, to the workspace.
//
// Kernel 2 (combine): for each (token, head) of a sequence with several
// segments, LSE-weighted merge of the partials: L = log2 sum_s 2^{lse_s}, out = sum_s 2^{lse_s - L} o_s --
// the merge by LSE that the MLA page's lse output exists for.

#include <type_traits>

#include <hip/hip_ext.h>

#include "device.h"
#include "kernels.h"

namespace mpa {

namespace {

constexpr int kDq = 576;        // query / key width
constexpr int kDv = 512;        // latent value width
constexpr int kBN = 32;         // keys per tile
constexpr int kRows = 128;      // query rows per workgroup (4 wave pairs x 32)
constexpr int kWaves = 8;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.0f;  // log2 units of growth tolerated before rescaling
constexpr float kSumLimit = 256.0f;    // 2^kRescaleSlack

// LDS layout of one key tile.  Latent part: key k sits in row slot
// lat_slot(k), 512 values + 8 of padding = 1040 bytes = 65 16-byte chunks.  An
// odd chunk count puts slot s at a distinct bank group for every s mod 16 in a
// given column; the slot order (a 4x4 transpose inside each 16-key block) puts
// the 4 keys of a transpose read at slots 4 apart.  So the QK operand reads (16
// keys, one 16-byte column) and the V^T transpose reads (4 keys x 64 bytes per
// half wave) both hit 16 distinct bank groups, and every address is one per-lane
// base plus an immediate offset.  A key's latent part is written by one direct
// load (64 lanes x 16 contiguous bytes).  Rope part: 32 rows of 128 bytes after
// the latent slots, 16-byte chunks XOR-swizzled by rope_swz (conflict-free for
// 16 rows in one column), 8 keys per direct load.
constexpr int kLatRow = kDv + 8;  // elements per latent slot
__device__ __forceinline__ int lat_slot(int k) {
  return (k & ~15) | ((k & 15) >> 2) | ((k & 3) << 2);
}
__device__ __forceinline__ int rope_swz(int r) { return (r >> 1) & 7; }
// The rope part of the 128 query rows: rows of 64 values + 8 of padding (9
// chunks, odd), read 32 rows at a time as the B operand.
constexpr int kQRopeRow = 72;

// int8 latent cache: slot s (key lat_slot(s)) holds the key's 512 bytes at
// byte 1040 (s % 16) + 512 (s / 16): slots s and s + 16 are adjacent, so one
// direct load (lanes 0..31 and 32..63) fills both, and the 16-byte padding per
// pair puts slot s at bank group s % 16 (+ column) for both read patterns --
// the QK operand (16 slots, one 16-byte column) and the 8-bit transpose read
// (8 slots, 16 bytes each).
constexpr int kQ8PairBytes = 2 * kDv + 16;
constexpr int kQ8LatBytes = 16 * kQ8PairBytes;
__device__ __forceinline__ int q8_slot_byte(int s) { return kQ8PairBytes * (s & 15) + kDv * (s >> 4); }

// 8 signed bytes -> the 8 fp16 values x + 1152, exact: byte x ^ 0x80 = x + 128
// placed under the fp16 exponent byte 0x64 is the value 1024 + (x + 128).  The
// bias is taken off the output once (1152 times the sum of the fp16 P that
// multiplied it) instead of off every value.
__device__ __forceinline__ f16x8 i8x8_biased_f16x8(i32x2 t) {
  const unsigned a = (unsigned)t[0] ^ 0x80808080u;
  const unsigned b = (unsigned)t[1] ^ 0x80808080u;
  // v_perm_b32 byte selectors: 0-3 pick bytes of the second operand, 4-7 of the
  // first (here the exponent byte 0x64), so each pair is one instruction.
  constexpr unsigned kExp = 0x64646464u;
  u32x4 w;
  w[0] = __builtin_amdgcn_perm(kExp, a, 0x04010400u);  // [a0, 0x64, a1, 0x64]
  w[1] = __builtin_amdgcn_perm(kExp, a, 0x04030402u);  // [a2, 0x64, a3, 0x64]
  w[2] = __builtin_amdgcn_perm(kExp, b, 0x04010400u);
  w[3] = __builtin_amdgcn_perm(kExp, b, 0x04030402u);
  return __builtin_bit_cast(f16x8, w);  // x + 1152, exact
}

// Q8: the int8 latent cache (qNope and ctKV int8, per-head descales) -- the
// nope part of the scores on the int8 MFMA (exact integer products), the value
// side through the 8-bit transpose read and an exact conversion to fp16 values
// biased by 1152; the output takes off 1152 times the row's sum of the fp16 P
// (the fp32 accumulation error this adds is bounded by 2^-24 x 1279 x sum P per
// MFMA accumulation step, far below the output rounding).
template <typename T, bool ONE_BLOCK, bool Q8>
__global__ void __launch_bounds__(512, 1)
    mla_split_kernel(MlaParams p, const int32_t* __restrict__ block_tables,
                     const int4* __restrict__ segs, const int32_t* __restrict__ piece_seg,
                     const int4* __restrict__ seqs, const int4* __restrict__ seqs2) {
  using V8 = typename Vec<T>::x8;
  using PV8 = std::conditional_t<Q8, f16x8, V8>;  // operands of O^T += V^T P^T
  using PT = std::conditional_t<Q8, _Float16, T>;
  constexpr int NCH = kDv / 16 / 2;  // 16 register-resident contraction chunks per wave of a pair
  constexpr int NCH8 = kDv / 32 / 2; // 8 int8 chunks (32 dims) per wave of a pair
  constexpr int NDT = kDv / 32 / 2;  // 8 O^T tiles per wave of a pair

  // Three key-tile buffers (latent rows, then rope rows), the pairs' partial
  // S^T exchange, and the rope part of the 128 query rows.
  constexpr int kLatElems = Q8 ? kQ8LatBytes / (int)sizeof(T) : kBN * kLatRow;
  constexpr int kBufElems = kLatElems + kBN * 64;
  __shared__ __attribute__((aligned(1024))) T tbuf[3 * kBufElems];
  __shared__ __attribute__((aligned(16))) float4 xch[kWaves][4 * 64];
  __shared__ __attribute__((aligned(16))) T qrope[kRows * kQRopeRow];

  // Workgroup -> (piece, row group): workgroups go round-robin to the 8 XCDs by
  // id; XCD x handles pieces [x * ppx, (x + 1) * ppx), the row groups of one
  // piece side by side.
  // (whole-sequence plans: workgroup i handles piece i / row_groups, so the row
  // groups of a sequence go round-robin to the XCDs)
  const int slot = blockIdx.x >> 3;
  const int piece = p.whole ? (int)blockIdx.x / p.row_groups : (blockIdx.x & 7) * p.pieces_per_xcd + slot / p.row_groups;
  const int rg = p.whole ? (int)blockIdx.x % p.row_groups : slot % p.row_groups;
  const int s_beg = piece_seg[piece];
  const int s_end = piece_seg[piece + 1];
  const int row_base = rg * kRows;  // first row (token-major (token, head) index) of this workgroup
  // Segments whose sequence has rows in this row group.
  // Plan records are read with scalar loads (see sload_int4).
  auto next_valid = [&](int s) -> int {
    while (s < s_end && sload_int4(&seqs2[sload_int4(&segs[s]).x]).y <= row_base) ++s;
    return s;
  };
  // End (exclusive) of the keys of segment sg that this row group visits: with
  // the SPEC mask a whole-sequence segment stops at its last row's limit,
  // ctx - q_len + t + 1 for the group's last token t (keys after it are hidden
  // from every row of the group); a partial segment keeps its end, since its
  // result is merged with the sequence's other segments.
  auto seg_keys_end = [&](const int4& sg) -> int {
    if (!p.spec_mask || sg.w >= 0) return sg.z;
    const int4 sq = sload_int4(&seqs[sg.x]);
    const int4 sq2 = sload_int4(&seqs2[sg.x]);
    const int t_last = min(sq2.y - 1, row_base + kRows - 1) / p.head_num;
    return min(sg.z, sq.x - sq.y + t_last + 1);
  };
  int n_total = 0;
  for (int s = next_valid(s_beg); s < s_end; s = next_valid(s + 1)) {
    const int4 sg = sload_int4(&segs[s]);
    n_total += (seg_keys_end(sg) - sg.y + kBN - 1) / kBN;
  }
  if (n_total == 0) return;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (uniform)
  const int pr = w >> 1;   // pair: 32 query rows
  const int hf = w & 1;    // half: contraction dims (nope [256hf, +256) + rope [32hf, +32)), output dims [256hf, +256)
  const int l = tid & 63;
  const int g = l >> 5;
  const int lq = l & 31;
  const int H = p.head_num;

  // ---- loader cursor (wave-uniform): the tile whose loads are issued next ----
  int ls = next_valid(s_beg);
  int lb, lj, lk1;
  {
    const int4 sg = sload_int4(&segs[ls]);
    lb = sg.x; lj = sg.y; lk1 = seg_keys_end(sg);
  }
  // ONE_BLOCK: a power-of-two block size >= 8 (>= 32 with the int8 cache): the 8
  // keys that a loader wave fetches of a tile (tiles start at multiples of 32)
  // lie in one cache block -- with the int8 cache the whole tile does -- so
  // each loader wave takes one wave-uniform block id per tile, that of its
  // first key (clamped into the group of the segment's last key on a tile
  // past it, so that no block-table entry past the keys is read).  Otherwise
  // each row looks its block up.
  auto wave_key0 = [&](int last) { return Q8 ? 0 : min(8 * w, last & ~7); };
  auto tile_block = [&]() -> int {
    return ONE_BLOCK ? block_tables[(long long)lb * p.max_blocks + ((lj + wave_key0(lk1 - 1 - lj)) >> p.bs_shift)]
                     : 0;
  };

  auto ld_advance = [&]() {
    lj += kBN;
    if (lj >= lk1) {
      ls = next_valid(ls + 1);
      if (ls < s_end) {
        const int4 sg = sload_int4(&segs[ls]);
        lb = sg.x; lj = sg.y; lk1 = seg_keys_end(sg);
      }
    }
  };
  // A tile whose loads are due: its block id (one-block tiles) and the loader
  // cursor at it (sequence, first key, segment end); the cursor moves on.
  struct TileRef {
    int blk, b, j, k1;
  };
  auto take_tile = [&]() -> TileRef {
    const TileRef r{tile_block(), lb, lj, lk1};
    ld_advance();
    return r;
  };
  // Row r of the cache: latent at lat_row(r), rope at rope_row(r).
  const bool split_rope = p.krope != nullptr;
  auto lat_row = [&](long long r) -> const T* { return (const T*)p.ckv + r * p.ckv_stride; };
  auto rope_row = [&](long long r) -> const T* {
    return split_rope ? (const T*)p.krope + r * 64 : (const T*)p.ckv + r * p.ckv_stride + kDv;
  };
  const unsigned lane16 = 16u * (unsigned)l;
  // Direct loads of the loader's tile into buffer `buf`, issued by waves 0..3
  // only: wave w fills the latent slots of keys 8w .. 8w+7 and the rope rows of
  // the same keys.  Keys at or beyond the segment end repeat its last key
  // (finite data, masked later).
  const long long lat_step = (long long)p.ckv_stride * (long long)sizeof(T);
  const long long rope_step = split_rope ? 64 * (long long)sizeof(T) : lat_step;
  auto issue = [&](const TileRef& tr, T* buf) __attribute__((always_inline)) {
    const int blk = tr.blk, tj = tr.j;  // the tile's block id and first key
    const int last = tr.k1 - 1 - tj;    // last key of the segment within the tile
    const unsigned m0buf = (unsigned)(unsigned long)(const __attribute__((address_space(3))) void*)buf;
    if constexpr (Q8) {
      // Latent: wave w fills slots 4w .. 4w+3 and the same + 16 (lanes 32..63),
      // 32 lanes x 16 bytes per key; rope as below.
      const int ln = opaque_lane();
      const int half = ln >> 5;
      const unsigned col = 16u * (unsigned)(ln & 31);
      const int ropekey = 8 * w + (ln >> 3);
      const unsigned ropecol = 16u * (unsigned)((ln & 7) ^ rope_swz(ropekey));
      if constexpr (ONE_BLOCK) {
        const long long rt = (long long)blk * p.block_size + (tj & (p.block_size - 1));
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int key = min(lat_slot(4 * w + k) + 16 * half, last);
          dma16s_m0((const char*)p.ckv + rt * kDv, (unsigned)key * kDv + col,
                    m0buf + (unsigned)q8_slot_byte(4 * w + k));
        }
        dma16s((const char*)p.krope + rt * 64 * (long long)sizeof(T),
               (unsigned)min(ropekey, last) * 64u * (unsigned)sizeof(T) + ropecol,
               buf + kLatElems + 64 * 8 * w);
      } else {
        const int32_t* bt = block_tables + (long long)tr.b * p.max_blocks;
        auto row_of = [&](int key) -> long long {
          const int j = tj + min(key, last);
          const int bi = j / p.block_size;
          return (long long)bt[bi] * p.block_size + (j - bi * p.block_size);
        };
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const long long row = row_of(lat_slot(4 * w + k) + 16 * half);
          dma16((const char*)p.ckv + row * kDv + col, (const char*)buf + q8_slot_byte(4 * w + k));
        }
        dma16((const char*)p.krope + row_of(ropekey) * 64 * (long long)sizeof(T) + ropecol,
              buf + kLatElems + 64 * 8 * w);
      }
      return;
    }
    if constexpr (ONE_BLOCK) {
      // The wave's keys lie in one cache block, from its key k0 on: consecutive rows.
      const int k0 = wave_key0(last);
      const long long rt = (long long)blk * p.block_size + ((tj + k0) & (p.block_size - 1));
      const char* a = (const char*)lat_row(rt + min(8 * w, last) - k0);
      const int advances = last - 8 * w;  // rows after the first that exist
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        dma16s_m0(a, lane16, m0buf + (unsigned)(lat_slot(8 * w + k) * kLatRow * sizeof(T)));
        if (k < advances) a += lat_step;
      }
      // Rope: lane l carries key 8w + l/8 (clamped), 16-byte chunk (l % 8) ^ rope_swz(key).
      const int ln = opaque_lane();
      const int key = 8 * w + (ln >> 3);
      const unsigned off = (unsigned)(min(key, last) - k0) * (unsigned)rope_step +
                           16u * (unsigned)((ln & 7) ^ rope_swz(key));
      dma16s(rope_row(rt), off, buf + kLatElems + 64 * 8 * w);
    } else {
      const int32_t* bt = block_tables + (long long)tr.b * p.max_blocks;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int j = tj + min(8 * w + k, last);
        const int bi = j / p.block_size;
        const long long row = (long long)bt[bi] * p.block_size + (j - bi * p.block_size);
        dma16s_m0(lat_row(row), lane16, m0buf + (unsigned)(lat_slot(8 * w + k) * kLatRow * sizeof(T)));
      }
      const int ln = opaque_lane();
      const int key = 8 * w + (ln >> 3);
      const int j = tj + min(key, last);
      const int bi = j / p.block_size;
      const long long row = (long long)bt[bi] * p.block_size + (j - bi * p.block_size);
      dma16((const char*)rope_row(row) + 16 * ((ln & 7) ^ rope_swz(key)),
            buf + kLatElems + 64 * 8 * w);
    }
  };
  // Waves 0..3 issue 9 direct loads per tile (5 with the int8 cache), so
  // "s_waitcnt vmcnt(9)" waits for every tile but the most recently issued one.  (Encoding: vmcnt | expcnt 7
  // << 4 | lgkmcnt 15 << 8, i.e. wait on vector memory only; through the
  // builtin so that the compiler's own wait tracking sees it.)  A loader wave
  // waits for its own loads; the barrier after it publishes the tile to all.
  auto wait_tiles = [&](bool newer_in_flight) __attribute__((always_inline)) {
    if (newer_in_flight) __builtin_amdgcn_s_waitcnt(0xF70 | (Q8 ? 5 : 9));  // Q8: 4 latent + 1 rope
    else __builtin_amdgcn_s_waitcnt(0xF70);
  };

  // ---- per-segment state ----
  V8 qreg[Q8 ? 1 : NCH];
  i32x4 qreg8[Q8 ? NCH8 : 1];
  float qk_desc = 1.0f, pv_desc = 1.0f, pv_desc_next = 1.0f;  // Q8: this lane's row's head
  float l16_run = 0.0f;  // Q8: sum of the fp16-rounded P (the values carry a bias of 1152)
  f32x16 o[NDT];
  float m_run = -INFINITY, l_run = 0.0f;
  bool row_ok = false, w_active = false;
  int lim = 0, w_lim_lo = 0;
  int cs = ls;           // compute cursor: segment, key start of the tile, segment end
  int cj = lj, ck1 = lk1;
  const float scale2 = p.scale2;
  float4* my_x = &xch[w][l];
  const float4* other_x = &xch[w ^ 1][l];
  const int tr_row = 4 * g + ((l & 15) >> 2);
  const int tr_col = 256 * hf + 16 * ((l >> 4) & 1) + 4 * (l & 3);

  // Loads the queries of segment `seg` into this wave: the nope part of this
  // lane's row (dims [256hf, +256)) into registers, and the rope part of the
  // pair's 32 rows that this wave reads (dims [32hf, +32)) into LDS.  A wave
  // writes only LDS it reads itself, so no barrier is involved.
  auto load_q = [&](int seg) __attribute__((always_inline)) {
    const int4 sg = sload_int4(&segs[seg]);
    const int4 sq = sload_int4(&seqs[sg.x]);
    const int4 sq2 = sload_int4(&seqs2[sg.x]);
    const int tok0 = sq.z, rows = sq2.y;
    const int ln = opaque_lane();
    const int mm_row = row_base + 32 * pr + (ln & 31);
    const bool ok = mm_row < rows;
    if constexpr (Q8) {
      // int8 nope: lane (row, g) holds dims 256hf + 32c + 16g .. +15 of chunk c;
      // the descales of the row's head (rows are (token, head) pairs).
      const int8_t* qn8 = (const int8_t*)p.q_nope + ((long long)tok0 * H + (ok ? mm_row : 0)) * kDv +
                          256 * hf + 16 * (ln >> 5);
#pragma unroll
      for (int c = 0; c < NCH8; ++c) qreg8[c] = ok ? *(const i32x4*)(qn8 + 32 * c) : i32x4{0, 0, 0, 0};
      const int hd = ok ? mm_row % H : 0;
      qk_desc = p.qk_descale[hd];
      pv_desc_next = p.pv_descale[hd];
    } else {
      const T* qn = (const T*)p.q_nope + ((long long)tok0 * H + (ok ? mm_row : 0)) * kDv + 8 * (ln >> 5);
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        if (ok) {
          qreg[c] = *(const V8*)(qn + 16 * (NCH * hf + c));
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) qreg[c][e] = (T)0.0f;
        }
      }
    }
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      const int r = 32 * pr + 16 * pass + (ln >> 2);  // row within the group of 128
      const int ch = 4 * hf + (ln & 3);               // 16-byte chunk of the 64-wide rope row
      const int mm = row_base + r;
      V8 v;
      if (mm < rows) {
        v = *(const V8*)((const T*)p.q_rope + ((long long)tok0 * H + mm) * 64 + 8 * ch);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (T)0.0f;
      }
      *(V8*)&qrope[r * kQRopeRow + 8 * ch] = v;
    }
    // The query loads complete here, so no later wait of the compiler's covers
    // direct loads issued after this point.
    __builtin_amdgcn_s_waitcnt(0xF70);
  };
  // Per-segment state of segment `seg`: row masks, key limits, accumulators.
  auto reset_state = [&](int seg) __attribute__((always_inline)) {
    const int4 sg = sload_int4(&segs[seg]);
    const int4 sq = sload_int4(&seqs[sg.x]);
    const int4 sq2 = sload_int4(&seqs2[sg.x]);
    const int ctx = sq.x, q_len = sq.y, rows = sq2.y;
    const int ln = opaque_lane();
    const int mm_row = row_base + 32 * pr + (ln & 31);
    row_ok = mm_row < rows;
    w_active = row_base + 32 * pr < rows;
    const int t_loc = row_ok ? mm_row / H : 0;
    lim = min(sg.z, p.spec_mask ? (ctx - q_len + t_loc + 1) : ctx);
    w_lim_lo = sg.z;
    if (p.spec_mask) w_lim_lo = min(sg.z, ctx - q_len + (row_base + 32 * pr) / H + 1);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[dt] = f32x16{};
    m_run = -INFINITY;
    l_run = 0.0f;
    l16_run = 0.0f;
    pv_desc = pv_desc_next;
  };

  // First half of a tile: the wave's partial S^T over its half of the 576
  // dims, written to its exchange slot.
  auto qk_part = [&](const T* lat) __attribute__((always_inline)) {
    if constexpr (Q8) {
      if (!w_active) return;
      // Nope: int8 A operands (key slot lat_slot(lq), dims 256hf + 32c + 16g ..
      // +15), loaded two chunks ahead; exact int32 sums, then the head's descale;
      // the rope MFMAs accumulate on top.
      const char* arow = (const char*)lat + q8_slot_byte(lat_slot(lq)) + 256 * hf + 16 * g;
      i32x4 ring[2];
      ring[0] = *(const i32x4*)(arow);
      ring[1] = *(const i32x4*)(arow + 32);
      i32x16 si = i32x16{};
      V8 ra0, ra1, bq0, bq1;
#pragma unroll
      for (int c = 0; c < NCH8; ++c) {
        const i32x4 a = ring[c & 1];
        if (c + 2 < NCH8) ring[c & 1] = *(const i32x4*)(arow + 32 * (c + 2));
        if (c == NCH8 - 3) {
          const int ln = opaque_lane();
          const int key = ln & 31;
          const int r0 = 2 * (2 * hf) + (ln >> 5);
          ra0 = *(const V8*)(lat + kLatElems + key * 64 + 8 * (r0 ^ rope_swz(key)));
          ra1 = *(const V8*)(lat + kLatElems + key * 64 + 8 * ((r0 + 2) ^ rope_swz(key)));
          const T* qrow = qrope + (32 * pr + lq) * kQRopeRow + 8 * g;
          bq0 = *(const V8*)(qrow + 8 * (4 * hf));
          bq1 = *(const V8*)(qrow + 8 * (4 * hf + 2));
        }
        si = mfma32_i8(a, qreg8[c], si);
        __builtin_amdgcn_sched_barrier(0);
      }
      f32x16 s0;
#pragma unroll
      for (int r = 0; r < 16; ++r) s0[r] = (float)si[r] * qk_desc;
      s0 = mfma32(ra0, bq0, s0);
      s0 = mfma32(ra1, bq1, s0);
#pragma unroll
      for (int r = 0; r < 16; r += 4)
        my_x[16 * r] = make_float4(s0[r], s0[r + 1], s0[r + 2], s0[r + 3]);
      return;
    }
    f32x16 s0 = f32x16{};
    // A operands: this lane's key row (slot), 16-byte chunks of this wave's half
    // of the contraction: 16 latent chunks, then 2 rope chunks.  Loads run
    // kQkDepth chunks ahead of the MFMA that consumes them.
    const T* arow = lat + lat_slot(lq) * kLatRow;
    auto load_a = [&](int c) -> V8 {
      if (c < NCH) return *(const V8*)(arow + 8 * (2 * (NCH * hf + c) + g));
      // Rope row lq, 16-byte chunk r16 (addresses recomputed here: registers).
      const int ln = opaque_lane();
      const int key = ln & 31;
      const int r16 = 2 * (2 * hf + c - NCH) + (ln >> 5);
      return *(const V8*)(lat + kLatElems + key * 64 + 8 * (r16 ^ rope_swz(key)));
    };
    constexpr int kQkDepth = 3;
    if (w_active) {
      V8 ring[kQkDepth];
#pragma unroll
      for (int c = 0; c < kQkDepth; ++c) ring[c] = load_a(c);
      V8 bq0, bq1;
#pragma unroll
      for (int c = 0; c < NCH + 2; ++c) {
        const V8 a = ring[c % kQkDepth];
        if (c + kQkDepth < NCH + 2) ring[c % kQkDepth] = load_a(c + kQkDepth);
        if (c == NCH - 4) {
          const T* qrow = qrope + (32 * pr + lq) * kQRopeRow + 8 * g;
          bq0 = *(const V8*)(qrow + 8 * (4 * hf));
          bq1 = *(const V8*)(qrow + 8 * (4 * hf + 2));
        }
        const V8 b = c < NCH ? qreg[c] : (c == NCH ? bq0 : bq1);
        s0 = mfma32(a, b, s0);
        // Keep the loads kQkDepth chunks ahead (the scheduler would otherwise
        // sink them next to their MFMA to save registers).
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int r = 0; r < 16; r += 4)
        my_x[16 * r] = make_float4(s0[r], s0[r + 1], s0[r + 2], s0[r + 3]);
    }
  };

  // Second half of a tile (after a barrier that made the partner's partial
  // scores visible): full scores, online softmax, O^T += V^T P^T.
  auto smpv_part = [&](const T* lat) __attribute__((always_inline)) {
    const int j0 = cj;
    f32x16 s0;
    if (w_active) {
      // V^T operands (keys 16kc + tr_row and the same + 8, i.e. slot + 2; dims
      // 32dt + tr_col .. +3), loaded kPvDepth MFMAs ahead; the first ones are in
      // flight during the softmax.
      // Q8: lane (group of 16, index s) points at key 4g + (e & 3) + 8 (e >> 2),
      // e = s / 2 (the key order of the P^T operand; key half i >> 3 is 512
      // bytes on), bytes 8 (s % 2) .. +7 of the group's 16 dims; the transpose
      // read returns this lane's dim over those 8 keys.
      const int e8 = (l & 15) >> 1;
      const char* vbase8 = (const char*)lat + q8_slot_byte(lat_slot(4 * g + (e8 & 3) + 8 * (e8 >> 2))) +
                           256 * hf + 16 * ((l >> 4) & 1) + 8 * (l & 1);
      const T* vbase = lat + lat_slot(tr_row) * kLatRow + tr_col;
      auto load_v = [&](int i) -> PV8 {
        if constexpr (Q8) {
          return i8x8_biased_f16x8(lds_read_tr8(vbase8 + kDv * (i >> 3) + 32 * (i & 7)));
        } else {
          const T* src0 = vbase + (i >> 3) * (16 * kLatRow) + 32 * (i & 7);
          const s16x4 lo = lds_read_tr16(src0);
          const s16x4 hi = lds_read_tr16(src0 + 2 * kLatRow);
          return __builtin_bit_cast(V8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
      };
      constexpr int kPvDepth = 2;
#pragma unroll
      for (int r = 0; r < 16; r += 4) {
        const float4 u = my_x[16 * r];
        const float4 v = other_x[16 * r];
        s0[r] = u.x + v.x; s0[r + 1] = u.y + v.y; s0[r + 2] = u.z + v.z; s0[r + 3] = u.w + v.w;
      }
      PV8 vring[kPvDepth];
#pragma unroll
      for (int c = 0; c < kPvDepth; ++c) vring[c] = load_v(c);
      // Fast path, on a tile every row of the wave sees once the reference max
      // is set: P against the running max at once, checked by the lane's sum
      // (a P above 2^slack only comes with a sum above it).  If some lane's
      // sum is larger, the scores are read back from the exchange slots (they
      // hold this tile's partial scores until the next tile) and take the path
      // with the row max.  Both waves of a pair see the same scores and take
      // the same branch.
      float psum = 0.0f;
      bool done = false;
      if (j0 + kBN <= w_lim_lo && __builtin_amdgcn_ballot_w64(m_run == -INFINITY) == 0) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s0[r] = fast_exp2(__builtin_fmaf(s0[r], scale2, -m_run));
          psum += s0[r];
        }
        done = __builtin_amdgcn_ballot_w64(!(psum <= kSumLimit)) == 0;
        if (!done) {
#pragma unroll
          for (int r = 0; r < 16; r += 4) {
            const float4 u = my_x[16 * r];
            const float4 v = other_x[16 * r];
            s0[r] = u.x + v.x; s0[r + 1] = u.y + v.y; s0[r + 2] = u.z + v.z; s0[r + 3] = u.w + v.w;
          }
          psum = 0.0f;
        }
      }
      if (!done) {
        // Row max of the scaled scores; the exponent below is fma(s, kmul, -m):
        // full tiles keep the raw scores (kmul = scale, max taken on the raw
        // values, exact since scaling is monotonic), partial tiles store the
        // scaled, masked scores (kmul = 1).
        float mx = -INFINITY;
        float kmul = scale2;
        if (j0 + kBN > w_lim_lo) {
          // Partial tile: key j0 + 4g + C is visible to this row iff C < vlim.
          const int vlim = lim - j0 - 4 * (opaque_lane() >> 5);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int C = 8 * (r >> 2) + (r & 3);
            const float x = (C < vlim) ? s0[r] * scale2 : -INFINITY;
            s0[r] = x;
            mx = fmaxf(mx, x);
          }
          kmul = 1.0f;
        } else if (scale2 >= 0.0f) {
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s0[r]);
          mx *= scale2;
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, -s0[r]);
          mx *= -scale2;
        }
        mx = max_with_other_half(mx);
        // Lazy rescale: keep the reference max unless a row grew by > 2^8.  Both
        // waves of a pair see the same scores and take the same decisions.
        const bool grow = mx > m_run + kRescaleSlack;
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
          const float m_new = fmaxf(m_run, mx);
          const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
          const float alpha = fast_exp2(m_run - m_use);
          l_run *= alpha;
          if constexpr (Q8) l16_run *= alpha;
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) o[dt] *= alpha;
          m_run = m_new;
        }
        const float m_use = (m_run == -INFINITY) ? 0.0f : m_run;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s0[r] = fast_exp2(__builtin_fmaf(s0[r], kmul, -m_use));
          psum += s0[r];
        }
      }
      l_run += psum;
      PV8 p0, p1;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p0[e] = (PT)s0[e];
        p1[e] = (PT)s0[8 + e];
      }
      if constexpr (Q8) {
        float q16 = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) q16 += (float)p0[e] + (float)p1[e];
        l16_run += q16;
      }
#pragma unroll
      for (int i = 0; i < 2 * NDT; ++i) {
        const PV8 a = vring[i % kPvDepth];
        if (i + kPvDepth < 2 * NDT) vring[i % kPvDepth] = load_v(i + kPvDepth);
        o[i & 7] = mfma32(a, (i >> 3) == 0 ? p0 : p1, o[i & 7]);
      }
    }
  };

  // Writes the segment's result: the final output (and natural-log LSE) when the
  // segment covers the whole sequence, else the normalised partial output and
  // its log2-domain LSE.
  auto seg_end = [&](int seg) __attribute__((always_inline)) {
    if (!w_active) return;
    const float l_tot = sum_with_other_half(l_run);
    const float bias = Q8 ? 1152.0f * sum_with_other_half(l16_run) : 0.0f;  // both halves take part
    if (!row_ok) return;
    const int4 sg = sload_int4(&segs[seg]);
    const int4 sq = sload_int4(&seqs[sg.x]);
    const int4 sq2 = sload_int4(&seqs2[sg.x]);
    const int ln = opaque_lane();
    const int mr = row_base + 32 * pr + (ln & 31);
    const int gl = ln >> 5;
    const float inv = (l_tot > 0.0f ? 1.0f / l_tot : 0.0f) * (Q8 ? pv_desc : 1.0f);
    const float lse2 = l_tot > 0.0f ? m_run + __builtin_amdgcn_logf(l_tot) : -INFINITY;
    if (sg.w < 0) {
      T* orow = (T*)p.out + ((long long)sq.z * H + mr) * kDv + 256 * hf + 4 * gl;
      if (p.lse != nullptr && gl == 0 && hf == 0) p.lse[(long long)sq.z * H + mr] = lse2 * kLn2;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          typename Vec<T>::x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = (T)((o[dt][4 * q + e] - bias) * inv);
          *(typename Vec<T>::x4*)(orow + 32 * dt + 8 * q) = v;
        }
      }
    } else {
      // A partial result stays in fp32: the merge rounds the sum to the output
      // type once, so that the split adds no rounding of its own.
      const long long prow = (long long)sq2.x + (long long)sg.w * sq2.y + mr;
      float* orow = (float*)p.part_o + prow * kDv + 256 * hf + 4 * gl;
      if (gl == 0 && hf == 0) p.part_lse[prow] = lse2;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float4 v;
          v.x = (o[dt][4 * q + 0] - bias) * inv;
          v.y = (o[dt][4 * q + 1] - bias) * inv;
          v.z = (o[dt][4 * q + 2] - bias) * inv;
          v.w = (o[dt][4 * q + 3] - bias) * inv;
          *(float4*)(orow + 32 * dt + 8 * q) = v;
        }
      }
    }
  };

  // Moves the compute cursor past its current tile; true when that tile was the
  // last of its segment.
  auto advance_cursor = [&]() -> bool {
    if (cj + kBN < ck1) {
      cj += kBN;
      return false;
    }
    cs = next_valid(cs + 1);
    if (cs < s_end) {
      const int4 sg = sload_int4(&segs[cs]);
      cj = sg.y; ck1 = seg_keys_end(sg);
    }
    return true;
  };

  // ---- prologue: loads of the first two tiles, queries of the first segment ----
  const bool loader = w < 4;
  if (loader) {
    issue(take_tile(), tbuf);
    if (n_total > 1) issue(take_tile(), tbuf + kBufElems);
  }
  load_q(cs);
  reset_state(cs);
  wait_tiles(false);
  lds_barrier();

  // ---- main loop ----
  // Waves 0..3 (group A) and 4..7 (group B) share the SIMDs one to one.  Both
  // run the same two-stage step per tile -- partial scores; barrier; loads of
  // tile t+2 (group A), softmax and PV; barrier -- but B enters one barrier
  // late, so B's partial scores of tile t overlap A's softmax and PV of tile t,
  // and B's softmax and PV of tile t overlap A's partial scores of tile t+1:
  // one wave's MFMA work runs beside the other's VALU work.  Only A loads
  // tiles: its wait before the barrier that ends its step t publishes tile
  // t+1 to both groups before either reads it, and the buffer it refills (that
  // of tile t-1) was last read by B before the barrier that ends A's stage of
  // tile t.  A group that finishes a segment writes its result and loads the
  // next segment's queries inside its own step.
  if (!loader) lds_barrier();
  for (int t = 0; t < n_total; ++t) {
    const T* cur = tbuf + (t % 3) * kBufElems;
    qk_part(cur);
    // Last tile of the segment: its queries are no longer needed; fetch the
    // next segment's now.
    if (cj + kBN >= ck1) {
      const int nxt = next_valid(cs + 1);
      if (nxt < s_end) load_q(nxt);
    }
    // The scalar reads behind tile t+2's loads (its block id; plan records
    // when the cursor enters the next segment) go here, where the wave is about
    // to wait for its partner anyway: scalar loads and LDS reads share one
    // counter, and scalar loads complete out of order, so any LDS wait behind a
    // scalar load in flight waits for that load too.
    TileRef nx{};
    const bool load_next = loader && t + 2 < n_total;
    if (load_next) nx = take_tile();
    lds_barrier();  // exchange slots written; the direct loads in flight stay in flight
    if (load_next) issue(nx, tbuf + ((t + 2) % 3) * kBufElems);
    smpv_part(cur);
    const int done = cs;
    if (advance_cursor()) {
      seg_end(done);
      if (cs < s_end) reset_state(cs);
    }
    if (loader) wait_tiles(t + 2 < n_total);
    asm volatile("s_barrier" ::: "memory");
  }
  if (loader) lds_barrier();
}

// Merge of a sequence's segment results: one wave per (token, head) row,
// 64 lanes x 8 values = 512; L = log2 sum_s 2^{lse_s}, out = sum_s 2^{lse_s - L} o_s.
template <typename T>
__global__ void __launch_bounds__(256) mla_combine_kernel(MlaParams p, const int4* __restrict__ seqs,
                                                         const int4* __restrict__ seqs2) {
  const int b = blockIdx.y;
  const int4 sq = seqs[b];
  const int n = sq.w;
  if (n < 2) return;
  const int4 sq2 = seqs2[b];
  const int rows = sq2.y;
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= rows) return;
  const int l = threadIdx.x & 63;
  const long long base = (long long)sq2.x + m;  // partial row of segment k: base + k * rows
  // One pass, 8 segments at a time (one memory round trip per group), the sum and
  // the accumulator kept relative to the running max mref.
  float mref = -INFINITY;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float tot = 0.0f;
  for (int k0 = 0; k0 < n; k0 += 8) {
    float4 a[8][2];
    float wgt[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (k0 + u < n) {
        const long long row = base + (long long)(k0 + u) * rows;
        wgt[u] = p.part_lse[row];
        const float4* src = (const float4*)((const float*)p.part_o + row * kDv + 8 * l);
        a[u][0] = src[0];
        a[u][1] = src[1];
      } else {
        wgt[u] = -INFINITY;
        a[u][0] = float4{0.0f, 0.0f, 0.0f, 0.0f};
        a[u][1] = float4{0.0f, 0.0f, 0.0f, 0.0f};
      }
    }
    float gm = mref;
#pragma unroll
    for (int u = 0; u < 8; ++u) gm = fmaxf(gm, wgt[u]);
    if (gm == -INFINITY) continue;  // nothing seen so far
    const float sc = fast_exp2(mref - gm);  // 0 while mref = -inf
    tot *= sc;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= sc;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (wgt[u] == -INFINITY) continue;  // an empty part: its values stay out of the sum
      const float wu = fast_exp2(wgt[u] - gm);
      tot += wu;
      acc[0] += wu * a[u][0].x;
      acc[1] += wu * a[u][0].y;
      acc[2] += wu * a[u][0].z;
      acc[3] += wu * a[u][0].w;
      acc[4] += wu * a[u][1].x;
      acc[5] += wu * a[u][1].y;
      acc[6] += wu * a[u][1].z;
      acc[7] += wu * a[u][1].w;
    }
    mref = gm;
  }
  const float inv = tot > 0.0f ? 1.0f / tot : 0.0f;
  typename Vec<T>::x8 v;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (T)(acc[e] * inv);
  const long long orow = (long long)sq.z * p.head_num + m;
  *(typename Vec<T>::x8*)((T*)p.out + orow * kDv + 8 * l) = v;
  if (p.lse != nullptr && l == 0) {
    p.lse[orow] = tot > 0.0f ? (mref + __builtin_amdgcn_logf(tot)) * kLn2 : -INFINITY;
  }
}

template <typename T, bool Q8>
void launch_split(const MlaParams& p, hipStream_t s, hipEvent_t start, hipEvent_t stop) {
  if (p.bs_shift >= (Q8 ? 5 : 3))
    hipExtLaunchKernelGGL((mla_split_kernel<T, true, Q8>), dim3(p.grid), dim3(512), 0, s, start, stop, 0, p,
                          p.block_tables, p.segs, p.piece_seg, p.seqs, p.seqs2);
  else
    hipExtLaunchKernelGGL((mla_split_kernel<T, false, Q8>), dim3(p.grid), dim3(512), 0, s, start, stop, 0, p,
                          p.block_tables, p.segs, p.piece_seg, p.seqs, p.seqs2);
}

template <typename T>
hipError_t launch_typed(const MlaParams& p, hipStream_t s, const LaunchEvents& ev) {
  // (the stop event goes on the combine when there is one)
  hipEvent_t split_stop = p.any_parts ? nullptr : ev.stop;
  if (p.quant)
    launch_split<T, true>(p, s, ev.start, split_stop);
  else
    launch_split<T, false>(p, s, ev.start, split_stop);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !p.any_parts) return e;
  hipExtLaunchKernelGGL(mla_combine_kernel<T>, dim3((p.max_rows + 3) / 4, p.batch), dim3(256), 0, s,
                        nullptr, ev.stop, 0, p, p.seqs, p.seqs2);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mla(const MlaParams& p, int dtype, hipStream_t stream, const LaunchEvents& ev) {
  if (p.grid <= 0) return hipSuccess;
  return dtype == 0 ? launch_typed<_Float16>(p, stream, ev) : launch_typed<__bf16>(p, stream, ev);
}

}  // namespace mpa
