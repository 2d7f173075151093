// Split-KV decode of multi-head latent attention (MLA) for gfx950.
//
// What it computes (Ascend ATB page "MLA", parameter table): query token t,
// head h: q = [qNope 512 | qRope 64]; key j = [ctKV_j 512 | kRope_j 64] of the
// single latent KV head; value j = ctKV_j (512);
//   s_j = qkScale * q.k_j over keys j < contextLens (maskType SPEC: j <=
//   contextLens - q_len + t), out = softmax(s) V, lse = ln sum_j exp(s_j).
//
// Kernel 1 (split): one workgroup per (key split, group of 64 query rows).
// The rows of a sequence are its (token, head) pairs; the 4 waves form two
// pairs, each pair owning 32 rows: one wave of a pair contracts the first 288
// of the 576 query/key dims and accumulates output dims 0..255, the other the
// rest; the two partial score tiles are summed through LDS.  Per tile of 32 keys the workgroup gathers the 576-wide latent
// rows through blockTables into LDS (16-byte coalesced loads, double
// buffered); each wave forms S^T = K Q^T with the 32x32x16 MFMA (Q^T stays in
// registers, 36 contraction chunks), runs the online softmax in the log2 domain
// and accumulates O^T += V^T P^T, reading V^T -- the first 512 columns of the
// same LDS rows -- with the LDS transpose read: every latent row is loaded from
// HBM once and serves as key and as value.  The running output is rescaled only
// when a row's max grows by more than 2^8 (exact: the final normalisation uses
// the same reference max).  It writes the split's normalised partial output
// (rounded to the input type) and log2-domain LSE (fp32) to the workspace.
//
// Kernel 2 (combine): for each (token, head), LSE-weighted merge of the partials
// of its sequence: L = log2 sum_s 2^{lse_s}, out = sum_s 2^{lse_s - L} o_s --
// the merge by LSE that the MLA page's lse output exists for.

#include <type_traits>

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

// LDS layout of one key tile: key k sits in row slot lat_slot(k); a slot holds
// the 576 values of the key (latent 512, then rope 64) and 8 values of padding,
// 1168 bytes = 73 16-byte chunks.  An odd chunk count puts slot s at a distinct
// bank group for every s mod 16 in a given column; the slot order (a 4x4
// transpose inside each 16-key block) puts the 4 keys of a transpose read at
// slots 4 apart.  So the QK operand reads (16 keys, one 16-byte column) and the
// V^T transpose reads (4 keys x 64 bytes per half wave) both hit 16 distinct
// bank groups, and every address is one per-lane base plus an immediate offset.
// A key's latent part is written by one direct load (64 lanes x 16 contiguous
// bytes), its rope part by one with 8 lanes active.
constexpr int kLatRow = kDq + 8;  // elements per key slot
__device__ __forceinline__ int lat_slot(int k) {
  return (k & ~15) | ((k & 15) >> 2) | ((k & 3) << 2);
}
// The rope part of the 128 query rows: rows of 64 values + 8 of padding (9
// chunks, odd), read 32 rows at a time as the B operand.
constexpr int kQRopeRow = 72;

template <typename T, bool ONE_BLOCK>
__global__ void __launch_bounds__(512, 1)
    mla_split_kernel(MlaParams p, const int32_t* __restrict__ block_tables,
                     const int4* __restrict__ segs, const int32_t* __restrict__ piece_seg,
                     const int4* __restrict__ seqs, const int4* __restrict__ seqs2) {
  using V8 = typename Vec<T>::x8;
  constexpr int NCH = kDv / 16 / 2;  // 16 register-resident contraction chunks per wave of a pair
  constexpr int NDT = kDv / 32 / 2;  // 8 O^T tiles per wave of a pair

  // Three key-tile buffers (latent rows, then rope rows), the pairs' partial
  // S^T exchange, and the rope part of the 128 query rows.
  constexpr int kBufElems = kBN * kLatRow;
  __shared__ __attribute__((aligned(1024))) T tbuf[3 * kBufElems];
  __shared__ __attribute__((aligned(16))) float4 xch[kWaves][4 * 64];
  __shared__ __attribute__((aligned(16))) T qrope[kRows * kQRopeRow];

  // Workgroup -> (piece, row group): workgroups go round-robin to the 8 XCDs by
  // id; XCD x handles pieces [x * ppx, (x + 1) * ppx), the row groups of one
  // piece side by side.
  const int slot = blockIdx.x >> 3;
  const int piece = (blockIdx.x & 7) * p.pieces_per_xcd + slot / p.row_groups;
  const int rg = slot % p.row_groups;
  const int s_beg = piece_seg[piece];
  const int s_end = piece_seg[piece + 1];
  const int row_base = rg * kRows;  // first row (token-major (token, head) index) of this workgroup
  // Segments whose sequence has rows in this row group.
  // Plan records are read with scalar loads (see sload_int4).
  auto next_valid = [&](int s) -> int {
    while (s < s_end && sload_int4(&seqs2[sload_int4(&segs[s]).x]).y <= row_base) ++s;
    return s;
  };
  int n_total = 0;
  for (int s = next_valid(s_beg); s < s_end; s = next_valid(s + 1)) {
    const int4 sg = sload_int4(&segs[s]);
    n_total += (sg.z - sg.y + kBN - 1) / kBN;
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
  const int m = row_base + 32 * pr + lq;  // this lane's row within its sequence

  // ---- loader cursor (wave-uniform): the tile whose loads are issued next ----
  int ls = next_valid(s_beg);
  int lb, lj, lk1;
  {
    const int4 sg = sload_int4(&segs[ls]);
    lb = sg.x; lj = sg.y; lk1 = sg.z;
  }
  // With a power-of-two block size >= 32 every tile lies inside one cache block
  // (tiles start at multiples of 32): one wave-uniform block id per tile.
  // Otherwise each row looks its block up.
  auto tile_block = [&]() -> int {
    return ONE_BLOCK ? block_tables[(long long)lb * p.max_blocks + (lj >> p.bs_shift)] : 0;
  };
  auto ld_advance = [&]() {
    lj += kBN;
    if (lj >= lk1) {
      ls = next_valid(ls + 1);
      if (ls < s_end) {
        const int4 sg = sload_int4(&segs[ls]);
        lb = sg.x; lj = sg.y; lk1 = sg.z;
      }
    }
  };
  // Row r of the cache: latent at lat_row(r), rope at rope_row(r).
  const bool split_rope = p.krope != nullptr;
  auto lat_row = [&](long long r) -> const T* { return (const T*)p.ckv + r * p.ckv_stride; };
  auto rope_row = [&](long long r) -> const T* {
    return split_rope ? (const T*)p.krope + r * 64 : (const T*)p.ckv + r * p.ckv_stride + kDv;
  };
  const unsigned lane16 = 16u * (unsigned)l;
  // Direct loads of the loader's tile into buffer `buf`: wave w fills the slots
  // of keys 4w .. 4w+3 (latent: 64 lanes; rope: lanes 0..7).  Keys at or beyond
  // the segment end repeat its last key (finite data, masked later).
  auto issue_tile = [&](int blk, T* buf) __attribute__((always_inline)) {
    const int last = lk1 - 1 - lj;
    long long rows[4];
    if constexpr (ONE_BLOCK) {
      const long long base = (long long)blk * p.block_size + (lj & (p.block_size - 1));
#pragma unroll
      for (int k = 0; k < 4; ++k) rows[k] = base + min(4 * w + k, last);
    } else {
      const int32_t* bt = block_tables + (long long)lb * p.max_blocks;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int j = lj + min(4 * w + k, last);
        const int bi = j / p.block_size;
        rows[k] = (long long)bt[bi] * p.block_size + (j - bi * p.block_size);
      }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      T* slot = buf + lat_slot(4 * w + k) * kLatRow;
      dma16s(lat_row(rows[k]), lane16, slot);
      if (l < 8) dma16s(rope_row(rows[k]), lane16, slot + kDv);
    }
  };
  // Every wave issues 8 direct loads per tile, so "s_waitcnt vmcnt(8)" waits
  // for every tile but the most recently issued one.  (Encoding: vmcnt |
  // expcnt 7 << 4 | lgkmcnt 15 << 8, i.e. wait on vector memory only; through
  // the builtin so that the compiler's own wait tracking sees it.)
  auto end_of_tile = [&](bool newer_in_flight) __attribute__((always_inline)) {
    if (newer_in_flight) __builtin_amdgcn_s_waitcnt(0xF70 | 8);
    else __builtin_amdgcn_s_waitcnt(0xF70);
    asm volatile("s_barrier" ::: "memory");
  };
  // ---- per-segment state ----
  V8 qreg[NCH];
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

  // Loads the queries of the compute cursor's segment: the nope part of this
  // lane's row into registers, the rope part of all 128 rows into LDS.
  auto seg_begin = [&]() __attribute__((always_inline)) {
    const int4 sg = sload_int4(&segs[cs]);
    const int4 sq = sload_int4(&seqs[sg.x]);
    const int4 sq2 = sload_int4(&seqs2[sg.x]);
    const int ctx = sq.x, q_len = sq.y, tok0 = sq.z, rows = sq2.y;
    row_ok = m < rows;
    w_active = row_base + 32 * pr < rows;
    const int t_loc = row_ok ? m / H : 0;
    lim = min(sg.z, p.spec_mask ? (ctx - q_len + t_loc + 1) : ctx);
    w_lim_lo = sg.z;
    if (p.spec_mask) w_lim_lo = min(sg.z, ctx - q_len + (row_base + 32 * pr) / H + 1);
    const T* qn = (const T*)p.q_nope + ((long long)tok0 * H + (row_ok ? m : 0)) * kDv + 8 * g;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      if (row_ok) {
        qreg[c] = *(const V8*)(qn + 16 * (NCH * hf + c));
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qreg[c][e] = (T)0.0f;
      }
    }
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      const int r = (tid >> 3) + 64 * pass;
      const int ch = tid & 7;
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
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[dt] = f32x16{};
    m_run = -INFINITY;
    l_run = 0.0f;
    // The query loads complete here (behind the loads already in flight), so
    // no later wait of the compiler's covers the direct loads issued next.
    __builtin_amdgcn_s_waitcnt(0xF70);
    lds_barrier();
  };

  auto compute = [&](const T* lat) __attribute__((always_inline)) {
    const int j0 = cj;
    f32x16 s0 = f32x16{};
    if (w_active) {
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const int q16 = 2 * (NCH * hf + c) + g;  // 16-byte chunk of the latent row
        const V8 a = *(const V8*)&lat[lat_slot(lq) * kLatRow + 8 * q16];
        s0 = mfma32(a, qreg[c], s0);
      }
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int r16 = 2 * (2 * hf + c) + g;   // 16-byte chunk of the 64-wide rope part
        const V8 a = *(const V8*)&lat[lat_slot(lq) * kLatRow + kDv + 8 * r16];
        const V8 bq = *(const V8*)&qrope[(32 * pr + lq) * kQRopeRow + 8 * r16];
        s0 = mfma32(a, bq, s0);
      }
#pragma unroll
      for (int r = 0; r < 16; r += 4)
        my_x[16 * r] = make_float4(s0[r], s0[r + 1], s0[r + 2], s0[r + 3]);
    }
    lds_barrier();  // the direct loads in flight stay in flight
    if (w_active) {
#pragma unroll
      for (int r = 0; r < 16; r += 4) {
        const float4 v = other_x[16 * r];
        s0[r] += v.x; s0[r + 1] += v.y; s0[r + 2] += v.z; s0[r + 3] += v.w;
      }
      const bool partial = j0 + kBN > w_lim_lo;
      const int vlim = lim - j0 - 4 * g;  // key j0 + 4g + C visible <=> C < vlim
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int C = 8 * (r >> 2) + (r & 3);
        float x = s0[r] * scale2;
        if (partial) x = (C < vlim) ? x : -INFINITY;
        s0[r] = x;
        mx = fmaxf(mx, x);
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
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[dt] *= alpha;
        m_run = m_new;
      }
      const float m_use = (m_run == -INFINITY) ? 0.0f : m_run;
      float psum = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s0[r] = fast_exp2(s0[r] - m_use);
        psum += s0[r];
      }
      l_run += psum;
      V8 p0, p1;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p0[e] = (T)s0[e];
        p1[e] = (T)s0[8 + e];
      }
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          // Keys 16kc + tr_row and the same + 8 (slot + 2), dims d .. d+3.
          const int d = 32 * dt + tr_col;
          const T* src0 = &lat[lat_slot(16 * kc + tr_row) * kLatRow + d];
          const T* src1 = src0 + 2 * kLatRow;
          const s16x4 lo = lds_read_tr16(src0);
          const s16x4 hi = lds_read_tr16(src1);
          const s16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          o[dt] = mfma32(__builtin_bit_cast(V8, both), kc == 0 ? p0 : p1, o[dt]);
        }
      }
    }
  };

  // Writes the segment's result: the final output (and natural-log LSE) when the
  // segment covers the whole sequence, else the normalised partial output and
  // its log2-domain LSE.
  auto seg_end = [&]() __attribute__((always_inline)) {
    if (!w_active) return;
    const float l_tot = sum_with_other_half(l_run);
    if (!row_ok) return;
    const int4 sg = sload_int4(&segs[cs]);
    const int4 sq = sload_int4(&seqs[sg.x]);
    const int4 sq2 = sload_int4(&seqs2[sg.x]);
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    const float lse2 = l_tot > 0.0f ? m_run + __builtin_amdgcn_logf(l_tot) : -INFINITY;
    T* orow;
    if (sg.w < 0) {
      orow = (T*)p.out + ((long long)sq.z * H + m) * kDv;
      if (p.lse != nullptr && g == 0 && hf == 0) p.lse[(long long)sq.z * H + m] = lse2 * kLn2;
    } else {
      const long long prow = (long long)sq2.x + (long long)sg.w * sq2.y + m;
      orow = (T*)p.part_o + prow * kDv;
      if (g == 0 && hf == 0) p.part_lse[prow] = lse2;
    }
    orow += 256 * hf + 4 * g;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        typename Vec<T>::x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (T)(o[dt][4 * q + e] * inv);
        *(typename Vec<T>::x4*)(orow + 32 * dt + 8 * q) = v;
      }
    }
  };

  // ---- prologue: loads of the first two tiles ----
  issue_tile(tile_block(), tbuf);
  ld_advance();
  if (n_total > 1) {
    issue_tile(tile_block(), tbuf + kBufElems);
    ld_advance();
  }
  int blk_next = (n_total > 2) ? tile_block() : 0;
  end_of_tile(false);
  bool first = true;  // the compute cursor sits on the first tile of a segment

  // ---- main loop: tile t computes from buffer t % 3 while tiles t+1 and t+2 load ----
  for (int t = 0; t < n_total; ++t) {
    if (first) seg_begin();
    const int buf = t % 3;
    if (t + 2 < n_total) {
      issue_tile(blk_next, tbuf + ((t + 2) % 3) * kBufElems);
      ld_advance();
      if (t + 3 < n_total) blk_next = tile_block();
    }
    compute(tbuf + buf * kBufElems);
    first = cj + kBN >= ck1;
    if (first) {
      seg_end();
      cs = next_valid(cs + 1);
      if (cs < s_end) {
        const int4 sg = sload_int4(&segs[cs]);
        cj = sg.y; ck1 = sg.z;
      }
    } else {
      cj += kBN;
    }
    end_of_tile(t + 2 < n_total);
  }
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
  float mx = -INFINITY;
  for (int k = l; k < n; k += 64) mx = fmaxf(mx, p.part_lse[base + (long long)k * rows]);
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  const float mref = (mx == -INFINITY) ? 0.0f : mx;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float tot = 0.0f;
  for (int k0 = 0; k0 < n; k0 += 8) {
    typename Vec<T>::x8 a[8];
    float wgt[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (k0 + u < n) {
        const long long row = base + (long long)(k0 + u) * rows;
        wgt[u] = p.part_lse[row];
        a[u] = *(const typename Vec<T>::x8*)((const T*)p.part_o + row * kDv + 8 * l);
      } else {
        wgt[u] = -INFINITY;
#pragma unroll
        for (int e = 0; e < 8; ++e) a[u][e] = (T)0.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float wu = fast_exp2(wgt[u] - mref);
      tot += wu;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += wu * (float)a[u][e];
    }
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

template <typename T>
hipError_t launch_typed(const MlaParams& p, hipStream_t s) {
  if (p.bs_shift >= 5)
    hipLaunchKernelGGL((mla_split_kernel<T, true>), dim3(p.grid), dim3(512), 0, s, p, p.block_tables,
                       p.segs, p.piece_seg, p.seqs, p.seqs2);
  else
    hipLaunchKernelGGL((mla_split_kernel<T, false>), dim3(p.grid), dim3(512), 0, s, p, p.block_tables,
                       p.segs, p.piece_seg, p.seqs, p.seqs2);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !p.any_parts) return e;
  hipLaunchKernelGGL(mla_combine_kernel<T>, dim3((p.max_rows + 3) / 4, p.batch), dim3(256), 0, s, p,
                     p.seqs, p.seqs2);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mla(const MlaParams& p, int dtype, hipStream_t stream) {
  if (p.grid <= 0) return hipSuccess;
  return dtype == 0 ? launch_typed<_Float16>(p, stream) : launch_typed<__bf16>(p, stream);
}

}  // namespace mpa
