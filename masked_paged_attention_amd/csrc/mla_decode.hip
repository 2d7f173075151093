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
constexpr int kRows = 64;       // query rows per workgroup (2 wave pairs x 32)
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.0f;  // log2 units of growth tolerated before rescaling

// LDS layout of one key tile (32 latent rows): the 512-wide part as 32 rows of
// 1024 bytes and the 64-wide rope part as 32 rows of 128 bytes, both filled by
// direct global->LDS loads (one wave instruction = 1024 contiguous LDS bytes).
// 16-byte chunks are XOR-swizzled inside each row so that the QK operand reads
// (16 rows, one chunk) and the V^T transpose reads (4 rows, 4 chunks) both hit
// 16 distinct bank groups.
__device__ __forceinline__ int lat_swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int rope_swz(int r) { return (r >> 1) & 7; }

template <typename T>
__global__ void __launch_bounds__(256, 1) mla_split_kernel(MlaParams p,
                                                         const int32_t* __restrict__ block_tables) {
  using V8 = typename Vec<T>::x8;
  constexpr int NCH = kDq / 16 / 2;      // 18 contraction chunks per wave of a pair
  constexpr int NDT = kDv / 32 / 2;      // 8 O^T tiles per wave of a pair

  // Three tile buffers, each one LDS object holding the latent rows followed by
  // the rope rows: while tile t is computed, the loads of tiles t+1 and t+2 are
  // in flight.
  constexpr int kBufElems = kBN * kDv + kBN * 64;
  __shared__ __attribute__((aligned(1024))) T tb0[kBufElems];
  __shared__ __attribute__((aligned(1024))) T tb1[kBufElems];
  __shared__ __attribute__((aligned(1024))) T tb2[kBufElems];
  // Partial S^T of each wave, register-major ([4 float4][64 lanes]) so that
  // consecutive lanes touch consecutive 16-byte slots.
  __shared__ __attribute__((aligned(16))) float4 xch[4][4 * 64];

  // 1-D grid.  Workgroups go round-robin to the 8 XCDs by id; ids are laid out
  // so that the row groups of one split are dispatched back to back on the same
  // XCD: they stream the same keys at the same time and share them through L2.
  const int rg = p.row_groups;
  const int lin = blockIdx.x;
  const int blk8 = lin / (8 * rg);
  const int within = lin - blk8 * 8 * rg;
  const int split_id = 8 * blk8 + (within & 7);
  const int row_group = within >> 3;
  const int4 sp = p.splits[split_id];
  const int b = sp.x;
  if (b < 0) return;
  const int k0 = sp.y, k1 = sp.z, part_row = sp.w;
  const int4 sq = p.seqs[b];
  const int ctx = sq.x, q_len = sq.y, tok0 = sq.z;
  const int H = p.head_num;
  const int M = q_len * H;                  // rows of this sequence
  const int row_base = row_group * kRows;  // first row of this workgroup
  if (row_base >= M) return;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (uniform)
  const int pr = w >> 1;   // pair: 32 query rows
  const int hf = w & 1;    // half: contraction dims [288hf, +288) and output dims [256hf, +256)
  const int l = tid & 63;
  const int g = l >> 5;
  const int lq = l & 31;

  const int m = row_base + 32 * pr + lq;  // this lane's query row
  const bool row_ok = m < M;
  const int t_loc = row_ok ? m / H : 0;
  const int hh = row_ok ? m % H : 0;
  const bool w_active = row_base + 32 * pr < M;
  // Keys this lane's row may see: [k0, lim).
  const int lim_full = p.spec_mask ? (ctx - q_len + t_loc + 1) : ctx;
  const int lim = min(k1, lim_full);
  // Keys every row of the pair sees (tiles below need no predicate).
  int w_lim_lo = k1;
  if (p.spec_mask) w_lim_lo = min(k1, ctx - q_len + (row_base + 32 * pr) / H + 1);

  // Q^T operand: row m, dims 16(18hf + c) + 8g .. +8 (qNope below 512, then qRope).
  V8 qreg[NCH];
  {
    const long long qrow = (long long)(tok0 + t_loc) * H + hh;
    const T* qn = (const T*)p.q_nope + qrow * kDv + 8 * g;
    const T* qr = (const T*)p.q_rope + qrow * 64 + 8 * g;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int cc = NCH * hf + c;
      if (row_ok) {
        qreg[c] = (cc < 32) ? *(const V8*)(qn + 16 * cc) : *(const V8*)(qr + 16 * (cc - 32));
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qreg[c][e] = (T)0.0f;
      }
    }
  }

  // The block table is read-only for the kernel: wave-uniform lookups become
  // scalar loads, which do not wait for the direct loads in flight.
  const int32_t* __restrict__ btab = block_tables + (long long)b * p.max_blocks;
  // Splits start at multiples of the 32-key tile, so with a power-of-two block
  // size >= 32 a tile lies inside one cache block: one wave-uniform block id per
  // tile, fetched two tiles ahead.  Otherwise each row looks its block up.
  const bool one_block = p.bs_shift >= 5;
  // Issues the direct loads of the tile starting at key j0 into (lat, rope).
  // Rows at or beyond k1 repeat row k1 - 1 (finite data; masked later).
  auto issue_tile = [&](int j0, int blk, T* lat, T* rope) __attribute__((always_inline)) {
    const T* rope_base = p.krope != nullptr ? (const T*)p.krope : (const T*)p.ckv + kDv;
    const int rope_stride = p.krope != nullptr ? 64 : p.ckv_stride;
    const int rr = 8 * w + (l >> 3);  // rope row of this lane
    const int rc = (l & 7) ^ rope_swz(rr);
    if (one_block) {
      const long long base = (long long)blk * p.block_size + (j0 & (p.block_size - 1));
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int r = 8 * w + k;
        const long long rowi = base + min(r, k1 - 1 - j0);
        const T* src = (const T*)p.ckv + rowi * p.ckv_stride + 8 * (l ^ lat_swz(r));
        dma16(src, lat + r * kDv);
      }
      const long long rowi = base + min(rr, k1 - 1 - j0);
      dma16(rope_base + rowi * rope_stride + 8 * rc, rope + 64 * 8 * w);
    } else {
      // Block lookups first (scalar for the latent rows), then the loads.
      long long rows[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int j = min(j0 + 8 * w + k, k1 - 1);
        const int bi = j / p.block_size;
        rows[k] = (long long)btab[bi] * p.block_size + (j - bi * p.block_size);
      }
      const int jr = min(j0 + rr, k1 - 1);
      const int bir = jr / p.block_size;
      const long long rowr = (long long)btab[bir] * p.block_size + (jr - bir * p.block_size);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int r = 8 * w + k;
        const T* src = (const T*)p.ckv + rows[k] * p.ckv_stride + 8 * (l ^ lat_swz(r));
        dma16(src, lat + r * kDv);
      }
      dma16(rope_base + rowr * rope_stride + 8 * rc, rope + 64 * 8 * w);
    }
  };
  auto tile_block = [&](int j0) -> int { return one_block ? btab[j0 >> p.bs_shift] : 0; };

  f32x16 o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) o[dt] = f32x16{};
  float m_run = -INFINITY;
  float l_run = 0.0f;
  const float scale2 = p.scale2;
  const int n_tiles = (k1 - k0 + kBN - 1) / kBN;
  float4* my_x = &xch[w][l];
  const float4* other_x = &xch[w ^ 1][l];
  const int tr_row = 4 * g + ((l & 15) >> 2);
  const int tr_col = 256 * hf + 16 * ((l >> 4) & 1) + 4 * (l & 3);

  auto compute = [&](int t, const T* lat, const T* rope) __attribute__((always_inline)) {
    const int j0 = k0 + t * kBN;
    // Partial S^T (32 keys x 32 rows) over this wave's half of the 576 dims.
    f32x16 s0 = f32x16{}, s1 = f32x16{};
    if (w_active) {
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const int q16 = 2 * (NCH * hf + c) + g;  // 16-byte chunk of the 576-wide row
        const V8 a = q16 < 64 ? *(const V8*)&lat[lq * kDv + 8 * (q16 ^ lat_swz(lq))]
                              : *(const V8*)&rope[lq * 64 + 8 * ((q16 - 64) ^ rope_swz(lq))];
        if (c & 1) s1 = mfma32(a, qreg[c], s1); else s0 = mfma32(a, qreg[c], s0);
      }
      s0 += s1;
#pragma unroll
      for (int r = 0; r < 16; r += 4)
        my_x[16 * r] = make_float4(s0[r], s0[r + 1], s0[r + 2], s0[r + 3]);
    }
    lds_barrier();  // the next tile's direct loads stay in flight
    if (w_active) {
#pragma unroll
      for (int r = 0; r < 16; r += 4) {
        const float4 v = other_x[16 * r];
        s0[r] += v.x; s0[r + 1] += v.y; s0[r + 2] += v.z; s0[r + 3] += v.w;
      }
      const bool partial = j0 + kBN > w_lim_lo;
      const int vlim = lim - j0 - 4 * g;  // key j0 + 4g + C visible <=> C < vlim
      float sc[16];
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int C = 8 * (r >> 2) + (r & 3);
        float x = s0[r] * scale2;
        if (partial) x = (C < vlim) ? x : -INFINITY;
        sc[r] = x;
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
        if (t > 0) {
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) o[dt] *= alpha;
        }
        m_run = m_new;
      }
      const float m_use = (m_run == -INFINITY) ? 0.0f : m_run;
      float psum = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sc[r] = fast_exp2(sc[r] - m_use);
        psum += sc[r];
      }
      l_run += psum;
      const V8 p0 = pack8<T>(&sc[0]);
      const V8 p1 = pack8<T>(&sc[8]);
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const int d = 32 * dt + tr_col;       // first of the 4 values this lane supplies
          const int r0 = 16 * kc + tr_row;
          const int r1 = r0 + 8;
          const T* src0 = &lat[r0 * kDv + 8 * ((d >> 3) ^ lat_swz(r0)) + (d & 7)];
          const T* src1 = &lat[r1 * kDv + 8 * ((d >> 3) ^ lat_swz(r1)) + (d & 7)];
          const s16x4 lo = lds_read_tr16(src0);
          const s16x4 hi = lds_read_tr16(src1);
          const s16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          o[dt] = mfma32(__builtin_bit_cast(V8, both), kc == 0 ? p0 : p1, o[dt]);
        }
      }
    }
  };

  // Each wave issues kLoadsPerTile direct loads per tile (8 latent rows + one
  // rope block); "s_waitcnt vmcnt(kLoadsPerTile)" therefore waits for every
  // tile but the most recently issued one.
  auto end_of_tile = [&](bool newer_in_flight) {
    // s_waitcnt through the builtin (encoding vmcnt | expcnt 7 << 4 | lgkmcnt
    // 15 << 8: wait on vector memory only) so the compiler's own wait tracking
    // sees it; the barrier itself is a memory clobber.
    if (newer_in_flight) __builtin_amdgcn_s_waitcnt(0xF70 | 9);
    else __builtin_amdgcn_s_waitcnt(0xF70);
    asm volatile("s_barrier" ::: "memory");
  };
  auto lat_buf = [&](auto I) -> T* {
    if constexpr (decltype(I)::value == 0) return tb0;
    else if constexpr (decltype(I)::value == 1) return tb1;
    else return tb2;
  };
  auto rope_buf = [&](auto I) -> T* { return lat_buf(I) + kBN * kDv; };
  std::integral_constant<int, 0> B0;
  std::integral_constant<int, 1> B1;
  std::integral_constant<int, 2> B2;

  issue_tile(k0, tile_block(k0), tb0, tb0 + kBN * kDv);
  if (n_tiles > 1) issue_tile(k0 + kBN, tile_block(k0 + kBN), tb1, tb1 + kBN * kDv);
  int blk_ahead = n_tiles > 2 ? tile_block(k0 + 2 * kBN) : 0;
  // Everything issued so far -- the query operands included -- completes here,
  // so no load from before the loop is still pending inside it.
  end_of_tile(false);
  // One step: start the loads of tile t+2 into the buffer tile t-1 used, compute
  // tile t, wait until tile t+1 has landed.  Unrolled by three so that every
  // buffer is a distinct LDS object and no load forces a wait on another
  // buffer's reads.
  auto step = [&](int t, auto cur, auto ahead) __attribute__((always_inline)) {
    if (t + 2 < n_tiles) {
      issue_tile(k0 + (t + 2) * kBN, blk_ahead, lat_buf(ahead), rope_buf(ahead));
      if (t + 3 < n_tiles) blk_ahead = tile_block(k0 + (t + 3) * kBN);
    }
    compute(t, lat_buf(cur), rope_buf(cur));
    end_of_tile(t + 2 < n_tiles);
  };
  for (int t = 0; t < n_tiles; t += 3) {
    step(t, B0, B2);
    if (t + 1 < n_tiles) step(t + 1, B1, B0);
    if (t + 2 < n_tiles) step(t + 2, B2, B1);
  }

  if (!w_active) return;
  const float l_tot = sum_with_other_half(l_run);
  if (!row_ok) return;
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  T* orow = (T*)p.part_o + (long long)(part_row + m) * kDv + 256 * hf + 4 * g;
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
  if (g == 0 && hf == 0) {
    p.part_lse[part_row + m] =
        l_tot > 0.0f ? m_run + __builtin_amdgcn_logf(l_tot) : -INFINITY;
  }
}

// One wave per (token, head): 64 lanes x 8 values = 512.
template <typename T>
__global__ void __launch_bounds__(256) mla_combine_kernel(MlaParams p) {
  const int wv = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int l = threadIdx.x & 63;
  const int H = p.head_num;
  if (wv >= p.tokens * H) return;
  const int tok = wv / H;
  const int h = wv % H;
  // Sequence of this token: binary search over the token starts.
  int lo = 0, hi = p.batch;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (p.seqs[mid].z <= tok) lo = mid; else hi = mid;
  }
  const int b = lo;
  const int4 sq = p.seqs[b];
  const int4 sq2 = p.seqs2[b];
  const int n = sq.w;
  const int m = (tok - sq.z) * H + h;
  // Pass 1: the largest partial LSE (lanes fetch different splits in parallel).
  float mx = -INFINITY;
  for (int k = l; k < n; k += 64) {
    const int s = p.seq_splits[sq2.x + k];
    mx = fmaxf(mx, p.part_lse[p.splits[s].w + m]);
  }
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  const float mref = (mx == -INFINITY) ? 0.0f : mx;
  // Pass 2: weighted sum, four splits' loads in flight at a time.
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float tot = 0.0f;
  for (int k0 = 0; k0 < n; k0 += 4) {
    typename Vec<T>::x8 a[4];
    float wgt[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (k0 + u < n) {
        const int s = p.seq_splits[sq2.x + k0 + u];
        const int row = p.splits[s].w + m;
        wgt[u] = fast_exp2(p.part_lse[row] - mref);
        a[u] = *(const typename Vec<T>::x8*)((const T*)p.part_o + (long long)row * kDv + 8 * l);
      } else {
        wgt[u] = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) a[u][e] = (T)0.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      tot += wgt[u];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += wgt[u] * (float)a[u][e];
    }
  }
  const float inv = tot > 0.0f ? 1.0f / tot : 0.0f;
  typename Vec<T>::x8 v;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (T)(acc[e] * inv);
  *(typename Vec<T>::x8*)((T*)p.out + (long long)wv * kDv + 8 * l) = v;
  if (p.lse != nullptr && l == 0) {
    p.lse[wv] = tot > 0.0f ? (mref + __builtin_amdgcn_logf(tot)) * kLn2 : -INFINITY;
  }
}

template <typename T>
hipError_t launch_typed(const MlaParams& p, hipStream_t s) {
  hipLaunchKernelGGL(mla_split_kernel<T>, dim3(p.n_splits * p.row_groups), dim3(256), 0, s, p,
                     p.block_tables);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int rows = p.tokens * p.head_num;
  hipLaunchKernelGGL(mla_combine_kernel<T>, dim3((rows + 3) / 4), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mla(const MlaParams& p, int dtype, hipStream_t stream) {
  if (p.n_splits <= 0 || p.tokens <= 0) return hipSuccess;
  return dtype == 0 ? launch_typed<_Float16>(p, stream) : launch_typed<__bf16>(p, stream);
}

}  // namespace mpa
