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
// (fp32) and log2-domain LSE to the workspace.
//
// Kernel 2 (combine): for each (token, head), LSE-weighted merge of the partials
// of its sequence: L = log2 sum_s 2^{lse_s}, out = sum_s 2^{lse_s - L} o_s --
// the merge by LSE that the MLA page's lse output exists for.

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

template <typename T>
__global__ void __launch_bounds__(256, 1) mla_split_kernel(MlaParams p) {
  using V8 = typename Vec<T>::x8;
  constexpr int KSTR = kDq + 8;          // LDS row stride (elements)
  constexpr int NCH = kDq / 16 / 2;      // 18 contraction chunks per wave of a pair
  constexpr int NDT = kDv / 32 / 2;      // 8 O^T tiles per wave of a pair
  constexpr int CPR = kDq / 8;           // 72 16-byte chunks per latent row
  constexpr int CHUNKS = kBN * CPR;      // 2304 chunks per tile
  constexpr int CPT = (CHUNKS + 255) / 256;

  __shared__ __attribute__((aligned(16))) T k_lds[2][kBN * KSTR];
  __shared__ __attribute__((aligned(16))) float xch[4][64 * 16];  // partial S^T of each wave

  const int4 sp = p.splits[blockIdx.x];
  const int b = sp.x;
  if (b < 0) return;
  const int k0 = sp.y, k1 = sp.z, part_row = sp.w;
  const int4 sq = p.seqs[b];
  const int ctx = sq.x, q_len = sq.y, tok0 = sq.z;
  const int H = p.head_num;
  const int M = q_len * H;                  // rows of this sequence
  const int row_base = blockIdx.y * kRows;  // first row of this workgroup
  if (row_base >= M) return;

  const int tid = threadIdx.x;
  const int w = tid >> 6;
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

  const int32_t* btab = p.block_tables + (long long)b * p.max_blocks;
  uint4 kr[CPT];
  auto load_tile = [&](int j0) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int x = tid + 256 * i;
      const int row = x / CPR;
      const int c = x % CPR;
      const int j = j0 + row;
      if (x < CHUNKS && j < k1) {
        int bi, slot;
        if (p.bs_shift >= 0) {
          bi = j >> p.bs_shift;
          slot = j & (p.block_size - 1);
        } else {
          bi = j / p.block_size;
          slot = j - bi * p.block_size;
        }
        const long long rowi = (long long)btab[bi] * p.block_size + slot;
        const T* src;
        if (p.krope == nullptr || c < 64) {
          src = (const T*)p.ckv + rowi * p.ckv_stride + 8 * c;
        } else {
          src = (const T*)p.krope + rowi * 64 + 8 * (c - 64);
        }
        kr[i] = *(const uint4*)src;
      } else {
        kr[i] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int x = tid + 256 * i;
      if (x < CHUNKS) {
        const int row = x / CPR;
        const int c = x % CPR;
        *(uint4*)&k_lds[buf][row * KSTR + 8 * c] = kr[i];
      }
    }
  };

  f32x16 o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) o[dt] = f32x16{};
  float m_run = -INFINITY;
  float l_run = 0.0f;
  const float scale2 = p.scale2;
  const int n_tiles = (k1 - k0 + kBN - 1) / kBN;
  float* my_x = &xch[w][l * 16];
  const float* other_x = &xch[w ^ 1][l * 16];

  load_tile(k0);
  store_tile(0);
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    const int j0 = k0 + t * kBN;
    if (t + 1 < n_tiles) load_tile(j0 + kBN);

    // Partial S^T (32 keys x 32 rows) over this wave's half of the 576 dims.
    f32x16 s0 = f32x16{}, s1 = f32x16{};
    if (w_active) {
#pragma unroll
      for (int c = 0; c < NCH; c += 2) {
        const int cc = NCH * hf + c;
        const V8 a0 = *(const V8*)&k_lds[buf][lq * KSTR + 16 * cc + 8 * g];
        const V8 a1 = *(const V8*)&k_lds[buf][lq * KSTR + 16 * (cc + 1) + 8 * g];
        s0 = mfma32(a0, qreg[c], s0);
        s1 = mfma32(a1, qreg[c + 1], s1);
      }
      s0 += s1;
#pragma unroll
      for (int r = 0; r < 16; r += 4)
        *(float4*)&my_x[r] = make_float4(s0[r], s0[r + 1], s0[r + 2], s0[r + 3]);
    }
    __syncthreads();
    if (w_active) {
#pragma unroll
      for (int r = 0; r < 16; r += 4) {
        const float4 v = *(const float4*)&other_x[r];
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
      const int tr_row = 4 * g + ((l & 15) >> 2);
      const int tr_col = 256 * hf + 16 * ((l >> 4) & 1) + 4 * (l & 3);
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const T* src = &k_lds[buf][(16 * kc + tr_row) * KSTR + 32 * dt + tr_col];
          const s16x4 lo = lds_read_tr16(src);
          const s16x4 hi = lds_read_tr16(src + 8 * KSTR);
          const s16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          o[dt] = mfma32(__builtin_bit_cast(V8, both), kc == 0 ? p0 : p1, o[dt]);
        }
      }
    }

    if (t + 1 < n_tiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  if (!w_active) return;
  const float l_tot = sum_with_other_half(l_run);
  if (!row_ok) return;
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  float* orow = p.part_o + (long long)(part_row + m) * kDv + 256 * hf + 4 * g;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      float4 v = make_float4(o[dt][4 * rg] * inv, o[dt][4 * rg + 1] * inv,
                             o[dt][4 * rg + 2] * inv, o[dt][4 * rg + 3] * inv);
      *(float4*)(orow + 32 * dt + 8 * rg) = v;
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
  float mx = -INFINITY;
  for (int k = 0; k < n; ++k) {
    const int s = p.seq_splits[sq2.x + k];
    mx = fmaxf(mx, p.part_lse[p.splits[s].w + m]);
  }
  const float mref = (mx == -INFINITY) ? 0.0f : mx;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float tot = 0.0f;
  for (int k = 0; k < n; ++k) {
    const int s = p.seq_splits[sq2.x + k];
    const int row = p.splits[s].w + m;
    const float wgt = fast_exp2(p.part_lse[row] - mref);
    tot += wgt;
    const float4* src = (const float4*)(p.part_o + (long long)row * kDv + 8 * l);
    const float4 a = src[0], c = src[1];
    acc[0] += wgt * a.x; acc[1] += wgt * a.y; acc[2] += wgt * a.z; acc[3] += wgt * a.w;
    acc[4] += wgt * c.x; acc[5] += wgt * c.y; acc[6] += wgt * c.z; acc[7] += wgt * c.w;
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
  hipLaunchKernelGGL(mla_split_kernel<T>, dim3(p.n_splits, p.row_groups), dim3(256), 0, s, p);
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
