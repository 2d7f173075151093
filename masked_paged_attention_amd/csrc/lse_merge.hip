// Merge of attention partials over disjoint key ranges by their log-sum-exp
// (the Ascend ATB page "MLA", parameter table: the lse output that the RING
// calcType requires; the same merge as the split-KV combine).  For row r and
// parts s = 0 .. S-1:
//   LSE_r = ln sum_s exp(lse[s][r]),  out[r] = sum_s exp(lse[s][r] - LSE_r) * o[s][r].
// A part with lse = -inf (no key in its range) weighs nothing and its values are
// not read into the sum (they may be undefined); a row whose parts are all -inf
// gets out = 0 and LSE = -inf.
//
// Streaming, HBM-bound: one thread per 16-byte chunk (8 elements) of one row;
// the threads of a row read the same LSE values (cached) and accumulate their
// chunk of every part in fp32, weighted relative to a running max.

#include "device.h"
#include "kernels.h"

namespace mpa {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <typename T>
__global__ void __launch_bounds__(256) lse_merge_kernel(LseMergeParams p) {
  using V8 = typename Vec<T>::x8;
  constexpr int kGroup = 8;  // parts whose LSEs and chunks are loaded together
  const long long chunks_per_row = p.head_dim / 8;
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= p.rows * chunks_per_row) return;
  const long long r = idx / chunks_per_row;
  const int c = (int)(idx - r * chunks_per_row);
  const float* lse = p.lse_parts + r;
  const T* o = (const T*)p.o_parts + r * p.head_dim + 8 * c;
  const long long part_stride = p.rows * p.head_dim;
  // One pass, a group of parts at a time (one memory round trip per group): the
  // running sum and accumulator are kept relative to the running max m.
  float m = -INFINITY;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float tot = 0.0f;
  for (int s0 = 0; s0 < p.n_parts; s0 += kGroup) {
    V8 v[kGroup];
    float lk[kGroup];
#pragma unroll
    for (int k = 0; k < kGroup; ++k) {
      const bool ok = s0 + k < p.n_parts;
      v[k] = ok ? *(const V8*)(o + (long long)(s0 + k) * part_stride) : V8{};
      lk[k] = ok ? lse[(long long)(s0 + k) * p.rows] : -INFINITY;
    }
    float gm = m;
#pragma unroll
    for (int k = 0; k < kGroup; ++k) gm = fmaxf(gm, lk[k]);
    if (gm == -INFINITY) continue;  // nothing seen so far
    const float sc = __builtin_amdgcn_exp2f((m - gm) * kLog2e);  // 0 when m = -inf
    tot *= sc;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= sc;
#pragma unroll
    for (int k = 0; k < kGroup; ++k) {
      // a part with LSE = -inf is left out entirely: its values may be anything
      // (NaN included) and must not reach the sum
      if (lk[k] == -INFINITY) continue;
      const float w = __builtin_amdgcn_exp2f((lk[k] - gm) * kLog2e);
      tot += w;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = __builtin_fmaf(w, (float)v[k][e], acc[e]);
    }
    m = gm;
  }
  const float inv = tot > 0.0f ? 1.0f / tot : 0.0f;
  V8 out;
#pragma unroll
  for (int e = 0; e < 8; ++e) out[e] = (T)(acc[e] * inv);
  *(V8*)((T*)p.out + r * p.head_dim + 8 * c) = out;
  if (c == 0 && p.lse_out != nullptr)
    p.lse_out[r] = tot > 0.0f ? m + __builtin_amdgcn_logf(tot) * kLn2 : -INFINITY;
}

}  // namespace

hipError_t launch_lse_merge(const LseMergeParams& p, int dtype, hipStream_t stream) {
  const long long total = p.rows * (p.head_dim / 8);
  if (total == 0) return hipSuccess;
  const long long blocks = (total + 255) / 256;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  if (dtype == 0) {
    hipLaunchKernelGGL(lse_merge_kernel<_Float16>, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  } else {
    hipLaunchKernelGGL(lse_merge_kernel<__bf16>, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace mpa
