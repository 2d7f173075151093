// C ABI of libmpa (declared in include/mpa.h): argument validation, operation
// objects holding the launch plan, and the launches.
//
// Phase 1 (…GetWorkspaceSize) validates every argument on the host first --
// nothing touches HIP until all checks pass -- then plans the launch on the host
// and keeps the plan in pinned host memory owned by the operation; the
// workspace size it reports covers the plan (and, for MLA, the split-KV
// partials).  Phase 2 copies the plan into the head of the caller's workspace
// with one asynchronous copy on the caller's stream and launches the kernels
// there: the library allocates no device memory.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "../../include/mpa.h"
#include "kernels.h"
#include "planner.h"

namespace {

thread_local std::string g_last_error;

mpaStatus fail(mpaStatus st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

mpaStatus hip_fail(hipError_t e, const char* what) {
  return fail(MPA_ERROR_HIP, "%s failed: %s", what, hipGetErrorString(e));
}

int shift_of(int bs) {
  if (bs > 0 && (bs & (bs - 1)) == 0) {
    int s = 0;
    while ((1 << s) < bs) ++s;
    return s;
  }
  return -1;
}

constexpr float kLog2e = 1.4426950408889634f;
static_assert(MPA_MLA_STATIC_SCRATCH_BYTES == mpa::kStaticScratchBytes, "static scratch size");
// kernel mask type of the chunked local causal mask (selected through the
// chunked entry point; not a PrefixEncoder maskType value)
constexpr int kMaskChunkedCausal = 10;

}  // namespace

struct mpaOperation {
  enum Kind { kPrefill, kMla } kind;
  int dtype = 0;
  // prefill
  mpa::PrefillParams pp{};
  int head_size = 0;
  int mask_type = 0;
  int grid = 0;
  // mla
  mpa::MlaParams mp{};
  uint64_t part_o_off = 0, part_lse_off = 0;
  // launch plan: pinned host copy, copied to workspace[0, plan_bytes) by every
  // execution; blob i sits at plan_offs[i]
  void* hplan = nullptr;
  uint64_t plan_bytes = 0;
  std::vector<size_t> plan_offs;
  uint64_t ws_bytes = 0;       // workspace bytes an execution needs
  uint64_t tile_f32_off = 0;   // prefill: fp32 tile copy at this workspace offset, if any
  bool tile_f32 = false;
  mpa::LaunchEvents events{};  // timing hooks (mpaOperationSetLaunchEvents)

  ~mpaOperation() {
    if (hplan) (void)hipHostFree(hplan);
  }
};

namespace {

constexpr uint64_t kWsAlign = 256;
uint64_t align_up(uint64_t x) { return (x + kWsAlign - 1) & ~(kWsAlign - 1); }

// Byte offsets of plan blobs laid out one after another, each 256-byte aligned;
// returns the total.
uint64_t plan_layout(const std::vector<size_t>& sizes, std::vector<size_t>& offs) {
  uint64_t total = 0;
  offs.clear();
  for (size_t n : sizes) {
    offs.push_back(total);
    total += align_up(n);
  }
  return total;
}

// Workspace bytes of a prefill plan of n_items work items over `batch` sequences
// (the items, then one 16-byte record per sequence).
uint64_t prefill_plan_bytes(size_t n_items, int batch) {
  std::vector<size_t> offs;
  return plan_layout({n_items * sizeof(mpa::PrefillItem), (size_t)batch * 4 * sizeof(int32_t)}, offs);
}

// Copies a host plan (a list of byte blobs) into pinned host memory owned by the
// operation, in the layout of plan_layout.
mpaStatus stage_plan(mpaOperation* op, const std::vector<std::pair<const void*, size_t>>& blobs) {
  std::vector<size_t> sizes;
  for (auto& bl : blobs) sizes.push_back(bl.second);
  op->plan_bytes = plan_layout(sizes, op->plan_offs);
  const size_t alloc = op->plan_bytes ? op->plan_bytes : kWsAlign;
  hipError_t e = hipHostMalloc(&op->hplan, alloc, hipHostMallocDefault);
  if (e != hipSuccess) {
    op->hplan = nullptr;
    return hip_fail(e, "hipHostMalloc (operation plan)");
  }
  std::memset(op->hplan, 0, alloc);
  for (size_t i = 0; i < blobs.size(); ++i)
    if (blobs[i].second) std::memcpy((char*)op->hplan + op->plan_offs[i], blobs[i].first, blobs[i].second);
  return MPA_OK;
}

// Checks the caller's workspace and queues the copy of the plan into its head.
mpaStatus bind_workspace(const mpaOperation* op, void* workspace, uint64_t workspaceSize, hipStream_t stream) {
  if (workspaceSize < op->ws_bytes)
    return fail(MPA_ERROR_WORKSPACE_TOO_SMALL, "workspace of %llu bytes, %llu needed",
                (unsigned long long)workspaceSize, (unsigned long long)op->ws_bytes);
  if (op->ws_bytes && !workspace) return fail(MPA_ERROR_INVALID_ARG, "workspace is NULL");
  if (((uintptr_t)workspace) & (kWsAlign - 1))
    return fail(MPA_ERROR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (op->plan_bytes) {
    hipError_t e = hipMemcpyAsync(workspace, op->hplan, op->plan_bytes, hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync (plan to workspace)");
  }
  return MPA_OK;
}

mpaStatus check_prefill(const void* query, const void* key, const void* value,
                        const int32_t* blockTables, const int32_t* seqLen, const int32_t* kvSeqLen,
                        const float* slopes, int maskType, int32_t headNum, int32_t kvHeadNum,
                        float qkScale, int32_t batch, int32_t headSize, int32_t numBlocks,
                        int32_t blockSize, int32_t maxBlockNum, int dtype, const int64_t* qStartLoc,
                        int64_t nTokens, void* attnOut, uint64_t* workspaceSize, mpaOperation** op) {
  if (!op || !workspaceSize) return fail(MPA_ERROR_INVALID_ARG, "workspaceSize and op must not be NULL");
  if (!query || !key || !value || !blockTables || !attnOut)
    return fail(MPA_ERROR_INVALID_ARG, "query, key, value, blockTables and attnOut are required");
  if (!seqLen || !kvSeqLen) return fail(MPA_ERROR_INVALID_ARG, "seqLen and kvSeqLen (host) are required");
  if (batch < 1) return fail(MPA_ERROR_INVALID_ARG, "batch must be >= 1 (got %d)", batch);
  if (headNum <= 0) return fail(MPA_ERROR_INVALID_ARG, "headNum must be > 0 (got %d)", headNum);
  if (kvHeadNum <= 0 || headNum % kvHeadNum != 0)
    return fail(MPA_ERROR_INVALID_ARG, "kvHeadNum must be > 0 and divide headNum (%d / %d)", headNum,
                kvHeadNum);
  if (dtype != MPA_FP16 && dtype != MPA_BF16)
    return fail(MPA_ERROR_INVALID_ARG, "dtype must be MPA_FP16 or MPA_BF16 (got %d)", dtype);
  if (maskType != MPA_MASK_NONE && maskType != MPA_MASK_ALIBI_COMPRESS &&
      maskType != MPA_MASK_ALIBI_COMPRESS_SQRT && maskType != MPA_MASK_ALIBI_COMPRESS_LEFT_ALIGN &&
      maskType != MPA_MASK_CAUSAL)
    return fail(MPA_ERROR_UNSUPPORTED, "maskType %d is not supported (0, 3, 4, 5, 9)", maskType);
  const bool alibi = maskType == MPA_MASK_ALIBI_COMPRESS || maskType == MPA_MASK_ALIBI_COMPRESS_SQRT ||
                     maskType == MPA_MASK_ALIBI_COMPRESS_LEFT_ALIGN;
  if (alibi && !slopes) return fail(MPA_ERROR_INVALID_ARG, "ALiBi mask types need slopes");
  if (!alibi && slopes) return fail(MPA_ERROR_INVALID_ARG, "slopes must be NULL for maskType %d", maskType);
  if (headSize != 64 && headSize != 128)
    return fail(MPA_ERROR_UNSUPPORTED, "headSize %d is not supported (64 or 128)", headSize);
  if (!(qkScale == qkScale) || qkScale == INFINITY || qkScale == -INFINITY)
    return fail(MPA_ERROR_INVALID_ARG, "qkScale must be finite");
  if (numBlocks < 1 || blockSize < 1 || maxBlockNum < 1)
    return fail(MPA_ERROR_INVALID_ARG, "numBlocks, blockSize and maxBlockNum must be >= 1");
  if (nTokens < 0) return fail(MPA_ERROR_INVALID_ARG, "nTokens must be >= 0");
  int64_t packed = 0;
  for (int b = 0; b < batch; ++b) {
    const int64_t L = seqLen[b], kv = kvSeqLen[b];
    if (L < 0 || kv < L)
      return fail(MPA_ERROR_INVALID_ARG, "sequence %d: need 0 <= seqLen (%lld) <= kvSeqLen (%lld)", b,
                  (long long)L, (long long)kv);
    if ((kv + blockSize - 1) / blockSize > maxBlockNum)
      return fail(MPA_ERROR_INVALID_ARG, "sequence %d: kvSeqLen %lld needs more than maxBlockNum=%d blocks",
                  b, (long long)kv, maxBlockNum);
    const int64_t start = qStartLoc ? qStartLoc[b] : packed;
    if (start < 0 || start + L > nTokens)
      return fail(MPA_ERROR_INVALID_ARG, "sequence %d: rows [%lld, %lld) exceed nTokens=%lld", b,
                  (long long)start, (long long)(start + L), (long long)nTokens);
    packed += L;
  }
  if (qStartLoc) {
    // Row ranges of different sequences must not overlap (outputs would race).
    std::vector<std::pair<int64_t, int64_t>> r;
    for (int b = 0; b < batch; ++b)
      if (seqLen[b] > 0) r.push_back({qStartLoc[b], qStartLoc[b] + seqLen[b]});
    std::sort(r.begin(), r.end());
    for (size_t i = 1; i < r.size(); ++i)
      if (r[i].first < r[i - 1].second)
        return fail(MPA_ERROR_INVALID_ARG, "qStartLoc: row ranges of two sequences overlap");
  }
  return MPA_OK;
}

}  // namespace

extern "C" {

const char* mpaGetErrorString(mpaStatus s) {
  switch (s) {
    case MPA_OK: return "success";
    case MPA_ERROR_INVALID_ARG: return "invalid argument";
    case MPA_ERROR_UNSUPPORTED: return "unsupported argument value";
    case MPA_ERROR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MPA_ERROR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* mpaGetLastErrorMessage(void) { return g_last_error.c_str(); }

mpaStatus mpaOperationSetLaunchEvents(mpaOperation* op, void* startEvent, void* stopEvent) {
  g_last_error.clear();
  if (!op) return fail(MPA_ERROR_INVALID_ARG, "op must not be NULL");
  op->events.start = (hipEvent_t)startEvent;
  op->events.stop = (hipEvent_t)stopEvent;
  return MPA_OK;
}

mpaStatus mpaDestroyOperation(mpaOperation* op) {
  delete op;
  return MPA_OK;
}

namespace {

// Phase 1 of the prefix encoder after validation; chunk > 0 selects the chunked
// local causal mask (kernel mask 10).
mpaStatus make_prefill_op(const void* query, const void* key, const void* value,
                          const int32_t* blockTables, const int32_t* seqLen, const int32_t* kvSeqLen,
                          const float* slopes, int maskType, int32_t chunk, int32_t headNum,
                          int32_t kvHeadNum, float qkScale, int32_t batch, int32_t headSize,
                          int32_t blockSize, int32_t maxBlockNum, int dtype, const int64_t* qStartLoc,
                          void* attnOut, float* lse, uint64_t* workspaceSize, mpaOperation** op,
                          const void* mask = nullptr, int32_t maskStride = 0) {
  const bool causal = maskType != MPA_MASK_NONE;
  mpa::PrefillPlan plan = mpa::plan_prefill(seqLen, kvSeqLen, batch, causal, headNum, kvHeadNum, chunk);
  std::vector<int32_t> seqs(4 * (size_t)batch);
  int64_t packed = 0;
  for (int b = 0; b < batch; ++b) {
    const int64_t start = qStartLoc ? qStartLoc[b] : packed;
    packed += seqLen[b];
    seqs[4 * b + 0] = seqLen[b];
    seqs[4 * b + 1] = kvSeqLen[b];
    seqs[4 * b + 2] = (int32_t)(uint32_t)(start & 0xffffffffll);
    seqs[4 * b + 3] = (int32_t)(start >> 32);
  }
  mpaOperation* o = new (std::nothrow) mpaOperation();
  if (!o) return fail(MPA_ERROR_HIP, "out of host memory");
  mpaStatus st;
  o->kind = mpaOperation::kPrefill;
  o->dtype = dtype;
  o->head_size = headSize;
  o->mask_type = chunk > 0 ? kMaskChunkedCausal : mask ? (maskType | mpa::kMaskTileFlag) : maskType;
  o->grid = (int)plan.items.size();
  st = stage_plan(o, {{plan.items.data(), plan.items.size() * sizeof(mpa::PrefillItem)},
                      {seqs.data(), seqs.size() * sizeof(int32_t)}});
  if (st != MPA_OK) {
    delete o;
    return st;
  }
  o->ws_bytes = o->plan_bytes;
  // (ALiBi tiles on the direct-load kernel: their fp32 copy follows the plan)
  const size_t tile_f32 = mpa::prefill_tile_f32_bytes(headSize, shift_of(blockSize), o->mask_type, maskStride);
  if (tile_f32 > 0) {
    o->tile_f32 = true;
    o->tile_f32_off = o->ws_bytes;
    o->ws_bytes += align_up(tile_f32);
  }
  mpa::PrefillParams& p = o->pp;
  p.q = query;
  p.k = key;
  p.v = value;
  p.out = attnOut;
  p.lse = lse;
  p.block_tables = blockTables;
  p.slopes = slopes;
  p.items = nullptr;  // in the workspace (bound at execution)
  p.seqs = nullptr;
  p.head_num = headNum;
  p.kv_head_num = kvHeadNum;
  p.block_size = blockSize;
  p.bs_shift = shift_of(blockSize);
  p.max_blocks = maxBlockNum;
  p.heads_per_item = plan.heads_per_item;
  p.chunk = chunk;
  p.mask = mask;
  p.mask_stride = maskStride;
  p.scale2 = qkScale * kLog2e;
  *workspaceSize = o->ws_bytes;
  *op = o;
  return MPA_OK;
}

}  // namespace

mpaStatus mpaSelfAttentionPrefixEncoderGetWorkspaceSize(
    const void* query, const void* key, const void* value, const int32_t* blockTables,
    const int32_t* seqLen, const int32_t* kvSeqLen, const float* slopes, int maskType,
    int32_t headNum, int32_t kvHeadNum, float qkScale, int32_t batch, int32_t headSize,
    int32_t numBlocks, int32_t blockSize, int32_t maxBlockNum, int dtype, const int64_t* qStartLoc,
    int64_t nTokens, void* attnOut, float* lse, uint64_t* workspaceSize, mpaOperation** op) {
  g_last_error.clear();
  if (op) *op = nullptr;
  mpaStatus st = check_prefill(query, key, value, blockTables, seqLen, kvSeqLen, slopes, maskType,
                               headNum, kvHeadNum, qkScale, batch, headSize, numBlocks, blockSize,
                               maxBlockNum, dtype, qStartLoc, nTokens, attnOut, workspaceSize, op);
  if (st != MPA_OK) return st;
  return make_prefill_op(query, key, value, blockTables, seqLen, kvSeqLen, slopes, maskType, 0, headNum,
                         kvHeadNum, qkScale, batch, headSize, blockSize, maxBlockNum, dtype, qStartLoc,
                         attnOut, lse, workspaceSize, op);
}

mpaStatus mpaSelfAttentionPrefixEncoderChunkedGetWorkspaceSize(
    const void* query, const void* key, const void* value, const int32_t* blockTables,
    const int32_t* seqLen, const int32_t* kvSeqLen, int32_t attentionChunkSize, int32_t headNum,
    int32_t kvHeadNum, float qkScale, int32_t batch, int32_t headSize, int32_t numBlocks,
    int32_t blockSize, int32_t maxBlockNum, int dtype, const int64_t* qStartLoc, int64_t nTokens,
    void* attnOut, float* lse, uint64_t* workspaceSize, mpaOperation** op) {
  g_last_error.clear();
  if (op) *op = nullptr;
  if (attentionChunkSize < 1)
    return fail(MPA_ERROR_INVALID_ARG, "attentionChunkSize must be >= 1 (got %d)", attentionChunkSize);
  mpaStatus st = check_prefill(query, key, value, blockTables, seqLen, kvSeqLen, nullptr, MPA_MASK_CAUSAL,
                               headNum, kvHeadNum, qkScale, batch, headSize, numBlocks, blockSize,
                               maxBlockNum, dtype, qStartLoc, nTokens, attnOut, workspaceSize, op);
  if (st != MPA_OK) return st;
  return make_prefill_op(query, key, value, blockTables, seqLen, kvSeqLen, nullptr, MPA_MASK_CAUSAL,
                         attentionChunkSize, headNum, kvHeadNum, qkScale, batch, headSize, blockSize,
                         maxBlockNum, dtype, qStartLoc, attnOut, lse, workspaceSize, op);
}

mpaStatus mpaSelfAttentionPrefixEncoderCompressedMaskGetWorkspaceSize(
    const void* query, const void* key, const void* value, const int32_t* blockTables,
    const int32_t* seqLen, const int32_t* kvSeqLen, const void* mask, int32_t maskRows,
    int32_t maskCols, const float* slopes, int maskType, int32_t headNum, int32_t kvHeadNum,
    float qkScale, int32_t batch, int32_t headSize, int32_t numBlocks, int32_t blockSize,
    int32_t maxBlockNum, int dtype, const int64_t* qStartLoc, int64_t nTokens, void* attnOut,
    float* lse, uint64_t* workspaceSize, mpaOperation** op) {
  g_last_error.clear();
  if (op) *op = nullptr;
  if (maskType == MPA_MASK_NONE)
    return fail(MPA_ERROR_UNSUPPORTED, "maskType 0 has no compressed mask (3, 4, 5 or 9)");
  mpaStatus st = check_prefill(query, key, value, blockTables, seqLen, kvSeqLen, slopes, maskType,
                               headNum, kvHeadNum, qkScale, batch, headSize, numBlocks, blockSize,
                               maxBlockNum, dtype, qStartLoc, nTokens, attnOut, workspaceSize, op);
  if (st != MPA_OK) return st;
  if (!mask) return fail(MPA_ERROR_INVALID_ARG, "mask is required");
  if ((reinterpret_cast<uintptr_t>(mask) & 15) != 0)
    return fail(MPA_ERROR_INVALID_ARG, "mask must be 16-byte aligned");
  const int edge = maskType == MPA_MASK_CAUSAL ? mpa::kMaskTile : 2 * mpa::kMaskTile;
  if (maskRows != edge || maskCols != edge)
    return fail(MPA_ERROR_UNSUPPORTED,
                "maskType %d takes a [%d, %d] compressed mask (got [%d, %d]); the [headNum, seqLen, 128] "
                "form is not supported",
                maskType, edge, edge, maskRows, maskCols);
  return make_prefill_op(query, key, value, blockTables, seqLen, kvSeqLen, slopes, maskType, 0, headNum,
                         kvHeadNum, qkScale, batch, headSize, blockSize, maxBlockNum, dtype, qStartLoc,
                         attnOut, lse, workspaceSize, op, mask, edge);
}

mpaStatus mpaSelfAttentionPrefixEncoder(void* workspace, uint64_t workspaceSize, mpaOperation* op,
                                        void* stream) {
  g_last_error.clear();
  if (!op || op->kind != mpaOperation::kPrefill)
    return fail(MPA_ERROR_INVALID_ARG, "op is not a PrefixEncoder operation");
  mpaStatus st = bind_workspace(op, workspace, workspaceSize, (hipStream_t)stream);
  if (st != MPA_OK) return st;
  mpa::PrefillParams p = op->pp;
  p.items = (const int4*)((char*)workspace + op->plan_offs[0]);
  p.seqs = (const int4*)((char*)workspace + op->plan_offs[1]);
  p.mask_f32 = op->tile_f32 ? (float*)((char*)workspace + op->tile_f32_off) : nullptr;
  hipError_t e = mpa::launch_prefill(p, op->dtype, op->head_size, op->mask_type, op->grid,
                                     (hipStream_t)stream, op->events);
  if (e != hipSuccess) return hip_fail(e, "prefill launch");
  return MPA_OK;
}

namespace {

// Phase 1 of MLA after the entry point's own checks; quant selects the int8
// latent cache (qNope / ctKV int8, separate kRope, per-head descales).
mpaStatus make_mla_op(const void* qNope, const void* qRope, const void* ctKV, const void* kRope,
                      const int32_t* blockTables, const int32_t* contextLens, const int32_t* qSeqLen,
                      int32_t headNum, float qkScale, int32_t kvHeadNum, int maskType, int calcType,
                      int cacheMode, int32_t batch, int32_t numBlocks, int32_t blockSize,
                      int32_t maxBlockNum, int dtype, int64_t nTokens, void* attenOut, float* lse,
                      uint64_t* workspaceSize, mpaOperation** op, bool quant, const float* qkDescale,
                      const float* pvDescale) {
  if (!op || !workspaceSize) return fail(MPA_ERROR_INVALID_ARG, "workspaceSize and op must not be NULL");
  if (!qNope || !qRope || !ctKV || !blockTables || !attenOut)
    return fail(MPA_ERROR_INVALID_ARG, "qNope, qRope, ctKV, blockTables and attenOut are required");
  if (!contextLens) return fail(MPA_ERROR_INVALID_ARG, "contextLens (host) is required");
  if (batch < 1) return fail(MPA_ERROR_INVALID_ARG, "batch must be >= 1");
  if (headNum <= 0) return fail(MPA_ERROR_INVALID_ARG, "headNum must be > 0");
  if (kvHeadNum != 1) return fail(MPA_ERROR_UNSUPPORTED, "MLA supports kvHeadNum == 1 only (got %d)", kvHeadNum);
  if (dtype != MPA_FP16 && dtype != MPA_BF16) return fail(MPA_ERROR_INVALID_ARG, "dtype must be fp16 or bf16");
  if (quant && (!qkDescale || !pvDescale))
    return fail(MPA_ERROR_INVALID_ARG, "the int8 cache needs qkDescale and pvDescale");
  if (cacheMode != MPA_MLA_CACHE_KVCACHE && cacheMode != MPA_MLA_CACHE_KROPE_CTKV)
    return fail(MPA_ERROR_UNSUPPORTED,
                "cacheMode %d is not supported (0, 1; the int8 cache has its own entry point, "
                "mpaMLAInt8GetWorkspaceSize, on the ND layout)",
                cacheMode);
  if (cacheMode == MPA_MLA_CACHE_KROPE_CTKV && !kRope)
    return fail(MPA_ERROR_INVALID_ARG, "cacheMode 1 needs kRope");
  if (cacheMode == MPA_MLA_CACHE_KVCACHE && kRope)
    return fail(MPA_ERROR_INVALID_ARG, "cacheMode 0 keeps the rope part inside ctKV: kRope must be NULL");
  if (calcType != MPA_MLA_CALC_UNDEFINED && calcType != MPA_MLA_CALC_SPEC && calcType != MPA_MLA_CALC_PREFILL)
    return fail(MPA_ERROR_UNSUPPORTED, "calcType %d is not supported (0, 1, 3)", calcType);
  const bool many_tokens = calcType == MPA_MLA_CALC_SPEC || calcType == MPA_MLA_CALC_PREFILL;
  if (maskType != MPA_MLA_MASK_UNDEFINED && maskType != MPA_MLA_MASK_SPEC)
    return fail(MPA_ERROR_UNSUPPORTED, "maskType %d is not supported (0, 1)", maskType);
  if (many_tokens && !qSeqLen)
    return fail(MPA_ERROR_INVALID_ARG, "calcType SPEC / PREFILL needs qSeqLen");
  if (!many_tokens && qSeqLen)
    return fail(MPA_ERROR_INVALID_ARG, "qSeqLen must be NULL unless calcType is SPEC or PREFILL");
  if (!(qkScale == qkScale) || qkScale == INFINITY || qkScale == -INFINITY)
    return fail(MPA_ERROR_INVALID_ARG, "qkScale must be finite");
  if (numBlocks < 1 || blockSize < 1 || maxBlockNum < 1)
    return fail(MPA_ERROR_INVALID_ARG, "numBlocks, blockSize and maxBlockNum must be >= 1");
  std::vector<int32_t> qlen(batch, 1);
  int64_t tokens = 0;
  for (int b = 0; b < batch; ++b) {
    if (qSeqLen) qlen[b] = qSeqLen[b];
    tokens += qlen[b] > 0 ? qlen[b] : 0;
    if (contextLens[b] < 1) return fail(MPA_ERROR_INVALID_ARG, "sequence %d: contextLens must be >= 1", b);
    if (qlen[b] < 1 || qlen[b] > contextLens[b])
      return fail(MPA_ERROR_INVALID_ARG, "sequence %d: need 1 <= qSeqLen (%d) <= contextLens (%d)", b,
                  qlen[b], contextLens[b]);
    if ((int64_t)(contextLens[b] + blockSize - 1) / blockSize > maxBlockNum)
      return fail(MPA_ERROR_INVALID_ARG, "sequence %d: contextLens %d needs more than maxBlockNum=%d blocks",
                  b, contextLens[b], maxBlockNum);
  }
  if (nTokens != tokens)
    return fail(MPA_ERROR_INVALID_ARG,
                "nTokens (%lld) must equal the query tokens of the batch (%lld: %s)", (long long)nTokens,
                (long long)tokens, many_tokens ? "the sum of qSeqLen" : "one per sequence");

  int dev = 0, cus = 256;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
  mpa::MlaPlan plan = mpa::plan_mla(contextLens, qlen.data(), batch, headNum, cus);
  if (plan.part_rows >= ((int64_t)1 << 31))
    return fail(MPA_ERROR_UNSUPPORTED, "MLA plan needs %lld partial rows (limit 2^31)", (long long)plan.part_rows);
  std::vector<int32_t> seqs(4 * (size_t)batch), seqs2(4 * (size_t)batch, 0);
  bool any_parts = false;
  for (int b = 0; b < batch; ++b) {
    const mpa::MlaSeq& q = plan.seqs[b];
    seqs[4 * b + 0] = q.ctx;
    seqs[4 * b + 1] = q.q_len;
    seqs[4 * b + 2] = q.tok0;
    seqs[4 * b + 3] = q.n_parts;
    seqs2[4 * b + 0] = q.part_row0;
    seqs2[4 * b + 1] = q.rows;
    any_parts = any_parts || q.n_parts > 1;
  }
  mpaOperation* o = new (std::nothrow) mpaOperation();
  if (!o) return fail(MPA_ERROR_HIP, "out of host memory");
  o->kind = mpaOperation::kMla;
  o->dtype = dtype;
  mpaStatus st = stage_plan(o, {{plan.segs.data(), plan.segs.size() * sizeof(mpa::MlaSegment)},
                                {plan.piece_seg.data(), plan.piece_seg.size() * 4},
                                {seqs.data(), seqs.size() * 4},
                                {seqs2.data(), seqs2.size() * 4}});
  if (st != MPA_OK) {
    delete o;
    return st;
  }
  mpa::MlaParams& p = o->mp;
  p.q_nope = qNope;
  p.q_rope = qRope;
  p.ckv = ctKV;
  p.krope = kRope;
  p.block_tables = blockTables;
  p.segs = nullptr;  // plan and partials live in the workspace (bound at execution)
  p.piece_seg = nullptr;
  p.seqs = nullptr;
  p.seqs2 = nullptr;
  p.out = attenOut;
  p.lse = lse;
  p.head_num = headNum;
  p.block_size = blockSize;
  p.bs_shift = shift_of(blockSize);
  p.max_blocks = maxBlockNum;
  p.ckv_stride = cacheMode == MPA_MLA_CACHE_KVCACHE ? 576 : 512;
  p.spec_mask = maskType == MPA_MLA_MASK_SPEC ? 1 : 0;
  p.grid = plan.grid;
  p.row_groups = plan.row_groups;
  p.pieces_per_xcd = plan.pieces_per_xcd;
  p.batch = batch;
  p.max_rows = plan.max_rows;
  p.any_parts = any_parts ? 1 : 0;
  p.whole = plan.whole ? 1 : 0;
  p.scale2 = qkScale * kLog2e;
  p.quant = quant ? 1 : 0;
  p.qk_descale = qkDescale;
  p.pv_descale = pvDescale;
  // workspace: plan, partial outputs (input type), partial LSEs (fp32)
  o->part_o_off = o->plan_bytes;
  o->part_lse_off = o->part_o_off + align_up((uint64_t)plan.part_rows * 512 * 4);  // fp32 partials
  o->ws_bytes = o->part_lse_off + align_up((uint64_t)plan.part_rows * 4);
  *workspaceSize = o->ws_bytes;
  *op = o;
  return MPA_OK;
}

}  // namespace

mpaStatus mpaMLAGetWorkspaceSize(const void* qNope, const void* qRope, const void* ctKV,
                                 const void* kRope, const int32_t* blockTables,
                                 const int32_t* contextLens, const int32_t* qSeqLen, int32_t headNum,
                                 float qkScale, int32_t kvHeadNum, int maskType, int calcType,
                                 int cacheMode, int32_t batch, int32_t numBlocks, int32_t blockSize,
                                 int32_t maxBlockNum, int dtype, int64_t nTokens, void* attenOut,
                                 float* lse, uint64_t* workspaceSize, mpaOperation** op) {
  g_last_error.clear();
  if (op) *op = nullptr;
  return make_mla_op(qNope, qRope, ctKV, kRope, blockTables, contextLens, qSeqLen, headNum, qkScale,
                     kvHeadNum, maskType, calcType, cacheMode, batch, numBlocks, blockSize, maxBlockNum,
                     dtype, nTokens, attenOut, lse, workspaceSize, op, false, nullptr, nullptr);
}

mpaStatus mpaMLAInt8GetWorkspaceSize(const void* qNope, const void* qRope, const void* ctKV,
                                     const void* kRope, const int32_t* blockTables,
                                     const int32_t* contextLens, const int32_t* qSeqLen,
                                     const float* qkDescale, const float* pvDescale, int32_t headNum,
                                     float qkScale, int32_t kvHeadNum, int maskType, int calcType,
                                     int32_t batch, int32_t numBlocks, int32_t blockSize,
                                     int32_t maxBlockNum, int dtype, int64_t nTokens, void* attenOut,
                                     float* lse, uint64_t* workspaceSize, mpaOperation** op) {
  g_last_error.clear();
  if (op) *op = nullptr;
  if (!kRope) return fail(MPA_ERROR_INVALID_ARG, "the int8 cache keeps the rope part in kRope: it is required");
  return make_mla_op(qNope, qRope, ctKV, kRope, blockTables, contextLens, qSeqLen, headNum, qkScale,
                     kvHeadNum, maskType, calcType, MPA_MLA_CACHE_KROPE_CTKV, batch, numBlocks, blockSize,
                     maxBlockNum, dtype, nTokens, attenOut, lse, workspaceSize, op, true, qkDescale,
                     pvDescale);
}

namespace {

// Execution of an MLA operation with its plan and partials in `workspace`.
mpaStatus run_mla(mpaOperation* op, void* workspace, uint64_t workspaceSize, void* stream) {
  mpaStatus st = bind_workspace(op, workspace, workspaceSize, (hipStream_t)stream);
  if (st != MPA_OK) return st;
  mpa::MlaParams p = op->mp;
  char* ws = (char*)workspace;
  p.segs = (const int4*)(ws + op->plan_offs[0]);
  p.piece_seg = (const int32_t*)(ws + op->plan_offs[1]);
  p.seqs = (const int4*)(ws + op->plan_offs[2]);
  p.seqs2 = (const int4*)(ws + op->plan_offs[3]);
  p.part_o = (char*)workspace + op->part_o_off;
  p.part_lse = (float*)((char*)workspace + op->part_lse_off);
  hipError_t e = mpa::launch_mla(p, op->dtype, (hipStream_t)stream, op->events);
  if (e != hipSuccess) return hip_fail(e, "MLA launch");
  return MPA_OK;
}

}  // namespace

mpaStatus mpaMLA(void* workspace, uint64_t workspaceSize, mpaOperation* op, void* stream) {
  g_last_error.clear();
  if (!op || op->kind != mpaOperation::kMla) return fail(MPA_ERROR_INVALID_ARG, "op is not an MLA operation");
  return run_mla(op, workspace, workspaceSize, stream);
}

mpaStatus mpaMLAStaticScratch(mpaOperation* op, void* stream) {
  g_last_error.clear();
  if (!op || op->kind != mpaOperation::kMla) return fail(MPA_ERROR_INVALID_ARG, "op is not an MLA operation");
  void* scratch = nullptr;
  size_t bytes = 0;
  hipError_t e = mpa::static_scratch(&scratch, &bytes);
  if (e != hipSuccess) return hip_fail(e, "static scratch lookup");
  if (op->ws_bytes > bytes)
    return fail(MPA_ERROR_WORKSPACE_TOO_SMALL,
                "the operation needs %llu bytes of scratch; the static scratch holds %llu (use mpaMLA with a "
                "workspace)",
                (unsigned long long)op->ws_bytes, (unsigned long long)bytes);
  return run_mla(op, scratch, bytes, stream);
}

mpaStatus mpaLseMerge(const void* oParts, const float* lseParts, int32_t nParts, int64_t rows,
                      int32_t headDim, int dtype, void* out, float* lse, void* stream) {
  g_last_error.clear();
  if (nParts < 1) return fail(MPA_ERROR_INVALID_ARG, "nParts must be >= 1 (got %d)", nParts);
  if (rows < 0) return fail(MPA_ERROR_INVALID_ARG, "rows must be >= 0 (got %lld)", (long long)rows);
  if (rows > 0 && (!oParts || !lseParts || !out))
    return fail(MPA_ERROR_INVALID_ARG, "oParts, lseParts and out are required");
  if (headDim < 8 || headDim > 4096 || headDim % 8)
    return fail(MPA_ERROR_INVALID_ARG, "headDim must be a multiple of 8 in [8, 4096] (got %d)", headDim);
  if (dtype != MPA_FP16 && dtype != MPA_BF16) return fail(MPA_ERROR_INVALID_ARG, "dtype must be fp16 or bf16");
  if (rows > ((int64_t)1 << 40) / headDim) return fail(MPA_ERROR_INVALID_ARG, "rows * headDim too large");
  const uintptr_t mis = (uintptr_t)oParts | (uintptr_t)out;
  if (mis & 15) return fail(MPA_ERROR_INVALID_ARG, "oParts and out must be 16-byte aligned");
  mpa::LseMergeParams p;
  p.o_parts = oParts;
  p.lse_parts = lseParts;
  p.out = out;
  p.lse_out = lse;
  p.rows = rows;
  p.n_parts = nParts;
  p.head_dim = headDim;
  if (rows == 0) return MPA_OK;
  hipError_t e = mpa::launch_lse_merge(p, dtype, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "LSE merge launch");
  return MPA_OK;
}

mpaStatus mpaPrefixEncoderPlanInspect(const int32_t* seqLen, const int32_t* kvSeqLen, int32_t batch,
                                      int maskType, int32_t headNum, int32_t kvHeadNum,
                                      int32_t headSize, int32_t* items, int64_t capacity,
                                      int64_t* nItems, int32_t* rowsPerItem, int32_t* keysPerTile,
                                      int32_t* headsPerItem, uint64_t* workspaceSize) {
  g_last_error.clear();
  (void)headSize;
  if (!seqLen || !kvSeqLen || batch < 1 || headNum <= 0 || kvHeadNum <= 0 || headNum % kvHeadNum)
    return fail(MPA_ERROR_INVALID_ARG, "invalid lengths or head counts");
  mpa::PrefillPlan plan =
      mpa::plan_prefill(seqLen, kvSeqLen, batch, maskType != MPA_MASK_NONE, headNum, kvHeadNum);
  if (nItems) *nItems = (int64_t)plan.items.size();
  if (rowsPerItem) *rowsPerItem = plan.rows_per_item;
  if (keysPerTile) *keysPerTile = mpa::kKeysPerTile;
  if (headsPerItem) *headsPerItem = plan.heads_per_item;
  if (workspaceSize) *workspaceSize = prefill_plan_bytes(plan.items.size(), batch);
  if (!items || capacity < (int64_t)plan.items.size())
    return fail(MPA_ERROR_INVALID_ARG, "capacity %lld < %zu items", (long long)capacity, plan.items.size());
  std::memcpy(items, plan.items.data(), plan.items.size() * sizeof(mpa::PrefillItem));
  return MPA_OK;
}

mpaStatus mpaMLAPlanInspect(const int32_t* contextLens, const int32_t* qSeqLen, int32_t batch,
                            int32_t headNum, int calcType, int32_t* splits, int64_t capacity,
                            int64_t* nSplits) {
  g_last_error.clear();
  if (!contextLens || batch < 1 || headNum <= 0) return fail(MPA_ERROR_INVALID_ARG, "invalid arguments");
  std::vector<int32_t> qlen(batch, 1);
  if (calcType == MPA_MLA_CALC_SPEC || calcType == MPA_MLA_CALC_PREFILL) {
    if (!qSeqLen) return fail(MPA_ERROR_INVALID_ARG, "calcType SPEC / PREFILL needs qSeqLen");
    for (int b = 0; b < batch; ++b) qlen[b] = qSeqLen[b];
  }
  mpa::MlaPlan plan = mpa::plan_mla(contextLens, qlen.data(), batch, headNum, 256);
  if (nSplits) *nSplits = (int64_t)plan.segs.size();
  if (!splits || capacity < (int64_t)plan.segs.size())
    return fail(MPA_ERROR_INVALID_ARG, "capacity %lld < %zu segments", (long long)capacity, plan.segs.size());
  std::vector<int32_t> seen(batch, 0);
  for (size_t pc = 0; pc + 1 < plan.piece_seg.size(); ++pc) {
    for (int32_t i = plan.piece_seg[pc]; i < plan.piece_seg[pc + 1]; ++i) {
      const mpa::MlaSegment& s = plan.segs[i];
      splits[5 * i + 0] = s.b;
      splits[5 * i + 1] = s.k0;
      splits[5 * i + 2] = s.k1;
      splits[5 * i + 3] = seen[s.b]++;
      splits[5 * i + 4] = (int32_t)pc;
    }
  }
  return MPA_OK;
}

}  // extern "C"
