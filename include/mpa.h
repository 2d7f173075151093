/*
 * mpa.h -- C ABI of libmpa: masked attention over a paged KV cache on AMD
 * Instinct MI355X (gfx950).
 *
 * Two operations, each called in two phases like the Ascend ATB C interface
 * (pages "PrefixEncoder" and "MLA", section 定义 / definition): a first call
 * validates the arguments, plans the launch on the host and returns an opaque
 * operation plus the workspace size it needs; a second call runs it
 * asynchronously on a HIP stream.
 *
 *   mpaSelfAttentionPrefixEncoderGetWorkspaceSize / mpaSelfAttentionPrefixEncoder
 *       fused masked self-attention of new query rows over a paged cache that
 *       already holds their prefix (ATB page "PrefixEncoder", parameter table);
 *       causal, right-aligned / sqrt / left-aligned ALiBi and padding masks are
 *       generated inside the kernel (ATB page "压缩mask", sections 开启方式 and
 *       约束说明); a separate phase-1 call reads an explicit compressed mask
 *       tile instead.
 *   mpaMLAGetWorkspaceSize / mpaMLA
 *       split-KV decode of multi-head latent attention: 576-wide query/key
 *       (qNope 512 + qRope 64), 512-wide latent value, one KV head (ATB page
 *       "MLA", parameter table).
 *
 * Conventions shared by every call:
 *   - "dev" pointers are HIP device pointers, "HOST" pointers are ordinary host
 *     memory read during the call that receives them (the host arrays are copied
 *     into the operation, so the caller may free them afterwards);
 *   - the caller owns every tensor and the workspace, and the library allocates
 *     no device memory: it owns only the mpaOperation (a host object and its
 *     launch plan, kept in pinned host memory), released by mpaDestroyOperation.
 *     Every execution first copies the plan into the head of the workspace
 *     (one asynchronous host-to-device copy on the execution's stream), then
 *     launches the kernels, which read the plan there;
 *   - all shape and argument checks happen in the first phase, on the host,
 *     before any HIP call; on error *op is set to NULL and a status != MPA_OK is
 *     returned; mpaGetLastErrorMessage() then describes the failure (per thread);
 *   - block ids inside blockTables live on the device and are NOT checked: every
 *     entry a sequence uses must name a block < numBlocks;
 *   - the execute phase is asynchronous on the given stream (a hipStream_t, NULL
 *     = the null stream); every pointer captured in the operation and the
 *     workspace must stay valid until the stream passes the call.  An operation
 *     may be executed any number of times; executions on different streams must
 *     not share a workspace concurrently.
 */
#ifndef MPA_H_
#define MPA_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t mpaStatus;
#define MPA_OK 0
#define MPA_ERROR_INVALID_ARG 1       /* a null required pointer, a bad size or shape */
#define MPA_ERROR_UNSUPPORTED 2       /* a valid value this build does not implement */
#define MPA_ERROR_WORKSPACE_TOO_SMALL 3
#define MPA_ERROR_HIP 4               /* a HIP runtime call failed (message has details) */

typedef struct mpaOperation mpaOperation; /* opaque, library-owned */

/* Element type of query/key/value and of the attention output. */
#define MPA_FP16 0
#define MPA_BF16 1

/* PrefixEncoder maskType.  3, 4, 5 and 9 carry the numbers of the ATB
 * PrefixEncoder parameter table (row maskType); 0 is this library's: no causal
 * rule, keys limited only by kvSeqLen (padding mask).  The ATB compressed norm
 * mask used for RoPE models (MASK_TYPE_NORM_COMPRESS, number not given on the
 * pages) has causal semantics: pass MPA_MASK_CAUSAL. */
#define MPA_MASK_NONE 0
#define MPA_MASK_ALIBI_COMPRESS 3            /* bias slope_h * (j - a_i), causal */
#define MPA_MASK_ALIBI_COMPRESS_SQRT 4       /* bias -slope_h * sqrt(a_i - j), causal */
#define MPA_MASK_ALIBI_COMPRESS_LEFT_ALIGN 5 /* bias slope_h * j, causal */
#define MPA_MASK_CAUSAL 9                    /* generated inside the operator */

/*
 * PrefixEncoder, phase 1.  Sequence b has seqLen[b] new query rows and
 * kvSeqLen[b] >= seqLen[b] keys in the paged cache; the first kvSeqLen[b] -
 * seqLen[b] keys are its cached prefix and its query row i sits at absolute
 * position a_i = kvSeqLen[b] - seqLen[b] + i (ATB page "PrefixEncoder",
 * parameter table, rows seqLen and kvSeqLen).  For every query head h and
 * row i it computes
 *     s_j  = qkScale * (q_i . k_j) + bias(i, j)     over the visible keys j
 *     out_i = sum_j softmax(s)_j v_j,   lse_i = ln sum_j exp(s_j)
 * with key j of sequence b at key[blockTables[b][j / blockSize]][j % blockSize]
 * [h / (headNum / kvHeadNum)] (GQA, contiguous head groups).  Visible: j <
 * kvSeqLen[b] and, for maskType 3/4/5/9, j <= a_i.
 *
 *   query        dev  [nTokens, headNum, headSize]  dtype; sequence b's rows
 *                     start at row qStartLoc[b] (or packed, see qStartLoc)
 *   key, value   dev  [numBlocks, blockSize, kvHeadNum, headSize] dtype
 *   blockTables  dev  [batch, maxBlockNum] int32; entries at and beyond
 *                     ceil(kvSeqLen[b] / blockSize) are never read
 *   seqLen       HOST [batch] int32, >= 0
 *   kvSeqLen     HOST [batch] int32, >= seqLen[b], ceil(kvSeqLen/blockSize) <= maxBlockNum
 *   slopes       dev  [headNum] fp32 ALiBi coefficients; required for maskType
 *                     3/4/5, must be NULL otherwise
 *   maskType     one of MPA_MASK_*
 *   headNum      query heads (> 0); kvHeadNum KV heads, headNum % kvHeadNum == 0
 *   qkScale      scale applied to q.k before the bias
 *   batch        number of sequences (>= 1)
 *   headSize     64 or 128
 *   numBlocks, blockSize, maxBlockNum   paged cache geometry (blockSize >= 1)
 *   dtype        MPA_FP16 or MPA_BF16
 *   qStartLoc    HOST [batch] int64 first query row of each sequence, or NULL
 *                for the packed layout (prefix sums of seqLen).  With a padded
 *                layout (qStartLoc[b] = b * Lpad) the rows between sequences
 *                are neither read nor written.
 *   nTokens      rows of query and attnOut (>= every qStartLoc[b] + seqLen[b])
 *   attnOut      dev  [nTokens, headNum, headSize] dtype (output)
 *   lse          dev  [nTokens, headNum] fp32 natural-log LSE (output), or NULL
 *   workspaceSize, op  outputs: bytes of device workspace phase 2 needs (the
 *                launch plan: 16 bytes per workgroup plus 16 per sequence, each
 *                part rounded up to 256 bytes) and the new operation
 */
mpaStatus mpaSelfAttentionPrefixEncoderGetWorkspaceSize(
    const void *query, const void *key, const void *value, const int32_t *blockTables,
    const int32_t *seqLen, const int32_t *kvSeqLen, const float *slopes, int maskType,
    int32_t headNum, int32_t kvHeadNum, float qkScale, int32_t batch, int32_t headSize,
    int32_t numBlocks, int32_t blockSize, int32_t maxBlockNum, int dtype,
    const int64_t *qStartLoc, int64_t nTokens, void *attnOut, float *lse,
    uint64_t *workspaceSize, mpaOperation **op);

/*
 * PrefixEncoder, phase 1, with a chunked local causal mask (a library extension:
 * the LLaMA 4 chunked attention of the page "终极指南：LLaMA模型的Transformer注意力掩码与
 * 填充处理技术解析", section "本地注意力掩码生成").  With C = attentionChunkSize, row i
 * of sequence b (absolute position a_i as above) sees the keys j with
 *     j <= a_i  and  floor(j / C) == floor(a_i / C)
 * (and j < kvSeqLen[b]); no bias.  The other arguments, outputs and errors are
 * those of mpaSelfAttentionPrefixEncoderGetWorkspaceSize with maskType causal and
 * no slopes; attentionChunkSize < 1 is MPA_ERROR_INVALID_ARG.  Phase 2 is
 * mpaSelfAttentionPrefixEncoder.
 */
mpaStatus mpaSelfAttentionPrefixEncoderChunkedGetWorkspaceSize(
    const void *query, const void *key, const void *value, const int32_t *blockTables,
    const int32_t *seqLen, const int32_t *kvSeqLen, int32_t attentionChunkSize, int32_t headNum,
    int32_t kvHeadNum, float qkScale, int32_t batch, int32_t headSize, int32_t numBlocks,
    int32_t blockSize, int32_t maxBlockNum, int dtype, const int64_t *qStartLoc, int64_t nTokens,
    void *attnOut, float *lse, uint64_t *workspaceSize, mpaOperation **op);

/*
 * PrefixEncoder, phase 1, with an explicit compressed mask tensor (ATB page
 * "压缩mask", section 约束说明, and ATB page "PrefixEncoder", parameter table,
 * row mask): the bias and the visibility inside the diagonal block come from
 * `mask` instead of being generated.  Same computation, arguments, outputs and
 * errors as mpaSelfAttentionPrefixEncoderGetWorkspaceSize, plus:
 *
 *   mask         dev  dtype, row-major [maskRows, maskCols], 16-byte aligned;
 *                     read only.  maskType 9 (the compressed norm mask of RoPE
 *                     models, which has causal semantics): [128, 128].
 *                     maskType 3, 4, 5: [256, 256].  The [headNum, seqLen, 128]
 *                     ALiBi form is MPA_ERROR_UNSUPPORTED, and so is maskType 0.
 *
 * Expansion, on a grid of 128 absolute positions (query a_i: block bq = a_i /
 * 128, row r = a_i % 128; key j: block bk, column c = j % 128; dk = bq - bk):
 * keys of a later block (dk < 0) and keys j >= kvSeqLen[b] are hidden, an
 * entry of -inf hides its key, and otherwise
 *   maskType 9:  bias 0 for dk >= 1, mask[r][c] for dk = 0;
 *   maskType 3:  y = mask[r][c] for dk = 0, mask[128 + r][c] - 128 (dk - 1)
 *                for dk >= 1; bias = slopes[h] * y;
 *   maskType 4:  the same y, a distance (entries <= 0 or -inf); bias =
 *                -slopes[h] * sqrt(-y);
 *   maskType 5:  y = mask[r][c] (dk = 0) or mask[128 + r][c] (dk >= 1), plus
 *                the key block origin 128 bk; bias = slopes[h] * y.
 * With the tiles the page describes, as read here (norm: 0 on and below the
 * diagonal, -inf above; right-aligned: col - row on and below the diagonal of
 * the 256 x 256 tile, -inf above; left-aligned: col there) the result equals
 * the generated mask of the same maskType.  A row whose tile hides every key
 * gets out = 0 and lse = -inf.  Phase 2 is mpaSelfAttentionPrefixEncoder; the operation keeps the
 * mask pointer, which must stay valid until the launches that use it end.
 * For maskType 3, 4 and 5 with headSize 128 and a power-of-two blockSize >= 16,
 * the workspace also holds an fp32 copy of the tile (256 KB after the plan),
 * which each execution fills from `mask` in a launch of its own before the
 * attention launch; the tile's contents are read at execution, not here.
 */
mpaStatus mpaSelfAttentionPrefixEncoderCompressedMaskGetWorkspaceSize(
    const void *query, const void *key, const void *value, const int32_t *blockTables,
    const int32_t *seqLen, const int32_t *kvSeqLen, const void *mask, int32_t maskRows,
    int32_t maskCols, const float *slopes, int maskType, int32_t headNum, int32_t kvHeadNum,
    float qkScale, int32_t batch, int32_t headSize, int32_t numBlocks, int32_t blockSize,
    int32_t maxBlockNum, int dtype, const int64_t *qStartLoc, int64_t nTokens, void *attnOut,
    float *lse, uint64_t *workspaceSize, mpaOperation **op);

/* PrefixEncoder, phase 2: copy of the plan into `workspace` (dev, >= the size
 * phase 1 returned, 256-byte aligned) and one kernel launch (two for the
 * compressed ALiBi tiles that get an fp32 copy), all on `stream`
 * (hipStream_t).  Errors: MPA_ERROR_INVALID_ARG for a NULL or misaligned
 * workspace or another kind of operation, MPA_ERROR_WORKSPACE_TOO_SMALL,
 * MPA_ERROR_HIP if the copy or the launch fails. */
mpaStatus mpaSelfAttentionPrefixEncoder(void *workspace, uint64_t workspaceSize,
                                        mpaOperation *op, void *stream);

/* MLA maskType / calcType / cacheMode (ATB page "MLA", parameter table).  Only
 * CALC_TYPE_UNDEFINED = 0 and KVCACHE = 0 carry numbers on the page; the others
 * follow the order the page lists them in. */
#define MPA_MLA_MASK_UNDEFINED 0   /* all-zero mask: every token sees keys < contextLens */
#define MPA_MLA_MASK_SPEC 1        /* token t of q_len sees keys j <= contextLens - q_len + t */
#define MPA_MLA_CALC_UNDEFINED 0   /* one query token per sequence */
#define MPA_MLA_CALC_SPEC 1        /* qSeqLen tokens per sequence (speculative decode) */
#define MPA_MLA_CALC_PREFILL 3     /* qSeqLen tokens per sequence (a whole new prompt); same masks */
#define MPA_MLA_CACHE_KVCACHE 0    /* one concatenated cache ctKV [NB, BS, 1, 576], kRope NULL */
#define MPA_MLA_CACHE_KROPE_CTKV 1 /* separate ctKV [NB, BS, 1, 512] and kRope [NB, BS, 1, 64] */

/*
 * MLA, phase 1.  Query token t of sequence b (tokens are batch-major: the
 * qSeqLen[b] tokens of sequence b follow those of b - 1) and head h attend
 * over keys j < contextLens[b] of the one latent KV head:
 *     s_j = qkScale * ([qNope|qRope]_{t,h} . [ctKV|kRope]_j),
 *     attenOut_{t,h} = sum_j softmax(s)_j ctKV_j[0:512],  lse = ln sum_j exp(s_j)
 * with the visibility of maskType.  The keys of a sequence are split over
 * several workgroups; their partial results are merged by their LSE.
 *
 *   qNope      dev [T, headNum, 512] dtype     qRope  dev [T, headNum, 64] dtype
 *   ctKV       dev [numBlocks, blockSize, 1, 512] (cacheMode 1) or
 *                  [numBlocks, blockSize, 1, 576] (cacheMode 0) dtype
 *   kRope      dev [numBlocks, blockSize, 1, 64] dtype (cacheMode 1), NULL for 0
 *   blockTables dev [batch, maxBlockNum] int32
 *   contextLens HOST [batch] int32 >= 1 (keys of each sequence, speculative
 *               tokens included)
 *   qSeqLen    HOST [batch] int32 in [1, contextLens[b]]; required iff calcType
 *              is MPA_MLA_CALC_SPEC or MPA_MLA_CALC_PREFILL, else NULL (one token
 *              per sequence)
 *   headNum    query heads (1..128 per token; > 0); kvHeadNum must be 1
 *   qkScale, maskType, calcType, cacheMode  see above (cacheMode 2 and 3, the
 *              page's int8 and fp16/bf16 NZ layouts, and calcType RING return
 *              MPA_ERROR_UNSUPPORTED; the int8 cache is served on the ND layout by
 *              mpaMLAInt8GetWorkspaceSize, RING's single-GPU part by mpaLseMerge)
 *   batch, numBlocks, blockSize, maxBlockNum, dtype   as for PrefixEncoder
 *   nTokens    T, the query tokens: batch for calcType UNDEFINED, the sum of
 *              qSeqLen otherwise (anything else is MPA_ERROR_INVALID_ARG)
 *   attenOut   dev [T, headNum, 512] dtype (output)
 *   lse        dev [T, headNum] fp32 natural-log LSE (output), or NULL
 *   workspaceSize, op  outputs: device workspace bytes (the launch plan, then
 *              the split-KV partial results, kept in fp32 with their fp32 LSE
 *              so that the merge rounds to dtype once) and the new operation
 */
mpaStatus mpaMLAGetWorkspaceSize(
    const void *qNope, const void *qRope, const void *ctKV, const void *kRope,
    const int32_t *blockTables, const int32_t *contextLens, const int32_t *qSeqLen,
    int32_t headNum, float qkScale, int32_t kvHeadNum, int maskType, int calcType,
    int cacheMode, int32_t batch, int32_t numBlocks, int32_t blockSize, int32_t maxBlockNum,
    int dtype, int64_t nTokens, void *attenOut, float *lse, uint64_t *workspaceSize,
    mpaOperation **op);

/*
 * MLA, phase 1, over an int8 latent cache (ATB page "MLA", parameter table:
 * qNope and ctKV int8, qkDescale and pvDescale [num_heads] float, the
 * quantised INT8_NZCACHE cache mode) -- on the ND layout instead of the
 * page's NZ one:
 *     s_j = qkScale * (qkDescale[h] * (qNope_{t,h} . ctKV_j) + qRope_{t,h} . kRope_j)
 *     attenOut_{t,h} = pvDescale[h] * sum_j softmax(s)_j ctKV_j,  lse = ln sum_j exp(s_j)
 * (qNope . ctKV an exact integer dot product over 512 dims; h the query head).
 *
 *   qNope      dev [T, headNum, 512] int8      qRope  dev [T, headNum, 64] dtype
 *   ctKV       dev [numBlocks, blockSize, 1, 512] int8
 *   kRope      dev [numBlocks, blockSize, 1, 64] dtype (required)
 *   qkDescale, pvDescale  dev [headNum] fp32 (required)
 *   dtype      MPA_FP16 or MPA_BF16: the type of qRope, kRope and attenOut
 * The other arguments, outputs, errors and phase 2 (mpaMLA) are those of
 * mpaMLAGetWorkspaceSize with cacheMode KROPE_CTKV.
 */
mpaStatus mpaMLAInt8GetWorkspaceSize(
    const void *qNope, const void *qRope, const void *ctKV, const void *kRope,
    const int32_t *blockTables, const int32_t *contextLens, const int32_t *qSeqLen,
    const float *qkDescale, const float *pvDescale, int32_t headNum, float qkScale,
    int32_t kvHeadNum, int maskType, int calcType, int32_t batch, int32_t numBlocks,
    int32_t blockSize, int32_t maxBlockNum, int dtype, int64_t nTokens, void *attenOut,
    float *lse, uint64_t *workspaceSize, mpaOperation **op);

/* MLA, phase 2, on `stream`: copy of the plan into the workspace (dev, >= the
 * size phase 1 returned, 256-byte aligned), the split kernel (partials into the
 * workspace) and, when a sequence was split, their LSE-weighted merge into
 * attenOut / lse.  Errors as for mpaSelfAttentionPrefixEncoder. */
mpaStatus mpaMLA(void *workspace, uint64_t workspaceSize, mpaOperation *op, void *stream);

/*
 * MLA, phase 2, without any allocation: for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid it).  The same launches as mpaMLA, with the plan and the split-KV
 * partials in a buffer the library owns: a static device array of
 * MPA_MLA_STATIC_SCRATCH_BYTES bytes (128 MiB), one per GPU, held until the
 * process ends.  Nothing is allocated and nothing must be zeroed: every
 * execution first copies its plan into the buffer and writes every partial it
 * reads.  All executions on one GPU share that GPU's buffer: executions that
 * may overlap on one GPU (different streams, or streams of different threads)
 * race and must be serialised by the caller.
 *   op      an operation from mpaMLAGetWorkspaceSize / mpaMLAInt8GetWorkspaceSize
 *           whose workspace size is at most MPA_MLA_STATIC_SCRATCH_BYTES
 *   stream  hipStream_t of the launches
 * Errors: MPA_ERROR_INVALID_ARG (op NULL or not MLA), MPA_ERROR_WORKSPACE_TOO_SMALL
 * (the operation needs more than the static buffer: use mpaMLA), MPA_ERROR_HIP.
 */
#define MPA_MLA_STATIC_SCRATCH_BYTES (128ull << 20)
mpaStatus mpaMLAStaticScratch(mpaOperation *op, void *stream);

/*
 * Merge of attention partials over disjoint key ranges by their log-sum-exp
 * (page "MLA", parameter table: the lse output, which the RING calcType requires;
 * the same merge the MLA call applies to its split-KV partials).  Each part is
 * the (output, LSE) of one call of this library over one key range, e.g. the
 * chunks of a long prefix, or one GPU's range of a ring.  For row r and part s:
 *   LSE_r = ln sum_s exp(lseParts[s][r]),
 *   out[r] = sum_s exp(lseParts[s][r] - LSE_r) * oParts[s][r].
 * A part with LSE = -inf (no key in its range) weighs nothing and its output
 * values are ignored (they may be undefined, NaN included); a row whose parts
 * are all -inf gets out = 0 and LSE = -inf.  One launch on `stream`;
 * nothing is allocated.
 *   oParts    dev [nParts, rows, headDim] dtype, contiguous (parts stacked)
 *   lseParts  dev [nParts, rows] fp32, natural log (as written by the lse
 *             outputs of PrefixEncoder and MLA)
 *   nParts    >= 1;  rows >= 0 ((token, head) pairs);  headDim a multiple of 8,
 *             8 .. 4096
 *   dtype     MPA_FP16 or MPA_BF16
 *   out       dev [rows, headDim] dtype (output); may not overlap the parts
 *   lse       dev [rows] fp32 natural-log LSE (output), or NULL
 * With rows = 0 nothing is launched and the pointers may be NULL.
 * Errors: MPA_ERROR_INVALID_ARG for NULL pointers or out-of-range sizes (checked
 * before any HIP call), MPA_ERROR_HIP if the launch fails.
 */
mpaStatus mpaLseMerge(const void *oParts, const float *lseParts, int32_t nParts, int64_t rows,
                      int32_t headDim, int dtype, void *out, float *lse, void *stream);

/* Timing hooks, for callers that profile an operation's executions without
 * adding commands to the stream between them.  startEvent / stopEvent are
 * hipEvent_t handles created by the caller with timing enabled, or NULL (none).
 * Each later execution of op records startEvent when its first kernel starts
 * and stopEvent when its last kernel ends, on the kernels' own dispatch packets
 * (hipExtLaunchKernel); an execution that launches nothing records neither.
 * The events must stay valid while executions that record them are queued; the
 * caller owns and destroys them.  Nothing is launched or allocated here.
 * Errors: MPA_ERROR_INVALID_ARG if op is NULL. */
mpaStatus mpaOperationSetLaunchEvents(mpaOperation *op, void *startEvent, void *stopEvent);

/* Releases an operation (NULL is accepted).  Must not be called while an
 * execution of it may still be running on a stream. */
mpaStatus mpaDestroyOperation(mpaOperation *op);

/* Static description of a status code. */
const char *mpaGetErrorString(mpaStatus status);

/* Detail of the last failure on the calling thread ("" if none). */
const char *mpaGetLastErrorMessage(void);

/*
 * Host-only inspection of the PrefixEncoder launch plan (no HIP call; for tests
 * and tools).  Fills items[0 .. *nItems) with 4 int32 each, one per workgroup in
 * launch order: {b, first query head, first query row, number of key tiles the
 * workgroup visits}, and reports the tile geometry and the workspace bytes
 * phase 1 would return for the plan (any output pointer may be NULL).  Returns
 * MPA_ERROR_INVALID_ARG if capacity (in items) is too small; *nItems and the
 * scalar outputs are set either way.
 */
mpaStatus mpaPrefixEncoderPlanInspect(const int32_t *seqLen, const int32_t *kvSeqLen,
                                      int32_t batch, int maskType, int32_t headNum,
                                      int32_t kvHeadNum, int32_t headSize, int32_t *items,
                                      int64_t capacity, int64_t *nItems, int32_t *rowsPerItem,
                                      int32_t *keysPerTile, int32_t *headsPerItem,
                                      uint64_t *workspaceSize);

/*
 * Host-only inspection of the MLA split plan (as planned for 256 compute
 * units).  The key tiles (32 keys) of all sequences, laid end to end, are cut
 * into pieces of near-equal tile counts; a piece's part of one sequence is a
 * segment.  Fills splits[0 .. *nSplits) with 5 int32 per segment, in piece
 * order: {b, first key, end key, index of the segment among those of sequence
 * b, piece}.  A sequence with one segment gets its output written directly;
 * the others are merged by LSE.  Returns MPA_ERROR_INVALID_ARG if capacity (in
 * segments) is too small; *nSplits is set either way.
 */
mpaStatus mpaMLAPlanInspect(const int32_t *contextLens, const int32_t *qSeqLen, int32_t batch,
                            int32_t headNum, int calcType, int32_t *splits, int64_t capacity,
                            int64_t *nSplits);

#ifdef __cplusplus
}
#endif

#endif /* MPA_H_ */
