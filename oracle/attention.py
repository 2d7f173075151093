"""fp64 reference attention over a paged KV cache.  TEST INFRASTRUCTURE ONLY.

What is computed (plainest reading of the pages, see ``oracle/__init__``):

    s_ij  = qkScale * (q_i . k_j) + bias(i, j)       over visible keys j only
    O_i   = sum_j exp(s_ij - m_i) v_j / sum_j exp(s_ij - m_i),  m_i = max_j s_ij
    LSE_i = m_i + ln(sum_j exp(s_ij - m_i))           (natural log, fp64)

i.e. A = softmax(qkScale * Q K^T + M), O = A V (nalar.dev article, section "Masking
mengubah kelayakan relasi attention"), with M from ``oracle.masks``.

Layouts follow the Ascend ATB page "PrefixEncoder", parameter table: query
[nTokens, headNum, headSize]; key/value [numBlocks, blockSize, kvHeadNum,
headSize] (the 4-D shape on the page names headNum; read as kvHeadNum);
blockTables [batch, maxBlockNum] int32 (the page says the first dimension is the
token index; read as the batch index); seqLen / kvSeqLen per sequence, host side.
Query head h reads KV head h // (headNum / kvHeadNum) (grouped-query attention;
the page is silent on the grouping, contiguous groups are taken).  Sequence b's
rows start at q_start_loc[b] (default: packed, prefix sums of seqLen).

The MLA variant follows the Ascend ATB page "MLA", parameter table: query =
[qNope 512 | qRope 64], key = [ctKV 512 | kRope 64] (or one concatenated 576-wide
cache with cacheMode 0), value = ctKV (512), one KV head, keys limited by
contextLens, speculative tokens (calcType 1, qseqlen) either all see every cached
key (maskType 0, the all-zero mask) or see a causal tail (maskType SPEC): token t
of q_len sees keys j <= ctx - q_len + t.  LSE is fp64 here (the page lists an
fp16/bf16 [num_tokens, num_heads, 1] tensor; this build keeps it fp32 on the GPU).

qkScale and slopes are taken at their fp32 values, as the operator receives them.
"""

import numpy as np

from . import masks as _m

MASK_NONE = _m.MASK_NONE
MASK_ALIBI = _m.MASK_ALIBI
MASK_ALIBI_SQRT = _m.MASK_ALIBI_SQRT
MASK_ALIBI_LEFT = _m.MASK_ALIBI_LEFT
MASK_CAUSAL = _m.MASK_CAUSAL
MASK_CHUNKED_CAUSAL = _m.MASK_CHUNKED_CAUSAL

MLA_MASK_UNDEFINED = 0
MLA_MASK_SPEC = 1
MLA_CALC_UNDEFINED = 0
MLA_CALC_SPEC = 1
MLA_CALC_PREFILL = 3  # listing order on the MLA page: UNDEFINED, SPEC, RING, PREFILL

ROW_CHUNK = 1024


def _f32(x):
    return float(np.float32(x))


def attend(q, k, v, scale, mask):
    """Masked softmax attention of a block of query rows, in fp64.

    q [R, Dq], k [N, Dq], v [N, Dv], mask [R, N] additive (-inf = masked).
    Returns (O [R, Dv], LSE [R]).  A row with no visible key gets O = 0 and
    LSE = -inf (cannot happen for valid rows of a well-formed call).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    s = scale * (q @ k.T) + mask
    vis = np.isfinite(mask)
    s = np.where(vis, s, -np.inf)
    m = s.max(axis=1)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    w = np.exp(s - m_safe[:, None])
    w = np.where(vis, w, 0.0)
    l = w.sum(axis=1)
    l_safe = np.where(empty, 1.0, l)
    o = (w @ v) / l_safe[:, None]
    o = np.where(empty[:, None], 0.0, o)
    lse = np.where(empty, -np.inf, m_safe + np.log(l_safe))
    return o, lse


def lse_merge(outs, lses):
    """Merge attention results over disjoint key sets.

    For disjoint key sets S_1..S_n of one query row with partial results (O_s,
    LSE_s): LSE = ln sum_s exp(LSE_s) and O = sum_s exp(LSE_s - LSE) O_s.  This is
    the quantity the MLA page's LSE output exists for (calcType RING).
    outs [n, ..., Dv], lses [n, ...].
    """
    outs = np.asarray(outs, dtype=np.float64)
    lses = np.asarray(lses, dtype=np.float64)
    mx = lses.max(axis=0)
    mx_safe = np.where(np.isfinite(mx), mx, 0.0)
    w = np.exp(lses - mx_safe)
    tot = w.sum(axis=0)
    lse = np.where(tot > 0, mx_safe + np.log(np.where(tot > 0, tot, 1.0)), -np.inf)
    coef = np.where(tot > 0, w / np.where(tot > 0, tot, 1.0), 0.0)
    o = (coef[..., None] * outs).sum(axis=0)
    return o, lse


def _gather(cache, block_tables, b, n, block_size, head):
    """Rows 0..n-1 of sequence b's paged cache for one KV head: [n, D] fp64."""
    j = np.arange(n)
    blocks = np.asarray(block_tables)[b, j // block_size]
    slots = j % block_size
    return np.asarray(cache[blocks, slots, head, :], dtype=np.float64)


def _q_starts(seq_len, q_start_loc):
    if q_start_loc is not None:
        return [int(x) for x in q_start_loc]
    starts, acc = [], 0
    for L in seq_len:
        starts.append(acc)
        acc += int(L)
    return starts


def _check_prefix_args(seq_len, kv_seq_len, head_num, kv_head_num, mask_type, slopes):
    if head_num <= 0 or kv_head_num <= 0 or head_num % kv_head_num:
        raise ValueError("headNum must be > 0 and a multiple of kvHeadNum")
    for L, kv in zip(seq_len, kv_seq_len):
        if not 0 <= int(L) <= int(kv):
            raise ValueError("need 0 <= seqLen <= kvSeqLen")
    if mask_type in _m.ALIBI_TYPES and slopes is None:
        raise ValueError("ALiBi mask types need slopes")


def prefix_encoder_rows(query, key, value, block_tables, seq_len, kv_seq_len,
                        slopes, mask_type, head_num, kv_head_num, qk_scale,
                        rows, q_start_loc=None, chunk=None, mask_tile=None):
    """Oracle output for selected (b, i, h) triples only.

    ``mask_tile``: an explicit compressed mask (ATB page "压缩mask", section
    约束说明) whose expansion gives the bias and visibility in place of the
    full rule of ``mask_type``.

    ``rows`` is an iterable of (b, i, h) with 0 <= i < seq_len[b].  Returns
    (O [n, D] fp64, LSE [n] fp64) in the order given.  Rows of the same (b, h) are
    batched into one fp64 product.
    """
    _check_prefix_args(seq_len, kv_seq_len, head_num, kv_head_num, mask_type, slopes)
    starts = _q_starts(seq_len, q_start_loc)
    block_size = key.shape[1]
    group = head_num // kv_head_num
    scale = _f32(qk_scale)
    rows = [tuple(int(x) for x in r) for r in rows]
    d_v = value.shape[-1]
    out = np.zeros((len(rows), d_v))
    lse = np.zeros(len(rows))
    by_bh = {}
    for n, (b, i, h) in enumerate(rows):
        if not 0 <= i < int(seq_len[b]):
            raise ValueError(f"row {i} outside sequence {b}")
        by_bh.setdefault((b, h), []).append((n, i))
    for (b, h), items in by_bh.items():
        kv = int(kv_seq_len[b])
        L = int(seq_len[b])
        kvh = h // group
        k_all = _gather(key, block_tables, b, kv, block_size, kvh)
        v_all = _gather(value, block_tables, b, kv, block_size, kvh)
        slope = _f32(slopes[h]) if mask_type in _m.ALIBI_TYPES else 0.0
        idx = np.array([it[0] for it in items])
        ii = np.array([it[1] for it in items])
        for c0 in range(0, len(ii), ROW_CHUNK):
            sel = ii[c0:c0 + ROW_CHUNK]
            a = (kv - L) + sel[:, None]
            j = np.arange(kv)[None, :]
            if mask_tile is not None:
                msk = _m.compressed_bias(mask_type, mask_tile, slope, a, j, kv)
            else:
                vis = _m.visible(mask_type, a, j, kv, chunk)
                msk = np.where(vis, _m.bias(mask_type, slope, a, j), -np.inf)
            q = np.asarray(query[starts[b] + sel, h, :], dtype=np.float64)
            o, ls = attend(q, k_all, v_all, scale, msk)
            out[idx[c0:c0 + ROW_CHUNK]] = o
            lse[idx[c0:c0 + ROW_CHUNK]] = ls
    return out, lse


def prefix_encoder(query, key, value, block_tables, seq_len, kv_seq_len, slopes,
                   mask_type, head_num, kv_head_num, qk_scale, q_start_loc=None,
                   heads=None, chunk=None, mask_tile=None):
    """Full oracle of the PrefixEncoder operation (``mask_tile``: see
    ``prefix_encoder_rows``).

    Returns (O [nTokens, headNum, D] fp64, LSE [nTokens, headNum] fp64).  Rows that
    belong to no sequence (padding rows of a padded layout) are NaN: they are not
    part of the result.  ``heads`` optionally restricts the heads computed (the
    others stay NaN).
    """
    n_tokens = query.shape[0]
    d_v = value.shape[-1]
    out = np.full((n_tokens, head_num, d_v), np.nan)
    lse = np.full((n_tokens, head_num), np.nan)
    starts = _q_starts(seq_len, q_start_loc)
    heads = range(head_num) if heads is None else heads
    for b in range(len(seq_len)):
        L = int(seq_len[b])
        if L == 0:
            continue
        for h in heads:
            rows = [(b, i, h) for i in range(L)]
            o, ls = prefix_encoder_rows(query, key, value, block_tables, seq_len,
                                        kv_seq_len, slopes, mask_type, head_num,
                                        kv_head_num, qk_scale, rows, q_start_loc, chunk,
                                        mask_tile)
            out[starts[b]:starts[b] + L, h] = o
            lse[starts[b]:starts[b] + L, h] = ls
    return out, lse


# ---------------------------------------------------------------------------
# MLA
# ---------------------------------------------------------------------------

def _mla_qlens(batch, q_seq_len, calc_type):
    if calc_type == MLA_CALC_UNDEFINED:
        return [1] * batch
    if calc_type in (MLA_CALC_SPEC, MLA_CALC_PREFILL):
        # SPEC: a few speculative tokens; PREFILL ("prefill全量"): all new tokens of
        # a prompt.  Both take qseqlen tokens per sequence with the same masks.
        if q_seq_len is None:
            raise ValueError("calcType SPEC / PREFILL needs qseqlen")
        return [int(x) for x in q_seq_len]
    raise ValueError(f"unsupported calcType {calc_type}")


def mla_rows(q_nope, q_rope, ct_kv, k_rope, block_tables, context_lens, q_seq_len,
             head_num, qk_scale, mask_type, calc_type, rows, qk_descale=None, pv_descale=None):
    """MLA oracle for selected (token, head) pairs.  Returns (O [n,512], LSE [n]).

    With ``qk_descale`` / ``pv_descale`` ([headNum]) the cache is the int8 one of
    the MLA page's parameter table (qNope and ctKV int8, rows qkDescale and
    pvDescale): for head h the nope part of the score is qkDescale[h] times the
    integer dot product qNope . ctKV, the rope part stays as it is, and the output
    is pvDescale[h] times the softmax-weighted ctKV rows.
    """
    quant = qk_descale is not None
    if quant != (pv_descale is not None):
        raise ValueError("qk_descale and pv_descale go together")
    batch = len(context_lens)
    qlens = _mla_qlens(batch, q_seq_len, calc_type)
    block_size = ct_kv.shape[1]
    d_v = 512
    scale = _f32(qk_scale)
    tok_b, tok_t = [], []
    for b in range(batch):
        for t in range(qlens[b]):
            tok_b.append(b)
            tok_t.append(t)
    rows = [(int(t), int(h)) for t, h in rows]
    out = np.zeros((len(rows), d_v))
    lse = np.zeros(len(rows))
    by_b = {}
    for n, (tok, h) in enumerate(rows):
        by_b.setdefault(tok_b[tok], []).append((n, tok, h))
    for b, items in by_b.items():
        ctx = int(context_lens[b])
        ql = qlens[b]
        if ql > ctx:
            raise ValueError("qseqlen larger than contextLens")
        lat = _gather(ct_kv, block_tables, b, ctx, block_size, 0)
        if k_rope is None:  # cacheMode 0: one 576-wide cache
            k = lat
            v = lat[:, :d_v]
        else:
            k = np.concatenate([lat, _gather(k_rope, block_tables, b, ctx, block_size, 0)], axis=1)
            v = lat
        idx = np.array([it[0] for it in items])
        qk_d = [float(np.float32(qk_descale[h])) if quant else 1.0 for _, _, h in items]
        qs = np.stack([np.concatenate([np.asarray(q_nope[tok, h], dtype=np.float64) * qd,
                                       np.asarray(q_rope[tok, h], dtype=np.float64)])
                       for (_, tok, h), qd in zip(items, qk_d)])
        t = np.array([tok_t[tok] for _, tok, _ in items])
        j = np.arange(ctx)[None, :]
        if mask_type == MLA_MASK_SPEC:
            vis = j <= (ctx - ql + t)[:, None]
        elif mask_type == MLA_MASK_UNDEFINED:
            vis = np.broadcast_to(j < ctx, (len(items), ctx))
        else:
            raise ValueError(f"unsupported MLA maskType {mask_type}")
        msk = np.where(vis, 0.0, -np.inf)
        o, ls = attend(qs, np.asarray(k, dtype=np.float64), np.asarray(v, dtype=np.float64), scale, msk)
        if quant:
            o = o * np.array([float(np.float32(pv_descale[h])) for _, _, h in items])[:, None]
        out[idx] = o
        lse[idx] = ls
    return out, lse


def mla(q_nope, q_rope, ct_kv, k_rope, block_tables, context_lens, q_seq_len,
        head_num, qk_scale, mask_type=MLA_MASK_UNDEFINED, calc_type=MLA_CALC_UNDEFINED,
        qk_descale=None, pv_descale=None):
    """Full MLA oracle: (O [T, headNum, 512] fp64, LSE [T, headNum] fp64)."""
    n_tok = q_nope.shape[0]
    rows = [(t, h) for t in range(n_tok) for h in range(head_num)]
    o, ls = mla_rows(q_nope, q_rope, ct_kv, k_rope, block_tables, context_lens,
                     q_seq_len, head_num, qk_scale, mask_type, calc_type, rows,
                     qk_descale, pv_descale)
    return o.reshape(n_tok, head_num, -1), ls.reshape(n_tok, head_num)
