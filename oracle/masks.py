"""Mask and bias definitions of the oracle (fp64, numpy).  TEST INFRASTRUCTURE ONLY.

Two things live here:

1. The *full* rule -- which (query, key) pairs are visible and which additive bias
   each visible pair gets -- written on absolute positions.  This is what the
   oracle's attention uses.
2. The *compressed* masks of the Ascend ATB page "压缩mask" (compressed mask),
   section "约束说明" (constraints), together with the expansion of a compressed
   tile back to a full [seqLen, kvSeqLen] mask.  They exist only so that a test can
   check that an expanded compressed mask equals the full rule; the HIP path never
   reads a mask tensor.

Notation.  Sequence b has ``seq_len`` new query rows and ``kv_len`` keys (cached
prefix plus the new rows, ATB page "PrefixEncoder", parameter table, rows seqLen
and kvSeqLen).  Query row i sits at absolute position a_i = (kv_len - seq_len) + i;
key j sits at position j.

Readings taken where the pages are silent, garbled or lost:

* masked pairs are excluded exactly (weight 0), i.e. -inf semantics -- the nalar.dev
  article, section "Masking mengubah kelayakan relasi attention", allows either a
  large negative or -inf; the fp16/bf16 mask figures of the compressed-mask page are
  not available;
* the ALiBi mask is slope_h x bias plus a triangular (causal) mask -- the
  decomposition formula of the compressed-mask page is lost; its surrounding text
  says the mask tensor carries the bias and ``slopes`` carries the per-head
  coefficient;
* right-aligned ALiBi (maskType 3): bias = slope_h * (j - a_i)  (0 on the diagonal,
  more negative further back);
* sqrt ALiBi (maskType 4): the same bias with the distance square-rooted,
  bias = -slope_h * sqrt(a_i - j)  (the garbled sentence of the compressed-mask page
  says only that the bias itself is square-rooted);
* left-aligned ALiBi (maskType 5): bias = slope_h * j  (grows with the key
  position from column 0); softmax output equals the right-aligned one because the
  two differ by the per-row constant slope_h * a_i;
* causal (maskType 9, generated inside the operator) and the compressed norm mask
  used for RoPE models: j <= a_i;
* maskType 0 (ours): no causal rule, keys limited only by kv_len (padding mask);
* chunked local causal mask (ours, number 10): the LLaMA 4 chunked attention of
  the page "终极指南：LLaMA模型的Transformer注意力掩码与填充处理技术解析", section
  "本地注意力掩码生成" (the function body is elided there; the plainest reading
  of a per-token chunk restriction combined with causality): with chunk size C,
  a query at absolute position a sees the keys j <= a of its own chunk,
  floor(j / C) == floor(a / C);
* every type also hides keys j >= kv_len (padding / varlen boundary, nalar.dev
  article, sections "Causal mask dan padding mask menangani batas yang berbeda" and
  "Packing mengeluarkan padding dari representasi").
"""

import numpy as np

MASK_NONE = 0
MASK_ALIBI = 3
MASK_ALIBI_SQRT = 4
MASK_ALIBI_LEFT = 5
MASK_CAUSAL = 9
MASK_CHUNKED_CAUSAL = 10

CAUSAL_TYPES = (MASK_ALIBI, MASK_ALIBI_SQRT, MASK_ALIBI_LEFT, MASK_CAUSAL, MASK_CHUNKED_CAUSAL)
ALIBI_TYPES = (MASK_ALIBI, MASK_ALIBI_SQRT, MASK_ALIBI_LEFT)

# Edge of the compressed tiles (the [128,128] norm mask and the [256,256] ALiBi
# mask, which holds a 2x2 arrangement of 128-wide tiles).
TILE = 128


def visible(mask_type, a, j, kv_len, chunk=None):
    """Boolean visibility of key position ``j`` for a query at absolute ``a``.

    ``a`` and ``j`` broadcast against each other (e.g. a[:, None], j[None, :]).
    ``chunk`` is the chunk size of MASK_CHUNKED_CAUSAL (required for it only).
    """
    a = np.asarray(a)
    j = np.asarray(j)
    vis = np.broadcast_to(j < kv_len, np.broadcast(a, j).shape)
    if mask_type in CAUSAL_TYPES:
        vis = vis & (j <= a)
    elif mask_type != MASK_NONE:
        raise ValueError(f"unknown mask type {mask_type}")
    if mask_type == MASK_CHUNKED_CAUSAL:
        if chunk is None or int(chunk) < 1:
            raise ValueError("the chunked mask needs a chunk size >= 1")
        vis = vis & (j // int(chunk) == a // int(chunk))
    elif chunk is not None:
        raise ValueError("a chunk size goes with the chunked mask only")
    return vis


def bias(mask_type, slope, a, j):
    """Additive fp64 bias of the pair (a, j).  Only meaningful where visible."""
    a = np.asarray(a, dtype=np.float64)
    j = np.asarray(j, dtype=np.float64)
    slope = float(slope)
    if mask_type in (MASK_NONE, MASK_CAUSAL, MASK_CHUNKED_CAUSAL):
        return np.zeros(np.broadcast(a, j).shape)
    if mask_type == MASK_ALIBI:
        return slope * (j - a)
    if mask_type == MASK_ALIBI_SQRT:
        # The distance is >= 0 on visible pairs; clip so masked pairs stay finite.
        return -slope * np.sqrt(np.maximum(a - j, 0.0))
    if mask_type == MASK_ALIBI_LEFT:
        return slope * j
    raise ValueError(f"unknown mask type {mask_type}")


def full_mask(mask_type, slope, seq_len, kv_len):
    """[seq_len, kv_len] fp64 additive mask M: bias where visible, -inf elsewhere."""
    prefix = kv_len - seq_len
    a = prefix + np.arange(seq_len)[:, None]
    j = np.arange(kv_len)[None, :]
    vis = visible(mask_type, a, j, kv_len)
    m = np.where(vis, bias(mask_type, slope, a, j), -np.inf)
    return m


# ---------------------------------------------------------------------------
# Compressed masks (compressed-mask page, section "约束说明").  The figures that
# hold the exact tensor contents are not available; these are the readings:
#   norm   [128,128]: 0 on and below the diagonal, masked above it;
#   ALiBi  [256,256]: the unscaled right-aligned bias y - x on and below the
#                     diagonal (so the second 128-row band holds the bias of a key
#                     tile one tile behind the query tile), masked above;
#   sqrt   [256,256]: same tile in distance form, square root taken after the
#                     tile is expanded (a square root cannot be shifted linearly);
#   left   [256,256]: the unscaled left-aligned bias y on and below the diagonal.
# A tile grid of TILE on absolute positions: bq = a // TILE, bk = j // TILE,
# r = a % TILE, c = j % TILE, k = bq - bk (how many tiles the key lies behind).
# ---------------------------------------------------------------------------


def compressed_norm():
    """[128,128] compressed causal mask: 0 where c <= r, -inf where c > r."""
    r = np.arange(TILE)[:, None]
    c = np.arange(TILE)[None, :]
    return np.where(c <= r, 0.0, -np.inf)


def compressed_alibi():
    """[256,256] unscaled right-aligned bias: y - x where y <= x, -inf above."""
    x = np.arange(2 * TILE)[:, None]
    y = np.arange(2 * TILE)[None, :]
    return np.where(y <= x, (y - x).astype(np.float64), -np.inf)


def compressed_alibi_left():
    """[256,256] unscaled left-aligned bias: y where y <= x, -inf above."""
    x = np.arange(2 * TILE)[:, None]
    y = np.arange(2 * TILE)[None, :]
    return np.where(y <= x, y.astype(np.float64), -np.inf)


def compressed_bias(mask_type, tile, slope, a, j, kv_len):
    """Additive mask of the pairs (a, j) read from a compressed tile: the bias,
    or -inf where the pair is hidden.  ``a`` (absolute query positions) and ``j``
    (key positions) broadcast against each other.

    ``tile`` is what ``compressed_norm`` / ``compressed_alibi`` /
    ``compressed_alibi_left`` return, or any tile of the same shape (the sqrt
    type uses the ``compressed_alibi`` tile in distance form).  Keys at or beyond
    kv_len are masked (padding).
    """
    a = np.asarray(a)
    j = np.asarray(j)
    shape = np.broadcast(a, j).shape
    tile = np.asarray(tile, dtype=np.float64)
    bq, r = a // TILE, a % TILE
    bk, c = j // TILE, j % TILE
    k = bq - bk
    if mask_type in (MASK_CAUSAL,):
        assert tile.shape == (TILE, TILE)
        diag = tile[np.broadcast_to(r, shape), np.broadcast_to(c, shape)]
        out = np.where(k > 0, 0.0, np.where(k == 0, diag, -np.inf))
    elif mask_type in (MASK_ALIBI, MASK_ALIBI_SQRT):
        assert tile.shape == (2 * TILE, 2 * TILE)
        rows = np.broadcast_to(np.where(k == 0, r, TILE + r), shape)
        cols = np.broadcast_to(c, shape)
        val = tile[rows, cols]
        # A key k >= 1 tiles behind reuses the second band, shifted by 128 per
        # extra tile of distance.
        shift = np.where(k >= 1, -TILE * (k - 1), 0).astype(np.float64)
        val = np.where(k >= 0, val + shift, -np.inf)
        if mask_type == MASK_ALIBI:
            with np.errstate(invalid="ignore"):  # slope 0 times a -inf entry (not selected)
                out = np.where(np.isfinite(val), slope * val, -np.inf)
        else:
            dist = -val
            with np.errstate(invalid="ignore"):
                out = np.where(np.isfinite(val), -slope * np.sqrt(np.where(np.isfinite(dist), dist, 0.0)),
                               -np.inf)
    elif mask_type == MASK_ALIBI_LEFT:
        assert tile.shape == (2 * TILE, 2 * TILE)
        rows = np.broadcast_to(np.where(k == 0, r, TILE + r), shape)
        cols = np.broadcast_to(c, shape)
        val = tile[rows, cols]
        # The tile holds the in-tile column; the key tile's origin is added back.
        val = np.where(k >= 0, val + TILE * bk, -np.inf)
        with np.errstate(invalid="ignore"):  # slope 0 times a -inf entry (not selected)
            out = np.where(np.isfinite(val), slope * val, -np.inf)
    else:
        raise ValueError(f"mask type {mask_type} has no compressed form")
    return np.where(j < kv_len, out, -np.inf)


def expand_compressed(mask_type, tile, slope, seq_len, kv_len):
    """Expand a compressed tile to the full [seq_len, kv_len] additive mask
    (rows at absolute positions kv_len - seq_len + i, see ``compressed_bias``)."""
    prefix = kv_len - seq_len
    a = prefix + np.arange(seq_len)[:, None]
    j = np.arange(kv_len)[None, :]
    return compressed_bias(mask_type, tile, slope, a, j, kv_len)
