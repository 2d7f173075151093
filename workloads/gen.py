"""Seeded generators for the prefill (PrefixEncoder) and MLA decode workloads.

Recipe:

* lengths and the block permutation come from ``numpy.random.default_rng(seed_len)``;
* values are fp32 ``torch.randn`` from ``torch.Generator('cpu').manual_seed(seed_val)``,
  times ``std``, cast round-to-nearest-even to fp16/bf16; the oracle reads exactly
  these cast values;
* the paged cache: sequence b needs ceil(alloc_b / blockSize) blocks; the cache has
  N = sum of those plus max(4, N // 8) spare blocks; a random permutation of all
  block ids is dealt out to the sequences in order, the first spare id fills unused
  block-table entries;
* ``poison=True`` writes NaN into every byte the operator must never read: spare
  blocks, slots at or beyond kvSeqLen in a sequence's blocks, and the padding rows
  of a padded query layout.

Nothing here computes attention, masks or biases.
"""

from dataclasses import dataclass, replace
from typing import Optional

import numpy as np
import torch

FP16 = "fp16"
BF16 = "bf16"
TORCH_DTYPE = {FP16: torch.float16, BF16: torch.bfloat16}

MASK_NONE, MASK_ALIBI, MASK_ALIBI_SQRT, MASK_ALIBI_LEFT, MASK_CAUSAL = 0, 3, 4, 5, 9
MLA_MASK_UNDEFINED, MLA_MASK_SPEC = 0, 1
MLA_CALC_UNDEFINED, MLA_CALC_SPEC = 0, 1
MLA_CACHE_KVCACHE, MLA_CACHE_KROPE_CTKV = 0, 1


def alibi_slopes(head_num):
    """Per-head ALiBi coefficients 2^(-8(h+1)/H) as fp32 (the workloads' recipe)."""
    h = np.arange(head_num, dtype=np.float64)
    return (2.0 ** (-8.0 * (h + 1) / head_num)).astype(np.float32)


def _randn(gen, shape, std, dtype):
    x = torch.randn(*shape, generator=gen, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(TORCH_DTYPE[dtype])


def _deal_blocks(rng, alloc_lens, block_size, spare_min=4, max_block_num=None):
    need = [max(0, -(-int(n) // block_size)) for n in alloc_lens]
    n_used = sum(need)
    n_blocks = n_used + max(spare_min, n_used // 8)
    perm = rng.permutation(n_blocks).astype(np.int32)
    width = max(1, max(need) if need else 1)
    if max_block_num is not None:
        assert max_block_num >= width
        width = max_block_num
    spare = perm[n_used:]
    table = np.full((len(alloc_lens), width), spare[0], dtype=np.int32)
    pos = 0
    for b, nb in enumerate(need):
        table[b, :nb] = perm[pos:pos + nb]
        pos += nb
    return n_blocks, table, spare, need


def _poison_cache(cache, table, kv_lens, need, spare, block_size):
    """NaN every slot the operator must not read (cache is modified in place)."""
    cache[torch.as_tensor(spare, dtype=torch.long)] = float("nan")
    for b, kv in enumerate(kv_lens):
        kv = int(kv)
        for blk in range(need[b]):
            lo = blk * block_size
            first_bad = max(0, kv - lo)
            if first_bad < block_size:
                cache[int(table[b, blk]), first_bad:] = float("nan")


@dataclass
class PrefillCase:
    """One PrefixEncoder call: tensors in the operator's layouts plus host metadata."""
    name: str
    dtype: str
    seq_len: np.ndarray          # int32 [B], host
    kv_seq_len: np.ndarray       # int32 [B], host
    head_num: int
    kv_head_num: int
    head_size: int
    block_size: int
    mask_type: int
    qk_scale: float
    slopes: Optional[np.ndarray]       # float32 [headNum] or None
    q_start_loc: Optional[np.ndarray]  # int64 [B] or None (packed)
    query: torch.Tensor          # [nTokens, headNum, headSize]
    key: torch.Tensor            # [numBlocks, blockSize, kvHeadNum, headSize]
    value: torch.Tensor
    block_tables: torch.Tensor   # int32 [B, maxBlockNum]
    chunk: int = 0               # chunk size of the chunked local causal mask, 0: none
    mask_tile: Optional[torch.Tensor] = None  # explicit compressed mask ([128,128] / [256,256]), dtype

    @property
    def batch(self):
        return len(self.seq_len)

    @property
    def n_tokens(self):
        return self.query.shape[0]

    @property
    def num_blocks(self):
        return self.key.shape[0]

    @property
    def max_block_num(self):
        return self.block_tables.shape[1]

    def row_starts(self):
        if self.q_start_loc is not None:
            return [int(x) for x in self.q_start_loc]
        return [int(x) for x in np.concatenate([[0], np.cumsum(self.seq_len)[:-1]])]

    def to(self, device):
        return replace(self, query=self.query.to(device), key=self.key.to(device),
                       value=self.value.to(device), block_tables=self.block_tables.to(device),
                       mask_tile=None if self.mask_tile is None else self.mask_tile.to(device))

    def oracle_args(self):
        """Numpy views of the same values (fp16 stays fp16; bf16 is widened to fp32 exactly)."""
        def npy(t):
            t = t.detach().cpu()
            if t.dtype == torch.bfloat16:
                t = t.float()
            return t.numpy()
        # the chunked local causal mask is mask type 10 on the oracle side (the
        # library selects it by its own entry point with causal maskType 9)
        return dict(query=npy(self.query), key=npy(self.key), value=npy(self.value),
                    block_tables=self.block_tables.cpu().numpy(), seq_len=self.seq_len,
                    kv_seq_len=self.kv_seq_len, slopes=self.slopes,
                    mask_type=10 if self.chunk else self.mask_type,
                    head_num=self.head_num, kv_head_num=self.kv_head_num,
                    qk_scale=self.qk_scale, q_start_loc=self.q_start_loc,
                    chunk=self.chunk if self.chunk else None,
                    mask_tile=None if self.mask_tile is None else npy(self.mask_tile).astype(np.float64))


def compressed_tile(mask_type, dtype, seed=None):
    """An explicit compressed mask tile as the ATB page "压缩mask" (section 约束说明)
    describes it, in the reading used throughout: [128,128] norm (0 on and below
    the diagonal, -inf above) for the causal type; [256,256] with col - row
    (right-aligned ALiBi, linear and sqrt) or col (left-aligned) on and below the
    diagonal, -inf above.  With ``seed``, a perturbed copy: an extra bias in steps
    of 1/4 (kept <= 0 for the right-aligned distance form) and -inf holes in about
    3% of the entries below the diagonal, so that every entry a call reads
    matters.  Returned on the CPU in the input type."""
    n = 128 if mask_type == MASK_CAUSAL else 256
    r = torch.arange(n, dtype=torch.float32)[:, None]
    c = torch.arange(n, dtype=torch.float32)[None, :]
    below = c <= r
    if mask_type == MASK_CAUSAL:
        val = torch.zeros(n, n)
    elif mask_type in (MASK_ALIBI, MASK_ALIBI_SQRT):
        val = c - r
    elif mask_type == MASK_ALIBI_LEFT:
        val = c.expand(n, n).clone()
    else:
        raise ValueError(f"mask type {mask_type} has no compressed tile")
    if seed is not None:
        g = torch.Generator("cpu").manual_seed(seed)
        hi = {MASK_CAUSAL: 9, MASK_ALIBI: 1, MASK_ALIBI_SQRT: 1, MASK_ALIBI_LEFT: 13}[mask_type]
        val = val + torch.randint(-12, hi, (n, n), generator=g).float() / 4
        below = below & ~((torch.rand(n, n, generator=g) < 0.03) & (c < r))
    return torch.where(below, val, torch.tensor(float("-inf"))).to(TORCH_DTYPE[dtype]).contiguous()


def make_prefill(seed, seq_len, kv_seq_len, head_num, kv_head_num, head_size, block_size,
                 dtype, mask_type, qk_scale, slopes=None, std=1.0, poison=False,
                 pad_to=None, max_block_num=None, name="custom", seed_val=None, chunk=0):
    """Build a PrefillCase with explicit lengths.

    ``pad_to``: lay the query rows out padded (row offset pad_to * b) and allocate
    ceil(pad_to / blockSize) blocks per sequence; otherwise rows are packed.
    ``slopes``: None, "alibi" (the 2^(-8(h+1)/H) recipe) or an explicit array.
    """
    seq_len = np.asarray(seq_len, dtype=np.int32)
    kv_seq_len = np.asarray(kv_seq_len, dtype=np.int32)
    rng = np.random.default_rng(seed)
    gen = torch.Generator("cpu").manual_seed(seed if seed_val is None else seed_val)
    alloc = kv_seq_len if pad_to is None else np.full_like(kv_seq_len, max(pad_to, int(kv_seq_len.max(initial=0))))
    n_blocks, table, spare, need = _deal_blocks(rng, alloc, block_size, max_block_num=max_block_num)
    total = int(seq_len.sum())
    if pad_to is None:
        n_tokens, q_start = total, None
    else:
        n_tokens = pad_to * len(seq_len)
        q_start = (np.arange(len(seq_len), dtype=np.int64) * pad_to)
    q_valid = _randn(gen, (total, head_num, head_size), std, dtype)
    key = _randn(gen, (n_blocks, block_size, kv_head_num, head_size), std, dtype)
    value = _randn(gen, (n_blocks, block_size, kv_head_num, head_size), std, dtype)
    if pad_to is None:
        query = q_valid
    else:
        query = torch.full((n_tokens, head_num, head_size), float("nan") if poison else 0.0,
                           dtype=TORCH_DTYPE[dtype])
        off = 0
        for b, L in enumerate(seq_len):
            query[q_start[b]:q_start[b] + L] = q_valid[off:off + L]
            off += int(L)
    if poison:
        _poison_cache(key, table, kv_seq_len, need, spare, block_size)
        _poison_cache(value, table, kv_seq_len, need, spare, block_size)
    if isinstance(slopes, str) and slopes == "alibi":
        slopes = alibi_slopes(head_num)
    elif slopes is not None:
        slopes = np.asarray(slopes, dtype=np.float32)
    return PrefillCase(name=name, dtype=dtype, seq_len=seq_len, kv_seq_len=kv_seq_len,
                       head_num=head_num, kv_head_num=kv_head_num, head_size=head_size,
                       block_size=block_size, mask_type=mask_type, qk_scale=float(qk_scale),
                       slopes=slopes, q_start_loc=q_start, query=query, key=key, value=value,
                       block_tables=torch.from_numpy(table), chunk=int(chunk))


def pad_prefill_case(case, pad_to, seed, poison=False, device=None):
    """Re-lay a packed case into the padded layout (rows at pad_to * b, pad_to keys
    allocated per sequence), carrying the same query/key/value values so that the
    valid rows of the two calls must agree.  Work happens on ``device``."""
    device = device or case.query.device
    rng = np.random.default_rng(seed)
    B = case.batch
    alloc = np.full(B, pad_to, dtype=np.int64)
    n_blocks, table, spare, need = _deal_blocks(rng, alloc, case.block_size)
    dt = case.query.dtype
    fill = float("nan") if poison else 0.0
    H, D, KVH, bs = case.head_num, case.head_size, case.kv_head_num, case.block_size
    query = torch.full((pad_to * B, H, D), fill, dtype=dt, device=device)
    key = torch.full((n_blocks, bs, KVH, D), fill, dtype=dt, device=device)
    value = torch.full((n_blocks, bs, KVH, D), fill, dtype=dt, device=device)
    src_q = case.query.to(device)
    src_k = case.key.to(device)
    src_v = case.value.to(device)
    old_t = case.block_tables.to(device).long()
    new_t = torch.from_numpy(table).to(device).long()
    starts = case.row_starts()
    for b in range(B):
        L, kv = int(case.seq_len[b]), int(case.kv_seq_len[b])
        query[pad_to * b:pad_to * b + L] = src_q[starts[b]:starts[b] + L]
        nb = -(-kv // bs)
        for blk in range(nb):
            n = min(bs, kv - blk * bs)
            key[new_t[b, blk], :n] = src_k[old_t[b, blk], :n]
            value[new_t[b, blk], :n] = src_v[old_t[b, blk], :n]
    return replace(case, name=case.name.replace("varlen", "padded"),
                   q_start_loc=np.arange(B, dtype=np.int64) * pad_to,
                   query=query, key=key, value=value, block_tables=torch.from_numpy(table).to(device))


# ---------------------------------------------------------------------------
# The measured workloads.  Index k of each configuration seeds its lengths with
# default_rng(1000 + k) and its values with manual_seed(2000 + k).
# ---------------------------------------------------------------------------

PREFILL_CONFIGS = {
    "tiny_causal": 0,
    "prefix_gqa_causal": 1,
    "alibi_right_4x4096": 2,
    "alibi_sqrt_16384": 3,
    "alibi_left_16384": 3,
    "alibi_sqrt_varlen16": 3,
    "alibi_left_varlen16": 3,
    "alibi_sqrt_padded16": 3,
    "alibi_left_padded16": 3,
}

MLA_CONFIGS = {
    "mla_decode_q1": 4,
    "mla_spec_q4": 4,
}


def _lognormal_lengths(rng, n=16, lo=128, hi=8192):
    x = np.exp(rng.normal(np.log(1024.0), 1.0, size=n))
    return np.clip(np.round(x), lo, hi).astype(np.int32)


def make_prefill_config(name, poison=False, device=None):
    """The named prefill workload, on ``device`` (CPU by default)."""
    k = PREFILL_CONFIGS[name]
    rng = np.random.default_rng(1000 + k)
    seed_blocks = 3000 + k
    if name == "tiny_causal":
        c = make_prefill(seed_blocks, [16, 37], [16, 37], 4, 4, 64, 16, FP16, MASK_CAUSAL,
                         0.125, poison=poison, name=name, seed_val=2000 + k)
    elif name == "prefix_gqa_causal":
        L = rng.integers(128, 1024, size=8, endpoint=True)
        P = rng.integers(0, 2048, size=8, endpoint=True)
        c = make_prefill(seed_blocks, L, L + P, 32, 8, 128, 128, BF16, MASK_CAUSAL,
                         1.0 / np.sqrt(128.0), poison=poison, name=name, seed_val=2000 + k)
    elif name == "alibi_right_4x4096":
        c = make_prefill(seed_blocks, [4096] * 4, [4096] * 4, 32, 32, 128, 128, FP16, MASK_ALIBI,
                         1.0 / np.sqrt(128.0), slopes="alibi", poison=poison, name=name,
                         seed_val=2000 + k)
    elif name in ("alibi_sqrt_16384", "alibi_left_16384"):
        mt = MASK_ALIBI_SQRT if "sqrt" in name else MASK_ALIBI_LEFT
        c = make_prefill(seed_blocks, [16384], [16384], 40, 40, 128, 128, BF16, mt,
                         1.0 / np.sqrt(128.0), slopes="alibi", poison=poison, name=name,
                         seed_val=2000 + k)
    else:
        mt = MASK_ALIBI_SQRT if "sqrt" in name else MASK_ALIBI_LEFT
        L = _lognormal_lengths(rng)
        c = make_prefill(seed_blocks + 10, L, L, 40, 40, 128, 128, BF16, mt,
                         1.0 / np.sqrt(128.0), slopes="alibi", poison=poison,
                         name=name.replace("padded", "varlen"), seed_val=2010 + k)
        if "padded" in name:
            c = pad_prefill_case(c, 8192, seed_blocks + 20, poison=poison, device=device)
    return c.to(device) if device is not None else c


@dataclass
class MLACase:
    """One MLA call: latent paged cache, split query, host lengths."""
    name: str
    dtype: str
    context_lens: np.ndarray            # int32 [B], host
    q_seq_len: Optional[np.ndarray]     # int32 [B], host (calcType SPEC) or None
    head_num: int
    block_size: int
    mask_type: int
    calc_type: int
    cache_mode: int
    qk_scale: float
    q_nope: torch.Tensor                # [T, H, 512]
    q_rope: torch.Tensor                # [T, H, 64]
    ct_kv: torch.Tensor                 # [NB, BS, 1, 512] (cacheMode 1) or [NB, BS, 1, 576] (cacheMode 0)
    k_rope: Optional[torch.Tensor]      # [NB, BS, 1, 64] or None (cacheMode 0)
    block_tables: torch.Tensor          # int32 [B, maxBlockNum]
    kv_head_num: int = 1
    qk_descale: Optional[np.ndarray] = None  # float32 [H], int8 cache only (q_nope, ct_kv int8)
    pv_descale: Optional[np.ndarray] = None

    @property
    def batch(self):
        return len(self.context_lens)

    @property
    def n_tokens(self):
        return self.q_nope.shape[0]

    @property
    def num_blocks(self):
        return self.ct_kv.shape[0]

    @property
    def max_block_num(self):
        return self.block_tables.shape[1]

    def to(self, device):
        return replace(self, q_nope=self.q_nope.to(device), q_rope=self.q_rope.to(device),
                       ct_kv=self.ct_kv.to(device),
                       k_rope=None if self.k_rope is None else self.k_rope.to(device),
                       block_tables=self.block_tables.to(device))

    def oracle_args(self):
        def npy(t):
            if t is None:
                return None
            t = t.detach().cpu()
            if t.dtype == torch.bfloat16:
                t = t.float()
            return t.numpy()
        return dict(q_nope=npy(self.q_nope), q_rope=npy(self.q_rope), ct_kv=npy(self.ct_kv),
                    k_rope=npy(self.k_rope), block_tables=self.block_tables.cpu().numpy(),
                    context_lens=self.context_lens, q_seq_len=self.q_seq_len,
                    head_num=self.head_num, qk_scale=self.qk_scale,
                    mask_type=self.mask_type, calc_type=self.calc_type,
                    qk_descale=self.qk_descale, pv_descale=self.pv_descale)


def make_mla(seed, context_lens, q_seq_len, head_num, block_size, dtype, mask_type,
             calc_type, cache_mode, qk_scale, std=0.5, poison=False, max_block_num=None,
             name="custom", seed_val=None):
    context_lens = np.asarray(context_lens, dtype=np.int32)
    B = len(context_lens)
    if calc_type == MLA_CALC_UNDEFINED:
        qlens = np.ones(B, dtype=np.int32)
        q_seq_len = None
    else:
        q_seq_len = np.asarray(q_seq_len, dtype=np.int32)
        qlens = q_seq_len
    rng = np.random.default_rng(seed)
    gen = torch.Generator("cpu").manual_seed(seed if seed_val is None else seed_val)
    n_blocks, table, spare, need = _deal_blocks(rng, context_lens, block_size,
                                                max_block_num=max_block_num)
    T = int(qlens.sum())
    q_nope = _randn(gen, (T, head_num, 512), std, dtype)
    q_rope = _randn(gen, (T, head_num, 64), std, dtype)
    if cache_mode == MLA_CACHE_KVCACHE:
        ct_kv = _randn(gen, (n_blocks, block_size, 1, 576), std, dtype)
        k_rope = None
    else:
        ct_kv = _randn(gen, (n_blocks, block_size, 1, 512), std, dtype)
        k_rope = _randn(gen, (n_blocks, block_size, 1, 64), std, dtype)
    if poison:
        _poison_cache(ct_kv, table, context_lens, need, spare, block_size)
        if k_rope is not None:
            _poison_cache(k_rope, table, context_lens, need, spare, block_size)
    return MLACase(name=name, dtype=dtype, context_lens=context_lens, q_seq_len=q_seq_len,
                   head_num=head_num, block_size=block_size, mask_type=mask_type,
                   calc_type=calc_type, cache_mode=cache_mode, qk_scale=float(qk_scale),
                   q_nope=q_nope, q_rope=q_rope, ct_kv=ct_kv, k_rope=k_rope,
                   block_tables=torch.from_numpy(table))


def make_mla_int8(seed, context_lens, q_seq_len, head_num, block_size, dtype, mask_type,
                  calc_type, qk_scale, poison=False, max_block_num=None, name="custom", seed_val=None):
    """An MLA call over an int8 latent cache: qNope and ctKV int8, drawn as
    round(32 * N(0, 1)) clipped to [-127, 127] (a latent of std 0.5 quantised with
    step 1/64), qRope / kRope N(0, 0.5^2) in ``dtype``, per-head descales
    qkDescale = U(0.5, 1.5) / 64^2 and pvDescale = U(0.5, 1.5) / 64.  ``poison``
    fills the cache slots the operator must not read with 127 (int8) and NaN
    (kRope)."""
    context_lens = np.asarray(context_lens, dtype=np.int32)
    B = len(context_lens)
    if calc_type == MLA_CALC_UNDEFINED:
        qlens = np.ones(B, dtype=np.int32)
        q_seq_len = None
    else:
        q_seq_len = np.asarray(q_seq_len, dtype=np.int32)
        qlens = q_seq_len
    rng = np.random.default_rng(seed)
    gen = torch.Generator("cpu").manual_seed(seed if seed_val is None else seed_val)
    n_blocks, table, spare, need = _deal_blocks(rng, context_lens, block_size,
                                                max_block_num=max_block_num)
    T = int(qlens.sum())

    def q8(shape):
        return torch.randn(*shape, generator=gen).mul_(32.0).round_().clamp_(-127, 127).to(torch.int8)

    q_nope = q8((T, head_num, 512))
    q_rope = _randn(gen, (T, head_num, 64), 0.5, dtype)
    ct_kv = q8((n_blocks, block_size, 1, 512))
    k_rope = _randn(gen, (n_blocks, block_size, 1, 64), 0.5, dtype)
    qk_descale = (rng.uniform(0.5, 1.5, size=head_num) / 64.0 ** 2).astype(np.float32)
    pv_descale = (rng.uniform(0.5, 1.5, size=head_num) / 64.0).astype(np.float32)
    if poison:
        wide = ct_kv.view(torch.uint8)  # poison through a byte view: 127 in every unread slot
        mark = torch.zeros(ct_kv.shape, dtype=torch.float32)
        _poison_cache(mark, table, context_lens, need, spare, block_size)
        wide[torch.isnan(mark)] = 127
        _poison_cache(k_rope, table, context_lens, need, spare, block_size)
    return MLACase(name=name, dtype=dtype, context_lens=context_lens, q_seq_len=q_seq_len,
                   head_num=head_num, block_size=block_size, mask_type=mask_type,
                   calc_type=calc_type, cache_mode=MLA_CACHE_KROPE_CTKV, qk_scale=float(qk_scale),
                   q_nope=q_nope, q_rope=q_rope, ct_kv=ct_kv, k_rope=k_rope,
                   block_tables=torch.from_numpy(table), qk_descale=qk_descale, pv_descale=pv_descale)


def make_mla_config(name, poison=False, device=None):
    """MLA decode on the latent paged cache: batch 64, 128 heads, blockSize 128,
    contextLens ~ U{1024..8192}, bf16 N(0, 0.5^2), qkScale 1/sqrt(192), cacheMode 1
    (separate ctKV / kRope).  q_len 1 (calcType 0, maskType 0) or q_len 4 (calcType
    SPEC, maskType SPEC)."""
    k = MLA_CONFIGS[name]
    rng = np.random.default_rng(1000 + k)
    ctx = rng.integers(1024, 8192, size=64, endpoint=True)
    if name == "mla_decode_q1":
        c = make_mla(3000 + k, ctx, None, 128, 128, BF16, MLA_MASK_UNDEFINED,
                     MLA_CALC_UNDEFINED, MLA_CACHE_KROPE_CTKV, 1.0 / np.sqrt(192.0),
                     poison=poison, max_block_num=64, name=name, seed_val=2000 + k)
    else:
        c = make_mla(3000 + k, ctx, np.full(64, 4), 128, 128, BF16, MLA_MASK_SPEC,
                     MLA_CALC_SPEC, MLA_CACHE_KROPE_CTKV, 1.0 / np.sqrt(192.0),
                     poison=poison, max_block_num=64, name=name, seed_val=2000 + k)
    return c.to(device) if device is not None else c
