"""GPU parity of the split-KV MLA decode (split kernel + LSE combine) against the
fp64 oracle, through the C ABI."""

import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import check_mla, gpu_mla, log

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("cache_mode", [0, 1])
def test_small_decode(dtype, cache_mode):
    log(f"case mla small q_len 1 dtype={dtype} cacheMode={cache_mode}")
    c = W.make_mla(61, [100, 37, 300, 1], None, 16, 64, dtype, 0, 0, cache_mode, 0.07,
                   poison=True).to(DEV)
    out, lse = gpu_mla(c)
    check_mla(c, out, lse)


@pytest.mark.parametrize("mask", [0, 1])
def test_spec_decode_128_heads(mask):
    log(f"case mla spec q_len [4, 2, 3] H 128 mask={mask}")
    c = W.make_mla(63, [70, 500, 1029], [4, 2, 3], 128, 128, "bf16", mask, 1, 1, 1 / np.sqrt(192),
                   poison=True).to(DEV)
    out, lse = gpu_mla(c)
    check_mla(c, out, lse)


@pytest.mark.parametrize("bs", [8, 16])
@pytest.mark.parametrize("cache_mode", [0, 1])
def test_small_block_sizes(bs, cache_mode):
    # 8- and 16-key cache blocks: one block id per loader wave's 8 keys of a tile;
    # contexts ending in every 8-key group of a 32-key tile, q_len 1..4 with the
    # SPEC mask, sequences cut across pieces (128 heads), NaN in unread slots
    log(f"case mla blockSize {bs} cacheMode {cache_mode}")
    ctx = [100, 37, 300, 1, 9, 17, 26, 2049, 771]
    ql = [1, 2, 4, 1, 3, 1, 2, 4, 1]
    c = W.make_mla(75 + bs, ctx, ql, 128, bs, "bf16", 1, 1, cache_mode, 1 / np.sqrt(192), poison=True).to(DEV)
    out, lse = gpu_mla(c)
    rng = np.random.default_rng(9)
    T = c.n_tokens
    rows = sorted({(int(rng.integers(T)), int(rng.integers(128))) for _ in range(300)} |
                  {(t, h) for t in range(T) for h in (0, 127)})
    check_mla(c, out, lse, rows=rows)


def test_odd_block_size_and_heads():
    log("case mla blockSize 24, 20 heads, q_len 3")
    c = W.make_mla(65, [95, 48, 3], [3, 3, 3], 20, 24, "bf16", 1, 1, 0, 0.05, poison=True).to(DEV)
    out, lse = gpu_mla(c)
    check_mla(c, out, lse)


def test_deterministic():
    log("case mla determinism")
    c = W.make_mla(67, [800, 2100], None, 128, 128, "bf16", 0, 0, 1, 0.07).to(DEV)
    o1, l1 = gpu_mla(c)
    o2, l2 = gpu_mla(c)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("name", ["mla_decode_q1", "mla_spec_q4"])
def test_full_size_sampled(name):
    log(f"case mla full-size {name}")
    c = W.make_mla_config(name, poison=True, device=DEV)
    out, lse = gpu_mla(c)
    rng = np.random.default_rng(3)
    T, H = c.n_tokens, c.head_num
    rows = sorted({(int(rng.integers(T)), int(rng.integers(H))) for _ in range(160)} |
                  {(0, 0), (T - 1, H - 1)})
    check_mla(c, out, lse, rows=rows)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    # every head of every token of two whole sequences: the shortest and the longest
    qlens = [1] * c.batch if c.q_seq_len is None else [int(x) for x in c.q_seq_len]
    tok0 = np.concatenate([[0], np.cumsum(qlens)[:-1]])
    for b in (int(np.argmin(c.context_lens)), int(np.argmax(c.context_lens))):
        rows = [(int(tok0[b]) + t, h) for t in range(qlens[b]) for h in range(H)]
        check_mla(c, out, lse, rows=rows)


def test_many_short_sequences():
    """300 sequences of 1..40 keys: pieces hold many segments, most sequences are
    one segment (direct output), some are cut between pieces (merged)."""
    log("case mla 300 short sequences, 32 heads")
    rng = np.random.default_rng(71)
    ctx = [int(x) for x in rng.integers(1, 41, size=300)]
    c = W.make_mla(71, ctx, None, 32, 32, "bf16", 0, 0, 1, 0.08, poison=True).to(DEV)
    out, lse = gpu_mla(c)
    check_mla(c, out, lse)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_mixed_lengths_cross_pieces(dtype):
    """Long and short sequences side by side at 128 heads: segments cross piece
    boundaries at arbitrary tiles; ragged tails; cacheMode 0 (rope inside ctKV)."""
    log(f"case mla mixed lengths 128 heads {dtype}")
    ctx = [5000, 33, 1, 4096, 127, 7777, 64, 2500]
    c = W.make_mla(73, ctx, None, 128, 128, dtype, 0, 0, 0, 1 / np.sqrt(192), poison=True).to(DEV)
    out, lse = gpu_mla(c)
    rng = np.random.default_rng(5)
    rows = sorted({(int(rng.integers(len(ctx))), int(rng.integers(128))) for _ in range(200)} |
                  {(b, h) for b in range(len(ctx)) for h in (0, 127)})
    check_mla(c, out, lse, rows=rows)


@pytest.mark.parametrize("mask", [0, 1])
def test_prefill_calc_type(mask):
    # calcType PREFILL: whole prompts of new tokens (qSeqLen up to contextLens), with
    # the same masks as SPEC; full parity on every (token, head).
    log(f"case mla prefill q_len [40, 64, 9] H 16 mask={mask}")
    c = W.make_mla(69, [40, 700, 300], [40, 64, 9], 16, 128, "bf16", mask, 3, 1, 1 / np.sqrt(192),
                   poison=True).to(DEV)
    out, lse = gpu_mla(c)
    check_mla(c, out, lse)


def test_prefill_128_heads_sampled():
    log("case mla prefill q_len [256, 130] H 128 causal (sampled rows)")
    c = W.make_mla(71, [2048, 900], [256, 130], 128, 128, "bf16", 1, 3, 1, 1 / np.sqrt(192),
                   poison=True).to(DEV)
    out, lse = gpu_mla(c)
    rng = np.random.default_rng(4)
    T, H = c.n_tokens, c.head_num
    rows = sorted({(int(rng.integers(T)), int(rng.integers(H))) for _ in range(160)} |
                  {(0, 0), (T - 1, H - 1), (255, 5), (256, 7)})
    check_mla(c, out, lse, rows=rows)


def _prefill_rows(c, n, seed):
    rng = np.random.default_rng(seed)
    T, H = c.n_tokens, c.head_num
    tok0 = np.concatenate([[0], np.cumsum(c.q_seq_len)[:-1]])
    edge = {(int(t0) + t, h) for t0, q in zip(tok0, c.q_seq_len) for t in (0, 1, int(q) - 1) for h in (0, 63, 127)}
    return sorted({(int(rng.integers(T)), int(rng.integers(H))) for _ in range(n)} | edge)


@pytest.mark.parametrize("mask", [0, 1])
def test_prefill_whole_sequences(mask):
    # long prompts at 128 heads: the whole-sequence plan (no key split, no merge),
    # each row group's key range ending at its last token's limit under the mask
    log(f"case mla prefill whole sequences q_len 200..256 H 128 mask={mask}")
    c = W.make_mla(77 + mask, [1024, 2048, 700, 1500], [256, 256, 200, 256], 128, 128, "bf16", mask, 3, 1,
                   1 / np.sqrt(192), poison=True).to(DEV)
    out, lse = gpu_mla(c)
    check_mla(c, out, lse, rows=_prefill_rows(c, 300, 12 + mask))
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()


@pytest.mark.parametrize("bs", [16, 128])
def test_prefill_whole_sequences_fp16_concatenated_cache(bs):
    # the whole-sequence plan over the 576-wide cache (cacheMode 0) in fp16, with
    # 16-key blocks (one block id per loader wave's 8 keys) and 128-key blocks
    log(f"case mla prefill whole sequences fp16 cacheMode 0 blockSize {bs}")
    c = W.make_mla(85 + bs, [900, 1333, 2050, 420], [256, 256, 256, 256], 128, bs, "fp16", 1, 3, 0,
                   1 / np.sqrt(192), poison=True).to(DEV)
    out, lse = gpu_mla(c)
    check_mla(c, out, lse, rows=_prefill_rows(c, 200, 16 + bs))


def test_int8_prefill_whole_sequences():
    log("case mla int8 prefill whole sequences q_len 256 H 128 causal")
    c = W.make_mla_int8(79, [1024, 2048, 700, 1500], [256, 256, 200, 256], 128, 128, "bf16", 1, 3,
                        1 / np.sqrt(192), poison=True).to(DEV)
    out, lse = gpu_mla(c)
    check_mla(c, out, lse, rows=_prefill_rows(c, 200, 14))
    # 16-key blocks: the int8 cache's per-row block lookups
    c = W.make_mla_int8(80, [777, 1500, 1030, 96], [256, 256, 256, 96], 128, 16, "fp16", 1, 3,
                        1 / np.sqrt(192), poison=True).to(DEV)
    out, lse = gpu_mla(c)
    check_mla(c, out, lse, rows=_prefill_rows(c, 200, 15))


# ---- int8 latent cache (qNope / ctKV int8, per-head qkDescale / pvDescale) ----

@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_int8_small_decode(dtype):
    log(f"case mla int8 small q_len 1 dtype={dtype}")
    c = W.make_mla_int8(81, [100, 37, 300, 1], None, 16, 64, dtype, 0, 0, 0.07, poison=True).to(DEV)
    out, lse = gpu_mla(c)
    check_mla(c, out, lse)


@pytest.mark.parametrize("mask", [0, 1])
def test_int8_spec_128_heads(mask):
    log(f"case mla int8 spec q_len [4, 2, 3] H 128 mask={mask}")
    c = W.make_mla_int8(83, [70, 500, 1029], [4, 2, 3], 128, 128, "bf16", mask, 1, 1 / np.sqrt(192),
                        poison=True).to(DEV)
    out, lse = gpu_mla(c)
    check_mla(c, out, lse)


def test_int8_odd_block_size_and_heads():
    # blockSize 24: every key looks its block up (no one-block tiles)
    log("case mla int8 blockSize 24, 20 heads, q_len 3")
    c = W.make_mla_int8(85, [95, 48, 3], [3, 3, 3], 20, 24, "fp16", 1, 1, 0.05, poison=True).to(DEV)
    out, lse = gpu_mla(c)
    check_mla(c, out, lse)


def test_int8_mixed_lengths_cross_pieces():
    log("case mla int8 mixed lengths 128 heads")
    ctx = [5000, 33, 1, 4096, 127, 7777, 64, 2500]
    c = W.make_mla_int8(87, ctx, None, 128, 128, "bf16", 0, 0, 1 / np.sqrt(192), poison=True).to(DEV)
    out, lse = gpu_mla(c)
    rng = np.random.default_rng(6)
    rows = sorted({(int(rng.integers(len(ctx))), int(rng.integers(128))) for _ in range(200)} |
                  {(b, h) for b in range(len(ctx)) for h in (0, 127)})
    check_mla(c, out, lse, rows=rows)


def test_int8_full_size_sampled():
    # the decode workload's shape (64 sequences, contextLens U{1024..8192}, 128 heads)
    log("case mla int8 full-size decode (sampled rows)")
    rng = np.random.default_rng(1001)
    ctx = rng.integers(1024, 8192, size=64, endpoint=True)
    c = W.make_mla_int8(89, ctx, None, 128, 128, "bf16", 0, 0, 1 / np.sqrt(192), poison=True,
                        max_block_num=64).to(DEV)
    out, lse = gpu_mla(c)
    rng = np.random.default_rng(7)
    T, H = c.n_tokens, c.head_num
    rows = sorted({(int(rng.integers(T)), int(rng.integers(H))) for _ in range(160)} |
                  {(0, 0), (T - 1, H - 1)})
    check_mla(c, out, lse, rows=rows)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    # every head of every token of two whole sequences: the shortest and the longest
    qlens = [1] * c.batch if c.q_seq_len is None else [int(x) for x in c.q_seq_len]
    tok0 = np.concatenate([[0], np.cumsum(qlens)[:-1]])
    for b in (int(np.argmin(c.context_lens)), int(np.argmax(c.context_lens))):
        rows = [(int(tok0[b]) + t, h) for t in range(qlens[b]) for h in range(H)]
        check_mla(c, out, lse, rows=rows)


def test_int8_prefill_and_determinism():
    log("case mla int8 prefill q_len [40, 64, 9] H 16 causal, run twice")
    c = W.make_mla_int8(91, [40, 700, 300], [40, 64, 9], 16, 128, "bf16", 1, 3, 1 / np.sqrt(192),
                        poison=True).to(DEV)
    o1, l1 = gpu_mla(c)
    check_mla(c, o1, l1)
    o2, l2 = gpu_mla(c)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_long_context_sampled():
    # contexts up to 64K keys next to short ones
    log("case mla long contexts (sampled rows)")
    ctx = [65536, 300, 40000, 1]
    c = W.make_mla(95, ctx, None, 64, 128, "bf16", 0, 0, 1, 1 / np.sqrt(192), poison=True).to(DEV)
    out, lse = gpu_mla(c)
    rng = np.random.default_rng(8)
    rows = sorted({(int(rng.integers(len(ctx))), int(rng.integers(64))) for _ in range(64)} |
                  {(b, h) for b in range(len(ctx)) for h in (0, 63)})
    check_mla(c, out, lse, rows=rows)
