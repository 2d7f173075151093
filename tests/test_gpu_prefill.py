"""GPU parity of the prefill (PrefixEncoder) kernel against the fp64 oracle, through
the C ABI, plus GPU-side invariants.  Tolerances: max-abs 5e-3 (fp16), 2e-2
(bf16); LSE within 1e-3 * max(1, |LSE|)."""

import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import (check_prefill_full, check_prefill_heads, check_prefill_sampled, gpu_prefill, log)

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _case(seed, seq, prefix, H, KVH, D, bs, dtype, mask, poison=True, pad_to=None, scale=None):
    seq = np.asarray(seq)
    kv = seq + np.asarray(prefix)
    slopes = "alibi" if mask in (3, 4, 5) else None
    c = W.make_prefill(seed, seq, kv, H, KVH, D, bs, dtype, mask,
                       scale if scale is not None else 1.0 / np.sqrt(D), slopes=slopes,
                       poison=poison, pad_to=pad_to, name=f"s{seed}-{dtype}-D{D}-m{mask}-bs{bs}")
    return c.to(DEV)


def test_tiny_causal_config():
    log("case tiny_causal (batch 2, seqLen [16,37], fp16, D 64, blockSize 16)")
    c = W.make_prefill_config("tiny_causal", poison=True, device=DEV)
    out, lse = gpu_prefill(c)
    check_prefill_full(c, out, lse)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("mask", [0, 3, 4, 5, 9])
def test_small_all_masks(dtype, D, mask):
    bs = {64: 16, 128: 24}[D]
    log(f"case small dtype={dtype} D={D} mask={mask} bs={bs}")
    c = _case(10 + mask + D, [150, 67, 1], [0, 90, 200], 4, 2, D, bs, dtype, mask)
    out, lse = gpu_prefill(c)
    check_prefill_full(c, out, lse)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("bs", [16, 32])
@pytest.mark.parametrize("mask", [0, 3, 4, 5, 9])
def test_head_size_128_small_blocks(dtype, bs, mask):
    # headSize 128 with 16- and 32-key cache blocks (the direct-load kernel, one
    # block id per wave's 16 rows of a tile): kvSeqLen 150, 157, 201, 224, 256,
    # 180, 110 put the last key of the final tile in every 16-row group and on a
    # tile boundary, with prefixes, GQA and NaN in every slot not to be read
    log(f"case D=128 bs={bs} dtype={dtype} mask={mask}")
    c = _case(400 + bs + mask, [150, 67, 1, 211, 256, 100, 110], [0, 90, 200, 13, 0, 80, 0], 4, 2, 128, bs,
              dtype, mask)
    out, lse = gpu_prefill(c)
    check_prefill_full(c, out, lse)


@pytest.mark.parametrize("bs", [16, 32])
def test_head_size_128_small_blocks_gqa4(bs):
    log(f"case D=128 bs={bs} GQA 8/2 and MQA 4/1")
    for H, KVH in ((8, 2), (4, 1)):
        c = _case(420 + bs + H, [300, 129, 45], [700, 0, 19], H, KVH, 128, bs, "bf16", 4)
        out, lse = gpu_prefill(c)
        check_prefill_full(c, out, lse)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("bs", [64, 128, 256])
@pytest.mark.parametrize("mask", [0, 3, 4, 5, 9])
def test_head_size_64_whole_tile_blocks(dtype, bs, mask):
    # headSize 64 with a power-of-two blockSize >= 64: every 64-key tile inside one
    # cache block (one block id per tile, fetched ahead) -- random block
    # permutation, NaN in every slot that must not be read
    log(f"case D=64 bs={bs} dtype={dtype} mask={mask}")
    c = _case(300 + bs + mask, [333, 70, 1], [90, 400, 250], 4, 2, 64, bs, dtype, mask)
    out, lse = gpu_prefill(c)
    check_prefill_full(c, out, lse)


@pytest.mark.parametrize("bs", [64, 256])
def test_head_size_64_whole_tile_blocks_chunked(bs):
    log(f"case D=64 bs={bs} chunked")
    c = W.make_prefill(310 + bs, np.array([300, 200]), np.array([800, 200]), 8, 2, 64, bs, "bf16", 9,
                       0.125, poison=True, chunk=96, name=f"chunk96-D64-bs{bs}").to(DEV)
    out, lse = gpu_prefill(c)
    check_prefill_full(c, out, lse)


@pytest.mark.parametrize("H,KVH", [(8, 8), (8, 4), (8, 2), (16, 2), (24, 3), (6, 1)])
def test_gqa_ratios(H, KVH):
    log(f"case gqa H={H} KVH={KVH}")
    c = _case(40 + H + KVH, [300, 129], [700, 0], H, KVH, 128, 128, "bf16", 9)
    out, lse = gpu_prefill(c)
    check_prefill_full(c, out, lse)


def test_padded_layout_leaves_padding_rows_untouched():
    log("case padded layout with sentinel")
    c = _case(51, [200, 5, 129], [30, 0, 64], 4, 4, 128, 16, "fp16", 3, pad_to=256)
    out, lse = gpu_prefill(c, sentinel=7.0)
    check_prefill_full(c, out, lse)
    o = out.float().cpu().numpy()
    l = lse.cpu().numpy()
    for b, L in enumerate(c.seq_len):
        lo, hi = 256 * b + L, 256 * (b + 1)
        assert (o[lo:hi] == 7.0).all() and (l[lo:hi] == 7.0).all(), f"padding rows of sequence {b} written"


def test_empty_and_tiny_sequences():
    log("case empty / single-row sequences")
    c = _case(53, [0, 70, 0, 1, 33], [40, 30, 0, 0, 0], 4, 4, 64, 16, "bf16", 9)
    out, lse = gpu_prefill(c)
    check_prefill_full(c, out, lse)


def test_deterministic_and_paged_equals_contiguous():
    log("case determinism + paged vs contiguous")
    c = _case(55, [260, 190], [100, 333], 8, 2, 128, 32, "bf16", 3, poison=False)
    o1, l1 = gpu_prefill(c)
    o2, l2 = gpu_prefill(c)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # Same values, blocks laid out in order (identity block table).
    bs = c.block_size
    key = torch.zeros_like(c.key)
    value = torch.zeros_like(c.value)
    bt = torch.zeros_like(c.block_tables)
    nxt = 0
    for b in range(c.batch):
        for blk in range(-(-int(c.kv_seq_len[b]) // bs)):
            src = int(c.block_tables[b, blk])
            key[nxt] = c.key[src]
            value[nxt] = c.value[src]
            bt[b, blk] = nxt
            nxt += 1
    import dataclasses
    c2 = dataclasses.replace(c, key=key, value=value, block_tables=bt)
    o3, l3 = gpu_prefill(c2)
    assert torch.equal(o1, o3) and torch.equal(l1, l3)


def test_left_aligned_equals_right_aligned():
    log("case left vs right ALiBi")
    c = _case(57, [300, 80], [0, 500], 4, 4, 128, 128, "bf16", 3, poison=False)
    o_r, l_r = gpu_prefill(c)
    import dataclasses
    c5 = dataclasses.replace(c, mask_type=5)
    o_l, l_l = gpu_prefill(c5)
    assert torch.equal(o_r, o_l)
    starts = c.row_starts()
    for b in range(c.batch):
        a = (c.kv_seq_len[b] - c.seq_len[b]) + np.arange(c.seq_len[b])
        d = (l_l - l_r)[starts[b]:starts[b] + c.seq_len[b]].cpu().numpy()
        want = c.slopes[None, :].astype(np.float64) * a[:, None]
        assert np.abs(d - want).max() <= 1e-3 * max(1.0, np.abs(want).max())


def test_gqa_equals_mha_with_repeated_kv():
    log("case GQA vs MHA")
    c = _case(59, [200, 90], [64, 0], 8, 2, 128, 16, "fp16", 9, poison=False)
    o1, l1 = gpu_prefill(c)
    import dataclasses
    g = c.head_num // c.kv_head_num
    c2 = dataclasses.replace(c, key=c.key.repeat_interleave(g, dim=2).contiguous(),
                             value=c.value.repeat_interleave(g, dim=2).contiguous(),
                             kv_head_num=c.head_num)
    o2, l2 = gpu_prefill(c2)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("name", ["prefix_gqa_causal", "alibi_right_4x4096", "alibi_sqrt_16384",
                                  "alibi_left_16384", "alibi_sqrt_varlen16", "alibi_left_padded16"])
def test_full_size_configs_sampled(name):
    # sampled rows of every head, then every row of the first and the last head
    # (the launch configuration the benchmark times)
    log(f"case full-size {name}")
    c = W.make_prefill_config(name, poison=True, device=DEV)
    out, lse = gpu_prefill(c)
    check_prefill_sampled(c, out, lse, n=160, seed=1)
    check_prefill_heads(c, out, lse, [0, c.head_num - 1])


def test_packed_equals_padded_full_size():
    log("case packed vs padded (16 lognormal sequences, sqrt ALiBi)")
    c = W.make_prefill_config("alibi_sqrt_varlen16", poison=False, device=DEV)
    cp = W.pad_prefill_case(c, 8192, 123, poison=True, device=DEV)
    o1, l1 = gpu_prefill(c)
    o2, l2 = gpu_prefill(cp)
    s1, s2 = c.row_starts(), cp.row_starts()
    for b in range(c.batch):
        L = int(c.seq_len[b])
        assert torch.equal(o1[s1[b]:s1[b] + L], o2[s2[b]:s2[b] + L])
        assert torch.equal(l1[s1[b]:s1[b] + L], l2[s2[b]:s2[b] + L])


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("mask", [3, 5])
@pytest.mark.parametrize("scale", [0.0, 1e-35, -1.0 / np.sqrt(128)])
def test_linear_alibi_zero_tiny_and_negative_scales(dtype, mask, scale):
    # The linear-ALiBi kernel (headSize 128, blockSize 128) starts each tile's S^T
    # accumulator at slope*C/qkScale; at qkScale 0 and below 2^-100 it drops the
    # q.k part instead, and a negative qkScale flips that start's sign.
    log(f"case linear ALiBi dtype={dtype} mask={mask} qkScale={scale}")
    c = _case(420 + mask, [300, 129, 70], [200, 0, 520], 4, 2, 128, 128, dtype, mask, scale=scale)
    out, lse = gpu_prefill(c)
    check_prefill_full(c, out, lse)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("mask", [3, 4, 5])
def test_alibi_score_spikes_move_the_running_max(dtype, mask):
    # Keys far from the diagonal with very large dot products: the diagonal tiles
    # come first, so the running max is set early and these keys then exceed it
    # by far more than the rescale slack (2^10), which must move the reference
    # (the full path).
    log(f"case score spikes dtype={dtype} mask={mask}")
    c = W.make_prefill(71 + mask, np.array([700, 300]), np.array([700, 500]), 4, 4, 128, 128, dtype,
                       mask, 1.0 / np.sqrt(128), slopes="alibi", poison=False, name=f"spike-{dtype}-m{mask}")
    bs = c.block_size
    for b, keys in [(0, [5, 130, 131, 400]), (1, [3, 260])]:
        for j in keys:
            blk = int(c.block_tables[b, j // bs])
            c.key[blk, j % bs] *= 25
    c = c.to(DEV)
    out, lse = gpu_prefill(c)
    check_prefill_full(c, out, lse)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("D,bs,chunk", [(128, 128, 64), (128, 128, 100), (128, 64, 256), (128, 24, 37),
                                        (128, 16, 48), (128, 32, 100), (64, 16, 48)])
def test_chunked_local_mask(dtype, D, bs, chunk):
    # chunked local causal mask: row at absolute a sees keys j <= a of its own chunk
    log(f"case chunked dtype={dtype} D={D} bs={bs} chunk={chunk}")
    c = W.make_prefill(83 + chunk, np.array([300, 200, 17]), np.array([800, 200, 107]), 8, 2, D, bs, dtype,
                       9, 1.0 / np.sqrt(D), poison=True, chunk=chunk,
                       name=f"chunk{chunk}-{dtype}-D{D}-bs{bs}").to(DEV)
    out, lse = gpu_prefill(c)
    check_prefill_full(c, out, lse)


def test_chunked_mask_with_a_long_chunk_equals_causal():
    log("case chunked (chunk >= kvSeqLen) equals causal")
    c = W.make_prefill(85, np.array([260, 90]), np.array([700, 90]), 4, 4, 128, 128, "bf16", 9,
                       1.0 / np.sqrt(128), poison=False, chunk=4096).to(DEV)
    o1, l1 = gpu_prefill(c)
    import dataclasses
    o2, l2 = gpu_prefill(dataclasses.replace(c, chunk=0))
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_chunked_full_size_sampled():
    # the bench's chunked call: one 16384-token bf16 sequence, 40 heads, chunk 2048
    log("case chunked full-size 16384 chunk 2048 (sampled rows)")
    c = W.make_prefill(87, np.array([16384]), np.array([16384]), 40, 40, 128, 128, "bf16", 9,
                       1.0 / np.sqrt(128.0), poison=True, chunk=2048).to(DEV)
    out, lse = gpu_prefill(c)
    check_prefill_sampled(c, out, lse, n=160, seed=12)


@pytest.mark.parametrize("mask", [9, 3])
def test_long_prefix_sampled(mask):
    # a ~60K-key cached prefix: large block-table indices and offsets
    log(f"case prefill long prefix mask={mask} (sampled rows)")
    slopes = "alibi" if mask == 3 else None
    c = W.make_prefill(93, np.array([700, 33]), np.array([60000, 40000]), 8, 2, 128, 128, "bf16", mask,
                       1.0 / np.sqrt(128.0), slopes=slopes, poison=True).to(DEV)
    out, lse = gpu_prefill(c)
    check_prefill_sampled(c, out, lse, n=96, seed=13)
