"""GPU parity of the PrefixEncoder call that reads an explicit compressed mask
(ATB page "压缩mask", section 约束说明; ATB page "PrefixEncoder", parameter table,
row mask) against the fp64 oracle's expansion of the same tile.

The tiles are inputs (workloads.gen.compressed_tile): the page's tiles as read
here (lower-triangular 0 / -inf norm mask, right-aligned col - row and
left-aligned col below the diagonal), and perturbed copies (extra bias, holes of
-inf) so that the kernel has to read every entry it uses.  Both sides get the same tile values
after the cast to the input type."""

import dataclasses

import numpy as np
import pytest
import torch

import workloads.gen as W
from tests.gpu_helpers import check_prefill_full, check_prefill_heads, gpu_prefill, log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


CASES = [
    # (seq_len, kv_seq_len, head_num, kv_head_num, D, bs): prefixes that start inside,
    # at and across 128-position blocks, ragged ends, an empty sequence
    ([300, 1, 0, 129], [700, 128, 5, 129], 8, 2, 128, 128),
    ([200, 77], [457, 333], 4, 4, 64, 16),
    ([256, 40], [256, 300], 4, 1, 128, 24),
    # headSize 128 with 64- and 256-key cache blocks (the direct-load kernel)
    ([257, 64, 3], [513, 64, 200], 8, 2, 128, 64),
    ([130, 500], [700, 500], 4, 4, 128, 256),
    # headSize 128 with 16- and 32-key cache blocks (the direct-load kernel, one
    # block id per wave's 16 rows of a tile)
    ([200, 77, 9], [457, 333, 9], 8, 2, 128, 16),
    ([130, 64], [301, 64], 4, 4, 128, 32),
    # headSize 64 with 64- and 256-key cache blocks (one block id per 64-key tile)
    ([190, 70], [450, 70], 4, 2, 64, 64),
    ([300, 5], [520, 300], 4, 4, 64, 256),
]


@pytest.mark.parametrize("mask_type", [9, 3, 4, 5])
@pytest.mark.parametrize("perturbed", [False, True])
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("ci", range(len(CASES)))
def test_compressed_mask_matches_oracle(mask_type, perturbed, dtype, ci):
    L, kv, H, KVH, D, bs = CASES[ci]
    log(f"case compressed mask={mask_type} perturbed={perturbed} dtype={dtype} case={ci}")
    slopes = "alibi" if mask_type != 9 else None
    c = W.make_prefill(211 + ci, np.array(L), np.array(kv), H, KVH, D, bs, dtype, mask_type,
                       1.0 / np.sqrt(D), slopes=slopes, poison=True,
                       name=f"tile{mask_type}-{'pert' if perturbed else 'page'}-{dtype}-c{ci}")
    c = dataclasses.replace(c, mask_tile=W.compressed_tile(mask_type, dtype, 17 + ci if perturbed else None))
    c = c.to(DEV)
    out, lse = gpu_prefill(c)
    check_prefill_full(c, out, lse)


@pytest.mark.parametrize("mask_type", [9, 3, 4, 5])
def test_page_tile_equals_generated_mask(mask_type):
    # the page's tile gives the result of the generated mask of the same type (both
    # paths checked against one oracle, the generated one without any tile)
    log(f"case compressed page tile vs generated mask={mask_type}")
    slopes = "alibi" if mask_type != 9 else None
    c = W.make_prefill(230, np.array([390, 130]), np.array([1000, 130]), 4, 2, 128, 128, "bf16", mask_type,
                       1.0 / np.sqrt(128), slopes=slopes, poison=True, name=f"gen{mask_type}").to(DEV)
    o_gen, l_gen = gpu_prefill(c)
    check_prefill_full(c, o_gen, l_gen)
    ct = dataclasses.replace(c, mask_tile=W.compressed_tile(mask_type, "bf16").to(DEV))
    o_tile, l_tile = gpu_prefill(ct)
    check_prefill_full(c, o_tile, l_tile)


def test_row_hidden_by_the_tile_is_zero():
    # a norm tile whose row 5 is all -inf: query position 5 (no prefix) sees nothing
    log("case compressed norm tile with an empty row")
    tile = W.compressed_tile(9, "fp16")
    tile[5, :] = float("-inf")
    c = W.make_prefill(240, np.array([40]), np.array([40]), 2, 2, 64, 16, "fp16", 9, 0.125,
                       poison=True, name="empty-row")
    c = dataclasses.replace(c, mask_tile=tile).to(DEV)
    out, lse = gpu_prefill(c)
    assert torch.all(out[5] == 0)
    assert torch.all(torch.isneginf(lse[5]))
    keep = torch.ones(40, dtype=torch.bool)
    keep[5] = False
    import oracle
    ro, rl = oracle.prefix_encoder(**c.oracle_args())
    assert np.abs(out[keep].float().cpu().numpy() - ro[keep.numpy()]).max() <= 5e-3
    assert np.all(np.isneginf(rl[5]))


@pytest.mark.parametrize("name", ["prefix_gqa_causal", "alibi_right_4x4096", "alibi_sqrt_16384",
                                  "alibi_left_16384"])
def test_compressed_mask_full_size_sampled(name):
    # the bench's compressed-tile calls: the full workloads with the page's tile
    log(f"case compressed full-size {name} (sampled rows)")
    from tests.gpu_helpers import check_prefill_sampled
    c = W.make_prefill_config(name, poison=True)
    c = dataclasses.replace(c, mask_tile=W.compressed_tile(c.mask_type, c.dtype)).to(DEV)
    out, lse = gpu_prefill(c)
    check_prefill_sampled(c, out, lse, n=160, seed=11)
    assert torch.isfinite(out.float()).all()


def test_row_hidden_by_the_tile_is_zero_dma_path():
    # the same with headSize 128 and 128-key blocks (the direct-load kernel)
    log("case compressed norm tile with an empty row, headSize 128")
    tile = W.compressed_tile(9, "bf16")
    tile[5, :] = float("-inf")
    c = W.make_prefill(241, np.array([40, 200]), np.array([40, 300]), 8, 2, 128, 128, "bf16", 9,
                       1.0 / np.sqrt(128), poison=True, name="empty-row-128")
    c = dataclasses.replace(c, mask_tile=tile).to(DEV)
    out, lse = gpu_prefill(c)
    assert torch.all(out[5] == 0)
    assert torch.all(torch.isneginf(lse[5]))
    import oracle
    ro, rl = oracle.prefix_encoder(**c.oracle_args())
    keep = np.ones(240, dtype=bool)
    keep[5] = False
    assert np.abs(out.float().cpu().numpy()[keep] - ro[keep]).max() <= 2e-2
    l = lse.cpu().numpy()[keep]
    assert (np.abs(l - rl[keep]) / np.maximum(1.0, np.abs(rl[keep]))).max() <= 1e-3


@pytest.mark.parametrize("mask_type", [3, 4, 5])
def test_alibi_tile_zero_and_negative_slopes(mask_type):
    # heads with slope 0 and negative slopes: a -inf entry still hides its key
    # (slope * -inf is not -inf there), headSize 128 and 128-key blocks
    log(f"case compressed ALiBi tile mask={mask_type} with zero / negative slopes")
    slopes = np.array([0.5, 0.0, -0.03125, 0.125, 0.0, 0.0625, -0.0078125, 0.25], dtype=np.float32)
    c = W.make_prefill(250 + mask_type, np.array([300, 129]), np.array([700, 129]), 8, 2, 128, 128, "bf16",
                       mask_type, 1.0 / np.sqrt(128), slopes=slopes, poison=True, name=f"slopes{mask_type}")
    c = dataclasses.replace(c, mask_tile=W.compressed_tile(mask_type, "bf16", 31)).to(DEV)
    out, lse = gpu_prefill(c)
    check_prefill_full(c, out, lse)


@pytest.mark.parametrize("mask_type", [3, 4, 5])
def test_tile_contents_read_at_each_execution(mask_type):
    # one planned call run twice, the tile overwritten in place between the runs:
    # each run follows the tile it found (ALiBi tiles on the direct-load
    # kernel go through the execution's fp32 copy of the tile)
    import masked_paged_attention_amd as mpa
    log(f"case compressed tile rewritten between two executions mask={mask_type}")
    c = W.make_prefill(260 + mask_type, np.array([300, 129]), np.array([700, 129]), 8, 2, 128, 128, "bf16",
                       mask_type, 1.0 / np.sqrt(128), slopes="alibi", poison=True, name=f"rerun{mask_type}")
    t1 = W.compressed_tile(mask_type, "bf16")
    t2 = W.compressed_tile(mask_type, "bf16", 41)
    c = c.to(DEV)
    tile = t1.to(DEV).clone()
    op = mpa.PrefixEncoder(c.query, c.key, c.value, c.block_tables, c.seq_len, c.kv_seq_len,
                           mask_type=c.mask_type, qk_scale=c.qk_scale,
                           slopes=torch.as_tensor(c.slopes, device=DEV), return_lse=True,
                           compressed_mask=tile)
    for t in (t1, t2):
        tile.copy_(t.to(DEV))
        out, lse = op.run()
        torch.cuda.synchronize()
        check_prefill_full(dataclasses.replace(c, mask_tile=t), out.clone(), lse.clone())
    op.close()


@pytest.mark.parametrize("bias_seed", [None, 43])
def test_sqrt_tile_long_sequence(bias_seed):
    # the sqrt tile over 8192 positions, every row of three heads: key blocks up
    # to 63 behind a row's own 128-block, with the page's tile (distances 1..255
    # behind the diagonal) and with an extra bias on it that widens them (no
    # -inf behind the diagonal)
    log(f"case sqrt tile, 8192 tokens, extra bias seed {bias_seed}")
    c = W.make_prefill(270, np.array([8192]), np.array([8192]), 4, 4, 128, 128, "bf16", 4,
                       1.0 / np.sqrt(128), slopes="alibi", poison=True, name=f"sqrtfar{bias_seed}")
    tile = W.compressed_tile(4, "bf16")
    if bias_seed is not None:
        rng = np.random.default_rng(bias_seed)
        extra = torch.as_tensor(-0.25 * rng.integers(0, 200, size=tuple(tile.shape)), dtype=torch.float32)
        tile = (tile.float() + extra).to(tile.dtype)
    c = dataclasses.replace(c, mask_tile=tile).to(DEV)
    out, lse = gpu_prefill(c)
    check_prefill_heads(c, out, lse, [0, 1, 3])


@pytest.mark.parametrize("mask_type,D,bs", [(3, 128, 128), (4, 128, 16), (5, 128, 64), (9, 128, 128),
                                            (3, 64, 64), (4, 128, 24)])
def test_compressed_mask_workspace_size(mask_type, D, bs):
    # the workspace holds the launch plan, and for the ALiBi tiles on the
    # direct-load kernel (headSize 128, power-of-two blockSize >= 16) the tile's
    # 256 KB fp32 copy after it; other shapes read the tile in place
    import masked_paged_attention_amd as mpa
    log(f"case compressed-mask workspace size mask={mask_type} D={D} bs={bs}")
    L, kv = np.array([300, 129]), np.array([700, 129])
    c = W.make_prefill(280 + mask_type, L, kv, 4, 2, D, bs, "bf16", mask_type, 1.0 / np.sqrt(D),
                       slopes="alibi" if mask_type != 9 else None, poison=False, name="ws").to(DEV)
    tile = W.compressed_tile(mask_type, "bf16").to(DEV)
    slopes = None if c.slopes is None else torch.as_tensor(c.slopes, device=DEV)
    op = mpa.PrefixEncoder(c.query, c.key, c.value, c.block_tables, c.seq_len, c.kv_seq_len,
                           mask_type=mask_type, qk_scale=c.qk_scale, slopes=slopes, compressed_mask=tile)
    plan_ws = mpa.plan_prefill(L, kv, mask_type, 4, 2, head_size=D, with_workspace=True)[-1]
    copy = 256 * 256 * 4 if (mask_type != 9 and D == 128 and bs >= 16 and bs & (bs - 1) == 0) else 0
    assert op.workspace.numel() == plan_ws + copy
    op.close()
