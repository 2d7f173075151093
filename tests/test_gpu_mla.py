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
