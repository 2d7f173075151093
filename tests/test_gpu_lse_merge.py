"""GPU parity of the LSE merge of attention partials (mpaLseMerge, the merge behind
the MLA page's lse output and RING calcType) against the fp64 oracle merge, and its
use for chunked prefill: a causal prefix-encoder call split into key chunks and
merged by LSE equals the oracle of the whole call.  Tolerances as the other tests:
max-abs 5e-3 (fp16), 2e-2 (bf16); LSE within 1e-3 * max(1, |LSE|)."""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import TOL, LSE_REL, check_prefill_full, gpu_prefill, log

pytestmark = pytest.mark.gpu

DEV = "cuda"
TORCH_DT = {"fp16": torch.float16, "bf16": torch.bfloat16}


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("S,rows,D", [(1, 37, 128), (3, 1000, 128), (5, 333, 512), (2, 64, 8), (4, 0, 64)])
def test_merge_matches_oracle(dtype, S, rows, D):
    import masked_paged_attention_amd as mpa
    log(f"case lse_merge dtype={dtype} parts={S} rows={rows} D={D}")
    g = torch.Generator().manual_seed(1000 * S + rows + D)
    o = torch.randn((S, rows, D), generator=g).to(TORCH_DT[dtype])
    lse = (torch.randn((S, rows), generator=g) * 4.0).float()
    if rows:
        lse[0, ::7] = -float("inf")       # parts that saw no key
        if rows > 5:
            lse[:, 5] = -float("inf")     # a row no part saw
    ro, rl = oracle.lse_merge(o.double().numpy(), lse.double().numpy())
    # the values of a part with LSE = -inf are undefined: NaN there must not matter
    o = torch.where(torch.isinf(lse)[..., None], torch.tensor(float("nan")).to(o.dtype), o)
    out, l = mpa.lse_merge(o.to(DEV), lse.to(DEV))
    torch.cuda.synchronize()
    got_o = out.float().cpu().numpy().astype(np.float64)
    got_l = l.cpu().numpy().astype(np.float64)
    assert np.isfinite(got_o).all()
    err = np.abs(got_o - ro).max() if rows else 0.0
    log(f"  max_abs_err={err:.3e} (tol {TOL[dtype]})")
    assert err <= TOL[dtype]
    fin = np.isfinite(rl)
    assert (np.isfinite(got_l) == fin).all() and (got_l[~fin] == -np.inf).all()
    if fin.any():
        lerr = (np.abs(got_l[fin] - rl[fin]) / np.maximum(1.0, np.abs(rl[fin]))).max()
        assert lerr <= LSE_REL, lerr


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_chunked_prefix_merge_equals_whole_call(dtype):
    # Causal prefill with a cached prefix, split at key `cut` (a block boundary, below
    # every prefix): keys [0, cut) are visible to every new row (mask NONE over that
    # chunk), keys [cut, kvSeqLen) form a causal call whose prefix is P - cut.
    import masked_paged_attention_amd as mpa
    log(f"case chunked prefix merge dtype={dtype}")
    L = np.array([300, 130])
    P = np.array([900, 600])
    c = W.make_prefill(91, L, P + L, 8, 2, 128, 128, dtype, 9, 1.0 / np.sqrt(128), poison=True,
                       name=f"chunked-{dtype}").to(DEV)
    cut, bs = 512, c.block_size
    bt = c.block_tables
    o1, l1 = mpa.prefix_encoder(c.query, c.key, c.value, bt[:, :cut // bs].contiguous(), L,
                                np.full_like(L, cut), mask_type=mpa.MASK_NONE, qk_scale=c.qk_scale,
                                return_lse=True)
    o2, l2 = mpa.prefix_encoder(c.query, c.key, c.value, bt[:, cut // bs:].contiguous(), L, P + L - cut,
                                mask_type=mpa.MASK_CAUSAL, qk_scale=c.qk_scale, return_lse=True)
    out, lse = mpa.lse_merge(torch.stack([o1, o2]), torch.stack([l1, l2]))
    torch.cuda.synchronize()
    check_prefill_full(c, out, lse)
    whole, wl = gpu_prefill(c)
    d = (out.float() - whole.float()).abs().max().item()
    log(f"  merged vs one call: max_abs_diff={d:.3e}")
    assert d <= 2 * TOL[dtype]
