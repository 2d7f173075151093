"""Timing hooks (mpaOperationSetLaunchEvents): events recorded on the kernels' own
dispatch packets bracket the call, lie inside stream events recorded around it,
and leave the results bit-identical."""

import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _created_events(n):
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in evs:
        e.record()  # creates the HIP event
    torch.cuda.synchronize()
    return evs


def _check_bracketed(op, outs):
    ref = [o.clone() for o in outs]
    k_start, k_stop, s_start, s_stop = _created_events(4)
    op.set_launch_events(k_start, k_stop)
    for o in outs:
        o.zero_()
    s_start.record()
    op.run()
    s_stop.record()
    torch.cuda.synchronize()
    k_ms = k_start.elapsed_time(k_stop)
    s_ms = s_start.elapsed_time(s_stop)
    log(f"  dispatch events {k_ms:.4f} ms, stream events {s_ms:.4f} ms")
    assert 0.0 < k_ms <= s_ms * 1.02 + 0.002
    for a, b in zip(outs, ref):
        assert torch.equal(a, b)
    # detached: later runs record nothing into them
    op.set_launch_events(None, None)
    op.run()
    torch.cuda.synchronize()


def test_prefill_launch_events():
    import masked_paged_attention_amd as mpa
    log("case launch events: prefix encoder, causal GQA, bf16, headSize 128")
    c = W.make_prefill(401, np.array([700, 129, 300]), np.array([1500, 129, 900]), 8, 2, 128, 128, "bf16",
                       9, 1.0 / np.sqrt(128), poison=True, name="events").to(DEV)
    out = torch.empty_like(c.query)
    lse = torch.empty((c.n_tokens, c.head_num), dtype=torch.float32, device=DEV)
    op = mpa.PrefixEncoder(c.query, c.key, c.value, c.block_tables, c.seq_len, c.kv_seq_len,
                           mask_type=c.mask_type, qk_scale=c.qk_scale, out=out, lse=lse)
    op.run()
    torch.cuda.synchronize()
    _check_bracketed(op, [out, lse])


@pytest.mark.parametrize("ctx", [[5000, 33, 1, 4096, 127, 7777, 64, 2500], [300]])
def test_mla_launch_events(ctx):
    # (several segments per sequence: split + combine; one short sequence: split only)
    import masked_paged_attention_amd as mpa
    log(f"case launch events: MLA decode, 128 heads, contexts {ctx}")
    m = W.make_mla(402, ctx, None, 128, 128, "bf16", 0, 0, 1, 1 / np.sqrt(192), poison=True).to(DEV)
    out = torch.empty((m.n_tokens, m.head_num, 512), dtype=m.q_rope.dtype, device=DEV)
    lse = torch.empty((m.n_tokens, m.head_num), dtype=torch.float32, device=DEV)
    op = mpa.MLA(m.q_nope, m.q_rope, m.ct_kv, m.k_rope, m.block_tables, m.context_lens,
                 qk_scale=m.qk_scale, out=out, lse=lse)
    op.run()
    torch.cuda.synchronize()
    _check_bracketed(op, [out, lse])


def test_events_need_creating():
    import masked_paged_attention_amd as mpa
    c = W.make_prefill(403, np.array([40]), np.array([40]), 2, 2, 64, 16, "fp16", 9, 0.125,
                       name="events-new").to(DEV)
    op = mpa.PrefixEncoder(c.query, c.key, c.value, c.block_tables, c.seq_len, c.kv_seq_len,
                           mask_type=c.mask_type, qk_scale=c.qk_scale)
    with pytest.raises(ValueError):
        op.set_launch_events(torch.cuda.Event(enable_timing=True), None)
