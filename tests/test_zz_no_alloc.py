"""mpaMLAStaticScratch -- the MLA execution that allocates nothing (its plan and
split-KV partials in the library's static device buffer) -- against mpaMLA with
a caller workspace, through the C ABI: identical outputs on two calls in a row,
the second over a smaller input; an operation that needs more scratch than the
buffer holds is refused before anything is launched."""

import ctypes

import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import check_mla, log

pytestmark = pytest.mark.gpu
DEV = "cuda"
STATIC_BYTES = 128 << 20


def _pair(case):
    """Workspace call and static-scratch call of the same operation inputs, into
    separate outputs."""
    import masked_paged_attention_amd as mpa
    outs = []
    for static in (False, True):
        out = torch.full((case.n_tokens, case.head_num, 512), 7.0, dtype=case.q_rope.dtype, device=DEV)
        lse = torch.full((case.n_tokens, case.head_num), 7.0, dtype=torch.float32, device=DEV)
        op = mpa.MLA(case.q_nope, case.q_rope, case.ct_kv, case.k_rope, case.block_tables, case.context_lens,
                     qk_scale=case.qk_scale, q_seq_len=case.q_seq_len, mask_type=case.mask_type,
                     calc_type=case.calc_type, out=out, lse=lse)
        assert op.workspace is not None and op.workspace.numel() <= STATIC_BYTES
        if static:
            st = mpa.LIB.mpaMLAStaticScratch(op._op, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
            assert st == 0, mpa.LIB.mpaGetLastErrorMessage()
        else:
            op.run()
        torch.cuda.synchronize()
        outs.append((out, lse, op.workspace.numel()))
        op.close()
    return outs


def test_static_scratch_equals_workspace_two_calls():
    big = W.make_mla_config("mla_decode_q1", poison=True, device=DEV)
    small = W.make_mla(501, np.array([700, 33, 2048, 129, 64]), None, 128, 128, "bf16", 0, 0, 1,
                       1.0 / np.sqrt(192.0), poison=True, name="small").to(DEV)
    sizes = []
    for case in (big, small):
        log(f"case static scratch vs workspace: {case.name} batch {case.batch}")
        (o_ws, l_ws, ws), (o_st, l_st, _) = _pair(case)
        sizes.append(ws)
        assert torch.equal(o_ws, o_st) and torch.equal(l_ws, l_st)
        rows = [(t, h) for t in (0, case.n_tokens - 1) for h in range(case.head_num)]
        check_mla(case, o_st, l_st, rows=rows)
    assert sizes[1] < sizes[0]


def test_static_scratch_refuses_an_operation_that_does_not_fit():
    import masked_paged_attention_amd as mpa
    log("case static scratch: an operation larger than the buffer")
    # one sequence of 128 new tokens: 16384 (token, head) rows, split over 8
    # pieces of its keys -- 131072 fp32 partial rows (~268 MB)
    ctx = np.array([4096], dtype=np.int32)
    ql = np.array([128], dtype=np.int32)
    c = W.make_mla(503, ctx, ql, 128, 128, "bf16", 1, 1, 1, 1.0 / np.sqrt(192.0), name="big-spec").to(DEV)
    out = torch.full((c.n_tokens, 128, 512), 7.0, dtype=torch.bfloat16, device=DEV)
    op = mpa.MLA(c.q_nope, c.q_rope, c.ct_kv, c.k_rope, c.block_tables, c.context_lens, qk_scale=c.qk_scale,
                 q_seq_len=c.q_seq_len, mask_type=c.mask_type, out=out)
    assert op.workspace.numel() > STATIC_BYTES
    st = mpa.LIB.mpaMLAStaticScratch(op._op, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 3, st  # MPA_ERROR_WORKSPACE_TOO_SMALL
    assert b"static scratch" in mpa.LIB.mpaGetLastErrorMessage()
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)  # nothing launched
    op.close()
