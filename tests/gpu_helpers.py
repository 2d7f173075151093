"""Shared helpers of the GPU parity tests: run the HIP path through the binding and
compare with the fp64 oracle at the tolerances of the build (max-abs 5e-3 for
fp16 outputs, 2e-2 for bf16; LSE within 1e-3 * max(1, |LSE|))."""

import sys

import numpy as np
import torch

import oracle

TOL = {"fp16": 5e-3, "bf16": 2e-2}
LSE_REL = 1e-3


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def gpu_prefill(case, return_lse=True, sentinel=None):
    import masked_paged_attention_amd as mpa
    out = torch.empty_like(case.query)
    if sentinel is not None:
        out.fill_(sentinel)
    lse = None
    if return_lse:
        lse = torch.full((case.n_tokens, case.head_num), float("nan") if sentinel is None else sentinel,
                         dtype=torch.float32, device=case.query.device)
    slopes = None
    if case.slopes is not None:
        slopes = torch.as_tensor(case.slopes, device=case.query.device)
    mpa.prefix_encoder(case.query, case.key, case.value, case.block_tables, case.seq_len,
                       case.kv_seq_len, mask_type=case.mask_type, qk_scale=case.qk_scale,
                       slopes=slopes, q_start_loc=case.q_start_loc, out=out, lse=lse,
                       attention_chunk=case.chunk if case.chunk else None,
                       compressed_mask=case.mask_tile)
    torch.cuda.synchronize()
    return out, lse


def compare_rows(name, dtype, got_o, got_l, ref_o, ref_l):
    """got_* / ref_* are [n, D] / [n] arrays of the same rows."""
    got_o = np.asarray(got_o, dtype=np.float64)
    assert np.isfinite(got_o).all(), f"{name}: non-finite output"
    err = np.abs(got_o - ref_o).max() if got_o.size else 0.0
    log(f"{name}: rows={len(ref_o)} max_abs_err={err:.3e} (tol {TOL[dtype]})")
    assert err <= TOL[dtype], f"{name}: max abs error {err} > {TOL[dtype]}"
    if got_l is not None:
        got_l = np.asarray(got_l, dtype=np.float64)
        lerr = (np.abs(got_l - ref_l) / np.maximum(1.0, np.abs(ref_l))).max() if got_l.size else 0.0
        log(f"{name}: lse max rel err={lerr:.3e}")
        assert lerr <= LSE_REL, f"{name}: LSE error {lerr}"


def check_prefill_full(case, out, lse):
    """Element-wise parity on every valid row of every head."""
    args = case.oracle_args()
    ro, rl = oracle.prefix_encoder(**args)
    starts = case.row_starts()
    rows = np.concatenate([np.arange(s, s + L) for s, L in zip(starts, case.seq_len)]) \
        if case.seq_len.sum() else np.zeros(0, dtype=np.int64)
    o = out.float().cpu().numpy()[rows]
    l = lse.cpu().numpy()[rows] if lse is not None else None
    compare_rows(case.name, case.dtype, o.reshape(-1, case.head_size), None if l is None else l.reshape(-1),
                 ro[rows].reshape(-1, case.head_size), rl[rows].reshape(-1))


def sample_rows(case, n, seed):
    """n (b, i, h) triples, with the first and last row of every sequence included."""
    rng = np.random.default_rng(seed)
    rows = set()
    for b, L in enumerate(case.seq_len):
        if L > 0:
            rows.add((b, 0, int(rng.integers(case.head_num))))
            rows.add((b, int(L) - 1, int(rng.integers(case.head_num))))
    valid = [b for b in range(case.batch) if case.seq_len[b] > 0]
    while len(rows) < n:
        b = int(rng.choice(valid))
        rows.add((b, int(rng.integers(case.seq_len[b])), int(rng.integers(case.head_num))))
    return sorted(rows)


def check_prefill_sampled(case, out, lse, n=192, seed=0):
    args = case.oracle_args()
    rows = sample_rows(case, n, seed)
    ro, rl = oracle.prefix_encoder_rows(rows=rows, **args)
    starts = case.row_starts()
    toks = np.array([starts[b] + i for b, i, _ in rows])
    heads = np.array([h for _, _, h in rows])
    o = out[torch.as_tensor(toks, device=out.device), torch.as_tensor(heads, device=out.device)].float().cpu().numpy()
    l = lse[torch.as_tensor(toks, device=out.device), torch.as_tensor(heads, device=out.device)].cpu().numpy() \
        if lse is not None else None
    compare_rows(case.name + " (sampled)", case.dtype, o, l, ro, rl)


def check_prefill_heads(case, out, lse, heads):
    """Element-wise parity on every row of the given heads, all sequences."""
    args = case.oracle_args()
    rows = [(b, i, h) for h in heads for b in range(case.batch) for i in range(int(case.seq_len[b]))]
    ro, rl = oracle.prefix_encoder_rows(rows=rows, **args)
    starts = case.row_starts()
    toks = torch.as_tensor([starts[b] + i for b, i, _ in rows], device=out.device)
    hs = torch.as_tensor([h for _, _, h in rows], device=out.device)
    o = out[toks, hs].float().cpu().numpy()
    l = lse[toks, hs].cpu().numpy() if lse is not None else None
    compare_rows(f"{case.name} (heads {list(heads)}, every row)", case.dtype, o, l, ro, rl)


def gpu_mla(case, return_lse=True):
    import masked_paged_attention_amd as mpa
    lse = None
    out = torch.empty((case.n_tokens, case.head_num, 512), dtype=case.q_rope.dtype, device=case.q_rope.device)
    if return_lse:
        lse = torch.full((case.n_tokens, case.head_num), float("nan"), dtype=torch.float32,
                         device=case.q_nope.device)
    qkd = pvd = None
    if case.qk_descale is not None:
        qkd = torch.as_tensor(case.qk_descale, device=case.q_nope.device)
        pvd = torch.as_tensor(case.pv_descale, device=case.q_nope.device)
    mpa.mla(case.q_nope, case.q_rope, case.ct_kv, case.k_rope, case.block_tables, case.context_lens,
            qk_scale=case.qk_scale, q_seq_len=case.q_seq_len, mask_type=case.mask_type,
            calc_type=case.calc_type, cache_mode=case.cache_mode, out=out, lse=lse,
            qk_descale=qkd, pv_descale=pvd)
    torch.cuda.synchronize()
    return out, lse


def check_mla(case, out, lse, rows=None):
    args = case.oracle_args()
    if rows is None:
        rows = [(t, h) for t in range(case.n_tokens) for h in range(case.head_num)]
    ro, rl = oracle.mla_rows(rows=rows, **args)
    t = torch.as_tensor([r[0] for r in rows], device=out.device)
    h = torch.as_tensor([r[1] for r in rows], device=out.device)
    o = out[t, h].float().cpu().numpy()
    l = lse[t, h].cpu().numpy() if lse is not None else None
    compare_rows(case.name, case.dtype, o, l, ro, rl)
