"""CPU tests of the C ABI: exported symbols, constants, argument validation (which
runs before any HIP call) and the host launch planners.  No kernel runs here."""

import ctypes
import json
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mpa.h")


@pytest.fixture(scope="module")
def lib():
    from masked_paged_attention_amd._lib import LIB
    return LIB


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mpa[A-Z]\w*)\s*\(", text)))


def _header_defines():
    out = {}
    for name, val in re.findall(r"#define\s+(MPA_\w+)\s+(-?\d+)", open(HEADER).read()):
        out[name] = int(val)
    return out


def test_every_declared_symbol_is_exported(lib):
    names = _declared_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/mpa.h but not exported"
    from masked_paged_attention_amd._lib import SIGNATURES
    assert sorted(SIGNATURES) == names


def test_no_kernel_spills_to_scratch(lib):
    """Every device kernel of the library fits its registers: the compiler's
    resource report, written by the build, shows no scratch (private memory)
    for any of them, and no kernel asks for more than 512 registers."""
    from masked_paged_attention_amd.build import RESOURCES
    assert os.path.exists(RESOURCES), "build the library first (its build writes the report)"
    res = json.load(open(RESOURCES))
    names = " ".join(res)
    for k in ("prefill_dma_kernel", "prefill_fwd_kernel", "mla_split_kernel", "mla_combine_kernel",
              "lse_merge_kernel"):
        assert k in names, k
    assert len(res) >= 60
    for name, r in res.items():
        assert r["scratch"] == 0, f"{name} spills {r['scratch']} bytes per lane"
        assert r["vgpr"] + r["agpr"] <= 512, name


def test_constants_match_pages():
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "atb_constants.json")))
    d = _header_defines()
    m = g["prefix_encoder_mask_types"]
    assert d["MPA_MASK_ALIBI_COMPRESS"] == m["MASK_TYPE_ALIBI_COMPRESS"]
    assert d["MPA_MASK_ALIBI_COMPRESS_SQRT"] == m["MASK_TYPE_ALIBI_COMPRESS_SQRT"]
    assert d["MPA_MASK_ALIBI_COMPRESS_LEFT_ALIGN"] == m["MASK_TYPE_ALIBI_COMPRESS_LEFT_ALIGN"]
    assert d["MPA_MASK_CAUSAL"] == m["MASK_TYPE_CAUSAL_MASK"]
    assert d["MPA_MLA_CALC_UNDEFINED"] == g["mla"]["CALC_TYPE_UNDEFINED"]
    assert d["MPA_MLA_CACHE_KVCACHE"] == g["mla"]["KVCACHE"]
    import masked_paged_attention_amd as mpa
    assert (mpa.MASK_ALIBI, mpa.MASK_ALIBI_SQRT, mpa.MASK_ALIBI_LEFT, mpa.MASK_CAUSAL) == (3, 4, 5, 9)


def test_error_strings(lib):
    for s in range(5):
        assert lib.mpaGetErrorString(s)
    assert lib.mpaGetErrorString(99) == b"unknown status"
    assert lib.mpaDestroyOperation(None) == 0


FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: validation fails first


def _i32(a):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.int32))
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _prefill(lib, **kw):
    args = dict(query=FAKE, key=FAKE, value=FAKE, bt=FAKE, seq=[4, 7], kv=[4, 9], slopes=None,
                mask=9, H=4, KVH=2, scale=0.125, batch=2, D=64, nb=8, bs=16, maxb=2, dtype=0,
                qstart=None, ntok=11, out=FAKE, lse=None)
    args.update(kw)
    seq, ps = _i32(args["seq"]) if args["seq"] is not None else (None, ctypes.POINTER(ctypes.c_int32)())
    kv, pk = _i32(args["kv"]) if args["kv"] is not None else (None, ctypes.POINTER(ctypes.c_int32)())
    if args["qstart"] is not None:
        qs = np.ascontiguousarray(np.asarray(args["qstart"], dtype=np.int64))
        pq = qs.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    else:
        pq = ctypes.POINTER(ctypes.c_int64)()
    ws = ctypes.c_uint64(123)
    op = ctypes.c_void_p(0xdead)
    st = lib.mpaSelfAttentionPrefixEncoderGetWorkspaceSize(
        args["query"], args["key"], args["value"], args["bt"], ps, pk, args["slopes"], args["mask"],
        args["H"], args["KVH"], args["scale"], args["batch"], args["D"], args["nb"], args["bs"],
        args["maxb"], args["dtype"], pq, args["ntok"], args["out"], args["lse"],
        ctypes.byref(ws), ctypes.byref(op))
    return st, op


@pytest.mark.parametrize("kw,status", [
    (dict(query=None), 1),
    (dict(out=None), 1),
    (dict(bt=None), 1),
    (dict(seq=None), 1),
    (dict(H=0), 1),
    (dict(KVH=3), 1),
    (dict(KVH=0), 1),
    (dict(dtype=2), 1),
    (dict(mask=7), 2),
    (dict(mask=3), 1),                  # ALiBi without slopes
    (dict(slopes=FAKE), 1),             # slopes with causal
    (dict(D=96), 2),
    (dict(seq=[5, 7], kv=[4, 9]), 1),   # kvSeqLen < seqLen
    (dict(seq=[-1, 7]), 1),
    (dict(kv=[4, 40]), 1),              # needs 3 blocks > maxBlockNum 2
    (dict(ntok=10), 1),                 # rows exceed nTokens
    (dict(qstart=[0, 2], ntok=20), 1),  # overlapping padded rows
    (dict(batch=0), 1),
    (dict(scale=float("nan")), 1),
    (dict(bs=0), 1),
])
def test_prefill_validation(lib, kw, status):
    st, op = _prefill(lib, **kw)
    assert st == status, lib.mpaGetLastErrorMessage()
    assert op.value is None or op.value == 0
    assert lib.mpaGetLastErrorMessage()


def test_prefill_valid_args_reach_hip_or_succeed(lib):
    st, op = _prefill(lib)
    # With no GPU the first HIP call fails; with a GPU phase 1 succeeds (no kernel runs).
    assert st in (0, 4), lib.mpaGetLastErrorMessage()
    if st == 0:
        assert lib.mpaDestroyOperation(op) == 0


def _mla(lib, **kw):
    args = dict(qn=FAKE, qr=FAKE, ckv=FAKE, kr=FAKE, bt=FAKE, ctx=[100, 300], ql=None, H=16,
                scale=0.07, KVH=1, mask=0, calc=0, cache=1, batch=2, nb=8, bs=64, maxb=5, dtype=1,
                ntok=None, out=FAKE, lse=None)
    args.update(kw)
    ctx, pc = _i32(args["ctx"]) if args["ctx"] is not None else (None, ctypes.POINTER(ctypes.c_int32)())
    ql, pq = _i32(args["ql"]) if args["ql"] is not None else (None, ctypes.POINTER(ctypes.c_int32)())
    ntok = args["ntok"]
    if ntok is None:  # the token count the other arguments imply
        ntok = int(np.sum(args["ql"])) if args["ql"] is not None and args["calc"] in (1, 3) else args["batch"]
    ws = ctypes.c_uint64(0)
    op = ctypes.c_void_p(0)
    st = lib.mpaMLAGetWorkspaceSize(args["qn"], args["qr"], args["ckv"], args["kr"], args["bt"], pc, pq,
                                    args["H"], args["scale"], args["KVH"], args["mask"], args["calc"],
                                    args["cache"], args["batch"], args["nb"], args["bs"], args["maxb"],
                                    args["dtype"], ntok, args["out"], args["lse"], ctypes.byref(ws),
                                    ctypes.byref(op))
    return st, op


@pytest.mark.parametrize("kw,status", [
    (dict(qn=None), 1),
    (dict(ctx=None), 1),
    (dict(KVH=2), 2),
    (dict(cache=2), 2),
    (dict(cache=3), 2),
    (dict(calc=2), 2),                   # RING
    (dict(calc=3), 1),                   # PREFILL without qSeqLen
    (dict(calc=4), 2),
    (dict(mask=2), 2),                   # MASK_FREE
    (dict(calc=1), 1),                   # SPEC without qSeqLen
    (dict(ql=[1, 1]), 1),                # qSeqLen without SPEC / PREFILL
    (dict(calc=3, ql=[101, 2]), 1),      # PREFILL: more tokens than keys
    (dict(calc=1, ql=[0, 2]), 1),
    (dict(calc=1, ql=[101, 2]), 1),      # more tokens than keys
    (dict(kr=None), 1),                  # cacheMode 1 needs kRope
    (dict(cache=0), 1),                  # cacheMode 0 with kRope
    (dict(ctx=[0, 5]), 1),
    (dict(ctx=[100, 400]), 1),           # 7 blocks > maxBlockNum 5
    (dict(H=0), 1),
    (dict(dtype=5), 1),
    (dict(ntok=3), 1),                   # decode: one token per sequence
    (dict(calc=1, ql=[2, 3], ntok=4), 1),  # SPEC: sum of qSeqLen
])
def test_mla_validation(lib, kw, status):
    st, op = _mla(lib, **kw)
    assert st == status, lib.mpaGetLastErrorMessage()
    assert op.value is None or op.value == 0


def test_mla_valid_args_reach_hip_or_succeed(lib):
    for kw in (dict(), dict(calc=1, ql=[2, 3], mask=1), dict(calc=3, ql=[100, 7], mask=1)):
        st, op = _mla(lib, **kw)
        assert st in (0, 4), lib.mpaGetLastErrorMessage()
        if st == 0:
            assert lib.mpaDestroyOperation(op) == 0


def test_mla_execute_rejects_small_workspace_and_wrong_op(lib):
    assert lib.mpaMLA(None, 0, None, None) == 1
    assert lib.mpaSelfAttentionPrefixEncoder(None, 0, None, None) == 1


@pytest.mark.parametrize("seed", range(4))
def test_prefill_workspace_covers_plan(seed):
    """The workspace phase 1 asks for holds the launch plan the kernels read from
    it: 16 bytes per workgroup item and 16 per sequence, each part 256-aligned."""
    import masked_paged_attention_amd as mpa
    rng = np.random.default_rng(100 + seed)
    B = int(rng.integers(1, 9))
    L = rng.integers(0, 3000, size=B)
    P = rng.integers(0, 3000, size=B)
    H, KVH = [(32, 8), (40, 40), (8, 1), (4, 4)][seed]
    items, _, _, _, ws = mpa.plan_prefill(L, L + P, 9, H, KVH, with_workspace=True)
    need = -(-16 * len(items) // 256) * 256 + -(-16 * B // 256) * 256
    assert ws == need and ws >= 16 * (len(items) + B) and ws % 256 == 0


def test_launch_events_need_an_operation(lib):
    assert lib.mpaOperationSetLaunchEvents(None, None, None) == 1


# ---------------------------------------------------------------------------
# Planners (host only).
# ---------------------------------------------------------------------------

def _visible_keys(kv, L, i, causal):
    return min(kv, kv - L + i + 1) if causal else kv


@pytest.mark.parametrize("seed", range(6))
def test_prefill_plan_covers_every_row_once(seed):
    import masked_paged_attention_amd as mpa
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 7))
    L = rng.integers(0, 600, size=B)
    P = rng.integers(0, 900, size=B)
    H, KVH = [(4, 4), (8, 2), (32, 8), (6, 2), (12, 3), (16, 1)][seed]
    mask = [9, 0, 3, 9, 4, 5][seed]
    causal = mask != 0
    items, rows, keys, hpi = mpa.plan_prefill(L, L + P, mask, H, KVH)
    assert keys == 64 and rows * hpi == 128
    seen = {}
    group_xcd = {}
    for pos, (b, h0, r0, nt) in enumerate(items):
        if b < 0:
            continue
        for h in range(h0, h0 + hpi):
            assert h // (H // KVH) == h0 // (H // KVH), "a workgroup mixes KV heads"
            for i in range(r0, min(r0 + rows, L[b])):
                seen[(b, h, i)] = seen.get((b, h, i), 0) + 1
        last = min(r0 + rows, L[b]) - 1
        want = -(-_visible_keys(L[b] + P[b], L[b], last, causal) // 64)
        assert nt == want
        key = (b, h0 // (H // KVH))
        group_xcd.setdefault(key, set()).add(pos % 8)
    expect = {(b, h, i) for b in range(B) for h in range(H) for i in range(L[b])}
    assert set(seen) == expect
    assert all(v == 1 for v in seen.values())
    # every (sequence, KV head) group lands on one XCD (workgroup id mod 8)
    assert all(len(x) == 1 for x in group_xcd.values())


@pytest.mark.parametrize("spec", [False, True])
def test_mla_plan_segments_partition_keys(spec):
    import masked_paged_attention_amd as mpa
    rng = np.random.default_rng(5)
    ctx = rng.integers(1, 9000, size=37)
    ql = rng.integers(1, 5, size=37) if spec else None
    segs = mpa.plan_mla(ctx, ql, 128, 1 if spec else 0)
    by_b = {}
    for b, k0, k1, idx, piece in segs:
        assert 0 <= b < len(ctx) and k1 > k0
        by_b.setdefault(b, []).append((k0, k1, idx, piece))
    for b in range(len(ctx)):
        parts = by_b[b]
        # in piece order, each sequence's segments are consecutive key ranges
        assert parts[0][0] == 0 and parts[-1][1] == ctx[b]
        for (a0, a1, i0, p0), (c0, c1, i1, p1) in zip(parts, parts[1:]):
            assert a1 == c0 and i1 == i0 + 1 and p1 > p0
        for k0, k1, _, _ in parts:
            assert k0 % 32 == 0
        for _, k1, _, _ in parts[:-1]:
            assert k1 % 32 == 0


@pytest.mark.parametrize("spec", [False, True])
def test_mla_plan_pieces_are_balanced(spec):
    """Pieces cover the flattened 32-key tiles in order with near-equal counts:
    256 pieces at q_len 1 (one per compute unit), 64 at q_len 4 with 128 heads
    (4 row groups per piece)."""
    import masked_paged_attention_amd as mpa
    rng = np.random.default_rng(11)
    ctx = rng.integers(1024, 8193, size=64)
    ql = np.full(64, 4) if spec else None
    segs = mpa.plan_mla(ctx, ql, 128, 1 if spec else 0)
    tiles = {}
    order = []
    for b, k0, k1, idx, piece in segs:
        tiles[piece] = tiles.get(piece, 0) + (k1 - k0 + 31) // 32
        order.append((piece, b, k0))
    assert order == sorted(order)
    n_pieces = 64 if spec else 256
    assert set(tiles) == set(range(n_pieces))
    total = sum((int(c) + 31) // 32 for c in ctx)
    assert sum(tiles.values()) == total
    assert max(tiles.values()) - min(tiles.values()) <= 1


def test_mla_plan_whole_sequences_for_long_prompts():
    """A prefill of long prompts at 128 heads has many (sequence, row group) pairs
    whose longest-first schedule balances: one segment per sequence, longest
    first, no key split.  The decode shapes keep the split (checked above)."""
    import masked_paged_attention_amd as mpa
    ctx = np.array([1024, 4096, 2048, 3072])
    segs = mpa.plan_mla(ctx, np.full(4, 256), 128, 3)
    assert [tuple(int(v) for v in x) for x in segs] == [(1, 0, 4096, 0, 0), (3, 0, 3072, 0, 1),
                                                       (2, 0, 2048, 0, 2), (0, 0, 1024, 0, 3)]
    # a few sequences whose row groups cannot balance stay split
    segs = mpa.plan_mla(np.array([9000, 300]), np.array([2, 256]), 128, 3)
    assert len(segs) > 2


def test_mla_plan_small_problem_uses_few_pieces():
    import masked_paged_attention_amd as mpa
    segs = mpa.plan_mla(np.array([65, 130, 9]), None, 16, 0)
    pieces = sorted(set(int(x[4]) for x in segs))
    assert len(pieces) == 3            # 9 tiles, at least 4 tiles per piece
    assert all(x[1] % 32 == 0 for x in segs)


def _merge(lib, o=16, l=32, n=2, rows=10, d=128, dtype=1, out=48, lse=64):
    return lib.mpaLseMerge(ctypes.c_void_p(o), ctypes.c_void_p(l), n, rows, d, dtype,
                           ctypes.c_void_p(out), ctypes.c_void_p(lse), ctypes.c_void_p(0))


@pytest.mark.parametrize("kw", [
    dict(o=0), dict(l=0), dict(out=0), dict(n=0), dict(rows=-1), dict(d=12), dict(d=0),
    dict(d=8192), dict(dtype=2), dict(o=24), dict(out=40),
])
def test_lse_merge_validation(lib, kw):
    # every case is rejected on the host, before any HIP call
    assert _merge(lib, **kw) == 1, lib.mpaGetLastErrorMessage()
    assert lib.mpaGetLastErrorMessage()


def test_lse_merge_zero_rows_is_a_no_op(lib):
    assert _merge(lib, rows=0) == 0, lib.mpaGetLastErrorMessage()
    assert _merge(lib, rows=0, o=0, l=0, out=0, lse=0) == 0, lib.mpaGetLastErrorMessage()


def _prefill_tile(lib, tile=0x10000, rows=128, cols=128, mask=9, slopes=None):
    seq, ps = _i32([4, 7])
    kv, pk = _i32([4, 9])
    ws = ctypes.c_uint64(123)
    op = ctypes.c_void_p(0xdead)
    st = lib.mpaSelfAttentionPrefixEncoderCompressedMaskGetWorkspaceSize(
        FAKE, FAKE, FAKE, FAKE, ps, pk, ctypes.c_void_p(tile), rows, cols, slopes, mask,
        4, 2, 0.125, 2, 64, 8, 16, 2, 0, ctypes.POINTER(ctypes.c_int64)(), 11, FAKE, None,
        ctypes.byref(ws), ctypes.byref(op))
    return st, op


@pytest.mark.parametrize("kw,status", [
    (dict(tile=0), 1),                               # no mask
    (dict(tile=0x10008), 1),                         # not 16-byte aligned
    (dict(rows=256, cols=256), 2),                   # norm mask is [128, 128]
    (dict(mask=3, slopes=FAKE), 2),                  # ALiBi takes [256, 256]
    (dict(mask=4, slopes=FAKE, rows=256, cols=128), 2),  # [headNum, seqLen, 128] form: unsupported
    (dict(mask=0), 2),                               # no compressed form
    (dict(mask=5, rows=256, cols=256), 1),           # ALiBi without slopes
])
def test_compressed_mask_validation(lib, kw, status):
    st, op = _prefill_tile(lib, **kw)
    assert st == status, lib.mpaGetLastErrorMessage()
    assert op.value is None or op.value == 0
    assert lib.mpaGetLastErrorMessage()


def test_compressed_mask_head_seq_form_is_refused_by_name(lib):
    # the [headNum, seqLen, 128] ALiBi form is out of scope: refused as unsupported,
    # with a message that names the form, before anything else happens
    st, op = _prefill_tile(lib, mask=4, slopes=FAKE, rows=256, cols=128)
    assert st == 2
    assert b"[headNum, seqLen, 128]" in lib.mpaGetLastErrorMessage()
    assert op.value is None or op.value == 0


def test_compressed_mask_valid_args_reach_hip_or_succeed(lib):
    for kw in (dict(), dict(mask=4, slopes=FAKE, rows=256, cols=256)):
        st, op = _prefill_tile(lib, **kw)
        assert st in (0, 4), lib.mpaGetLastErrorMessage()
        if st == 0:
            assert lib.mpaDestroyOperation(op) == 0


def _mla8(lib, qkd=FAKE, pvd=FAKE, kr=FAKE, KVH=1, calc=0, ql=None, dtype=1, ntok=2):
    ctx, pc = _i32([100, 300])
    pq = _i32(ql)[1] if ql is not None else ctypes.POINTER(ctypes.c_int32)()
    ws = ctypes.c_uint64(0)
    op = ctypes.c_void_p(0xdead)
    st = lib.mpaMLAInt8GetWorkspaceSize(FAKE, FAKE, FAKE, kr, FAKE, pc, pq, qkd, pvd, 16, 0.07, KVH,
                                        0, calc, 2, 8, 64, 5, dtype, ntok, FAKE, None,
                                        ctypes.byref(ws), ctypes.byref(op))
    return st, op


@pytest.mark.parametrize("kw,status", [
    (dict(qkd=None), 1), (dict(pvd=None), 1), (dict(kr=None), 1), (dict(KVH=2), 2),
    (dict(calc=1), 1),                   # SPEC without qSeqLen
    (dict(dtype=2), 1),
    (dict(ntok=1), 1),                   # one token per sequence
])
def test_mla_int8_validation(lib, kw, status):
    st, op = _mla8(lib, **kw)
    assert st == status, lib.mpaGetLastErrorMessage()
    assert op.value is None or op.value == 0


def test_mla_int8_valid_args_reach_hip_or_succeed(lib):
    st, op = _mla8(lib)
    assert st in (0, 4), lib.mpaGetLastErrorMessage()
    if st == 0:
        assert lib.mpaDestroyOperation(op) == 0


def test_prefill_plan_order_per_xcd():
    """Within an XCD the plan keeps a group's items together unless running them
    longest first ends the modelled schedule clearly earlier: the short-item GQA
    prefix workload comes out longest first, the single long MHA sequence keeps
    each head's items adjacent."""
    import masked_paged_attention_amd as mpa
    import workloads as W
    c = W.make_prefill_config("prefix_gqa_causal")
    items, _, _, _ = mpa.plan_prefill(c.seq_len, c.kv_seq_len, 9, 32, 8)
    for x in range(8):
        mine = items[x::8]
        mine = mine[mine[:, 0] >= 0]
        assert np.all(np.diff(mine[:, 3]) <= 0)
    items, _, _, _ = mpa.plan_prefill([16384], [16384], 4, 40, 40)
    for x in range(8):
        mine = items[x::8]
        heads = mine[mine[:, 0] >= 0][:, 1]
        changes = int(np.count_nonzero(np.diff(heads)))
        assert changes == len(set(heads.tolist())) - 1   # each head's items form one run
