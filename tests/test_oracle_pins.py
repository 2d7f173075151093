"""Pins of the fp64 oracle against things other than itself (CPU only).

* brute force: pure-Python loops, one key at a time through the block table,
  math.exp / math.fsum, on tiny inputs for every mask type, GQA, prefixes,
  padded layouts and random block permutations;
* closed forms: q = 0 rows (mean of the visible values, ln(count)), the
  geometric series of right-aligned ALiBi, the single-visible-key row;
* invariants: rows of A sum to one and are zero on masked keys, slope 0 ALiBi equals
  causal, left- and right-aligned ALiBi give the same output with LSE shifted by
  slope * a_i, GQA equals MHA with repeated K/V, paged equals contiguous, keys
  outside a row's visible set do not matter, packed equals padded, prefix
  consistency, the LSE merge identity, expanded compressed masks equal the full
  rule, MLA equals the generic rule with concatenated Q/K.
"""

import math

import numpy as np
import pytest

import oracle
from oracle import masks as M

TYPES = [M.MASK_NONE, M.MASK_ALIBI, M.MASK_ALIBI_SQRT, M.MASK_ALIBI_LEFT, M.MASK_CAUSAL]


def _case(rng, B, Lq, Lkv, H, KVH, D, bs, pad_to=None, dv=None, extra_blocks=3):
    """Small random paged case in fp64 (values are not rounded: the oracle is fp64)."""
    need = [-(-int(kv) // bs) for kv in Lkv]
    nb = sum(need) + extra_blocks
    perm = rng.permutation(nb)
    width = max(need) + 1
    bt = np.full((B, width), perm[-1], dtype=np.int32)
    pos = 0
    for b in range(B):
        bt[b, :need[b]] = perm[pos:pos + need[b]]
        pos += need[b]
    dv = D if dv is None else dv
    key = rng.standard_normal((nb, bs, KVH, D))
    value = rng.standard_normal((nb, bs, KVH, dv))
    if pad_to is None:
        nt = int(sum(Lq))
        qs = None
    else:
        nt = pad_to * B
        qs = np.arange(B) * pad_to
    query = rng.standard_normal((nt, H, D))
    return query, key, value, bt, qs


def brute_prefix(query, key, value, bt, seq_len, kv_seq_len, slopes, mask_type, H, KVH,
                 scale, q_start=None):
    """Pure-Python reference, one (row, key) pair at a time."""
    bs = key.shape[1]
    g = H // KVH
    if q_start is None:
        q_start, acc = [], 0
        for L in seq_len:
            q_start.append(acc)
            acc += int(L)
    scale = float(np.float32(scale))
    res = {}
    for b in range(len(seq_len)):
        L, kv = int(seq_len[b]), int(kv_seq_len[b])
        for h in range(H):
            kvh = h // g
            slope = float(np.float32(slopes[h])) if slopes is not None else 0.0
            for i in range(L):
                pos = kv - L + i
                q = query[q_start[b] + i][h]
                scores, vals = [], []
                for j in range(kv):
                    if mask_type != M.MASK_NONE and j > pos:
                        continue
                    blk = int(bt[b][j // bs])
                    k = key[blk][j % bs][kvh]
                    v = value[blk][j % bs][kvh]
                    dot = math.fsum(float(q[d]) * float(k[d]) for d in range(len(q)))
                    if mask_type == M.MASK_ALIBI:
                        bias = slope * (j - pos)
                    elif mask_type == M.MASK_ALIBI_SQRT:
                        bias = -slope * math.sqrt(pos - j)
                    elif mask_type == M.MASK_ALIBI_LEFT:
                        bias = slope * j
                    else:
                        bias = 0.0
                    scores.append(scale * dot + bias)
                    vals.append(v)
                m = max(scores)
                w = [math.exp(s - m) for s in scores]
                tot = math.fsum(w)
                o = [math.fsum(w[n] * float(vals[n][d]) for n in range(len(w))) / tot
                     for d in range(len(vals[0]))]
                res[(q_start[b] + i, h)] = (np.array(o), m + math.log(tot))
    return res


@pytest.mark.parametrize("mask_type", TYPES)
@pytest.mark.parametrize("layout", ["mha", "gqa", "mqa_pad"])
def test_brute_force(mask_type, layout):
    rng = np.random.default_rng(100 + mask_type * 7 + len(layout))
    if layout == "mha":
        B, Lq, Lkv, H, KVH, D, bs, pad = 3, [5, 17, 1], [5, 29, 40], 2, 2, 8, 4, None
    elif layout == "gqa":
        B, Lq, Lkv, H, KVH, D, bs, pad = 2, [13, 9], [21, 9], 4, 2, 16, 8, None
    else:
        B, Lq, Lkv, H, KVH, D, bs, pad = 2, [7, 11], [12, 11], 3, 1, 8, 5, 16
    query, key, value, bt, qs = _case(rng, B, Lq, Lkv, H, KVH, D, bs, pad_to=pad)
    slopes = rng.uniform(0.05, 0.9, size=H) if mask_type in M.ALIBI_TYPES else None
    scale = 0.37
    o, lse = oracle.prefix_encoder(query, key, value, bt, Lq, Lkv, slopes, mask_type, H, KVH,
                                   scale, q_start_loc=qs)
    ref = brute_prefix(query, key, value, bt, Lq, Lkv, slopes, mask_type, H, KVH, scale, qs)
    for (t, h), (ro, rl) in ref.items():
        np.testing.assert_allclose(o[t, h], ro, rtol=0, atol=1e-12)
        assert abs(lse[t, h] - rl) <= 1e-12 * max(1.0, abs(rl))
    # rows that belong to no sequence stay NaN
    covered = np.zeros(o.shape[:2], dtype=bool)
    for (t, h) in ref:
        covered[t, h] = True
    assert np.isnan(o[~covered]).all() and np.isnan(lse[~covered]).all()


def _zero_q_case(prefix, L, D=6, H=3, bs=4, seed=0):
    rng = np.random.default_rng(seed)
    kv = prefix + L
    query, key, value, bt, _ = _case(rng, 1, [L], [kv], H, H, D, bs)
    query[:] = 0.0
    return query, key, value, bt, kv


def _contig(value, bt, kv, bs, head):
    return np.stack([value[bt[0][j // bs]][j % bs][head] for j in range(kv)])


@pytest.mark.parametrize("prefix", [0, 9])
def test_closed_form_causal_zero_query(prefix):
    L, bs = 11, 4
    query, key, value, bt, kv = _zero_q_case(prefix, L, bs=bs)
    o, lse = oracle.prefix_encoder(query, key, value, bt, [L], [kv], None, M.MASK_CAUSAL, 3, 3, 0.5)
    for h in range(3):
        V = _contig(value, bt, kv, bs, h)
        for i in range(L):
            a = prefix + i
            np.testing.assert_allclose(o[i, h], V[:a + 1].mean(axis=0), atol=1e-13)
            assert abs(lse[i, h] - math.log(a + 1)) < 1e-13


def test_closed_form_no_mask_zero_query():
    L, prefix, bs = 6, 5, 4
    query, key, value, bt, kv = _zero_q_case(prefix, L, bs=bs)
    o, lse = oracle.prefix_encoder(query, key, value, bt, [L], [kv], None, M.MASK_NONE, 3, 3, 0.5)
    for h in range(3):
        V = _contig(value, bt, kv, bs, h)
        np.testing.assert_allclose(o[:, h], np.broadcast_to(V.mean(axis=0), (L, V.shape[1])), atol=1e-13)
        np.testing.assert_allclose(lse[:, h], math.log(kv), atol=1e-13)


@pytest.mark.parametrize("prefix", [0, 13])
def test_closed_form_alibi_right_zero_query(prefix):
    """q = 0: weights exp(-m d), d = a_i - j = 0..a_i, a geometric series."""
    L, bs = 10, 4
    query, key, value, bt, kv = _zero_q_case(prefix, L, bs=bs)
    slopes = np.array([0.5, 0.125, 0.03125])
    o, lse = oracle.prefix_encoder(query, key, value, bt, [L], [kv], slopes, M.MASK_ALIBI, 3, 3, 1.0)
    for h in range(3):
        m = slopes[h]
        V = _contig(value, bt, kv, bs, h)
        for i in range(L):
            a = prefix + i
            want_lse = math.log((1 - math.exp(-m * (a + 1))) / (1 - math.exp(-m)))
            assert abs(lse[i, h] - want_lse) < 1e-12
            w = np.exp(-m * np.arange(a + 1))          # weight of key a - d
            want_o = (w[:, None] * V[a::-1][:a + 1]).sum(axis=0) / w.sum()
            np.testing.assert_allclose(o[i, h], want_o, atol=1e-12)


@pytest.mark.parametrize("prefix", [0, 7])
def test_closed_form_alibi_sqrt_and_left_zero_query(prefix):
    L, bs = 9, 4
    query, key, value, bt, kv = _zero_q_case(prefix, L, bs=bs)
    slopes = np.array([0.75, 0.25, 0.0625])
    o_s, lse_s = oracle.prefix_encoder(query, key, value, bt, [L], [kv], slopes,
                                       M.MASK_ALIBI_SQRT, 3, 3, 1.0)
    o_l, lse_l = oracle.prefix_encoder(query, key, value, bt, [L], [kv], slopes,
                                       M.MASK_ALIBI_LEFT, 3, 3, 1.0)
    for h in range(3):
        m = slopes[h]
        V = _contig(value, bt, kv, bs, h)
        for i in range(L):
            a = prefix + i
            ws = [math.exp(-m * math.sqrt(a - j)) for j in range(a + 1)]
            assert abs(lse_s[i, h] - math.log(math.fsum(ws))) < 1e-12
            np.testing.assert_allclose(o_s[i, h], np.dot(ws, V[:a + 1]) / math.fsum(ws), atol=1e-12)
            wl = [math.exp(m * j) for j in range(a + 1)]
            assert abs(lse_l[i, h] - math.log(math.fsum(wl))) < 1e-11
            np.testing.assert_allclose(o_l[i, h], np.dot(wl, V[:a + 1]) / math.fsum(wl), atol=1e-12)


def test_single_visible_key_row():
    """Causal, no prefix, row 0 sees only key 0: O = V_0 exactly, LSE = scale * q.k_0."""
    rng = np.random.default_rng(5)
    query, key, value, bt, _ = _case(rng, 2, [4, 6], [4, 6], 2, 2, 8, 4)
    scale = 0.3
    o, lse = oracle.prefix_encoder(query, key, value, bt, [4, 6], [4, 6], None, M.MASK_CAUSAL,
                                   2, 2, scale)
    for b, t0 in ((0, 0), (1, 4)):
        for h in range(2):
            k0 = key[bt[b][0]][0][h]
            v0 = value[bt[b][0]][0][h]
            assert np.array_equal(o[t0, h], v0)
            want = float(np.float32(scale)) * math.fsum(float(x) * float(y) for x, y in zip(query[t0, h], k0))
            assert abs(lse[t0, h] - want) < 1e-12


def test_rows_of_attention_sum_to_one_and_vanish_when_masked():
    """With V = identity (value row j = e_j) the output row is the attention row."""
    rng = np.random.default_rng(7)
    for mt in TYPES:
        L, prefix = 9, 6
        kv = L + prefix
        bs = 4
        query, key, _, bt, _ = _case(rng, 1, [L], [kv], 1, 1, 8, bs, dv=kv)
        value = np.zeros((key.shape[0], bs, 1, kv))
        for j in range(kv):
            value[bt[0][j // bs], j % bs, 0, j] = 1.0
        slopes = [0.4] if mt in M.ALIBI_TYPES else None
        o, _ = oracle.prefix_encoder(query, key, value, bt, [L], [kv], slopes, mt, 1, 1, 0.7)
        A = o[:, 0]
        np.testing.assert_allclose(A.sum(axis=1), 1.0, atol=1e-14)
        a = prefix + np.arange(L)[:, None]
        j = np.arange(kv)[None, :]
        masked = ~M.visible(mt, a, j, kv)
        assert (A[masked] == 0).all()
        assert (A[~masked] > 0).all()


def test_alibi_slope_zero_is_causal_and_left_equals_right():
    rng = np.random.default_rng(11)
    Lq, Lkv = [12, 30], [20, 30]
    query, key, value, bt, _ = _case(rng, 2, Lq, Lkv, 4, 2, 8, 8)
    zero = np.zeros(4)
    oc, lc = oracle.prefix_encoder(query, key, value, bt, Lq, Lkv, None, M.MASK_CAUSAL, 4, 2, 0.4)
    for mt in M.ALIBI_TYPES:
        oz, lz = oracle.prefix_encoder(query, key, value, bt, Lq, Lkv, zero, mt, 4, 2, 0.4)
        np.testing.assert_allclose(oz, oc, atol=1e-13)
        np.testing.assert_allclose(lz, lc, atol=1e-13)
    slopes = np.array([0.9, 0.3, 0.1, 0.02])
    o_r, l_r = oracle.prefix_encoder(query, key, value, bt, Lq, Lkv, slopes, M.MASK_ALIBI, 4, 2, 0.4)
    o_l, l_l = oracle.prefix_encoder(query, key, value, bt, Lq, Lkv, slopes, M.MASK_ALIBI_LEFT, 4, 2, 0.4)
    np.testing.assert_allclose(o_l, o_r, atol=1e-12)
    t = 0
    for b in range(2):
        for i in range(Lq[b]):
            a = Lkv[b] - Lq[b] + i
            np.testing.assert_allclose(l_l[t] - l_r[t], np.float32(slopes).astype(np.float64) * a, atol=1e-11)
            t += 1


def test_gqa_equals_mha_with_repeated_kv():
    rng = np.random.default_rng(13)
    Lq, Lkv = [9, 14], [15, 14]
    H, KVH = 6, 2
    query, key, value, bt, _ = _case(rng, 2, Lq, Lkv, H, KVH, 8, 4)
    key_r = np.repeat(key, H // KVH, axis=2)
    value_r = np.repeat(value, H // KVH, axis=2)
    slopes = rng.uniform(0.1, 0.5, size=H)
    for mt in (M.MASK_CAUSAL, M.MASK_ALIBI):
        sl = slopes if mt == M.MASK_ALIBI else None
        o1, l1 = oracle.prefix_encoder(query, key, value, bt, Lq, Lkv, sl, mt, H, KVH, 0.5)
        o2, l2 = oracle.prefix_encoder(query, key_r, value_r, bt, Lq, Lkv, sl, mt, H, H, 0.5)
        np.testing.assert_allclose(o1, o2, atol=1e-14)
        np.testing.assert_allclose(l1, l2, atol=1e-14)


def test_paged_equals_contiguous_under_block_permutation():
    rng = np.random.default_rng(17)
    Lq, Lkv, bs = [10, 23, 4], [19, 23, 31], 4
    query, key, value, bt, _ = _case(rng, 3, Lq, Lkv, 2, 2, 8, bs)
    # Identity layout: sequence b owns consecutive blocks in order.
    need = [-(-kv // bs) for kv in Lkv]
    key_c = np.zeros((sum(need) + 1, bs, 2, 8))
    value_c = np.zeros_like(key_c)
    bt_c = np.full_like(bt, sum(need))
    nxt = 0
    for b in range(3):
        for blk in range(need[b]):
            key_c[nxt] = key[bt[b][blk]]
            value_c[nxt] = value[bt[b][blk]]
            bt_c[b][blk] = nxt
            nxt += 1
    for mt in (M.MASK_CAUSAL, M.MASK_ALIBI_SQRT, M.MASK_NONE):
        sl = [0.3, 0.2] if mt in M.ALIBI_TYPES else None
        o1, l1 = oracle.prefix_encoder(query, key, value, bt, Lq, Lkv, sl, mt, 2, 2, 0.6)
        o2, l2 = oracle.prefix_encoder(query, key_c, value_c, bt_c, Lq, Lkv, sl, mt, 2, 2, 0.6)
        np.testing.assert_array_equal(o1, o2)
        np.testing.assert_array_equal(l1, l2)


def test_unread_keys_do_not_matter():
    """NaN in spare blocks / tail slots and changes to keys a row cannot see leave
    that row unchanged; a change to a key a row can see changes it."""
    rng = np.random.default_rng(19)
    Lq, Lkv, bs = [8], [21], 4
    query, key, value, bt, _ = _case(rng, 1, Lq, Lkv, 2, 2, 8, bs, extra_blocks=4)
    o0, l0 = oracle.prefix_encoder(query, key, value, bt, Lq, Lkv, None, M.MASK_CAUSAL, 2, 2, 0.5)
    key2, value2 = key.copy(), value.copy()
    used = set(int(x) for x in bt[0][:-(-21 // bs)])
    for blk in range(key.shape[0]):
        if blk not in used:
            key2[blk] = np.nan
            value2[blk] = np.nan
    last = int(bt[0][21 // bs])
    key2[last, 21 % bs:] = np.nan
    value2[last, 21 % bs:] = np.nan
    o1, l1 = oracle.prefix_encoder(query, key2, value2, bt, Lq, Lkv, None, M.MASK_CAUSAL, 2, 2, 0.5)
    np.testing.assert_array_equal(o0, o1)
    np.testing.assert_array_equal(l0, l1)
    # perturb key/value 17: rows with a_i < 17 (a_i = 13 + i) unchanged, others change
    jstar = 17
    key3, value3 = key.copy(), value.copy()
    key3[bt[0][jstar // bs], jstar % bs] += 3.0
    value3[bt[0][jstar // bs], jstar % bs] -= 2.0
    o3, l3 = oracle.prefix_encoder(query, key3, value3, bt, Lq, Lkv, None, M.MASK_CAUSAL, 2, 2, 0.5)
    for i in range(8):
        a = 13 + i
        if a < jstar:
            np.testing.assert_array_equal(o3[i], o0[i])
        else:
            assert np.abs(o3[i] - o0[i]).max() > 1e-6


def test_packed_equals_padded():
    rng = np.random.default_rng(23)
    Lq, Lkv = [5, 12, 3], [9, 12, 20]
    query, key, value, bt, _ = _case(rng, 3, Lq, Lkv, 2, 1, 8, 4)
    pad = 16
    qp = np.full((pad * 3, 2, 8), np.nan)
    off = 0
    for b in range(3):
        qp[pad * b:pad * b + Lq[b]] = query[off:off + Lq[b]]
        off += Lq[b]
    for mt in TYPES:
        sl = [0.5, 0.25] if mt in M.ALIBI_TYPES else None
        o1, l1 = oracle.prefix_encoder(query, key, value, bt, Lq, Lkv, sl, mt, 2, 1, 0.5)
        o2, l2 = oracle.prefix_encoder(qp, key, value, bt, Lq, Lkv, sl, mt, 2, 1, 0.5,
                                       q_start_loc=np.arange(3) * pad)
        off = 0
        for b in range(3):
            np.testing.assert_array_equal(o2[pad * b:pad * b + Lq[b]], o1[off:off + Lq[b]])
            np.testing.assert_array_equal(l2[pad * b:pad * b + Lq[b]], l1[off:off + Lq[b]])
            assert np.isnan(o2[pad * b + Lq[b]:pad * (b + 1)]).all()
            off += Lq[b]


def test_prefix_consistency():
    """Last L rows of a causal pass over P + L rows == a prefix pass with prefix P."""
    rng = np.random.default_rng(29)
    P, L = 13, 7
    query, key, value, bt, _ = _case(rng, 1, [P + L], [P + L], 2, 2, 8, 4)
    for mt in TYPES:
        sl = [0.3, 0.6] if mt in M.ALIBI_TYPES else None
        of, lf = oracle.prefix_encoder(query, key, value, bt, [P + L], [P + L], sl, mt, 2, 2, 0.5)
        op, lp = oracle.prefix_encoder(query[P:], key, value, bt, [L], [P + L], sl, mt, 2, 2, 0.5)
        np.testing.assert_allclose(op, of[P:], atol=1e-14)
        np.testing.assert_allclose(lp, lf[P:], atol=1e-14)


def test_lse_merge_identity():
    rng = np.random.default_rng(31)
    R, N, D = 5, 40, 6
    q = rng.standard_normal((R, D))
    k = rng.standard_normal((N, D))
    v = rng.standard_normal((N, D + 2))
    bias = rng.standard_normal((R, N))
    full = oracle.attend(q, k, v, 0.8, bias)
    cuts = [0, 7, 8, 25, 40]
    parts_o, parts_l = [], []
    for c0, c1 in zip(cuts[:-1], cuts[1:]):
        sub = np.full_like(bias, -np.inf)
        sub[:, c0:c1] = bias[:, c0:c1]
        o, l = oracle.attend(q, k, v, 0.8, sub)
        parts_o.append(o)
        parts_l.append(l)
    o, l = oracle.lse_merge(parts_o, parts_l)
    np.testing.assert_allclose(o, full[0], atol=1e-13)
    np.testing.assert_allclose(l, full[1], atol=1e-13)
    # A part that sees no key (LSE = -inf) contributes nothing.
    e = np.full((R,), -np.inf)
    o2, l2 = oracle.lse_merge(parts_o + [np.full_like(parts_o[0], 123.0)], parts_l + [e])
    np.testing.assert_allclose(o2, full[0], atol=1e-13)
    np.testing.assert_allclose(l2, full[1], atol=1e-13)


@pytest.mark.parametrize("prefix", [0, 100, 200])
@pytest.mark.parametrize("mt", [M.MASK_CAUSAL, M.MASK_ALIBI, M.MASK_ALIBI_SQRT, M.MASK_ALIBI_LEFT])
def test_expanded_compressed_mask_equals_full(prefix, mt):
    L = 300
    kv = prefix + L
    slope = 0.0625
    tile = {M.MASK_CAUSAL: M.compressed_norm(), M.MASK_ALIBI: M.compressed_alibi(),
            M.MASK_ALIBI_SQRT: M.compressed_alibi(), M.MASK_ALIBI_LEFT: M.compressed_alibi_left()}[mt]
    exp = M.expand_compressed(mt, tile, slope, L, kv)
    full = M.full_mask(mt, slope, L, kv)
    assert np.array_equal(np.isfinite(exp), np.isfinite(full))
    np.testing.assert_allclose(exp[np.isfinite(exp)], full[np.isfinite(full)], rtol=0, atol=1e-12)
    # The tiles have the printed sizes: [128,128] norm, [256,256] ALiBi.
    assert tile.shape == ((128, 128) if mt == M.MASK_CAUSAL else (256, 256))


def test_full_mask_values_small():
    """Spot values of the full rule on a 3-row, 5-key prefix case (prefix 2)."""
    m = M.full_mask(M.MASK_ALIBI, 0.5, 3, 5)
    inf = -np.inf
    want = np.array([[-1.0, -0.5, 0.0, inf, inf],
                     [-1.5, -1.0, -0.5, 0.0, inf],
                     [-2.0, -1.5, -1.0, -0.5, 0.0]])
    assert np.array_equal(m, want)
    s = M.full_mask(M.MASK_ALIBI_SQRT, 0.5, 3, 5)
    assert s[2, 0] == -0.5 * 2.0 and s[0, 2] == 0.0 and s[0, 3] == inf
    left = M.full_mask(M.MASK_ALIBI_LEFT, 0.5, 3, 5)
    assert np.array_equal(left[2], [0.0, 0.5, 1.0, 1.5, 2.0]) and left[0, 3] == inf
    none = M.full_mask(M.MASK_NONE, 0.5, 3, 5)
    assert (none == 0).all()


@pytest.mark.parametrize("cache_mode", [0, 1])
@pytest.mark.parametrize("spec", [False, True])
def test_mla_equals_generic_rule(cache_mode, spec):
    rng = np.random.default_rng(37 + cache_mode + 2 * spec)
    B, H, bs = 3, 4, 8
    ctx = np.array([19, 8, 33])
    qlens = np.array([3, 1, 4]) if spec else np.ones(3, dtype=int)
    T = int(qlens.sum())
    need = [-(-int(c) // bs) for c in ctx]
    nb = sum(need) + 2
    perm = rng.permutation(nb)
    bt = np.full((B, max(need)), perm[-1], dtype=np.int32)
    p = 0
    for b in range(B):
        bt[b, :need[b]] = perm[p:p + need[b]]
        p += need[b]
    q_nope = rng.standard_normal((T, H, 512))
    q_rope = rng.standard_normal((T, H, 64))
    lat = rng.standard_normal((nb, bs, 1, 512))
    rope = rng.standard_normal((nb, bs, 1, 64))
    full = np.concatenate([lat, rope], axis=3)
    if cache_mode == 0:
        ct, kr = full, None
    else:
        ct, kr = lat, rope
    mt = oracle.MLA_MASK_SPEC if spec else oracle.MLA_MASK_UNDEFINED
    ct_type = oracle.MLA_CALC_SPEC if spec else oracle.MLA_CALC_UNDEFINED
    o, l = oracle.mla(q_nope, q_rope, ct, kr, bt, ctx, qlens if spec else None, H, 0.07, mt, ct_type)
    q = np.concatenate([q_nope, q_rope], axis=2)
    ref_mask = M.MASK_CAUSAL if spec else M.MASK_NONE
    og, lg = oracle.prefix_encoder(q, full, lat, bt, qlens, ctx, None, ref_mask, H, 1, 0.07)
    np.testing.assert_allclose(o, og, atol=1e-13)
    np.testing.assert_allclose(l, lg, atol=1e-13)
    # Brute force for a few (token, head) rows: SPEC token t sees keys <= ctx - q_len + t.
    tok = 0
    for b in range(B):
        for t in range(qlens[b]):
            lim = ctx[b] - qlens[b] + t if spec else ctx[b] - 1
            h = (b + t) % H
            qv = q[tok, h]
            ks = [full[bt[b][j // bs], j % bs, 0] for j in range(lim + 1)]
            s = [float(np.float32(0.07)) * math.fsum(float(a) * float(c) for a, c in zip(qv, kk)) for kk in ks]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            tot = math.fsum(w)
            want = sum(wi * kk[:512] for wi, kk in zip(w, ks)) / tot
            np.testing.assert_allclose(o[tok, h], want, atol=1e-12)
            assert abs(l[tok, h] - (m + math.log(tot))) < 1e-12
            tok += 1


def test_oracle_rejects_bad_arguments():
    rng = np.random.default_rng(3)
    query, key, value, bt, _ = _case(rng, 1, [4], [4], 2, 2, 8, 4)
    with pytest.raises(ValueError):
        oracle.prefix_encoder(query, key, value, bt, [4], [4], None, M.MASK_ALIBI, 2, 2, 1.0)
    with pytest.raises(ValueError):
        oracle.prefix_encoder(query, key, value, bt, [5], [4], None, M.MASK_CAUSAL, 2, 2, 1.0)
    with pytest.raises(ValueError):
        oracle.prefix_encoder(query, key, value, bt, [4], [4], None, M.MASK_CAUSAL, 3, 2, 1.0)


def test_compressed_tile_shapes_match_page():
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "atb_constants.json")))
    shp = g["compressed_mask_shapes"]
    assert list(M.compressed_norm().shape) == shp["norm"]
    assert list(M.compressed_alibi().shape) == shp["alibi"]
    assert list(M.compressed_alibi_left().shape) == shp["alibi_left_align"]
    mt = g["prefix_encoder_mask_types"]
    assert (M.MASK_ALIBI, M.MASK_ALIBI_SQRT, M.MASK_ALIBI_LEFT, M.MASK_CAUSAL) == (
        mt["MASK_TYPE_ALIBI_COMPRESS"], mt["MASK_TYPE_ALIBI_COMPRESS_SQRT"],
        mt["MASK_TYPE_ALIBI_COMPRESS_LEFT_ALIGN"], mt["MASK_TYPE_CAUSAL_MASK"])


def test_mla_prefill_is_causal_self_attention():
    # calcType PREFILL (MLA page, calcType row: "prefill全量") with the SPEC mask and
    # whole prompts (qseqlen = contextLens) is causal self-attention over the prompt:
    # the prefix-encoder rule with no prefix, and a brute-force row.
    rng = np.random.default_rng(41)
    B, H, bs = 2, 3, 8
    ctx = np.array([13, 6])
    need = [-(-int(c) // bs) for c in ctx]
    nb = sum(need) + 1
    bt = np.full((B, max(need)), nb - 1, dtype=np.int32)
    bt[0, :need[0]] = [0, 1]
    bt[1, :need[1]] = [2]
    T = int(ctx.sum())
    q_nope = rng.standard_normal((T, H, 512))
    q_rope = rng.standard_normal((T, H, 64))
    lat = rng.standard_normal((nb, bs, 1, 512))
    rope = rng.standard_normal((nb, bs, 1, 64))
    full = np.concatenate([lat, rope], axis=3)
    o, l = oracle.mla(q_nope, q_rope, lat, rope, bt, ctx, ctx, H, 0.05, oracle.MLA_MASK_SPEC,
                      oracle.MLA_CALC_PREFILL)
    q = np.concatenate([q_nope, q_rope], axis=2)
    og, lg = oracle.prefix_encoder(q, full, lat, bt, ctx, ctx, None, M.MASK_CAUSAL, H, 1, 0.05)
    np.testing.assert_allclose(o, og, atol=1e-13)
    np.testing.assert_allclose(l, lg, atol=1e-13)
    # the first token of a prompt sees only key 0: its output is that key's latent row
    np.testing.assert_allclose(o[0, 1], lat[bt[0, 0], 0, 0], atol=1e-12)
    np.testing.assert_allclose(o[13, 2], lat[bt[1, 0], 0, 0], atol=1e-12)


def _brute_chunked(query, key, value, bt, seq_len, kv_seq_len, H, KVH, scale, chunk):
    """Pure-Python chunked-local causal attention: row at absolute a sees keys j <= a
    with j // chunk == a // chunk (one key at a time through the block table)."""
    bs = key.shape[1]
    g = H // KVH
    scale = float(np.float32(scale))
    res, row0 = {}, 0
    for b in range(len(seq_len)):
        L, kv = int(seq_len[b]), int(kv_seq_len[b])
        for h in range(H):
            for i in range(L):
                a = kv - L + i
                q = query[row0 + i][h]
                sc, vals = [], []
                for j in range((a // chunk) * chunk, a + 1):
                    blk = int(bt[b][j // bs])
                    k = key[blk][j % bs][h // g]
                    sc.append(scale * math.fsum(float(x) * float(y) for x, y in zip(q, k)))
                    vals.append(value[blk][j % bs][h // g])
                m = max(sc)
                w = [math.exp(s - m) for s in sc]
                tot = math.fsum(w)
                o = np.array([math.fsum(w[n] * float(vals[n][d]) for n in range(len(w))) / tot
                              for d in range(len(vals[0]))])
                res[(row0 + i, h)] = (o, m + math.log(tot))
        row0 += L
    return res


@pytest.mark.parametrize("chunk", [1, 3, 8, 64])
def test_chunked_mask_brute_force(chunk):
    rng = np.random.default_rng(50 + chunk)
    L, kv = [9, 5], [20, 5]
    query, key, value, bt, _ = _case(rng, 2, L, kv, 4, 2, 6, 4)
    o, l = oracle.prefix_encoder(query, key, value, bt, L, kv, None, M.MASK_CHUNKED_CAUSAL, 4, 2, 0.6,
                                 chunk=chunk)
    want = _brute_chunked(query, key, value, bt, L, kv, 4, 2, 0.6, chunk)
    for (r, h), (wo, wl) in want.items():
        np.testing.assert_allclose(o[r, h], wo, atol=1e-12)
        assert abs(l[r, h] - wl) < 1e-12


def test_chunked_mask_special_cases():
    rng = np.random.default_rng(57)
    L, kv = [12, 7], [30, 7]
    query, key, value, bt, _ = _case(rng, 2, L, kv, 2, 2, 5, 4)
    # a chunk at least as long as every sequence: plain causal
    oc, lc = oracle.prefix_encoder(query, key, value, bt, L, kv, None, M.MASK_CHUNKED_CAUSAL, 2, 2, 0.7,
                                   chunk=64)
    ref, lref = oracle.prefix_encoder(query, key, value, bt, L, kv, None, M.MASK_CAUSAL, 2, 2, 0.7)
    np.testing.assert_allclose(oc, ref, atol=1e-13)
    np.testing.assert_allclose(lc, lref, atol=1e-13)
    # chunk 1: every row sees only its own key -> that key's value, LSE = its score
    o1, l1 = oracle.prefix_encoder(query, key, value, bt, L, kv, None, M.MASK_CHUNKED_CAUSAL, 2, 2, 0.7,
                                   chunk=1)
    row = 0
    for b in range(2):
        for i in range(L[b]):
            a = kv[b] - L[b] + i
            blk, slot = bt[b][a // 4], a % 4
            for h in range(2):
                np.testing.assert_allclose(o1[row + i, h], value[blk, slot, h], atol=1e-13)
                s = float(np.float32(0.7)) * float(np.dot(query[row + i, h], key[blk, slot, h]))
                assert abs(l1[row + i, h] - s) < 1e-12
        row += L[b]
    with pytest.raises(ValueError):
        oracle.prefix_encoder(query, key, value, bt, L, kv, None, M.MASK_CHUNKED_CAUSAL, 2, 2, 0.7)


def _brute_mla_int8(qn, qr, ckv, kr, bt, ctx, qlens, H, scale, qkd, pvd, spec):
    """Pure-Python int8 MLA (MLA page, parameter table: int8 qNope / ctKV with
    per-head qkDescale / pvDescale): exact integer nope dot products, descales
    applied to the score and the output, softmax with math.exp."""
    bs = ckv.shape[1]
    out, lse = [], []
    tok = 0
    for b in range(len(ctx)):
        rows = [(int(bt[b][j // bs]), j % bs) for j in range(int(ctx[b]))]
        for t in range(int(qlens[b])):
            for h in range(H):
                lim = int(ctx[b]) - int(qlens[b]) + t + 1 if spec else int(ctx[b])
                s = []
                for j in range(lim):
                    blk, slot = rows[j]
                    nope = sum(int(qn[tok, h, d]) * int(ckv[blk, slot, 0, d]) for d in range(512))
                    rope = sum(float(qr[tok, h, d]) * float(kr[blk, slot, 0, d]) for d in range(64))
                    s.append(float(scale) * (float(qkd[h]) * nope + rope))
                m = max(s)
                w = [math.exp(x - m) for x in s]
                tot = sum(w)
                o = [float(pvd[h]) * sum(w[j] * int(ckv[rows[j][0], rows[j][1], 0, d]) for j in range(lim)) / tot
                     for d in range(512)]
                out.append(o)
                lse.append(m + math.log(tot))
            tok += 1
    return np.array(out), np.array(lse)


@pytest.mark.parametrize("spec", [False, True])
def test_mla_int8_brute_force(spec):
    import workloads as W
    qlens = [2, 3] if spec else None
    c = W.make_mla_int8(61, [7, 12], qlens, 2, 4, "bf16", 1 if spec else 0, 1 if spec else 0, 0.07)
    a = c.oracle_args()
    ro, rl = oracle.mla(**a)
    bo, bl = _brute_mla_int8(a["q_nope"], a["q_rope"], a["ct_kv"], a["k_rope"], a["block_tables"],
                             a["context_lens"], qlens or [1, 1], 2, np.float32(0.07),
                             np.float32(a["qk_descale"]), np.float32(a["pv_descale"]), spec)
    np.testing.assert_allclose(ro.reshape(-1, 512), bo, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(rl.reshape(-1), bl, rtol=1e-12, atol=1e-12)


def test_mla_int8_descale_invariants():
    import workloads as W
    c = W.make_mla_int8(62, [40, 9, 130], None, 3, 16, "fp16", 0, 0, 0.07)
    a = c.oracle_args()
    o1, l1 = oracle.mla(**a)
    # pvDescale scales the output linearly and leaves the LSE alone
    a2 = dict(a, pv_descale=a["pv_descale"] * np.float32(2.0))
    o2, l2 = oracle.mla(**a2)
    np.testing.assert_allclose(o2, 2.0 * o1, rtol=1e-12, atol=0)
    np.testing.assert_array_equal(l2, l1)
    # qkDescale 0 leaves the rope part alone: the float oracle with qNope = 0, and
    # pvDescale 1 reads ctKV as the values
    a3 = dict(a, qk_descale=np.zeros(3, np.float32), pv_descale=np.ones(3, np.float32))
    o3, l3 = oracle.mla(**a3)
    a4 = dict(a, q_nope=np.zeros(a["q_nope"].shape), ct_kv=a["ct_kv"].astype(np.float64),
              qk_descale=None, pv_descale=None)
    o4, l4 = oracle.mla(**a4)
    np.testing.assert_allclose(o3, o4, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l3, l4, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# Attention read through an explicit compressed tile (the mask_tile branch of
# oracle.prefix_encoder / prefix_encoder_rows).
# ---------------------------------------------------------------------------

_PAGE_TILES = {M.MASK_CAUSAL: M.compressed_norm, M.MASK_ALIBI: M.compressed_alibi,
               M.MASK_ALIBI_SQRT: M.compressed_alibi, M.MASK_ALIBI_LEFT: M.compressed_alibi_left}


@pytest.mark.parametrize("mt", [M.MASK_CAUSAL, M.MASK_ALIBI, M.MASK_ALIBI_SQRT, M.MASK_ALIBI_LEFT])
def test_prefix_encoder_with_page_tile_equals_generated_rule(mt):
    """The tiles as the compressed-mask page describes them, read through the
    tile branch, give the attention of the generated rule of the same type --
    with cached prefixes, so rows and keys span several 128-position blocks."""
    rng = np.random.default_rng(600 + mt)
    L, P = np.array([150, 70]), np.array([140, 300])
    kv = L + P
    H, KVH, D = 4, 2, 8
    q, k, v, bt, _ = _case(rng, 2, L, kv, H, KVH, D, 32)
    slopes = (2.0 ** (-8.0 * (np.arange(H) + 1) / H)).astype(np.float32) if mt != M.MASK_CAUSAL else None
    args = dict(query=q, key=k, value=v, block_tables=bt, seq_len=L, kv_seq_len=kv, slopes=slopes,
                mask_type=mt, head_num=H, kv_head_num=KVH, qk_scale=0.3)
    o_gen, l_gen = oracle.prefix_encoder(**args)
    o_tile, l_tile = oracle.prefix_encoder(mask_tile=_PAGE_TILES[mt](), **args)
    np.testing.assert_allclose(o_tile, o_gen, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l_tile, l_gen, rtol=0, atol=1e-12)


def _tile_pair(mt, tile, slope, a, j, kv):
    """The expansion of a compressed tile for one (query position a, key j), as
    the operation's contract states it: (visible, bias)."""
    T = 128
    if j >= kv:
        return False, 0.0
    bq, r, bk, c = a // T, a % T, j // T, j % T
    dk = bq - bk
    if dk < 0:
        return False, 0.0
    if mt == M.MASK_CAUSAL:
        if dk > 0:
            return True, 0.0
        y = float(tile[r][c])
        return (y != -math.inf), y
    y = float(tile[r][c] if dk == 0 else tile[T + r][c])
    if y == -math.inf:
        return False, 0.0
    if mt == M.MASK_ALIBI_LEFT:
        return True, slope * (y + T * bk)
    if dk >= 1:
        y -= T * (dk - 1)
    if mt == M.MASK_ALIBI:
        return True, slope * y
    return True, -slope * math.sqrt(-y)


@pytest.mark.parametrize("mt", [M.MASK_CAUSAL, M.MASK_ALIBI, M.MASK_ALIBI_SQRT, M.MASK_ALIBI_LEFT])
def test_prefix_encoder_with_perturbed_tile_brute_force(mt):
    """Arbitrary tile contents (extra bias, -inf holes that hide keys): the tile
    branch against a pure-Python pass, one (row, key) pair at a time."""
    rng = np.random.default_rng(700 + mt)
    T = 128
    n = T if mt == M.MASK_CAUSAL else 2 * T
    x = np.arange(n)[:, None]
    y = np.arange(n)[None, :]
    base = {M.MASK_CAUSAL: np.zeros((n, n)), M.MASK_ALIBI: (y - x).astype(float),
            M.MASK_ALIBI_SQRT: (y - x).astype(float), M.MASK_ALIBI_LEFT: np.broadcast_to(y, (n, n)).astype(float)}[mt]
    extra = rng.integers(-12, 1, size=(n, n)) / 4.0  # keeps the distance form <= 0
    tile = np.where(y <= x, base + extra, -np.inf)
    tile[(rng.random((n, n)) < 0.05) & (y < x)] = -np.inf
    L, P = np.array([40, 9]), np.array([230, 120])
    kv = L + P
    H, KVH, D = 2, 1, 4
    q, k, v, bt, _ = _case(rng, 2, L, kv, H, KVH, D, 16)
    slopes = np.array([0.75, 0.1], dtype=np.float32)
    scale = 0.4
    o, lse = oracle.prefix_encoder(q, k, v, bt, L, kv, slopes if mt != M.MASK_CAUSAL else None, mt, H, KVH,
                                   scale, mask_tile=tile)
    bs = k.shape[1]
    sc = float(np.float32(scale))
    starts = [0, int(L[0])]
    for b in range(2):
        for h in range(H):
            sl = float(np.float32(slopes[h])) if mt != M.MASK_CAUSAL else 0.0
            for i in range(int(L[b])):
                a = int(kv[b] - L[b]) + i
                qq = q[starts[b] + i][h]
                ss, vv = [], []
                for j in range(int(kv[b])):
                    vis, bias = _tile_pair(mt, tile, sl, a, j, int(kv[b]))
                    if not vis:
                        continue
                    blk = int(bt[b][j // bs])
                    dot = math.fsum(float(qq[d]) * float(k[blk][j % bs][0][d]) for d in range(D))
                    ss.append(sc * dot + bias)
                    vv.append(v[blk][j % bs][0])
                got_o, got_l = o[starts[b] + i][h], lse[starts[b] + i][h]
                if not ss:
                    assert got_l == -math.inf and np.all(got_o == 0.0)
                    continue
                m = max(ss)
                w = [math.exp(s - m) for s in ss]
                tot = math.fsum(w)
                want = [math.fsum(w[t] * float(vv[t][d]) for t in range(len(w))) / tot for d in range(D)]
                np.testing.assert_allclose(got_o, want, rtol=0, atol=1e-12)
                assert abs(got_l - (m + math.log(tot))) <= 1e-12 * max(1.0, abs(got_l))
