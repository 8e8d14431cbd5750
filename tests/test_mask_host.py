"""Host-side mask descriptor and block schedule of the HIP library, checked bit
for bit against the oracle's predicates (no GPU needed)."""

import numpy as np
import pytest

import attention_jvp_causal_attn_amd as aj
from oracle import block_causal_allowed, rects_allowed, tf_allowed


def csr_to_matrix(n_q, n_k, gq, rp, kb, ke):
    M = np.zeros((n_q, n_k), dtype=bool)
    for g in range(len(gq) - 1):
        for r in range(rp[g], rp[g + 1]):
            M[gq[g]:gq[g + 1], kb[r]:ke[r]] = True
    return M


def check_canonical(n_q, n_k, gq, rp, kb, ke):
    assert gq[0] == 0 and gq[-1] == n_q and np.all(np.diff(gq) > 0)
    assert rp[0] == 0 and np.all(np.diff(rp) >= 0) and rp[-1] == len(kb)
    for g in range(len(gq) - 1):
        ranges = list(zip(kb[rp[g]:rp[g + 1]], ke[rp[g]:rp[g + 1]]))
        for b, e in ranges:
            assert 0 <= b < e <= n_k                      # non-empty, in range
        for (b0, e0), (b1, e1) in zip(ranges, ranges[1:]):
            assert e0 < b1                                # sorted, disjoint, not touching
        if g > 0:
            prev = list(zip(kb[rp[g - 1]:rp[g]], ke[rp[g - 1]:rp[g]]))
            assert prev != ranges                         # adjacent groups differ


TF_CASES = [(4, 16, 1), (21, 3, 1), (21, 2, 3), (7, 5, 1), (33, 1, 3), (6, 7, 2), (1, 1, 1),
            (2, 37, 2)]


@pytest.mark.parametrize("nf,tpf,fpc", TF_CASES)
def test_tf_descriptor_matches_predicate(nf, tpf, fpc):
    m = aj.attn_jvp_mask_tf(nf, tpf, fpc)
    info = m.info()
    pred = tf_allowed(nf, tpf, fpc)
    assert info["n_q"] == info["n_k"] == pred.n_q
    gq, rp, kb, ke = aj.attn_jvp_mask_export(m)
    check_canonical(pred.n_q, pred.n_k, gq, rp, kb, ke)
    M = csr_to_matrix(pred.n_q, pred.n_k, gq, rp, kb, ke)
    np.testing.assert_array_equal(M, pred.matrix())
    F, C = nf // fpc, tpf * fpc
    assert info["n_visible_pairs"] == C * C * F * (F + 1) == int(M.sum())
    assert info["n_groups"] == 2 * F or (F == 1 and info["n_groups"] == 2)


@pytest.mark.parametrize("nf,tpf,fpc", [(21, 1560, 1), (21, 1560, 3), (7, 1560, 1),
                                        (33, 1560, 3)])
def test_tf_descriptor_full_size_intervals(nf, tpf, fpc):
    # Wan2.1-1.3B-shaped masks: compare each group's intervals with the
    # predicate's row on the group's first and last row.
    m = aj.attn_jvp_mask_tf(nf, tpf, fpc)
    pred = tf_allowed(nf, tpf, fpc)
    gq, rp, kb, ke = aj.attn_jvp_mask_export(m)
    for g in range(len(gq) - 1):
        row = np.zeros(pred.n_k, dtype=bool)
        for r in range(rp[g], rp[g + 1]):
            row[kb[r]:ke[r]] = True
        for q in (gq[g], gq[g + 1] - 1, (gq[g] + gq[g + 1]) // 2):
            np.testing.assert_array_equal(row, pred([q])[0])
    F, C = nf // fpc, tpf * fpc
    assert m.info()["n_visible_pairs"] == C * C * F * (F + 1)


def random_rects(rng, n_q, n_k, max_groups=6, max_ranges=4):
    n_groups = int(rng.integers(1, max_groups + 1))
    cuts = np.sort(rng.choice(np.arange(1, n_q), size=min(n_groups - 1, n_q - 1), replace=False))
    gq = np.concatenate([[0], cuts, [n_q]]).astype(np.int32)
    rp, kb, ke = [0], [], []
    for g in range(len(gq) - 1):
        nr = int(rng.integers(0, max_ranges + 1))
        pts = np.sort(rng.choice(np.arange(0, n_k + 1), size=min(2 * nr, n_k + 1), replace=False))
        for i in range(0, len(pts) - 1, 2):
            kb.append(pts[i])
            ke.append(pts[i + 1])
        rp.append(len(kb))
    return gq, np.array(rp, np.int32), np.array(kb, np.int32), np.array(ke, np.int32)


@pytest.mark.parametrize("seed", range(12))
def test_rect_descriptor_matches_predicate(seed):
    rng = np.random.default_rng(seed)
    n_q, n_k = int(rng.integers(1, 200)), int(rng.integers(1, 200))
    gq, rp, kb, ke = random_rects(rng, n_q, n_k)
    m = aj.attn_jvp_mask_rects(n_q, n_k, gq, rp, kb, ke)
    rects = [(gq[g], gq[g + 1], kb[r], ke[r]) for g in range(len(gq) - 1)
             for r in range(rp[g], rp[g + 1])]
    pred = rects_allowed(n_q, n_k, rects)
    egq, erp, ekb, eke = aj.attn_jvp_mask_export(m)
    check_canonical(n_q, n_k, egq, erp, ekb, eke)
    M = csr_to_matrix(n_q, n_k, egq, erp, ekb, eke)
    np.testing.assert_array_equal(M, pred.matrix())
    assert m.info()["n_visible_pairs"] == int(M.sum())


def brute_schedule(M, BM, BN):
    n_q, n_k = M.shape
    n_tiles = -(-n_q // BM)
    n_kb = -(-n_k // BN)
    out = []
    for t in range(n_tiles):
        rows = M[t * BM:(t + 1) * BM]
        ents = []
        for kb in range(n_kb):
            blk = np.zeros((rows.shape[0], BN), dtype=bool)
            sub = rows[:, kb * BN:(kb + 1) * BN]
            blk[:, :sub.shape[1]] = sub
            if blk.any():
                ents.append((kb, bool(blk.all()), blk))
        # full blocks first, then partial ones, each in increasing order
        out.append([e for e in ents if e[1]] + [e for e in ents if not e[1]])
    return out


def check_schedule(mask, M, BM, BN):
    s = aj.attn_jvp_mask_schedule(mask, BM, BN)
    ref = brute_schedule(M, BM, BN)
    assert len(s["tile_offsets"]) == len(ref) + 1
    words = BN // 32
    for t, ents in enumerate(ref):
        e0, e1 = s["tile_offsets"][t], s["tile_offsets"][t + 1]
        assert e1 - e0 == len(ents)
        for e, (kb, full, blk) in zip(range(e0, e1), ents):
            assert s["entry_block"][e] == kb
            p = s["entry_partial"][e]
            assert (p < 0) == full
            if not full:
                bits = s["partial_bits"][p]                 # [BM, words]
                got = np.zeros((BM, BN), dtype=bool)
                for w in range(words):
                    for i in range(32):
                        got[:, 32 * w + i] = (bits[:, w] >> np.uint32(i)) & np.uint32(1)
                want = np.zeros((BM, BN), dtype=bool)
                want[:blk.shape[0]] = blk
                np.testing.assert_array_equal(got, want)
    counts = np.diff(s["tile_offsets"])
    order = s["tile_order"]
    assert sorted(order.tolist()) == list(range(len(ref)))
    key = [(-counts[t], t) for t in order]
    assert key == sorted(key)


@pytest.mark.parametrize("nf,tpf,fpc", [(4, 16, 1), (5, 37, 1), (6, 23, 2), (3, 100, 3),
                                        (2, 1, 1)])
@pytest.mark.parametrize("BM,BN", [(128, 32), (64, 32), (128, 64), (16, 32)])
def test_tf_schedule_matches_brute_force(nf, tpf, fpc, BM, BN):
    m = aj.attn_jvp_mask_tf(nf, tpf, fpc)
    check_schedule(m, tf_allowed(nf, tpf, fpc).matrix(), BM, BN)


@pytest.mark.parametrize("seed", range(8))
def test_rect_schedule_matches_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    n_q, n_k = int(rng.integers(1, 300)), int(rng.integers(1, 300))
    gq, rp, kb, ke = random_rects(rng, n_q, n_k)
    m = aj.attn_jvp_mask_rects(n_q, n_k, gq, rp, kb, ke)
    M = csr_to_matrix(n_q, n_k, *aj.attn_jvp_mask_export(m))
    for BM, BN in [(128, 32), (64, 32), (32, 64)]:
        check_schedule(m, M, BM, BN)


@pytest.mark.parametrize("nf,tpf,fpc", [(21, 1560, 1), (21, 1560, 3), (7, 1560, 1),
                                        (33, 1560, 3)])
def test_full_size_schedule_covers_visible_pairs(nf, tpf, fpc):
    # Every admissible pair is covered exactly once by the scheduled blocks.
    m = aj.attn_jvp_mask_tf(nf, tpf, fpc)
    info = m.info()
    for dtype, tangent in ((aj.ATTN_JVP_BF16, True), (aj.ATTN_JVP_BF16, False),
                           (aj.ATTN_JVP_F32, True)):
        BM, BN = aj.attn_jvp_tile_shape(dtype, 128, tangent)
        s = aj.attn_jvp_mask_schedule(m, BM, BN)
        n_q, n_k = info["n_q"], info["n_k"]
        total = 0
        for t in range(len(s["tile_offsets"]) - 1):
            rows = min(n_q, (t + 1) * BM) - t * BM
            e0, e1 = s["tile_offsets"][t], s["tile_offsets"][t + 1]
            part = s["entry_partial"][e0:e1]
            total += int((part < 0).sum()) * rows * BN
        bits = s["partial_bits"]
        total += int(np.unpackbits(bits.view(np.uint8)).sum())
        assert total == info["n_visible_pairs"]


def test_mask_errors():
    E = aj.AttnJvpError
    with pytest.raises(E) as ei:
        aj.attn_jvp_mask_tf(5, 10, 2)          # frames not a multiple of the chunk
    assert ei.value.status == aj._lib.ATTN_JVP_ERR_SHAPE
    for args in [(0, 1, 1), (1, 0, 1), (1, 1, 0), (-3, 4, 1), (2 ** 20, 2 ** 10, 1)]:
        with pytest.raises(E) as ei:
            aj.attn_jvp_mask_tf(*args)
        assert ei.value.status == aj._lib.ATTN_JVP_ERR_SHAPE
    ok = dict(n_q=10, n_k=8, group_q_begin=[0, 4, 10], range_ptr=[0, 1, 2], k_begin=[0, 2],
              k_end=[3, 8])
    aj.attn_jvp_mask_rects(**ok)
    bad = [
        dict(group_q_begin=[1, 4, 10]),                      # partition does not start at 0
        dict(group_q_begin=[0, 4, 9]),                       # does not end at n_q
        dict(group_q_begin=[0, 4, 4]),                       # not strictly increasing
        dict(range_ptr=[0, 2, 1]),                           # decreasing CSR
        dict(k_begin=[0, 5], k_end=[3, 4]),                  # end < begin
        dict(k_begin=[0, 2], k_end=[3, 9]),                  # past n_k
        dict(range_ptr=[0, 2, 2], k_begin=[2, 0], k_end=[3, 1]),  # unsorted
        dict(range_ptr=[0, 2, 2], k_begin=[0, 2], k_end=[3, 5]),  # overlapping
        dict(k_begin=[-1, 2]),                               # negative
    ]
    for b in bad:
        args = dict(ok)
        args.update(b)
        with pytest.raises(E) as ei:
            aj.attn_jvp_mask_rects(**args)
        assert ei.value.status == aj._lib.ATTN_JVP_ERR_MASK, b
    # CSR pointers past the end of the key arrays are refused before the C
    # builder could read beyond them
    for rp in ([0, 1, 5], [0, 3, 3], [0, -1, 2]):
        with pytest.raises(ValueError):
            aj.attn_jvp_mask_rects(10, 8, [0, 4, 10], rp, [0, 2], [3, 8])
    with pytest.raises(E) as ei:
        aj.attn_jvp_mask_rects(0, 8, [0], [0], [], [])
    assert ei.value.status == aj._lib.ATTN_JVP_ERR_SHAPE
    with pytest.raises(E) as ei:
        aj.attn_jvp_mask_dense(4, 0)
    assert ei.value.status == aj._lib.ATTN_JVP_ERR_SHAPE
    m = aj.attn_jvp_mask_tf(2, 3, 1)
    with pytest.raises(E) as ei:
        aj.attn_jvp_mask_schedule(m, 64, 48)
    assert ei.value.status == aj._lib.ATTN_JVP_ERR_SHAPE


def test_canonical_merges():
    # touching ranges merge, empty ranges vanish, identical adjacent groups merge
    m = aj.attn_jvp_mask_rects(6, 10, [0, 2, 4, 6], [0, 3, 4, 5], [0, 3, 5, 0, 0],
                               [3, 3, 7, 7, 7])
    gq, rp, kb, ke = aj.attn_jvp_mask_export(m)
    assert gq.tolist() == [0, 2, 6]
    assert list(zip(kb, ke)) == [(0, 3), (5, 7), (0, 7)]
    m = aj.attn_jvp_mask_rects(3, 10, [0, 3], [0, 3], [0, 3, 5], [3, 5, 9])
    gq, rp, kb, ke = aj.attn_jvp_mask_export(m)
    assert list(zip(kb, ke)) == [(0, 9)]
    d = aj.attn_jvp_mask_dense(7, 9)
    assert d.info() == dict(n_q=7, n_k=9, n_groups=1, n_ranges=1, n_visible_pairs=63)


# ------------------------------------------------------------ transpose ----

@pytest.mark.parametrize("nf,tpf,fpc", TF_CASES)
def test_tf_transpose_is_matrix_transpose(nf, tpf, fpc):
    m = aj.attn_jvp_mask_tf(nf, tpf, fpc)
    t = aj.attn_jvp_mask_transpose(m)
    N = 2 * nf * tpf
    gq, rp, kb, ke = aj.attn_jvp_mask_export(t)
    check_canonical(N, N, gq, rp, kb, ke)
    np.testing.assert_array_equal(csr_to_matrix(N, N, gq, rp, kb, ke),
                                  tf_allowed(nf, tpf, fpc).matrix().T)
    assert t.info()["n_visible_pairs"] == m.info()["n_visible_pairs"]
    # transposing twice gives back the canonical original
    tt = aj.attn_jvp_mask_transpose(t)
    for a, b in zip(aj.attn_jvp_mask_export(tt), aj.attn_jvp_mask_export(m)):
        np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("seed", range(12))
def test_rect_transpose_is_matrix_transpose(seed):
    rng = np.random.default_rng(100 + seed)
    n_q, n_k = int(rng.integers(1, 200)), int(rng.integers(1, 200))
    gq, rp, kb, ke = random_rects(rng, n_q, n_k)
    m = aj.attn_jvp_mask_rects(n_q, n_k, gq, rp, kb, ke)
    t = aj.attn_jvp_mask_transpose(m)
    info = t.info()
    assert (info["n_q"], info["n_k"]) == (n_k, n_q)
    egq, erp, ekb, eke = aj.attn_jvp_mask_export(t)
    check_canonical(n_k, n_q, egq, erp, ekb, eke)
    M = csr_to_matrix(n_q, n_k, *aj.attn_jvp_mask_export(m))
    np.testing.assert_array_equal(csr_to_matrix(n_k, n_q, egq, erp, ekb, eke), M.T)
    # the backward's key-tile schedule is the schedule of the transpose
    check_schedule(t, M.T, 128, 32)


# ---------------------------------------------------- block-causal (DF) ----

@pytest.mark.parametrize("n_units,unit_tokens", [(1, 1), (5, 1), (4, 37), (21, 13), (3, 130)])
def test_block_causal_matches_predicate(n_units, unit_tokens):
    m = aj.attn_jvp_mask_block_causal(n_units, unit_tokens)
    N = n_units * unit_tokens
    gq, rp, kb, ke = aj.attn_jvp_mask_export(m)
    check_canonical(N, N, gq, rp, kb, ke)
    M = block_causal_allowed(n_units, unit_tokens).matrix()
    np.testing.assert_array_equal(csr_to_matrix(N, N, gq, rp, kb, ke), M)
    assert m.info()["n_visible_pairs"] == int(M.sum())
    check_schedule(m, M, 128, 32)


def test_block_causal_errors():
    for args in [(0, 4), (4, 0), (-1, 3), (1 << 16, 1 << 15)]:
        with pytest.raises(aj.AttnJvpError):
            aj.attn_jvp_mask_block_causal(*args)


# ------------------------------------------------ split-key unit lists ----

def check_split(mask, BM, BN, S):
    """The unit list of a split launch against the rule in the C header,
    recomputed here from the (separately tested) tile schedule."""
    s = aj.attn_jvp_mask_schedule(mask, BM, BN)
    u = aj.attn_jvp_mask_split_schedule(mask, BM, BN, S)
    toff = s["tile_offsets"]
    counts = np.diff(toff)
    L = max(1, -(-int(counts.max(initial=0)) // S))
    offs, tiles, parts, nparts = [0], [], [], 0
    for t, n in enumerate(counts):
        k = max(1, -(-int(n) // L))
        for j in range(k):
            offs.append(int(toff[t]) + (int(n) * (j + 1)) // k)
            tiles.append(t)
            parts.append(nparts + j if k > 1 else -1)
        if k > 1:
            nparts += k
    np.testing.assert_array_equal(u["unit_offsets"], offs)
    np.testing.assert_array_equal(u["unit_tile"], tiles)
    np.testing.assert_array_equal(u["unit_part"], parts)
    assert u["n_parts"] == nparts
    # every entry of every tile in exactly one unit, in order; no unit longer than L
    ucount = np.diff(u["unit_offsets"])
    assert ucount.max(initial=0) <= L and ucount.min(initial=0) >= 0
    for t in range(len(counts)):
        mine = np.nonzero(u["unit_tile"] == t)[0]
        assert len(mine) >= 1 and np.all(np.diff(mine) == 1)
        assert u["unit_offsets"][mine[0]] == toff[t] and u["unit_offsets"][mine[-1] + 1] == toff[t + 1]
    order = u["unit_order"]
    assert sorted(order.tolist()) == list(range(len(tiles)))
    key = [(-ucount[x], x) for x in order]
    assert key == sorted(key)
    return u


@pytest.mark.parametrize("S", [1, 2, 3, 8, 1000])
@pytest.mark.parametrize("nf,tpf,fpc", [(4, 16, 1), (6, 23, 2), (9, 60, 3)])
def test_split_units_follow_the_rule(nf, tpf, fpc, S):
    m = aj.attn_jvp_mask_tf(nf, tpf, fpc)
    for BM, BN in [(128, 32), (256, 32), (64, 32)]:
        u = check_split(m, BM, BN, S)
        if S == 1:   # one unit per tile, nothing to merge
            assert u["n_parts"] == 0 and np.all(u["unit_tile"] == np.arange(len(u["unit_tile"])))


@pytest.mark.parametrize("seed", range(8))
def test_split_units_random_rects(seed):
    rng = np.random.default_rng(100 + seed)
    n_q, n_k = int(rng.integers(1, 700)), int(rng.integers(1, 900))
    m = aj.attn_jvp_mask_rects(n_q, n_k, *random_rects(rng, n_q, n_k))
    for S in (1, 2, 5):
        check_split(m, 128, 32, S)


def test_split_units_kv_cache_rectangle():
    # one chunk of queries against a long key sequence: every tile has the
    # same list, cut into exactly max_splits pieces
    m = aj.attn_jvp_mask_rects(4680, 65520, [0, 4680], [0, 1], [0], [65520])
    u = check_split(m, 256, 32, 8)
    assert len(u["unit_tile"]) == 19 * 8 and u["n_parts"] == 19 * 8
    # a tile without any admissible key stays one empty unit
    m = aj.attn_jvp_mask_rects(600, 400, [0, 256, 600], [0, 0, 1], [0], [400])
    u = check_split(m, 256, 32, 4)
    assert np.diff(u["unit_offsets"])[0] == 0 and u["unit_part"][0] == -1


def test_split_errors():
    m = aj.attn_jvp_mask_tf(4, 16, 1)
    for args in [(128, 32, 0), (128, 32, -3), (128, 48, 2), (0, 32, 2)]:
        with pytest.raises(aj.AttnJvpError):
            aj.attn_jvp_mask_split_schedule(m, *args)


def test_schedule_larger_than_int32_entries_is_refused():
    # The device schedule indexes its (tile, key block) entries with int32: a
    # dense 2^26 x 2^26 mask would need 2^18 tiles x 2^21 blocks = 2^39
    # entries at 256 x 32 tiles.  The entries are counted (not built) first
    # and the schedule is refused with ERR_SHAPE, without allocating it.
    n = 1 << 26
    m = aj.attn_jvp_mask_dense(n, n)
    with pytest.raises(aj.AttnJvpError) as ei:
        aj.attn_jvp_mask_schedule(m, 256, 32)
    assert ei.value.status == aj._lib.ATTN_JVP_ERR_SHAPE
    with pytest.raises(aj.AttnJvpError) as ei:
        aj.attn_jvp_mask_split_schedule(m, 256, 32, 2)
    assert ei.value.status == aj._lib.ATTN_JVP_ERR_SHAPE
    # 2^31 - 1 entries is the largest schedule: 46,341 tiles of one row x
    # 46,341 blocks of 32 keys is 2,147,488,281 > 2^31 - 1 ...
    big = aj.attn_jvp_mask_dense(46341, 46341 * 32)
    with pytest.raises(aj.AttnJvpError) as ei:
        aj.attn_jvp_mask_schedule(big, 1, 32)
    assert ei.value.status == aj._lib.ATTN_JVP_ERR_SHAPE
