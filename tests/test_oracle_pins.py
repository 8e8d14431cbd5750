"""Pins of the CPU oracle to things other than itself.

Every check here ties ``oracle/`` to an independent fact: hand-written mask
matrices, a hand-derived worked example, closed forms, central finite
differences, PyTorch's own scaled-dot-product attention and its forward-mode
AD, and mask invariants.  A plausible mistake in the oracle (a dropped term,
a wrong sign or index, a transposed operand, an off-by-one unit boundary)
fails at least one of them.
"""

import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from torch.func import jvp
from torch.nn.attention import SDPBackend, sdpa_kernel

import oracle
from oracle import (block_causal_allowed, dense_allowed, masked_attention,
                    masked_attention_jvp, rects_allowed, tf_allowed)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed, std=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * std


def _six(B, N, H, D, seed, tstd=1.0):
    return [_rand((B, N, H, D), seed + t, 1.0 if t < 3 else tstd) for t in range(6)]


def _load_mask(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([int(x) for x in line.split()])
    params, mat = rows[0], np.array(rows[1:], dtype=bool)
    return params, mat


# ---------------------------------------------------------------- masks ----

@pytest.mark.parametrize("name", ["tf_mask_frame_F2_C1.txt",
                                  "tf_mask_frame_F3_C2.txt",
                                  "tf_mask_chunk_F4_C1_K2.txt"])
def test_tf_predicate_matches_hand_written(name):
    (nf, tpf, fpc), mat = _load_mask(name)
    pred = tf_allowed(nf, tpf, fpc)
    assert pred.matrix().shape == mat.shape
    np.testing.assert_array_equal(pred.matrix(), mat)


@pytest.mark.parametrize("nf,tpf,fpc", [(4, 16, 1), (21, 3, 1), (21, 2, 3),
                                        (7, 5, 1), (33, 1, 3), (6, 7, 2)])
def test_tf_visible_pair_count_closed_form(nf, tpf, fpc):
    # F units of C tokens per stream: clean unit u sees (u+1)C clean keys,
    # noisy unit u sees uC clean + C noisy = (u+1)C keys; 2F groups of C rows.
    F_, C = nf // fpc, tpf * fpc
    closed = 2 * sum(C * (u + 1) * C for u in range(F_))
    assert closed == C * C * F_ * (F_ + 1)
    assert int(tf_allowed(nf, tpf, fpc).matrix().sum()) == closed


def test_tf_semantics_statements():
    pred = tf_allowed(6, 3, 2)
    M = pred.matrix()
    Nc = pred.n_clean
    noisy_q, unit_q = pred.stream_and_unit(np.arange(pred.n_q))
    # clean rows never see noisy keys
    assert not M[:Nc, Nc:].any()
    for i in range(pred.n_q):
        for j in range(pred.n_k):
            if noisy_q[i] and noisy_q[j]:
                assert M[i, j] == (unit_q[i] == unit_q[j])
            if noisy_q[i] and not noisy_q[j]:
                assert M[i, j] == (unit_q[j] < unit_q[i])


def test_rect_and_block_causal_predicates():
    r = rects_allowed(4, 5, [(0, 2, 0, 1), (1, 4, 3, 5)])
    expect = np.array([[1, 0, 0, 0, 0], [1, 0, 0, 1, 1],
                       [0, 0, 0, 1, 1], [0, 0, 0, 1, 1]], dtype=bool)
    np.testing.assert_array_equal(r.matrix(), expect)
    bc = block_causal_allowed(3, 2).matrix()
    np.testing.assert_array_equal(bc, np.kron(np.tril(np.ones((3, 3))), np.ones((2, 2))).astype(bool))
    assert dense_allowed(3, 4).matrix().all()


# ----------------------------------------------------- worked example ----

def _ev(s):
    return float(eval(str(s), {"ln": math.log, "__builtins__": {}}))


def test_hand_derived_example():
    with open(os.path.join(GOLDEN, "hand_example_d1.json")) as f:
        g = json.load(f)
    arr = {n: np.array([[_ev(x) for x in row] for row in g[n]]).reshape(1, 2, 1, 1)
           for n in ("q", "k", "v", "dq", "dk", "dv")}
    O, dO, LSE = masked_attention_jvp(arr["q"], arr["k"], arr["v"], arr["dq"],
                                      arr["dk"], arr["dv"], dense_allowed(2, 2),
                                      scale=1.0)
    np.testing.assert_allclose(O.reshape(2), [_ev(r[0]) for r in g["O"]], rtol=0, atol=1e-14)
    np.testing.assert_allclose(dO.reshape(2), [_ev(r[0]) for r in g["dO"]], rtol=0, atol=1e-14)
    np.testing.assert_allclose(LSE.reshape(2), [_ev(x) for x in g["LSE"]], rtol=0, atol=1e-14)


# ------------------------------------------------ library cross-checks ----

def _torch_sdpa(q, k, v, mask, scale):
    # [B, N, H, D] -> [B, H, N, D] for torch
    t = lambda x: torch.from_numpy(x).permute(0, 2, 1, 3)
    return F.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=torch.from_numpy(mask),
                                          scale=scale)


MASKS = {
    "tf_frame": lambda: tf_allowed(3, 4, 1),
    "tf_chunk": lambda: tf_allowed(4, 3, 2),
    "dense": lambda: dense_allowed(16, 16),
    "rects": lambda: rects_allowed(20, 20, [(0, 7, 2, 9), (5, 20, 0, 3), (12, 20, 15, 20)]),
}


@pytest.mark.parametrize("mname", list(MASKS))
def test_primal_matches_torch_sdpa(mname):
    pred = MASKS[mname]()
    N = pred.n_q
    q, k, v, *_ = _six(2, N, 3, 8, seed=11)
    scale = 0.37
    M = pred.matrix()
    O, LSE = masked_attention(q, k, v, pred, scale=scale)
    with sdpa_kernel(SDPBackend.MATH):
        ref = _torch_sdpa(q, k, v, M, scale).permute(0, 2, 1, 3).numpy()
    np.testing.assert_allclose(O, ref, rtol=1e-12, atol=1e-12)
    # LSE against torch.logsumexp of the masked score matrix
    S = torch.einsum("bnhd,bmhd->bhnm", torch.from_numpy(q), torch.from_numpy(k)) * scale
    S = S.masked_fill(~torch.from_numpy(M), float("-inf"))
    np.testing.assert_allclose(LSE, torch.logsumexp(S, dim=-1).numpy(), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("mname", list(MASKS))
def test_tangent_matches_torch_forward_ad(mname):
    pred = MASKS[mname]()
    N = pred.n_q
    q, k, v, dq, dk, dv = _six(1, N, 2, 8, seed=21, tstd=0.3)
    M = torch.from_numpy(pred.matrix())
    t = lambda x: torch.from_numpy(x).permute(0, 2, 1, 3)

    def f(q_, k_, v_):
        return F.scaled_dot_product_attention(q_, k_, v_, attn_mask=M)

    with sdpa_kernel(SDPBackend.MATH):
        o_ref, do_ref = jvp(f, (t(q), t(k), t(v)), (t(dq), t(dk), t(dv)))
    O, dO, _ = masked_attention_jvp(q, k, v, dq, dk, dv, pred)
    np.testing.assert_allclose(O, o_ref.permute(0, 2, 1, 3).numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dO, do_ref.permute(0, 2, 1, 3).numpy(), rtol=1e-11, atol=1e-12)


# -------------------------------------------------- finite differences ----

@pytest.mark.parametrize("mname,D", [("tf_frame", 4), ("tf_chunk", 16), ("rects", 16),
                                     ("dense", 64)])
def test_tangent_central_finite_difference(mname, D):
    pred = MASKS[mname]()
    N = pred.n_q
    x = _six(1, N, 2, D, seed=31)
    eps = 1e-6
    plus = [a + eps * b for a, b in zip(x[:3], x[3:])]
    minus = [a - eps * b for a, b in zip(x[:3], x[3:])]
    Op, Lp = masked_attention(*plus, pred)
    Om, Lm = masked_attention(*minus, pred)
    fd = (Op - Om) / (2 * eps)
    _, dO, _ = masked_attention_jvp(*x, pred)
    rel = np.abs(dO - fd).max() / np.abs(fd).max()
    assert rel <= 1e-7, rel


@pytest.mark.parametrize("mname,D", [("tf_frame", 4), ("tf_chunk", 16), ("rects", 16)])
def test_lse_tangent_central_finite_difference(mname, D):
    pred = MASKS[mname]()
    x = _six(1, pred.n_q, 2, D, seed=33)
    eps = 1e-6
    plus = [a + eps * b for a, b in zip(x[:3], x[3:])]
    minus = [a - eps * b for a, b in zip(x[:3], x[3:])]
    _, Lp = masked_attention(*plus, pred)
    _, Lm = masked_attention(*minus, pred)
    live = np.isfinite(Lp)
    fd = np.where(live, (Lp - Lm) / (2 * eps), 0.0)
    *_, dL = masked_attention_jvp(*x, pred, lse_tangent=True)
    rel = np.abs(dL - fd).max() / np.abs(fd).max()
    assert rel <= 1e-7, rel


def test_lse_tangent_matches_torch_forward_ad():
    pred = MASKS["tf_chunk"]()
    q, k, v, dq, dk, dv = _six(1, pred.n_q, 2, 8, seed=35, tstd=0.3)
    M = torch.from_numpy(pred.matrix())
    sc = 1 / math.sqrt(8)

    def lse(q_, k_):
        S = (q_ @ k_.transpose(-1, -2)) * sc
        return torch.logsumexp(S.masked_fill(~M, float("-inf")), dim=-1)

    t = lambda x: torch.from_numpy(x).permute(0, 2, 1, 3)
    _, ref = jvp(lse, (t(q), t(k)), (t(dq), t(dk)))
    *_, dL = masked_attention_jvp(q, k, v, dq, dk, dv, pred, lse_tangent=True)
    np.testing.assert_allclose(dL, ref.numpy(), rtol=1e-11, atol=1e-13)


# ------------------------------------------------------- closed forms ----

def test_zero_query_key_tangents_gives_p_dv():
    pred = tf_allowed(3, 4, 1)
    q, k, v, _, _, dv = _six(1, pred.n_q, 2, 8, seed=41)
    z = np.zeros_like(q)
    _, dO, _ = masked_attention_jvp(q, k, v, z, z, dv, pred)
    # P from an independent softmax (scipy) over the masked score matrix
    from scipy.special import softmax
    M = pred.matrix()
    for h in range(2):
        S = (q[0, :, h] @ k[0, :, h].T) / math.sqrt(8)
        S = np.where(M, S, -np.inf)
        P = softmax(S, axis=1)
        np.testing.assert_allclose(dO[0, :, h], P @ dv[0, :, h], rtol=1e-12, atol=1e-13)


def test_single_visible_key():
    # diagonal rect mask: every row sees only itself
    N = 9
    pred = rects_allowed(N, N, [(i, i + 1, i, i + 1) for i in range(N)])
    q, k, v, dq, dk, dv = _six(2, N, 2, 16, seed=51)
    O, dO, LSE = masked_attention_jvp(q, k, v, dq, dk, dv, pred, scale=0.5)
    np.testing.assert_array_equal(O, v)
    np.testing.assert_allclose(dO, dv, rtol=0, atol=1e-15)
    np.testing.assert_allclose(LSE, 0.5 * np.einsum("bnhd,bnhd->bhn", q, k), rtol=1e-14)
    # TF mask with one token per frame: clean row 0 and noisy row Nc see only themselves
    pred = tf_allowed(5, 1, 1)
    q, k, v, dq, dk, dv = _six(1, pred.n_q, 1, 8, seed=52)
    O, dO, LSE = masked_attention_jvp(q, k, v, dq, dk, dv, pred)
    for r in (0, pred.n_clean):
        np.testing.assert_array_equal(O[0, r], v[0, r])
        np.testing.assert_allclose(dO[0, r], dv[0, r], atol=1e-15)


def test_zero_queries_give_uniform_weights():
    pred = tf_allowed(4, 3, 2)
    _, k, v, _, dk, dv = _six(1, pred.n_q, 2, 8, seed=61)
    z = np.zeros_like(k)
    O, dO, LSE = masked_attention_jvp(z, k, v, z, dk, dv, pred)
    M = pred.matrix()
    cnt = M.sum(1)
    for h in range(2):
        np.testing.assert_allclose(O[0, :, h], (M @ v[0, :, h]) / cnt[:, None], rtol=1e-13)
        np.testing.assert_allclose(dO[0, :, h], (M @ dv[0, :, h]) / cnt[:, None], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(LSE[0, h], np.log(cnt), rtol=1e-14)


def test_lse_tangent_closed_forms():
    pred = tf_allowed(3, 4, 1)
    q, k, v, dq, dk, dv = _six(1, pred.n_q, 2, 8, seed=63)
    z = np.zeros_like(q)
    # only dV moves: the scores, hence LSE, do not
    *_, dL = masked_attention_jvp(q, k, v, z, z, dv, pred, lse_tangent=True)
    assert np.all(dL == 0)
    # q = 0: uniform weights, dLSE = mean over J of scale <dq, k_j>
    *_, dL = masked_attention_jvp(z, k, v, dq, z, dv, pred, lse_tangent=True)
    M = pred.matrix()
    sc = 1 / math.sqrt(8)
    for h in range(2):
        ds = sc * (dq[0, :, h] @ k[0, :, h].T)
        np.testing.assert_allclose(dL[0, h], (M * ds).sum(1) / M.sum(1), rtol=1e-12, atol=1e-14)
    # a row without keys has dLSE = 0
    pr = rects_allowed(4, 4, [(0, 2, 0, 4)])
    *_, dL = masked_attention_jvp(*_six(1, 4, 1, 4, seed=64), pr, lse_tangent=True)
    assert np.all(dL[0, 0, 2:] == 0) and np.all(dL[0, 0, :2] != 0)


def test_zero_queries_covariance_form():
    # q = 0: p uniform over J; ds_j = scale <dq, k_j>; dO = cov_J(ds, v) + mean_J dv
    pred = tf_allowed(3, 5, 1)
    _, k, v, dq, _, dv = _six(1, pred.n_q, 1, 8, seed=71)
    z = np.zeros_like(k)
    _, dO, _ = masked_attention_jvp(z, k, v, dq, z, dv, pred)
    M = pred.matrix()
    sc = 1 / math.sqrt(8)
    for i in range(pred.n_q):
        J = np.nonzero(M[i])[0]
        ds = sc * (k[0, J, 0] @ dq[0, i, 0])
        vv = v[0, J, 0]
        cov = (ds[:, None] * vv).mean(0) - ds.mean() * vv.mean(0)
        np.testing.assert_allclose(dO[0, i, 0], cov + dv[0, J, 0].mean(0), rtol=1e-11, atol=1e-13)


def test_tangent_is_linear():
    pred = tf_allowed(4, 3, 1)
    q, k, v, *t1 = _six(1, pred.n_q, 2, 8, seed=81)
    t2 = _six(1, pred.n_q, 2, 8, seed=91)[3:]
    d1 = masked_attention_jvp(q, k, v, *t1, pred)[1]
    d2 = masked_attention_jvp(q, k, v, *t2, pred)[1]
    d12 = masked_attention_jvp(q, k, v, *[a + b for a, b in zip(t1, t2)], pred)[1]
    d3 = masked_attention_jvp(q, k, v, *[-2.5 * a for a in t1], pred)[1]
    np.testing.assert_allclose(d12, d1 + d2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(d3, -2.5 * d1, rtol=1e-12, atol=1e-13)


def test_noisy_rows_independent_of_later_chunks():
    pred = tf_allowed(6, 3, 2)   # 3 chunks
    q, k, v, dq, dk, dv = _six(1, pred.n_q, 2, 8, seed=101)
    base = masked_attention_jvp(q, k, v, dq, dk, dv, pred)
    Nc, C = pred.n_clean, pred.unit_tokens
    # perturb K, V, dK, dV of every token in chunks >= 1 (clean and noisy) and of
    # noisy chunk 0's neighbours that chunk-0 noisy rows may not see
    later = [t for t in range(pred.n_k) if (t % Nc) // C >= 1]
    k2, v2, dk2, dv2 = (x.copy() for x in (k, v, dk, dv))
    for x in (k2, v2, dk2, dv2):
        x[:, later] += 3.0
    pert = masked_attention_jvp(q, k2, v2, dq, dk2, dv2, pred)
    rows0 = [t for t in range(pred.n_q) if (t % Nc) // C == 0]
    for a, b in zip(base, pert):
        if a.ndim == 4:
            np.testing.assert_array_equal(a[:, rows0], b[:, rows0])
        else:
            np.testing.assert_array_equal(a[:, :, rows0], b[:, :, rows0])


def test_rows_without_keys():
    pred = rects_allowed(4, 4, [(0, 2, 0, 4)])   # rows 2, 3 see nothing
    x = _six(1, 4, 1, 4, seed=111)
    O, dO, LSE = masked_attention_jvp(*x, pred)
    assert np.all(O[0, 2:] == 0) and np.all(dO[0, 2:] == 0)
    assert np.all(np.isneginf(LSE[0, 0, 2:])) and np.all(np.isfinite(LSE[0, 0, :2]))


def test_row_subset_matches_full():
    pred = tf_allowed(4, 5, 2)
    x = _six(2, pred.n_q, 2, 8, seed=121)
    full = masked_attention_jvp(*x, pred)
    rows = np.array([0, 3, 9, 10, 21, 39])
    sub = masked_attention_jvp(*x, pred, rows=rows, row_block=4)
    # row blocks change BLAS call shapes, so equality is up to fp64 rounding
    np.testing.assert_allclose(sub[0], full[0][:, rows], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(sub[1], full[1][:, rows], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(sub[2], full[2][:, :, rows], rtol=1e-13, atol=1e-14)
