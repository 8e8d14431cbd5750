"""Pins of the CPU oracle's backward (gradients of the masked primal).

Each check ties ``oracle.masked_attention_grad`` to something other than
itself: PyTorch's reverse-mode autograd of its own scaled-dot-product
attention, central finite differences of the oracle's forward (a separately
pinned function), closed forms, and subset / mask invariants.  A dropped D_i
term, a missing scale, a transposed product or a wrong mask orientation fails
at least one of them.
"""

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from torch.nn.attention import SDPBackend, sdpa_kernel

from oracle import (dense_allowed, masked_attention, masked_attention_grad, rects_allowed,
                    tf_allowed)


def _rand(shape, seed, std=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * std


MASKS = {
    "tf_frame": lambda: tf_allowed(3, 4, 1),
    "tf_chunk": lambda: tf_allowed(4, 3, 2),
    "dense": lambda: dense_allowed(16, 16),
    "rects": lambda: rects_allowed(20, 20, [(0, 7, 2, 9), (5, 20, 0, 3), (12, 20, 15, 20)]),
}


@pytest.mark.parametrize("mname", list(MASKS))
def test_grad_matches_torch_autograd(mname):
    pred = MASKS[mname]()
    N = pred.n_q
    q, k, v, g = (_rand((2, N, 3, 8), 51 + i) for i in range(4))
    scale = 0.41
    M = torch.from_numpy(pred.matrix())
    t = lambda x: torch.from_numpy(x).permute(0, 2, 1, 3).clone().requires_grad_(True)
    tq, tk, tv = t(q), t(k), t(v)
    with sdpa_kernel(SDPBackend.MATH):
        o = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=M, scale=scale)
    (o * torch.from_numpy(g).permute(0, 2, 1, 3)).sum().backward()
    dQ, dK, dV, Dsum = masked_attention_grad(q, k, v, g, pred, scale=scale)
    back = lambda x: x.grad.permute(0, 2, 1, 3).numpy()
    np.testing.assert_allclose(dQ, back(tq), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dK, back(tk), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dV, back(tv), rtol=1e-11, atol=1e-12)
    # D_i = <g_i, O_i> with O from the (separately pinned) forward oracle
    O, _ = masked_attention(q, k, v, pred, scale=scale)
    np.testing.assert_allclose(Dsum, np.einsum("bnhd,bnhd->bhn", g, O), rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("mname,D", [("tf_frame", 4), ("tf_chunk", 16), ("rects", 8)])
def test_grad_central_finite_difference(mname, D):
    pred = MASKS[mname]()
    N = pred.n_q
    q, k, v, g = (_rand((1, N, 2, D), 61 + i) for i in range(4))
    dQ, dK, dV, _ = masked_attention_grad(q, k, v, g, pred)
    eps = 1e-6
    rng = np.random.default_rng(7)
    for which, grad in ((0, dQ), (1, dK), (2, dV)):
        # directional derivative along a random direction of one input
        u = rng.standard_normal(q.shape)
        xs_p, xs_m = [q, k, v], [q, k, v]
        xs_p = [x + eps * u if i == which else x for i, x in enumerate(xs_p)]
        xs_m = [x - eps * u if i == which else x for i, x in enumerate(xs_m)]
        Op, _ = masked_attention(*xs_p, pred)
        Om, _ = masked_attention(*xs_m, pred)
        fd = ((Op - Om) * g).sum() / (2 * eps)
        an = (grad * u).sum()
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (which, fd, an)


def test_single_visible_key_gradients():
    # every row sees exactly one key: p = 1, dS = 0, so dQ = dK = 0 and dV_j = sum of g
    N = 6
    rects = [(i, i + 1, (2 * i) % N, (2 * i) % N + 1) for i in range(N)]
    pred = rects_allowed(N, N, rects)
    q, k, v, g = (_rand((1, N, 2, 4), 71 + i) for i in range(4))
    dQ, dK, dV, _ = masked_attention_grad(q, k, v, g, pred)
    assert np.abs(dQ).max() < 1e-14 and np.abs(dK).max() < 1e-14
    want = np.zeros_like(v)
    for i in range(N):
        want[:, (2 * i) % N] += g[:, i]
    np.testing.assert_allclose(dV, want, rtol=0, atol=1e-14)


def test_unseen_keys_get_zero_gradient():
    # keys 12..19 are seen by no row
    pred = rects_allowed(10, 20, [(0, 10, 0, 12)])
    q, g = _rand((1, 10, 2, 8), 81), _rand((1, 10, 2, 8), 82)
    k, v = _rand((1, 20, 2, 8), 83), _rand((1, 20, 2, 8), 84)
    _, dK, dV, _ = masked_attention_grad(q, k, v, g, pred)
    assert np.abs(dK[:, 12:]).max() == 0 and np.abs(dV[:, 12:]).max() == 0
    assert np.abs(dK[:, :12]).max() > 0 and np.abs(dV[:, :12]).max() > 0


def test_zero_queries_uniform_weights():
    # q = 0: every admissible key of a row has weight 1/|J_i|, so dV_j = sum over
    # the rows admitting j of g_i / |J_i|, and dK = 0 (dS_ij = P (dP - D) sums
    # against q = 0)
    pred = tf_allowed(3, 4, 1)
    N = pred.n_q
    k, v, g = (_rand((1, N, 1, 8), 91 + i) for i in range(3))
    q = np.zeros_like(k)
    _, dK, dV, _ = masked_attention_grad(q, k, v, g, pred)
    M = pred.matrix().astype(np.float64)
    W = M / M.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(dV[0, :, 0], W.T @ g[0, :, 0], rtol=1e-13, atol=1e-14)
    assert np.abs(dK).max() < 1e-14


def test_subsets_match_full():
    pred = tf_allowed(4, 5, 2)
    N = pred.n_q
    q, k, v, g = (_rand((1, N, 2, 8), 101 + i) for i in range(4))
    dQ, dK, dV, Ds = masked_attention_grad(q, k, v, g, pred, row_block=7)
    rows = np.array([0, 3, 17, 39])
    keys = np.array([1, 5, 22, 38])
    dQs, dKs, dVs, Dss = masked_attention_grad(q, k, v, g, pred, rows=rows, keys=keys)
    np.testing.assert_allclose(dQs, dQ[:, rows], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(dKs, dK[:, keys], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(dVs, dV[:, keys], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(Dss, Ds[:, :, rows], rtol=1e-13, atol=1e-14)
