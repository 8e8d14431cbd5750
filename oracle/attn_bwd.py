"""Plain fp64 gradients of masked attention (the backward of the primal).

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed: the gradients of L = sum_i <g_i, O_i> with respect to Q, K
and V, for the same masked operator whose forward the oracle module
``attn_jvp`` defines ("Causal-rCM ..." Appendix B returns the row log-sum-exp
so that a backward of the masked forward can reuse it; the student is trained
through that TF-masked packed forward, Section 3).  The pages give no backward
formulas; the plain definition is the chain rule through the two-pass softmax,
written out per (batch, head) slice with J_i the admissible keys of row i and
I_j the rows that admit key j:

    P_ij  = exp(s_ij - LSE_i),   s_ij = scale * <q_i, k_j>       (j in J_i)
    dV_j  = sum_{i in I_j} P_ij g_i
    dP_ij = <g_i, v_j>
    D_i   = sum_{j in J_i} P_ij dP_ij
    dS_ij = P_ij (dP_ij - D_i)
    dQ_i  = scale * sum_{j in J_i} dS_ij k_j
    dK_j  = scale * sum_{i in I_j} dS_ij q_i

(D_i equals <g_i, O_i>.)  Masked pairs contribute nothing (no term at all).
A row with no admissible key has no gradient; a key that no row admits gets
zero dK and dV.
"""

import numpy as np

from .attn_jvp import _f64, _prep


def masked_attention_grad(q, k, v, g, allowed, scale=None, rows=None, keys=None,
                          row_block=512):
    """Gradients of sum(g * O) for the masked attention O(q, k, v).

    q, k, v : array-like [B, N, H, D] (numpy or torch, any float dtype)
    g       : array-like [B, N, H, D], the gradient flowing into O
    allowed : predicate object, ``allowed(rows) -> bool [len(rows), N]``
    rows    : query rows whose dQ is returned (default: all)
    keys    : key rows whose dK, dV are returned (default: all)
    returns (dQ [B, R, H, D], dK [B, K, H, D], dV [B, K, H, D], Dsum [B, H, R])
    with Dsum the row sums D_i of the rows returned.

    Every row's P and D_i are built from all of its admissible keys (first
    pass over all rows); the second pass sums over all rows that admit each
    requested key.
    """
    B, N, H, D = q.shape
    n_k = k.shape[1]
    scale, rows = _prep(q, scale, rows, N)
    keys = np.arange(n_k) if keys is None else np.asarray(keys, dtype=np.int64)
    all_rows = np.arange(N)
    blocks = []
    for r0 in range(0, N, row_block):
        rb = all_rows[r0:r0 + row_block]
        A = np.asarray(allowed(rb), dtype=bool)           # [r, n_k]
        blocks.append((rb, A))
    want = np.zeros(N, dtype=bool)
    want[rows] = True
    pos = np.full(N, -1, dtype=np.int64)
    pos[rows] = np.arange(len(rows))
    dQ = np.zeros((B, len(rows), H, D))
    dK = np.zeros((B, len(keys), H, D))
    dV = np.zeros((B, len(keys), H, D))
    Dsum = np.zeros((B, H, len(rows)))
    for b in range(B):
        for h in range(H):
            qs, ks, vs, gs = (_f64(x[b, :, h, :]) for x in (q, k, v, g))
            lse = np.full(N, -np.inf)
            dsum = np.zeros(N)
            # pass 1: every row's LSE and D_i; dQ of the requested rows
            for rb, A in blocks:
                live = A.any(axis=1)
                if not live.any():
                    continue
                s = np.where(A, scale * (qs[rb] @ ks.T), -np.inf)
                m = s.max(axis=1, keepdims=True)
                m = np.where(np.isfinite(m), m, 0.0)
                e = np.where(A, np.exp(s - m), 0.0)
                l = e.sum(axis=1, keepdims=True)
                p = np.where(A, e / np.where(l > 0, l, 1.0), 0.0)
                dp = np.where(A, gs[rb] @ vs.T, 0.0)
                d_i = (p * dp).sum(axis=1)
                lse[rb] = np.where(live, m[:, 0] + np.log(np.where(live, l[:, 0], 1.0)), -np.inf)
                dsum[rb] = d_i
                sel = want[rb]
                if sel.any():
                    ds = np.where(A, p * (dp - d_i[:, None]), 0.0)
                    dQ[b, pos[rb[sel]], h, :] = scale * (ds[sel] @ ks)
            Dsum[b, h, :] = dsum[rows]
            # pass 2: dK, dV of the requested keys, summed over the rows that admit them
            kk, vk = ks[keys], vs[keys]
            for rb, A in blocks:
                Ak = A[:, keys]
                if not Ak.any():
                    continue
                live = np.isfinite(lse[rb])
                s = np.where(Ak, scale * (qs[rb] @ kk.T), -np.inf)
                p = np.where(Ak & live[:, None],
                             np.exp(s - np.where(live, lse[rb], 0.0)[:, None]), 0.0)
                dp = np.where(Ak, gs[rb] @ vk.T, 0.0)
                ds = np.where(Ak, p * (dp - dsum[rb][:, None]), 0.0)
                dV[b, :, h, :] += p.T @ gs[rb]
                dK[b, :, h, :] += scale * (ds.T @ qs[rb])
    return dQ, dK, dV, Dsum
