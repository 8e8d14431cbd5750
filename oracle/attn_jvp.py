"""Plain fp64 masked attention and its forward-mode JVP (tangent).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Definition followed ("Causal-rCM ..." Appendix B, "FlashAttention-2 JVP Kernel
with Custom Masks"): the JVP must be the derivative of exactly the primal
masked attention operator; masked-out pairs contribute no tangent because the
discrete mask has no tangent; the outputs are the primal output O, the row
log-sum-exp and the tangent output dO.  The online-softmax pass of the kernel
reaches this same result up to rounding, so the oracle is the plain definition
written out (two-pass softmax, no tiling, no online rescaling):

For one (batch b, head h) slice and query row i, with J_i the admissible keys,

    s_j   = scale * <q_i, k_j>                              (j in J_i)
    m     = max_j s_j,   e_j = exp(s_j - m),   l = sum_j e_j,   p_j = e_j / l
    O_i   = sum_j p_j v_j
    LSE_i = m + ln l
    ds_j  = scale * (<dq_i, k_j> + <q_i, dk_j>)             (j in J_i)
    mu_i  = sum_j p_j ds_j
    dO_i  = sum_j p_j (ds_j - mu_i) v_j + sum_j p_j dv_j

The last line is the product rule applied to O_i = sum_j p_j v_j with
dp_j = p_j (ds_j - mu_i), the derivative of the normalised softmax.  The
tangent of the row log-sum-exp (returned on request: the appendix lists LSE
among the outputs, and its derivative is the softmax-weighted mean of the
score tangents) is

    dLSE_i = mu_i = sum_j p_j ds_j
``scale`` defaults to 1/sqrt(D) and carries no tangent (the pages are silent
on the scale; the usual attention default is taken).  A row with no admissible
key gets O = 0, dO = 0 and LSE = -inf (the pages are silent; TF masks never
produce such rows).

Rows are evaluated in blocks only to bound memory; every row's sums run over
its own admissible keys exactly as written above (entries outside J_i are
excluded by ``np.where`` before any sum, never multiplied by a weight).
"""

import numpy as np


def _f64(x):
    """Exact fp64 copy of an array-like (bf16 and fp32 widen exactly)."""
    if hasattr(x, "detach"):  # a torch tensor: widen through fp32 on the CPU
        x = x.detach().to("cpu").float().numpy()
    return np.asarray(x, dtype=np.float64)


def _prep(q, scale, rows, n):
    d = int(q.shape[-1])
    if scale is None or scale <= 0:
        scale = 1.0 / np.sqrt(d)
    if rows is None:
        rows = np.arange(n)
    rows = np.asarray(rows, dtype=np.int64)
    return float(scale), rows


def masked_attention_jvp(q, k, v, dq, dk, dv, allowed, scale=None, rows=None,
                         row_block=512, lse_tangent=False):
    """Masked attention and its tangent.

    q, k, v, dq, dk, dv : array-like [B, N, H, D] (numpy or torch, any float
                          dtype); one (b, h) slice at a time is widened to fp64
    allowed : predicate object, ``allowed(rows) -> bool [len(rows), N]``
    rows    : query rows to evaluate (default: all N)
    returns (O, dO, LSE) as fp64: O, dO [B, R, H, D], LSE [B, H, R]; with
    ``lse_tangent`` also dLSE [B, H, R] (0 for rows without keys)
    """
    B, N, H, D = q.shape
    scale, rows = _prep(q, scale, rows, N)
    R = len(rows)
    O = np.zeros((B, R, H, D))
    dO = np.zeros((B, R, H, D))
    LSE = np.full((B, H, R), -np.inf)
    dLSE = np.zeros((B, H, R))
    blocks = []
    for r0 in range(0, R, row_block):
        rb = rows[r0:r0 + row_block]
        A = np.asarray(allowed(rb), dtype=bool)          # [r, N]
        cols = np.nonzero(A.any(axis=0))[0]
        if cols.size:
            blocks.append((r0, rb, cols, A[:, cols]))
    for b in range(B):
        for h in range(H):
            qs, ks, vs = _f64(q[b, :, h, :]), _f64(k[b, :, h, :]), _f64(v[b, :, h, :])
            dqs, dks, dvs = _f64(dq[b, :, h, :]), _f64(dk[b, :, h, :]), _f64(dv[b, :, h, :])
            for r0, rb, cols, A in blocks:
                live = A.any(axis=1)
                qi, dqi = qs[rb], dqs[rb]
                kj, vj, dkj, dvj = ks[cols], vs[cols], dks[cols], dvs[cols]
                s = np.where(A, scale * (qi @ kj.T), -np.inf)
                m = s.max(axis=1, keepdims=True)
                m = np.where(np.isfinite(m), m, 0.0)
                e = np.where(A, np.exp(s - m), 0.0)
                l = e.sum(axis=1, keepdims=True)
                p = np.where(live[:, None], e / np.where(l > 0, l, 1.0), 0.0)
                ds = np.where(A, scale * (dqi @ kj.T + qi @ dkj.T), 0.0)
                mu = (p * ds).sum(axis=1, keepdims=True)
                dp = np.where(A, p * (ds - mu), 0.0)
                O[b, r0:r0 + len(rb), h, :] = p @ vj
                dO[b, r0:r0 + len(rb), h, :] = dp @ vj + p @ dvj
                lse = np.where(live, m[:, 0] + np.log(np.where(live, l[:, 0], 1.0)), -np.inf)
                LSE[b, h, r0:r0 + len(rb)] = lse
                dLSE[b, h, r0:r0 + len(rb)] = mu[:, 0]
    if lse_tangent:
        return O, dO, LSE, dLSE
    return O, dO, LSE


def masked_attention(q, k, v, allowed, scale=None, rows=None, row_block=512):
    """Primal only: (O, LSE) of the same masked operator (the first four
    lines of the definition in the module docstring)."""
    B, N, H, D = q.shape
    scale, rows = _prep(q, scale, rows, N)
    R = len(rows)
    O = np.zeros((B, R, H, D))
    LSE = np.full((B, H, R), -np.inf)
    blocks = []
    for r0 in range(0, R, row_block):
        rb = rows[r0:r0 + row_block]
        A = np.asarray(allowed(rb), dtype=bool)
        cols = np.nonzero(A.any(axis=0))[0]
        if cols.size:
            blocks.append((r0, rb, cols, A[:, cols]))
    for b in range(B):
        for h in range(H):
            qs, ks, vs = _f64(q[b, :, h, :]), _f64(k[b, :, h, :]), _f64(v[b, :, h, :])
            for r0, rb, cols, A in blocks:
                live = A.any(axis=1)
                s = np.where(A, scale * (qs[rb] @ ks[cols].T), -np.inf)
                m = s.max(axis=1, keepdims=True)
                m = np.where(np.isfinite(m), m, 0.0)
                e = np.where(A, np.exp(s - m), 0.0)
                l = e.sum(axis=1, keepdims=True)
                p = np.where(live[:, None], e / np.where(l > 0, l, 1.0), 0.0)
                O[b, r0:r0 + len(rb), h, :] = p @ vs[cols]
                LSE[b, h, r0:r0 + len(rb)] = np.where(
                    live, m[:, 0] + np.log(np.where(live, l[:, 0], 1.0)), -np.inf)
    return O, LSE
