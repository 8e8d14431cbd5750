"""GPU parity on seeded random query-group / key-range masks: random sizes
(ragged tiles), random groups and ranges (partial blocks, rows without keys,
keys nobody sees), both head dims and both dtypes.  Forward (unsplit and
split, with the LSE tangent) and backward, each against the fp64 oracle with
the tolerances of the other parity tests."""

import sys

import numpy as np
import pytest
import torch

import attention_jvp_causal_attn_amd as aj
from attention_jvp_causal_attn_amd.inputs import make_random
from oracle import masked_attention_grad, masked_attention_jvp, rects_allowed

pytestmark = pytest.mark.gpu
TOL = {"bf16": 2e-2, "f32": 1e-5}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def check(name, got, ref, tol):
    got = np.asarray(got, dtype=np.float64)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin), f"{name}: finite pattern differs"
    if not fin.any():
        return
    err = np.abs(got[fin] - ref[fin]).max()
    scale = np.abs(ref[fin]).max()
    rel = err / scale if scale > 0 else err
    say(f"  {name}: ratio {rel:.3e} (tol {tol})")
    assert rel <= tol, f"{name}: {rel:.3e} > {tol}"


def random_mask(rng, n_q, n_k):
    """Random partition of the rows into groups, each with up to 3 disjoint
    random key ranges (possibly none)."""
    n_groups = int(rng.integers(1, 7))
    cuts = np.sort(rng.choice(np.arange(1, n_q), size=min(n_groups - 1, n_q - 1), replace=False))
    gq = [0] + cuts.tolist() + [n_q]
    rp, kb, ke, rects = [0], [], [], []
    for g in range(len(gq) - 1):
        nr = int(rng.integers(0, 4))
        pts = np.sort(rng.choice(np.arange(0, n_k + 1), size=min(2 * nr, n_k + 1), replace=False))
        for i in range(0, len(pts) - 1, 2):
            kb.append(int(pts[i]))
            ke.append(int(pts[i + 1]))
            rects.append((gq[g], gq[g + 1], int(pts[i]), int(pts[i + 1])))
        rp.append(len(kb))
    return aj.attn_jvp_mask_rects(n_q, n_k, gq, rp, kb, ke), rects_allowed(n_q, n_k, rects)


CASES = [(seed, dtype, D) for seed in range(6) for dtype, D in
         [("bf16", 128), ("bf16", 64), ("f32", 64)]]


@pytest.mark.parametrize("seed,dtype,D", CASES)
def test_random_mask_forward_split_and_backward(seed, dtype, D):
    rng = np.random.default_rng(4000 + seed)
    n_q, n_k, H = int(rng.integers(1, 700)), int(rng.integers(1, 900)), int(rng.integers(1, 3))
    say(f"case: random mask seed={seed} {dtype} D={D} n_q={n_q} n_k={n_k} H={H}")
    mask, pred = random_mask(rng, n_q, n_k)
    xq = make_random(1, n_q, H, D, dtype=dtype, seed=5000 + seed, tangent_std=0.1)
    xk = make_random(1, n_k, H, D, dtype=dtype, seed=6000 + seed, tangent_std=0.1)
    x = dict(q=xq["q"], dq=xq["dq"], k=xk["k"], v=xk["v"], dk=xk["dk"], dv=xk["dv"])
    xd = {k: v.cuda() for k, v in x.items()}
    tol = TOL[dtype]
    O, dO, LSE, dL = masked_attention_jvp(x["q"], x["k"], x["v"], x["dq"], x["dk"], x["dv"],
                                          pred, lse_tangent=True)
    for S in (1, 3):
        o, do, lse, dlse = aj.attn_jvp_fwd(xd["q"], xd["k"], xd["v"], xd["dq"], xd["dk"],
                                           xd["dv"], mask, lse_tangent=True, max_splits=S)
        torch.cuda.synchronize()
        check(f"O (S={S})", f64(o), O, tol)
        check(f"dO (S={S})", f64(do), dO, tol)
        check(f"LSE (S={S})", f64(lse), LSE, tol)
        check(f"dLSE (S={S})", f64(dlse), dL, tol)
    g = make_random(1, n_q, H, D, dtype=dtype, seed=7000 + seed)["q"]
    o, _, lse = aj.attn_jvp_fwd(xd["q"], xd["k"], xd["v"], None, None, None, mask)
    gq, gk, gv, delta = aj.attn_jvp_bwd(xd["q"], xd["k"], xd["v"], o, g.cuda(), lse, mask)
    torch.cuda.synchronize()
    dQ, dK, dV, Ds = masked_attention_grad(x["q"], x["k"], x["v"], g, pred)
    check("dQ", f64(gq), dQ, tol)
    check("dK", f64(gk), dK, tol)
    check("dV", f64(gv), dV, tol)
    check("D", f64(delta), Ds, tol)
