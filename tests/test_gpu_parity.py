"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

Tolerances (per output tensor O, dO, LSE): max|gpu - ref| <= tol * max|ref|,
tol = 2e-2 for bf16 inputs and 1e-5 for fp32 inputs; every output finite
where the reference is.  Inputs are seeded; the oracle sees the exact values
the GPU sees (bf16 and fp32 widen to fp64 exactly).
"""

import math
import os
import sys
import types

import numpy as np
import pytest
import torch

import attention_jvp_causal_attn_amd as aj
from attention_jvp_causal_attn_amd.inputs import WORKLOADS, make_inputs, make_random
from oracle import (block_causal_allowed, dense_allowed, masked_attention,
                    masked_attention_jvp, rects_allowed, tf_allowed)

pytestmark = pytest.mark.gpu

TOL = {torch.bfloat16: 2e-2, torch.float32: 1e-5}
DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(x):
    return {k: v.to(DEV) for k, v in x.items()}


def run(xd, mask, tangent=True, scale=None):
    if tangent:
        o, do, lse = aj.attn_jvp_fwd(xd["q"], xd["k"], xd["v"], xd["dq"], xd["dk"], xd["dv"],
                                     mask, scale=scale)
    else:
        o, do, lse = aj.attn_jvp_fwd(xd["q"], xd["k"], xd["v"], None, None, None, mask,
                                     scale=scale)
    torch.cuda.synchronize()
    return o, do, lse


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def check(name, got, ref, tol):
    got = np.asarray(got, dtype=np.float64)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin), f"{name}: finite pattern differs"
    if not fin.any():
        return 0.0
    err = np.abs(got[fin] - ref[fin]).max()
    scale = np.abs(ref[fin]).max()
    rel = err / scale if scale > 0 else err
    say(f"  {name}: max|err| = {err:.3e}, max|ref| = {scale:.3e}, ratio = {rel:.3e} (tol {tol})")
    assert rel <= tol, f"{name}: {rel:.3e} > {tol}"
    return rel


def parity(x, pred, mask, tol, rows=None, scale=None):
    xd = to_dev(x)
    o, do, lse = run(xd, mask, scale=scale)
    O, dO, LSE = masked_attention_jvp(x["q"], x["k"], x["v"], x["dq"], x["dk"], x["dv"], pred,
                                      scale=scale, rows=rows)
    sel = slice(None) if rows is None else torch.as_tensor(rows)
    check("O", f64(o[:, sel]), O, tol)
    check("dO", f64(do[:, sel]), dO, tol)
    check("LSE", f64(lse[:, :, sel]), LSE, tol)
    return o, do, lse


# ------------------------------------------------------------ fp32 path ----

def test_tiny_tf_fp32_workload():
    w = WORKLOADS[1]
    say(f"case: {w.describe()}")
    x = make_inputs(w)
    parity(x, tf_allowed(w.n_frames, w.tokens_per_frame, w.frames_per_chunk),
           aj.attn_jvp_mask_tf(w.n_frames, w.tokens_per_frame, w.frames_per_chunk),
           TOL[torch.float32])


@pytest.mark.parametrize("nf,tpf,fpc,B,H,D", [(5, 37, 1, 2, 3, 128), (3, 21, 3, 1, 2, 64),
                                              (2, 1, 1, 1, 1, 64)])
def test_small_tf_fp32(nf, tpf, fpc, B, H, D):
    say(f"case: fp32 TF nf={nf} tpf={tpf} fpc={fpc} B={B} H={H} D={D}")
    pred = tf_allowed(nf, tpf, fpc)
    x = make_random(B, pred.n_q, H, D, dtype="f32", seed=7000 + nf * 10 + D)
    parity(x, pred, aj.attn_jvp_mask_tf(nf, tpf, fpc), TOL[torch.float32])


# ------------------------------------------------------------ bf16 path ----

SMALL_BF16 = [
    (5, 37, 1, 2, 3, 128),   # N=370: 3 query tiles, ragged tail, unaligned units
    (6, 23, 2, 1, 2, 64),    # chunk-wise, D=64
    (4, 64, 1, 1, 2, 128),   # tile-aligned units
    (3, 100, 3, 2, 1, 128),  # one chunk of 300 tokens per stream
    (2, 1, 1, 1, 1, 128),    # N=4: rows with a single admissible key
    (7, 50, 1, 1, 2, 64),
    (9, 33, 3, 1, 1, 128),
]


@pytest.mark.parametrize("nf,tpf,fpc,B,H,D", SMALL_BF16)
def test_small_tf_bf16(nf, tpf, fpc, B, H, D):
    say(f"case: bf16 TF nf={nf} tpf={tpf} fpc={fpc} B={B} H={H} D={D}")
    pred = tf_allowed(nf, tpf, fpc)
    x = make_random(B, pred.n_q, H, D, dtype="bf16", seed=8000 + nf * 10 + D, tangent_std=0.1)
    parity(x, pred, aj.attn_jvp_mask_tf(nf, tpf, fpc), TOL[torch.bfloat16])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_dense_and_rect_masks(dtype):
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    say(f"case: dense mask 200x200 {dtype}")
    x = make_random(1, 200, 2, 128, dtype=dtype, seed=9100, tangent_std=0.2)
    parity(x, dense_allowed(200, 200), aj.attn_jvp_mask_dense(200, 200), TOL[td], scale=0.05)
    # generic rectangles, including rows with no admissible key at all
    say(f"case: rect mask 150x150 {dtype}")
    gq = [0, 10, 70, 100, 150]
    rp = [0, 2, 3, 3, 5]
    kb = [5, 40, 0, 0, 120]
    ke = [20, 41, 150, 64, 150]
    rects = [(gq[g], gq[g + 1], kb[r], ke[r]) for g in range(4) for r in range(rp[g], rp[g + 1])]
    x = make_random(2, 150, 1, 64, dtype=dtype, seed=9200, tangent_std=0.1)
    o, do, lse = parity(x, rects_allowed(150, 150, rects),
                        aj.attn_jvp_mask_rects(150, 150, gq, rp, kb, ke), TOL[td])
    assert torch.all(o[:, 70:100] == 0) and torch.all(do[:, 70:100] == 0)
    assert torch.all(torch.isneginf(lse[:, :, 70:100]))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_queries_differ_from_keys(dtype):
    # n_q != n_k: a chunk of 80 queries attending to 300 cached + own keys
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    n_q, n_k, H, D = 80, 380, 2, 128
    say(f"case: rect n_q={n_q} n_k={n_k} {dtype}")
    xq = make_random(1, n_q, H, D, dtype=dtype, seed=9300, tangent_std=0.1)
    xk = make_random(1, n_k, H, D, dtype=dtype, seed=9400, tangent_std=0.1)
    x = dict(q=xq["q"], dq=xq["dq"], k=xk["k"], v=xk["v"], dk=xk["dk"], dv=xk["dv"])
    gq, rp, kb, ke = [0, 40, 80], [0, 1, 2], [0, 0], [340, 380]
    pred = rects_allowed(n_q, n_k, [(0, 40, 0, 340), (40, 80, 0, 380)])
    parity(x, pred, aj.attn_jvp_mask_rects(n_q, n_k, gq, rp, kb, ke), TOL[td])


# ------------------------------------------------- invariants and modes ----

def _tf_case(dtype="bf16", nf=6, tpf=29, fpc=2, B=1, H=2, D=128, seed=9500):
    pred = tf_allowed(nf, tpf, fpc)
    x = make_random(B, pred.n_q, H, D, dtype=dtype, seed=seed, tangent_std=0.1)
    return pred, aj.attn_jvp_mask_tf(nf, tpf, fpc), x


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_primal_only_matches_jvp_primal(dtype):
    pred, mask, x = _tf_case(dtype)
    xd = to_dev(x)
    o1, _, l1 = run(xd, mask, tangent=True)
    o2, d2, l2 = run(xd, mask, tangent=False)
    assert d2 is None
    same = torch.equal(o1, o2) and torch.equal(l1, l2)
    say(f"  primal-only O/LSE bitwise equal to the JVP run: {same}")
    td = xd["q"].dtype
    O, LSE = masked_attention(x["q"], x["k"], x["v"], pred)
    check("O(primal)", f64(o2), O, TOL[td])
    check("LSE(primal)", f64(l2), LSE, TOL[td])
    check("O(primal vs jvp)", f64(o2), f64(o1), TOL[td])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_deterministic(dtype):
    _, mask, x = _tf_case(dtype, seed=9600)
    xd = to_dev(x)
    a = run(xd, mask)
    b = run(xd, mask)
    for u, v in zip(a, b):
        assert torch.equal(u, v)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rows_blind_to_inadmissible_keys(dtype):
    # Rows of chunk 0 (clean and noisy) must be bitwise unchanged when K, V, dK,
    # dV of every later-chunk token change (a noisy token's output does not
    # depend on later chunks).
    pred, mask, x = _tf_case(dtype, nf=6, tpf=29, fpc=2, seed=9700)
    xd = to_dev(x)
    base = run(xd, mask)
    Nc, C = pred.n_clean, pred.unit_tokens
    later = torch.tensor([t for t in range(pred.n_k) if (t % Nc) // C >= 1])
    y = {k: v.clone() for k, v in xd.items()}
    for n in ("k", "v", "dk", "dv"):
        y[n][:, later.to(DEV)] = (y[n][:, later.to(DEV)] * -3.0 + 1.5).to(y[n].dtype)
    pert = run(y, mask)
    rows0 = torch.tensor([t for t in range(pred.n_q) if (t % Nc) // C == 0], device=DEV)
    assert torch.equal(base[0][:, rows0], pert[0][:, rows0])
    assert torch.equal(base[1][:, rows0], pert[1][:, rows0])
    assert torch.equal(base[2][:, :, rows0], pert[2][:, :, rows0])
    # and the rows that can see them did change
    assert not torch.equal(base[0], pert[0])


def test_head_and_batch_permutation_is_bitwise():
    pred, mask, x = _tf_case("bf16", B=2, H=3, seed=9800)
    xd = to_dev(x)
    a = run(xd, mask)
    perm_h = torch.tensor([2, 0, 1], device=DEV)
    y = {k: v[:, :, perm_h].flip(0).contiguous() for k, v in xd.items()}
    b = run(y, mask)
    assert torch.equal(a[0][:, :, perm_h].flip(0), b[0])
    assert torch.equal(a[1][:, :, perm_h].flip(0), b[1])
    assert torch.equal(a[2][:, perm_h].flip(0), b[2])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_tangent_linearity(dtype):
    # Doubling every tangent doubles every value the tangent path forms (the
    # products, exponent sums, the bf16 roundings of P*dS, mu and T), exactly,
    # in binary floating point away from overflow and subnormals: dO and the
    # LSE tangent double bit for bit and O, LSE do not change.
    _, mask, x = _tf_case(dtype, seed=9900)
    xd = to_dev(x)
    o1, d1, l1, g1 = aj.attn_jvp_fwd(xd["q"], xd["k"], xd["v"], xd["dq"], xd["dk"], xd["dv"],
                                     mask, lse_tangent=True)
    y = {n: xd[n] * 2 for n in ("dq", "dk", "dv")}
    assert all(torch.equal(y[n] / 2, xd[n]) for n in y)      # exact scaling of the inputs
    o2, d2, l2, g2 = aj.attn_jvp_fwd(xd["q"], xd["k"], xd["v"], y["dq"], y["dk"], y["dv"], mask,
                                     lse_tangent=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(d2, d1 * 2), "dO(2t) differs from 2 dO(t)"
    assert torch.equal(g2, g1 * 2), "dLSE(2t) differs from 2 dLSE(t)"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_single_visible_key(dtype):
    N, H, D = 100, 2, 128
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    mask = aj.attn_jvp_mask_rects(N, N, list(range(N + 1)), list(range(N + 1)),
                                  list(range(N)), list(range(1, N + 1)))
    x = make_random(1, N, H, D, dtype=dtype, seed=9950, tangent_std=0.1)
    xd = to_dev(x)
    o, do, lse = run(xd, mask, scale=0.125)
    assert torch.equal(o, xd["v"])                           # p = 1 exactly
    check("dO=dv", f64(do), f64(xd["dv"]), TOL[td])
    ref = 0.125 * (f64(xd["q"]) * f64(xd["k"])).sum(-1).transpose(0, 2, 1)
    check("LSE=s_jj", f64(lse), ref, TOL[td])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_zero_queries_uniform_weights(dtype):
    pred, mask, x = _tf_case(dtype, seed=9960)
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    x["q"] = torch.zeros_like(x["q"])
    x["dq"] = torch.zeros_like(x["dq"])
    xd = to_dev(x)
    o, do, lse = run(xd, mask)
    M = pred.matrix()
    cnt = M.sum(1)
    for h in range(x["q"].shape[2]):
        check(f"O=mean v (h{h})", f64(o)[0, :, h], (M @ f64(x["v"])[0, :, h]) / cnt[:, None], TOL[td])
        check(f"dO=mean dv (h{h})", f64(do)[0, :, h], (M @ f64(x["dv"])[0, :, h]) / cnt[:, None],
              TOL[td])
        check(f"LSE=ln|J| (h{h})", f64(lse)[0, h], np.log(cnt), TOL[td])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_outputs_fully_written_and_in_bounds(dtype):
    # NaN-poisoned outputs inside guard bands: every output element is written,
    # nothing past the ends is touched.
    pred, mask, x = _tf_case(dtype, nf=5, tpf=37, fpc=1, B=1, H=3, seed=9970)
    xd = to_dev(x)
    B, N, H, D = xd["q"].shape
    td = xd["q"].dtype
    G = 4096
    ob = torch.full((B * N * H * D + 2 * G,), float("nan"), dtype=td, device=DEV)
    db = torch.full_like(ob, float("nan"))
    lb = torch.full((B * H * N + 2 * G,), float("nan"), dtype=torch.float32, device=DEV)
    o = ob[G:G + B * N * H * D].view(B, N, H, D)
    do = db[G:G + B * N * H * D].view(B, N, H, D)
    lse = lb[G:G + B * H * N].view(B, H, N)
    aj.attn_jvp_fwd(xd["q"], xd["k"], xd["v"], xd["dq"], xd["dk"], xd["dv"], mask, o=o, d_o=do,
                    lse=lse)
    torch.cuda.synchronize()
    for buf in (ob, db, lb):
        assert torch.isnan(buf[:G]).all() and torch.isnan(buf[-G:]).all()
        assert torch.isfinite(buf[G:-G]).all()


# (B, H, n): the B*H slices and n / 256 query tiles (both bf16 head dims use
# 256-row tiles) select each branch of the workgroup -> work map: XCD groups
# of 8, 4, 2 and 1 slices' worth, and the identity map when the tiles do not
# split evenly over a group.
WORK_MAP_CASES = [
    (1, 3, 2048),  # 3 slices, 8 tiles: one group of 8 XCDs, 1 tile slot in 8 each
    (1, 2, 1024),  # groups of 4 XCDs
    (2, 3, 512),   # 6 slices: groups of 4 XCDs, 2 tiles -> identity map
    (1, 4, 600),   # groups of 2 XCDs, 3 tiles -> identity map
    (2, 5, 1024),  # 10 slices: groups of 4 XCDs, 5 slices per group
    (1, 2, 2048),  # groups of 4 XCDs, 2 tile slots each
    (4, 2, 400),   # 8 slices: one slice group per XCD
    (1, 12, 512),  # 12 slices, 2 tiles: groups of 2 XCDs (the 65,520-token workloads' map)
    (1, 4, 512),   # 4 slices, 2 tiles: groups of 2 XCDs, one slice per group
]


@pytest.mark.parametrize("B,H,n,D", [c + (d,) for d in (64, 128) for c in WORK_MAP_CASES])
def test_every_tile_of_every_slice_computed_once(B, H, n, D):
    say(f"case: dense bf16 B={B} H={H} n={n} D={D} (work map)")
    pred = dense_allowed(n, n)
    x = make_random(B, n, H, D, dtype="bf16", seed=9100 + 10 * B + H + D, tangent_std=0.1)
    xd = to_dev(x)
    o = torch.full_like(xd["q"], float("nan"))
    do = torch.full_like(xd["q"], float("nan"))
    lse = torch.full((B, H, n), float("nan"), dtype=torch.float32, device=DEV)
    aj.attn_jvp_fwd(xd["q"], xd["k"], xd["v"], xd["dq"], xd["dk"], xd["dv"],
                    aj.attn_jvp_mask_dense(n, n), o=o, d_o=do, lse=lse)
    torch.cuda.synchronize()
    O, dO, LSE = masked_attention_jvp(x["q"], x["k"], x["v"], x["dq"], x["dk"], x["dv"], pred)
    tol = TOL[torch.bfloat16]
    check("O", f64(o), O, tol)
    check("dO", f64(do), dO, tol)
    check("LSE", f64(lse), LSE, tol)


# Absent tangents are zero: a call with some of dq, dk, dv set to None equals,
# bit for bit, the call with explicit zero tensors, and matches the oracle.
TANGENT_SUBSETS = [("dq",), ("dk",), ("dv",), ("dk", "dv"), ("dq", "dk"), ("dq", "dv")]


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("f32", 64)])
@pytest.mark.parametrize("given", TANGENT_SUBSETS)
def test_absent_tangents_are_zero(dtype, D, given):
    say(f"case: {dtype} D={D} tangents given: {given}")
    pred = tf_allowed(5, 37, 1)
    x = make_random(1, pred.n_q, 2, D, dtype=dtype, seed=9300 + D + len(given), tangent_std=0.1)
    for name in ("dq", "dk", "dv"):
        if name not in given:
            x[name] = torch.zeros_like(x[name])
    xd = to_dev(x)
    mask = aj.attn_jvp_mask_tf(5, 37, 1)
    t = {name: (xd[name] if name in given else None) for name in ("dq", "dk", "dv")}
    o1, do1, lse1 = aj.attn_jvp_fwd(xd["q"], xd["k"], xd["v"], t["dq"], t["dk"], t["dv"], mask)
    o2, do2, lse2 = aj.attn_jvp_fwd(xd["q"], xd["k"], xd["v"], xd["dq"], xd["dk"], xd["dv"], mask)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(do1, do2) and torch.equal(lse1, lse2)
    O, dO, LSE = masked_attention_jvp(x["q"], x["k"], x["v"], x["dq"], x["dk"], x["dv"], pred)
    tol = TOL[torch.bfloat16 if dtype == "bf16" else torch.float32]
    check("O", f64(o1), O, tol)
    check("dO", f64(do1), dO, tol)
    check("LSE", f64(lse1), LSE, tol)


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("f32", 64)])
def test_block_causal_diffusion_forcing_mask(dtype, D):
    say(f"case: {dtype} D={D} block-causal 6 x 70")
    pred = block_causal_allowed(6, 70)
    x = make_random(1, pred.n_q, 2, D, dtype=dtype, seed=9400 + D, tangent_std=0.1)
    parity(x, pred, aj.attn_jvp_mask_block_causal(6, 70),
           TOL[torch.bfloat16 if dtype == "bf16" else torch.float32])


def test_strided_views_of_fused_buffers():
    # Q/dQ/O/dO and K/V/dK/dV as views of fused [B, N, 3, H, D]-style buffers
    pred = tf_allowed(4, 45, 1)
    B, N, H, D = 1, pred.n_q, 2, 128
    x = make_random(B, N, H, D, dtype="bf16", seed=9980, tangent_std=0.1)
    fused_k = torch.empty(B, N, 4, H, D, dtype=torch.bfloat16, device=DEV)
    fused_q = torch.empty(B, N, 4, H, D, dtype=torch.bfloat16, device=DEV)
    for i, n in enumerate(("k", "v", "dk", "dv")):
        fused_k[:, :, i] = x[n].to(DEV)
    fused_q[:, :, 0] = x["q"].to(DEV)
    fused_q[:, :, 1] = x["dq"].to(DEV)
    q, dq, o, do = (fused_q[:, :, i] for i in range(4))
    k, v, dk, dv = (fused_k[:, :, i] for i in range(4))
    mask = aj.attn_jvp_mask_tf(4, 45, 1)
    lse = torch.empty(B, H, N, dtype=torch.float32, device=DEV)
    aj.attn_jvp_fwd(q, k, v, dq, dk, dv, mask, o=o, d_o=do, lse=lse)
    torch.cuda.synchronize()
    O, dO, LSE = masked_attention_jvp(x["q"], x["k"], x["v"], x["dq"], x["dk"], x["dv"], pred)
    check("O", f64(o), O, 2e-2)
    check("dO", f64(do), dO, 2e-2)
    check("LSE", f64(lse), LSE, 2e-2)


# ------------------------------------------- full-size workloads, sampled ----

BF16_TILE = 256   # query rows per workgroup of both bf16 head dims


def sample_rows(w, n_random=48, seed=0):
    """The first and last row of every 256-row query tile, the first and last
    row of every unit of both streams, and random rows."""
    Nc, C = w.n_frames * w.tokens_per_frame, w.unit_tokens
    rows = set()
    for s in (0, Nc):
        for u in range(w.n_units):
            rows.update({s + u * C, s + u * C + C - 1})
    for t0 in range(0, w.N, BF16_TILE):
        rows.update({t0, min(w.N, t0 + BF16_TILE) - 1})
    rows.update({0, w.N - 1})
    rng = np.random.default_rng(seed)
    rows.update(rng.integers(0, w.N, size=n_random).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < w.N))


@pytest.mark.parametrize("wid", [2, 3, 4, 5])
def test_full_size_workload_every_tile(wid):
    # Every (b, h) slice of the full workload in the launch the benchmark
    # times, outputs NaN-filled beforehand: every element written and finite;
    # the first and last row of every query tile, every unit boundary and
    # random rows compared with the oracle element by element.
    w = WORKLOADS[wid]
    say(f"case: workload {wid}: {w.describe()}")
    x = make_inputs(w)
    xd = to_dev(x)
    mask = aj.attn_jvp_mask_tf(w.n_frames, w.tokens_per_frame, w.frames_per_chunk)
    pred = tf_allowed(w.n_frames, w.tokens_per_frame, w.frames_per_chunk)
    o = torch.full_like(xd["q"], float("nan"))
    do = torch.full_like(xd["q"], float("nan"))
    lse = torch.full((w.B, w.H, w.N), float("nan"), dtype=torch.float32, device=DEV)
    aj.attn_jvp_fwd(xd["q"], xd["k"], xd["v"], xd["dq"], xd["dk"], xd["dv"], mask, o=o, d_o=do,
                    lse=lse)
    torch.cuda.synchronize()
    for name, t in (("O", o), ("dO", do), ("LSE", lse)):
        assert bool(torch.isfinite(t).all()), f"{name}: an element is unwritten or not finite"
    rows = sample_rows(w, seed=wid)
    say(f"  every element written and finite; {len(rows)} rows per (b, h) against the oracle "
        f"({w.B * w.H} slices)")
    O, dO, LSE = masked_attention_jvp(x["q"], x["k"], x["v"], x["dq"], x["dk"], x["dv"], pred,
                                      rows=rows)
    sel = torch.as_tensor(rows)
    tol = TOL[torch.bfloat16]
    check("O", f64(o[:, sel]), O, tol)
    check("dO", f64(do[:, sel]), dO, tol)
    check("LSE", f64(lse[:, :, sel]), LSE, tol)


def test_chunkwise_65k_one_full_slice():
    # one whole (b, h) slice of the chunk-wise 65,520-token workload, every
    # row, compared with the oracle element by element
    w = WORKLOADS[3]
    h = 7
    say(f"case: workload 3, every row of slice (b=0, h={h}): {w.describe()}")
    x = make_inputs(w)
    xd = to_dev(x)
    mask = aj.attn_jvp_mask_tf(w.n_frames, w.tokens_per_frame, w.frames_per_chunk)
    pred = tf_allowed(w.n_frames, w.tokens_per_frame, w.frames_per_chunk)
    o, do, lse = run(xd, mask)
    sl = {k: v[:, :, h:h + 1] for k, v in x.items()}
    O, dO, LSE = masked_attention_jvp(sl["q"], sl["k"], sl["v"], sl["dq"], sl["dk"], sl["dv"],
                                      pred)
    tol = TOL[torch.bfloat16]
    check("O", f64(o[:, :, h:h + 1]), O, tol)
    check("dO", f64(do[:, :, h:h + 1]), dO, tol)
    check("LSE", f64(lse[:, h:h + 1]), LSE, tol)


def test_head_dim_64_long_sequence_sampled():
    # the chunk-wise 65,520-token sequence at head dim 64 (4 heads), sampled
    # rows of every (b, h)
    nf, tpf, fpc, H, D = 21, 1560, 3, 4, 64
    pred = tf_allowed(nf, tpf, fpc)
    say(f"case: chunk-wise TF nf={nf} tpf={tpf} fpc={fpc} H={H} D={D} (N={pred.n_q})")
    x = make_random(1, pred.n_q, H, D, dtype="bf16", seed=6464, tangent_std=0.1)
    w = types.SimpleNamespace(n_frames=nf, tokens_per_frame=tpf, unit_tokens=tpf * fpc,
                              n_units=nf // fpc, N=pred.n_q)
    rows = sample_rows(w, seed=64)
    say(f"  {len(rows)} sampled rows per (b, h)")
    parity(x, pred, aj.attn_jvp_mask_tf(nf, tpf, fpc), TOL[torch.bfloat16], rows=rows)


def test_rows_beyond_4gib_of_one_slice():
    # A (batch, head) slice whose rows span more than 4 GiB (row stride 2^20
    # elements, 2,100 rows): the tile staging must not wrap 32-bit byte
    # offsets.  Forward (dQ tile staging) and backward (V tile staging of the
    # dK/dV pass), checked against the oracle.
    from oracle import masked_attention_grad
    nf, tpf, D, SN = 7, 150, 128, 1 << 20
    pred = tf_allowed(nf, tpf, 1)
    N = pred.n_q
    assert (N - 1) * SN * 2 > (1 << 32)
    say(f"case: bf16 TF N={N} D={D}, row stride {SN} elements ({N * SN * 2 / 2**30:.1f} GiB per tensor)")
    x = make_random(1, N, 1, D, dtype="bf16", seed=9990, tangent_std=0.1)
    g = make_random(1, N, 1, D, dtype="bf16", seed=9991)["q"]

    def big(src=None):
        buf = torch.empty((N, SN), dtype=torch.bfloat16, device=DEV)
        v = buf[:, :D].unsqueeze(0).unsqueeze(2)          # [1, N, 1, D], strides (.., SN, .., 1)
        if src is not None:
            v.copy_(src.to(DEV))
        return v

    t = {n: big(x[n]) for n in ("q", "k", "v", "dq", "dk", "dv")}
    o, do, gq, gk, gv, gd = big(), big(), big(), big(), big(), big(g)
    mask = aj.attn_jvp_mask_tf(nf, tpf, 1)
    lse = torch.empty(1, 1, N, dtype=torch.float32, device=DEV)
    aj.attn_jvp_fwd(t["q"], t["k"], t["v"], t["dq"], t["dk"], t["dv"], mask, o=o, d_o=do, lse=lse)
    torch.cuda.synchronize()
    O, dO, LSE = masked_attention_jvp(x["q"], x["k"], x["v"], x["dq"], x["dk"], x["dv"], pred)
    check("O", f64(o), O, 2e-2)
    check("dO", f64(do), dO, 2e-2)
    check("LSE", f64(lse), LSE, 2e-2)
    po, _, plse = aj.attn_jvp_fwd(t["q"], t["k"], t["v"], None, None, None, mask, o=o, lse=lse)
    aj.attn_jvp_bwd(t["q"], t["k"], t["v"], po, gd, plse, mask, g_q=gq, g_k=gk, g_v=gv)
    torch.cuda.synchronize()
    dQ, dK, dV, _ = masked_attention_grad(x["q"], x["k"], x["v"], g, pred)
    check("dQ", f64(gq), dQ, 2e-2)
    check("dK", f64(gk), dK, 2e-2)
    check("dV", f64(gv), dV, 2e-2)


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("f32", 64)])
def test_head_major_memory_layout(dtype, D):
    # tensors stored [B, H, N, D] (row stride D, head stride N * D) and passed
    # as [B, N, H, D] views: forward, split forward and backward
    from oracle import masked_attention_grad
    pred = tf_allowed(5, 37, 1)
    B, H, N = 2, 3, pred.n_q
    say(f"case: head-major layout {dtype} D={D} B={B} H={H} N={N}")
    x = make_random(B, N, H, D, dtype=dtype, seed=13200 + D, tangent_std=0.1)
    hm = {k: v.permute(0, 2, 1, 3).contiguous().to(DEV).permute(0, 2, 1, 3) for k, v in x.items()}
    assert hm["q"].stride(1) == D and hm["q"].stride(2) == N * D
    mask = aj.attn_jvp_mask_tf(5, 37, 1)
    out = lambda: torch.empty(B, H, N, D, dtype=hm["q"].dtype, device=DEV).permute(0, 2, 1, 3)
    tol = TOL[hm["q"].dtype]
    O, dO, LSE = masked_attention_jvp(x["q"], x["k"], x["v"], x["dq"], x["dk"], x["dv"], pred)
    for S in (1, 3):
        o, do = out(), out()
        _, _, lse = aj.attn_jvp_fwd(hm["q"], hm["k"], hm["v"], hm["dq"], hm["dk"], hm["dv"], mask,
                                    o=o, d_o=do, max_splits=S)
        torch.cuda.synchronize()
        check(f"O (S={S})", f64(o), O, tol)
        check(f"dO (S={S})", f64(do), dO, tol)
        check(f"LSE (S={S})", f64(lse), LSE, tol)
    g = make_random(B, N, H, D, dtype=dtype, seed=13300 + D)["q"]
    gd = g.permute(0, 2, 1, 3).contiguous().to(DEV).permute(0, 2, 1, 3)
    o = out()
    _, _, lse = aj.attn_jvp_fwd(hm["q"], hm["k"], hm["v"], None, None, None, mask, o=o)
    gq, gk, gv = out(), out(), out()
    aj.attn_jvp_bwd(hm["q"], hm["k"], hm["v"], o, gd, lse, mask, g_q=gq, g_k=gk, g_v=gv)
    torch.cuda.synchronize()
    dQ, dK, dV, _ = masked_attention_grad(x["q"], x["k"], x["v"], g, pred)
    check("dQ", f64(gq), dQ, tol)
    check("dK", f64(gk), dK, tol)
    check("dV", f64(gv), dV, tol)


# A query tile whose key list holds more than two chunks of schedule entries
# (more than 1,024 key blocks of 32): the kernels restage the entry list in
# LDS while they walk it, so every refill is crossed here.  Dense masks with a
# ragged last key block, every element compared with the oracle.
@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("tangent", [True, False])
def test_long_key_list_crosses_entry_refills(D, tangent):
    n_q, n_k, H = 300, 40017, 2
    say(f"case: dense bf16 n_q={n_q} n_k={n_k} H={H} D={D} tangent={tangent}")
    pred = dense_allowed(n_q, n_k)
    xq = make_random(1, n_q, H, D, dtype="bf16", seed=14100 + D, tangent_std=0.1)
    xk = make_random(1, n_k, H, D, dtype="bf16", seed=14200 + D, tangent_std=0.1)
    x = dict(q=xq["q"], dq=xq["dq"], k=xk["k"], v=xk["v"], dk=xk["dk"], dv=xk["dv"])
    xd = to_dev(x)
    mask = aj.attn_jvp_mask_dense(n_q, n_k)
    o = torch.full_like(xd["q"], float("nan"))
    do = torch.full_like(xd["q"], float("nan"))
    lse = torch.full((1, H, n_q), float("nan"), dtype=torch.float32, device=DEV)
    if tangent:
        aj.attn_jvp_fwd(xd["q"], xd["k"], xd["v"], xd["dq"], xd["dk"], xd["dv"], mask, o=o,
                        d_o=do, lse=lse)
    else:
        aj.attn_jvp_fwd(xd["q"], xd["k"], xd["v"], None, None, None, mask, o=o, lse=lse)
    torch.cuda.synchronize()
    tol = TOL[torch.bfloat16]
    if tangent:
        O, dO, LSE = masked_attention_jvp(x["q"], x["k"], x["v"], x["dq"], x["dk"], x["dv"], pred)
        check("dO", f64(do), dO, tol)
    else:
        O, LSE = masked_attention(x["q"], x["k"], x["v"], pred)
    check("O", f64(o), O, tol)
    check("LSE", f64(lse), LSE, tol)
