"""GPU parity of the backward (gradients of the masked primal) against the
fp64 oracle, through the C ABI.  The GPU backward consumes the GPU forward's
O and LSE; the oracle sees only the seeded inputs.  Tolerance per output
tensor: max|gpu - ref| <= tol * max|ref|, tol = 2e-2 for bf16 inputs and
outputs, 1e-5 for fp32."""

import sys

import numpy as np
import pytest
import torch

import attention_jvp_causal_attn_amd as aj
from attention_jvp_causal_attn_amd.inputs import WORKLOADS, make_inputs, make_random
from oracle import (block_causal_allowed, dense_allowed, masked_attention_grad, rects_allowed,
                    tf_allowed)

pytestmark = pytest.mark.gpu
TOL = 2e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def check(name, got, ref, tol=TOL):
    got = np.asarray(got, dtype=np.float64)
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    err = np.abs(got - ref).max()
    scale = np.abs(ref).max()
    rel = err / scale if scale > 0 else err
    say(f"  {name}: max|err| = {err:.3e}, max|ref| = {scale:.3e}, ratio = {rel:.3e} (tol {tol})")
    assert rel <= tol, f"{name}: {rel:.3e} > {tol}"


def run_bwd(x, g, mask):
    xd = {k: v.cuda() for k, v in x.items()}
    gd = g.cuda()
    o, _, lse = aj.attn_jvp_fwd(xd["q"], xd["k"], xd["v"], None, None, None, mask)
    gq, gk, gv, delta = aj.attn_jvp_bwd(xd["q"], xd["k"], xd["v"], o, gd, lse, mask)
    torch.cuda.synchronize()
    return gq, gk, gv, delta


def parity(x, g, pred, mask, rows=None, keys=None, tol=TOL):
    gq, gk, gv, delta = run_bwd(x, g, mask)
    dQ, dK, dV, Ds = masked_attention_grad(x["q"], x["k"], x["v"], g, pred, rows=rows, keys=keys)
    rsel = slice(None) if rows is None else torch.as_tensor(rows)
    ksel = slice(None) if keys is None else torch.as_tensor(keys)
    check("dQ", f64(gq[:, rsel]), dQ, tol)
    check("dK", f64(gk[:, ksel]), dK, tol)
    check("dV", f64(gv[:, ksel]), dV, tol)
    check("D", f64(delta[:, :, rsel]), Ds, tol)


SMALL = [
    (5, 37, 1, 2, 3),   # N=370: 3 query tiles, ragged tail, unaligned units
    (4, 64, 1, 1, 2),   # tile-aligned units
    (3, 100, 3, 2, 1),  # one chunk of 300 tokens per stream
    (2, 1, 1, 1, 1),    # N=4: rows with a single admissible key
    (9, 33, 3, 1, 1),
    (8, 130, 2, 1, 2),  # N=1040: five 256-row tiles, ragged tail
]


@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("nf,tpf,fpc,B,H", SMALL)
def test_small_tf_bwd(nf, tpf, fpc, B, H, D):
    say(f"case: bwd bf16 TF nf={nf} tpf={tpf} fpc={fpc} B={B} H={H} D={D}")
    pred = tf_allowed(nf, tpf, fpc)
    x = make_random(B, pred.n_q, H, D, dtype="bf16", seed=9500 + nf * 10 + tpf)
    g = make_random(B, pred.n_q, H, D, dtype="bf16", seed=9600 + nf)["q"]
    parity(x, g, pred, aj.attn_jvp_mask_tf(nf, tpf, fpc))


@pytest.mark.parametrize("D", [128, 64])
def test_rect_bwd_queries_differ_from_keys(D):
    # queries of the current chunk against a longer key sequence, with keys
    # that no query sees (their gradients are zero)
    n_q, n_k = 150, 420
    rects = [(0, 70, 0, 300), (70, 150, 0, 140), (70, 150, 260, 330)]
    gq = [0, 70, 150]
    rp = [0, 1, 3]
    kb = [0, 0, 260]
    ke = [300, 140, 330]
    pred = rects_allowed(n_q, n_k, rects)
    mask = aj.attn_jvp_mask_rects(n_q, n_k, gq, rp, kb, ke)
    xq = make_random(1, n_q, 2, D, dtype="bf16", seed=9700)
    xk = make_random(1, n_k, 2, D, dtype="bf16", seed=9710)
    x = {"q": xq["q"], "k": xk["k"], "v": xk["v"]}
    g = xq["dq"]
    gq_, gk_, gv_, _ = run_bwd(x, g, mask)
    assert torch.count_nonzero(gk_[:, 330:]) == 0 and torch.count_nonzero(gv_[:, 330:]) == 0
    parity(x, g, pred, mask)


@pytest.mark.parametrize("D", [128, 64])
def test_dense_bwd(D):
    pred = dense_allowed(300, 300)
    x = make_random(2, 300, 2, D, dtype="bf16", seed=9800)
    g = make_random(2, 300, 2, D, dtype="bf16", seed=9810)["q"]
    parity(x, g, pred, aj.attn_jvp_mask_dense(300, 300))


@pytest.mark.parametrize("D", [128, 64])
def test_block_causal_bwd(D):
    pred = block_causal_allowed(6, 70)
    x = make_random(1, pred.n_q, 2, D, dtype="bf16", seed=9850 + D)
    g = make_random(1, pred.n_q, 2, D, dtype="bf16", seed=9860 + D)["q"]
    parity(x, g, pred, aj.attn_jvp_mask_block_causal(6, 70))


def test_bwd_deterministic():
    pred = tf_allowed(4, 50, 2)
    x = make_random(1, pred.n_q, 2, 128, dtype="bf16", seed=9900)
    g = make_random(1, pred.n_q, 2, 128, dtype="bf16", seed=9910)["q"]
    mask = aj.attn_jvp_mask_tf(4, 50, 2)
    a = run_bwd(x, g, mask)
    b = run_bwd(x, g, mask)
    for u, w in zip(a, b):
        assert torch.equal(u, w)


def test_full_size_batched_workload_bwd_sampled():
    # batched 22k workload with outlier rows, one (b, h) slice checked on
    # sampled rows (dQ) and sampled keys (dK, dV) against the oracle
    w = WORKLOADS[4]
    say(f"case: bwd {w.describe()}")
    x = make_inputs(w)
    g = make_random(w.B, w.N, w.H, w.D, dtype=w.dtype, seed=9950)["q"]
    mask = aj.attn_jvp_mask_tf(w.n_frames, w.tokens_per_frame, w.frames_per_chunk)
    gq, gk, gv, delta = run_bwd(x, g, mask)
    pred = tf_allowed(w.n_frames, w.tokens_per_frame, w.frames_per_chunk)
    rng = np.random.default_rng(5)
    rows = np.sort(rng.choice(w.N, size=48, replace=False))
    keys = np.sort(rng.choice(w.N, size=48, replace=False))
    b, h = 1, 5
    sl = {k: v[b:b + 1, :, h:h + 1] for k, v in x.items()}
    dQ, dK, dV, Ds = masked_attention_grad(sl["q"], sl["k"], sl["v"], g[b:b + 1, :, h:h + 1],
                                           pred, rows=rows, keys=keys, row_block=256)
    check("dQ", f64(gq[b:b + 1, rows, h:h + 1]), dQ)
    check("dK", f64(gk[b:b + 1, keys, h:h + 1]), dK)
    check("dV", f64(gv[b:b + 1, keys, h:h + 1]), dV)
    check("D", f64(delta[b:b + 1, h:h + 1, rows]), Ds)


@pytest.mark.parametrize("D", [64])
def test_chunkwise_11k_bwd_sampled(D):
    # 7 chunks of 3 frames x 520 tokens per stream (N = 21,840 with the clean
    # and noisy streams: 86 query tiles), one (b, h) slice checked on sampled
    # rows (dQ) and sampled keys (dK, dV), chunk boundaries included (head
    # dim 128 has the batched 22k case)
    nf, tpf, fpc, H = 21, 520, 3, 2
    pred = tf_allowed(nf, tpf, fpc)
    say(f"case: bwd chunk-wise TF nf={nf} tpf={tpf} fpc={fpc} H={H} D={D} (N={pred.n_q})")
    x = make_random(1, pred.n_q, H, D, dtype="bf16", seed=6400 + D)
    g = make_random(1, pred.n_q, H, D, dtype="bf16", seed=6401 + D)["q"]
    mask = aj.attn_jvp_mask_tf(nf, tpf, fpc)
    gq, gk, gv, delta = run_bwd(x, g, mask)
    C, Nc = tpf * fpc, nf * tpf
    edges = {s + u * C + o for s in (0, Nc) for u in range(nf // fpc) for o in (0, C - 1)}
    rng = np.random.default_rng(D)
    rows = np.array(sorted(edges | set(rng.integers(0, pred.n_q, size=24).tolist())))
    keys = np.array(sorted(edges | set(rng.integers(0, pred.n_q, size=24).tolist())))
    h = 1
    sl = {k: v[:, :, h:h + 1] for k, v in x.items()}
    dQ, dK, dV, Ds = masked_attention_grad(sl["q"], sl["k"], sl["v"], g[:, :, h:h + 1], pred,
                                           rows=rows, keys=keys, row_block=256)
    check("dQ", f64(gq[:, rows, h:h + 1]), dQ)
    check("dK", f64(gk[:, keys, h:h + 1]), dK)
    check("dV", f64(gv[:, keys, h:h + 1]), dV)
    check("D", f64(delta[:, h:h + 1, rows]), Ds)


# ------------------------------------------------------------ fp32 path ----

@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("nf,tpf,fpc,B,H", [(4, 16, 1, 1, 2), (5, 37, 1, 2, 1), (3, 50, 3, 1, 1)])
def test_small_tf_bwd_fp32(nf, tpf, fpc, B, H, D):
    say(f"case: bwd fp32 TF nf={nf} tpf={tpf} fpc={fpc} B={B} H={H} D={D}")
    pred = tf_allowed(nf, tpf, fpc)
    x = make_random(B, pred.n_q, H, D, dtype="f32", seed=9700 + nf * 10 + tpf + D)
    g = make_random(B, pred.n_q, H, D, dtype="f32", seed=9800 + nf)["q"]
    parity(x, g, pred, aj.attn_jvp_mask_tf(nf, tpf, fpc), tol=1e-5)


def test_tiny_tf_fp32_workload_bwd():
    w = WORKLOADS[1]
    say(f"case: bwd on {w.describe()}")
    x = make_inputs(w)
    g = make_random(w.B, w.N, w.H, w.D, dtype="f32", seed=9900)["q"]
    parity(x, g, tf_allowed(w.n_frames, w.tokens_per_frame, w.frames_per_chunk),
           aj.attn_jvp_mask_tf(w.n_frames, w.tokens_per_frame, w.frames_per_chunk), tol=1e-5)


def test_rect_bwd_fp32_unseen_keys_and_empty_rows():
    # rows 70..99 see nothing; keys 150..199 are seen by nobody
    n_q, n_k, H, D = 130, 200, 2, 64
    gq_, rp, kb, ke = [0, 70, 100, 130], [0, 1, 1, 2], [0, 10], [150, 120]
    pred = rects_allowed(n_q, n_k, [(0, 70, 0, 150), (100, 130, 10, 120)])
    xq = make_random(1, n_q, H, D, dtype="f32", seed=9910)
    xk = make_random(1, n_k, H, D, dtype="f32", seed=9911)
    x = dict(q=xq["q"], k=xk["k"], v=xk["v"])
    g = make_random(1, n_q, H, D, dtype="f32", seed=9912)["q"]
    gq, gk, gv, delta = run_bwd(x, g, aj.attn_jvp_mask_rects(n_q, n_k, gq_, rp, kb, ke))
    assert torch.all(gq[:, 70:100] == 0) and torch.all(gk[:, 150:] == 0) and torch.all(gv[:, 150:] == 0)
    dQ, dK, dV, Ds = masked_attention_grad(x["q"], x["k"], x["v"], g, pred)
    check("dQ", f64(gq), dQ, 1e-5)
    check("dK", f64(gk), dK, 1e-5)
    check("dV", f64(gv), dV, 1e-5)


@pytest.mark.parametrize("D", [128, 64])
def test_rect_bwd_bf16_unseen_keys_and_empty_rows(D):
    # rows 250..329 see nothing (LSE = -inf), keys 520..699 are seen by nobody;
    # partial blocks then hold rows and queries without any admissible key
    n_q, n_k, H = 600, 700, 2
    gq_, rp, kb, ke = [0, 250, 330, 600], [0, 1, 1, 3], [0, 37, 500], [400, 460, 520]
    pred = rects_allowed(n_q, n_k, [(0, 250, 0, 400), (330, 600, 37, 460), (330, 600, 500, 520)])
    xq = make_random(1, n_q, H, D, dtype="bf16", seed=9920 + D)
    xk = make_random(1, n_k, H, D, dtype="bf16", seed=9921 + D)
    x = dict(q=xq["q"], k=xk["k"], v=xk["v"])
    g = make_random(1, n_q, H, D, dtype="bf16", seed=9922 + D)["q"]
    mask = aj.attn_jvp_mask_rects(n_q, n_k, gq_, rp, kb, ke)
    gq, gk, gv, delta = run_bwd(x, g, mask)
    assert torch.all(gq[:, 250:330] == 0) and torch.all(gk[:, 520:] == 0) and torch.all(gv[:, 520:] == 0)
    assert torch.all(delta[:, :, 250:330] == 0)
    parity(x, g, pred, mask)


# More than 1,024 blocks of 32 along one tile's list in each pass: 40,017
# keys per query tile (dQ pass), then 40,017 queries per key tile (dK/dV
# pass); the entry list is restaged in LDS twice on the way.  Dense masks with
# a ragged last block, every element compared with the oracle.
@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("n_q,n_k", [(300, 40017), (40017, 300)])
def test_long_lists_cross_entry_refills_bwd(n_q, n_k, D):
    H = 2
    say(f"case: bwd dense bf16 n_q={n_q} n_k={n_k} H={H} D={D}")
    pred = dense_allowed(n_q, n_k)
    xq = make_random(1, n_q, H, D, dtype="bf16", seed=14300 + D)
    xk = make_random(1, n_k, H, D, dtype="bf16", seed=14400 + D)
    x = {"q": xq["q"], "k": xk["k"], "v": xk["v"]}
    g = xq["dq"]
    parity(x, g, pred, aj.attn_jvp_mask_dense(n_q, n_k))


def test_chunkwise_65k_bwd_every_tile():
    # The backward at the benchmarked shape (chunk-wise 65,520 tokens, B=1,
    # H=12, D=128), NaN-filled outputs: every element of every slice written
    # and finite.  Slice h=4 against the oracle: dQ and D on the first and
    # last row of every 256-row query tile and of every chunk, dK and dV on
    # the first and last key of every 256-key tile and of every chunk.
    w = WORKLOADS[3]
    say(f"case: bwd {w.describe()}")
    x = make_inputs(w)
    g = make_random(w.B, w.N, w.H, w.D, dtype=w.dtype, seed=9960)["q"]
    mask = aj.attn_jvp_mask_tf(w.n_frames, w.tokens_per_frame, w.frames_per_chunk)
    xd = {k: v.cuda() for k, v in x.items()}
    gd = g.cuda()
    o, _, lse = aj.attn_jvp_fwd(xd["q"], xd["k"], xd["v"], None, None, None, mask)
    gq, gk, gv = (torch.full_like(xd["q"], float("nan")) for _ in range(3))
    delta = torch.full_like(lse, float("nan"))
    aj.attn_jvp_bwd(xd["q"], xd["k"], xd["v"], o, gd, lse, mask, g_q=gq, g_k=gk, g_v=gv,
                    delta=delta)
    torch.cuda.synchronize()
    for name, t in (("dQ", gq), ("dK", gk), ("dV", gv), ("D", delta)):
        assert bool(torch.isfinite(t).all()), f"{name}: an element is unwritten or not finite"
    pred = tf_allowed(w.n_frames, w.tokens_per_frame, w.frames_per_chunk)
    C, Nc = w.unit_tokens, w.n_frames * w.tokens_per_frame
    edges = {s + u * C + o_ for s in (0, Nc) for u in range(w.n_units) for o_ in (0, C - 1)}
    edges |= {t0 + o_ for t0 in range(0, w.N, 256) for o_ in (0, 255) if t0 + o_ < w.N}
    idx = np.array(sorted(edges))
    h = 4
    say(f"  every element written and finite; {len(idx)} rows and keys of slice h={h} "
        "against the oracle")
    sl = {k: v[:, :, h:h + 1] for k, v in x.items()}
    dQ, dK, dV, Ds = masked_attention_grad(sl["q"], sl["k"], sl["v"], g[:, :, h:h + 1], pred,
                                           rows=idx, keys=idx)
    check("dQ", f64(gq[:, idx, h:h + 1]), dQ)
    check("dK", f64(gk[:, idx, h:h + 1]), dK)
    check("dV", f64(gv[:, idx, h:h + 1]), dV)
    check("D", f64(delta[:, h:h + 1, idx]), Ds)
