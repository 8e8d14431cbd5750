"""The allocation-free split-key forward (attn_jvp_fwd_split_noalloc, called
through the C ABI) against the split-key entry point it stands in for
(attn_jvp_fwd_split with a caller workspace): bit for bit equal outputs on
two calls in a row, the second with a smaller input (the fixed scratch array
keeps the first call's contents), plus the documented refusals: a schedule
that is not resident yet, and a launch larger than the scratch array."""

import ctypes
import sys

import numpy as np
import pytest
import torch

import attention_jvp_causal_attn_amd as aj
from attention_jvp_causal_attn_amd import _lib
from attention_jvp_causal_attn_amd.inputs import make_random
from oracle import masked_attention_jvp, rects_allowed, tf_allowed

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def args_of(x, o, do, lse, dlse):
    q, k = x["q"], x["k"]
    B, n_q, H, D = q.shape
    return _lib.AttnJvpArgs(
        dtype=_lib.ATTN_JVP_BF16 if q.dtype == torch.bfloat16 else _lib.ATTN_JVP_F32,
        B=B, H=H, n_q=n_q, n_k=k.shape[1], D=D,
        q=q.data_ptr(), k=k.data_ptr(), v=x["v"].data_ptr(), dq=x["dq"].data_ptr(),
        dk=x["dk"].data_ptr(), dv=x["dv"].data_ptr(), o=o.data_ptr(), d_o=do.data_ptr(),
        lse=lse.data_ptr(), q_stride_b=q.stride(0), q_stride_n=q.stride(1),
        q_stride_h=q.stride(2), k_stride_b=k.stride(0), k_stride_n=k.stride(1),
        k_stride_h=k.stride(2), scale=0.0, d_lse=dlse.data_ptr())


def outputs(x):
    q = x["q"]
    B, n_q, H, _ = q.shape
    o = torch.full_like(q, float("nan"))
    do = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, n_q), float("nan"), dtype=torch.float32, device=DEV)
    dlse = torch.full_like(lse, float("nan"))
    return o, do, lse, dlse


def via_split(x, mask, S):
    """The existing entry point, with a caller-owned workspace."""
    o, do, lse, dlse = outputs(x)
    a = args_of(x, o, do, lse, dlse)
    need = ctypes.c_uint64(0)
    L = _lib.lib()
    assert L.attn_jvp_fwd_split_workspace(ctypes.byref(a), mask.handle, S,
                                          ctypes.byref(need)) == _lib.ATTN_JVP_OK
    ws = torch.empty(max(16, need.value), dtype=torch.uint8, device=DEV)
    st = L.attn_jvp_fwd_split(ctypes.byref(a), mask.handle, S, ctypes.c_void_p(ws.data_ptr()),
                              ctypes.c_uint64(ws.numel()), None)
    assert st == _lib.ATTN_JVP_OK, aj.attn_jvp_status_str(st)
    torch.cuda.synchronize()
    return (o, do, lse, dlse), need.value


def via_noalloc(x, mask, S):
    o, do, lse, dlse = outputs(x)
    a = args_of(x, o, do, lse, dlse)
    st = _lib.lib().attn_jvp_fwd_split_noalloc(ctypes.byref(a), mask.handle, S, None)
    return st, (o, do, lse, dlse)


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def kv_case():
    # 1,000 queries (4 tiles of 256) against 20,000 keys, 8 heads, head dim
    # 128: every tile cut in 4 (16 partial slots, 34 MB of partial sums)
    n_q, n_k, H = 1000, 20000, 8
    xq = make_random(1, n_q, H, 128, dtype="bf16", seed=15100, tangent_std=0.1, device=DEV)
    xk = make_random(1, n_k, H, 128, dtype="bf16", seed=15200, tangent_std=0.1, device=DEV)
    x = dict(q=xq["q"], dq=xq["dq"], k=xk["k"], v=xk["v"], dk=xk["dk"], dv=xk["dv"])
    mask = aj.attn_jvp_mask_rects(n_q, n_k, [0, n_q], [0, 1], [0], [n_k])
    return x, mask, rects_allowed(n_q, n_k, [(0, n_q, 0, n_k)]), 4


def tf_case(dtype, D):
    # teacher-forcing mask, 1,370 tokens: smaller than the first call
    pred = tf_allowed(5, 137, 1)
    x = make_random(1, pred.n_q, 2, D, dtype=dtype, seed=15300 + D, tangent_std=0.1, device=DEV)
    return x, aj.attn_jvp_mask_tf(5, 137, 1), pred, 3


def test_noalloc_matches_split_entry_point_two_calls():
    cases = [("kv-cache rectangle 1000 x 20000, H=8, D=128, bf16", kv_case()),
             ("TF 1370 tokens, H=2, D=64, bf16", tf_case("bf16", 64)),
             ("TF 1370 tokens, H=2, D=64, fp32", tf_case("f32", 64))]
    for name, (x, mask, pred, S) in cases:
        say(f"case: {name}, max_splits={S}")
        # before any split call on this device the schedule is not resident
        st, _ = via_noalloc(x, mask, S)
        assert st == _lib.ATTN_JVP_ERR_NOT_READY, aj.attn_jvp_status_str(st)
        ref, need = via_split(x, mask, S)
        assert 0 < need <= _lib.NOALLOC_SCRATCH_BYTES
        st, got = via_noalloc(x, mask, S)
        assert st == _lib.ATTN_JVP_OK, aj.attn_jvp_status_str(st)
        torch.cuda.synchronize()
        for nm, u, v in zip(("O", "dO", "LSE", "dLSE"), got, ref):
            assert torch.equal(u, v), f"{nm} differs from attn_jvp_fwd_split"
        say(f"  {need} bytes of partial sums; O, dO, LSE, dLSE bitwise equal to "
            "attn_jvp_fwd_split")
        # and within the oracle's tolerance on a few rows
        rows = np.array([0, 255, 256, x["q"].shape[1] - 1])
        O, dO, LSE = masked_attention_jvp(*(x[n].cpu() for n in ("q", "k", "v", "dq", "dk", "dv")),
                                          pred, rows=rows)
        tol = 2e-2 if x["q"].dtype == torch.bfloat16 else 1e-5
        for nm, g, r in (("O", got[0][:, rows], O), ("dO", got[1][:, rows], dO),
                         ("LSE", got[2][:, :, rows], LSE)):
            err = np.abs(f64(g) - r).max() / np.abs(r).max()
            assert err <= tol, f"{nm}: {err:.3e} > {tol}"


def test_noalloc_refuses_launches_beyond_the_scratch_array():
    # one frame of 1,560 queries against 32,760 keys with 16 heads, cut in 3:
    # 21 partial slots x 16 heads x 256 rows x 1,040 bytes = 89 MB > 64 MiB
    n_q, n_k, H = 1560, 32760, 16
    xq = make_random(1, n_q, H, 128, dtype="bf16", seed=15400, tangent_std=0.1, device=DEV)
    xk = make_random(1, n_k, H, 128, dtype="bf16", seed=15500, tangent_std=0.1, device=DEV)
    x = dict(q=xq["q"], dq=xq["dq"], k=xk["k"], v=xk["v"], dk=xk["dk"], dv=xk["dv"])
    mask = aj.attn_jvp_mask_rects(n_q, n_k, [0, n_q], [0, 1], [0], [n_k])
    o, do, lse, dlse = outputs(x)
    a = args_of(x, o, do, lse, dlse)
    need = ctypes.c_uint64(0)
    L = _lib.lib()
    assert L.attn_jvp_fwd_split_workspace(ctypes.byref(a), mask.handle, 3,
                                          ctypes.byref(need)) == _lib.ATTN_JVP_OK
    assert need.value > _lib.NOALLOC_SCRATCH_BYTES
    st = L.attn_jvp_fwd_split_noalloc(ctypes.byref(a), mask.handle, 3, None)
    assert st == _lib.ATTN_JVP_ERR_SCRATCH, aj.attn_jvp_status_str(st)
    torch.cuda.synchronize()
    assert torch.isnan(o).all()   # nothing was launched
