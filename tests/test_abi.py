"""The C ABI library loads without a GPU, exports every declared entry point
and rejects bad arguments with the documented status codes before touching
the device."""

import ctypes
import os
import re

import pytest

import attention_jvp_causal_attn_amd as aj
from attention_jvp_causal_attn_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_jvp.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_jvp_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert "attn_jvp_fwd" in names and "attn_jvp_mask_tf" in names
    handle = ctypes.CDLL(_lib.LIB_PATH)
    for n in names:
        assert hasattr(handle, n), n
    assert set(names) == set(_lib.SIGNATURES)


def test_version_and_status_strings():
    assert aj.attn_jvp_version() == 2
    for st in range(-10, 1):
        assert aj.attn_jvp_status_str(st) not in ("", "unknown status")
    assert aj.attn_jvp_status_str(-99) == "unknown status"
    assert aj.attn_jvp_tile_shape(aj.ATTN_JVP_BF16, 128) == (256, 32)
    assert aj.attn_jvp_tile_shape(aj.ATTN_JVP_BF16, 128, tangent=False) == (256, 64)
    assert aj.attn_jvp_tile_shape(aj.ATTN_JVP_BF16, 64) == (256, 32)
    assert aj.attn_jvp_tile_shape(aj.ATTN_JVP_BF16, 64, tangent=False) == (256, 32)
    assert aj.attn_jvp_tile_shape(aj.ATTN_JVP_F32, 64) == (64, 32)
    assert aj.attn_jvp_tile_shape(aj.ATTN_JVP_F32, 128, tangent=False) == (64, 32)
    with pytest.raises(aj.AttnJvpError):
        aj.attn_jvp_tile_shape(aj.ATTN_JVP_BF16, 96)
    with pytest.raises(aj.AttnJvpError):
        aj.attn_jvp_tile_shape(7, 128)


def _gpu_present():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


def _args(mask, sp=0x10000, **kw):
    # placeholder addresses sp apart (the default tensors of the 128-token
    # masks below take exactly 0x10000 bytes each)
    info = mask.info()
    base = dict(dtype=0, B=1, H=2, n_q=info["n_q"], n_k=info["n_k"], D=128,
                q=sp, k=2 * sp, v=3 * sp, dq=4 * sp, dk=5 * sp, dv=6 * sp,
                o=7 * sp, d_o=8 * sp, lse=9 * sp,
                q_stride_b=0, q_stride_n=256, q_stride_h=128,
                k_stride_b=0, k_stride_n=256, k_stride_h=128, scale=0.0)
    base.update(kw)
    return _lib.AttnJvpArgs(**base)


def _fwd(a, mask):
    return _lib.lib().attn_jvp_fwd(ctypes.byref(a), mask.handle, None)


# Every case fails validation before any HIP call, so fake (never dereferenced)
# device addresses are safe here with or without a GPU.
BAD = [
    (dict(dtype=5), _lib.ATTN_JVP_ERR_DTYPE),
    (dict(q=None), _lib.ATTN_JVP_ERR_NULL),
    (dict(o=None), _lib.ATTN_JVP_ERR_NULL),
    (dict(lse=None), _lib.ATTN_JVP_ERR_NULL),
    (dict(d_o=None), _lib.ATTN_JVP_ERR_NULL),
    (dict(dk=None, d_o=None), _lib.ATTN_JVP_ERR_NULL),   # any tangent given needs d_o
    (dict(dq=None, dv=None, d_o=None), _lib.ATTN_JVP_ERR_NULL),
    (dict(D=96), _lib.ATTN_JVP_ERR_UNSUPPORTED),
    (dict(B=0), _lib.ATTN_JVP_ERR_SHAPE),
    (dict(H=-1), _lib.ATTN_JVP_ERR_SHAPE),
    (dict(n_q=37), _lib.ATTN_JVP_ERR_MASK),
    (dict(n_k=11), _lib.ATTN_JVP_ERR_MASK),
    (dict(q=0x10002), _lib.ATTN_JVP_ERR_ALIGN),
    (dict(lse=0x90004), _lib.ATTN_JVP_ERR_ALIGN),
    (dict(d_o=0x80008), _lib.ATTN_JVP_ERR_ALIGN),
    (dict(q_stride_n=257), _lib.ATTN_JVP_ERR_ALIGN),
    (dict(k_stride_h=132), _lib.ATTN_JVP_ERR_ALIGN),
    (dict(q_stride_h=64), _lib.ATTN_JVP_ERR_SHAPE),
    (dict(k_stride_b=-8), _lib.ATTN_JVP_ERR_SHAPE),
    (dict(k_stride_n=1 << 25), _lib.ATTN_JVP_ERR_SHAPE),
    (dict(o=0x10000), _lib.ATTN_JVP_ERR_UNSUPPORTED),      # output aliases q
    (dict(d_o=0x70000), _lib.ATTN_JVP_ERR_UNSUPPORTED),    # d_o aliases o
    (dict(scale=float("nan")), _lib.ATTN_JVP_ERR_SHAPE),
    (dict(scale=float("inf")), _lib.ATTN_JVP_ERR_SHAPE),
    (dict(d_lse=0xa0004), _lib.ATTN_JVP_ERR_ALIGN),
    (dict(d_lse=0xa0000, dq=None, dk=None, dv=None), _lib.ATTN_JVP_ERR_UNSUPPORTED),  # no tangent
    (dict(d_lse=0x90000), _lib.ATTN_JVP_ERR_UNSUPPORTED),   # d_lse aliases lse
    (dict(lse=0x70000), _lib.ATTN_JVP_ERR_UNSUPPORTED),     # lse aliases o
    (dict(d_lse=0x30000), _lib.ATTN_JVP_ERR_UNSUPPORTED),   # d_lse aliases v
    # outputs that share bytes with another tensor at an offset
    (dict(o=0x1fff0), _lib.ATTN_JVP_ERR_UNSUPPORTED),       # o's first row in q's last
    (dict(o=0x20010), _lib.ATTN_JVP_ERR_UNSUPPORTED),       # o inside k
    (dict(d_o=0x6ff00), _lib.ATTN_JVP_ERR_UNSUPPORTED),     # d_o over dv's tail
    (dict(lse=0x8fff0), _lib.ATTN_JVP_ERR_UNSUPPORTED),     # lse over d_o's tail
    (dict(d_lse=0x90200), _lib.ATTN_JVP_ERR_UNSUPPORTED),   # d_lse inside lse
    (dict(lse=0x2fff0, dq=None, dk=None, dv=None, d_o=None),
     _lib.ATTN_JVP_ERR_UNSUPPORTED),                        # primal: lse over k's tail
    (dict(q_stride_n=0), _lib.ATTN_JVP_ERR_UNSUPPORTED),    # o writes one row N times
]


@pytest.mark.parametrize("kw,status", BAD)
def test_fwd_rejects_bad_arguments(kw, status):
    mask = aj.attn_jvp_mask_tf(4, 16, 1)
    assert _fwd(_args(mask, **kw), mask) == status


def _split(a, mask, S, ws=None, nbytes=0):
    return _lib.lib().attn_jvp_fwd_split(ctypes.byref(a), mask.handle, S, ws, nbytes, None)


@pytest.mark.parametrize("kw,status", BAD)
def test_split_rejects_bad_arguments(kw, status):
    mask = aj.attn_jvp_mask_tf(4, 16, 1)
    assert _split(_args(mask, **kw), mask, 2, 0x100000, 1 << 30) == status


def test_split_workspace_checks():
    mask = aj.attn_jvp_mask_tf(8, 64, 1)   # n = 1024 rows at D=64
    L = _lib.lib()
    a = _args(mask, sp=1 << 24, D=64, q_stride_n=128, q_stride_h=64, k_stride_n=128,
              k_stride_h=64)
    need = ctypes.c_uint64(0)
    assert L.attn_jvp_fwd_split_workspace(ctypes.byref(a), mask.handle, 4,
                                          ctypes.byref(need)) == _lib.ATTN_JVP_OK
    bm, bn = aj.attn_jvp_tile_shape(aj.ATTN_JVP_BF16, 64)
    u = aj.attn_jvp_mask_split_schedule(mask, bm, bn, 4)
    assert u["n_parts"] > 0
    rows = 1 * 2 * u["n_parts"] * bm                       # B * H * parts * block_m
    assert need.value == rows * 16 + rows * 2 * 64 * 4      # float4 stats + A, T rows
    assert L.attn_jvp_fwd_split_workspace(ctypes.byref(a), mask.handle, 0,
                                          ctypes.byref(need)) == _lib.ATTN_JVP_ERR_SHAPE
    assert L.attn_jvp_fwd_split_workspace(ctypes.byref(a), mask.handle, 4,
                                          None) == _lib.ATTN_JVP_ERR_NULL
    assert L.attn_jvp_fwd_split_workspace(ctypes.byref(a), mask.handle, 1,
                                          ctypes.byref(need)) == _lib.ATTN_JVP_OK
    assert need.value == 0
    big = 1 << 40
    assert L.attn_jvp_fwd_split_workspace(ctypes.byref(a), mask.handle, 4,
                                          ctypes.byref(need)) == _lib.ATTN_JVP_OK
    assert _split(a, mask, 0, big, need.value) == _lib.ATTN_JVP_ERR_SHAPE
    assert _split(a, mask, 4, None, need.value) == _lib.ATTN_JVP_ERR_NULL
    assert _split(a, mask, 4, big + 8, need.value) == _lib.ATTN_JVP_ERR_ALIGN
    assert _split(a, mask, 4, big, need.value - 16) == _lib.ATTN_JVP_ERR_SHAPE
    # the workspace may not share a byte with a tensor
    assert _split(a, mask, 4, (1 << 24) - 16, need.value) == _lib.ATTN_JVP_ERR_UNSUPPORTED
    assert _split(a, mask, 4, (9 << 24) - 16, need.value) == _lib.ATTN_JVP_ERR_UNSUPPORTED  # lse


@pytest.mark.skipif(_gpu_present(), reason="needs a host without a HIP device")
def test_split_without_device_reports_hip_error():
    mask = aj.attn_jvp_mask_tf(4, 16, 1)
    a = _args(mask)
    assert _split(a, mask, 1) == _lib.ATTN_JVP_ERR_HIP
    assert _split(a, mask, 2, 1 << 40, 1 << 30) == _lib.ATTN_JVP_ERR_HIP


def test_noalloc_argument_checks():
    mask = aj.attn_jvp_mask_tf(4, 16, 1)
    L = _lib.lib()
    assert L.attn_jvp_fwd_split_noalloc(None, mask.handle, 2, None) == _lib.ATTN_JVP_ERR_NULL
    a = _args(mask)
    assert L.attn_jvp_fwd_split_noalloc(ctypes.byref(a), None, 2, None) == _lib.ATTN_JVP_ERR_NULL
    if not _gpu_present():
        # no device: the scratch array has no address to fetch
        assert L.attn_jvp_fwd_split_noalloc(ctypes.byref(a), mask.handle, 2, None) == \
            _lib.ATTN_JVP_ERR_HIP


def test_fwd_null_args_and_mask():
    mask = aj.attn_jvp_mask_tf(4, 16, 1)
    L = _lib.lib()
    assert L.attn_jvp_fwd(None, mask.handle, None) == _lib.ATTN_JVP_ERR_NULL
    a = _args(mask)
    assert L.attn_jvp_fwd(ctypes.byref(a), None, None) == _lib.ATTN_JVP_ERR_NULL


@pytest.mark.skipif(_gpu_present(), reason="needs a host without a HIP device")
def test_fwd_without_device_reports_hip_error():
    mask = aj.attn_jvp_mask_tf(4, 16, 1)
    assert _fwd(_args(mask), mask) == _lib.ATTN_JVP_ERR_HIP
    assert _fwd(_args(mask, dq=None, dk=None, dv=None, d_o=None), mask) == _lib.ATTN_JVP_ERR_HIP
    assert _fwd(_args(mask, dk=None, dv=None), mask) == _lib.ATTN_JVP_ERR_HIP


def test_python_binding_requires_gpu_tensors():
    import torch
    mask = aj.attn_jvp_mask_tf(2, 4, 1)
    x = torch.zeros(1, 16, 1, 64)
    with pytest.raises(ValueError):
        aj.attn_jvp_fwd(x, x, x, x, x, x, mask)
    with pytest.raises(ValueError):
        aj.attn_jvp_fwd(x, x, x, x, None, x, mask)


def _bwd_args(mask, sp=0x10000, **kw):
    info = mask.info()
    base = dict(dtype=0, B=1, H=2, n_q=info["n_q"], n_k=info["n_k"], D=128,
                q=sp, k=2 * sp, v=3 * sp, o=4 * sp, g_o=5 * sp, lse=6 * sp,
                g_q=7 * sp, g_k=8 * sp, g_v=9 * sp, delta=10 * sp,
                q_stride_b=0, q_stride_n=256, q_stride_h=128,
                k_stride_b=0, k_stride_n=256, k_stride_h=128, scale=0.0)
    base.update(kw)
    return _lib.AttnJvpBwdArgs(**base)


BAD_BWD = [
    (dict(dtype=5), _lib.ATTN_JVP_ERR_DTYPE),
    (dict(q=None), _lib.ATTN_JVP_ERR_NULL),
    (dict(o=None), _lib.ATTN_JVP_ERR_NULL),
    (dict(lse=None), _lib.ATTN_JVP_ERR_NULL),
    (dict(delta=None), _lib.ATTN_JVP_ERR_NULL),
    (dict(g_v=None), _lib.ATTN_JVP_ERR_NULL),
    (dict(D=96), _lib.ATTN_JVP_ERR_UNSUPPORTED),
    (dict(dtype=1, k_stride_n=258), _lib.ATTN_JVP_ERR_ALIGN),   # fp32: 1032-byte rows
    (dict(B=0), _lib.ATTN_JVP_ERR_SHAPE),
    (dict(n_k=11), _lib.ATTN_JVP_ERR_MASK),
    (dict(g_q=0x70008), _lib.ATTN_JVP_ERR_ALIGN),
    (dict(k_stride_n=257), _lib.ATTN_JVP_ERR_ALIGN),
    (dict(q_stride_h=64), _lib.ATTN_JVP_ERR_SHAPE),
    (dict(g_q=0x10000), _lib.ATTN_JVP_ERR_UNSUPPORTED),   # output aliases q
    (dict(g_v=0x80000), _lib.ATTN_JVP_ERR_UNSUPPORTED),   # g_v aliases g_k
    (dict(g_q=0x1fff0), _lib.ATTN_JVP_ERR_UNSUPPORTED),   # g_q over q's tail
    (dict(g_k=0x4fff0), _lib.ATTN_JVP_ERR_UNSUPPORTED),   # g_k over o's tail
    (dict(delta=0x60200), _lib.ATTN_JVP_ERR_UNSUPPORTED), # delta inside lse
    (dict(delta=0x9ff00), _lib.ATTN_JVP_ERR_UNSUPPORTED), # delta over g_v's tail
    (dict(k_stride_n=0), _lib.ATTN_JVP_ERR_UNSUPPORTED),  # g_k writes one row N times
    (dict(scale=float("nan")), _lib.ATTN_JVP_ERR_SHAPE),
]


@pytest.mark.parametrize("kw,status", BAD_BWD)
def test_bwd_rejects_bad_arguments(kw, status):
    mask = aj.attn_jvp_mask_tf(4, 16, 1)
    a = _bwd_args(mask, **kw)
    assert _lib.lib().attn_jvp_bwd(ctypes.byref(a), mask.handle, None) == status


@pytest.mark.skipif(_gpu_present(), reason="needs a host without a HIP device")
def test_bwd_without_device_reports_hip_error():
    mask = aj.attn_jvp_mask_tf(4, 16, 1)
    for dtype in (0, 1):
        a = _bwd_args(mask, sp=0x10000 * (1 + dtype), dtype=dtype)   # fp32 rows are twice as long
        assert _lib.lib().attn_jvp_bwd(ctypes.byref(a), mask.handle, None) == _lib.ATTN_JVP_ERR_HIP


def test_split_choose():
    import torch
    bf = lambda n, D=128: torch.empty(1, n, 12, D, dtype=torch.bfloat16)
    # one frame of queries (7 tiles of 256 rows) against 32,760 keys (1,024
    # blocks of 32), 12 heads, 256 compute units: 84 workgroups leave the chip
    # idle.  By hand: S = 3 gives 252 units of <= 342 blocks, one round
    # (342 + 2 + 2); S = 2: 168 units of 512; S = 4: 336 units, two rounds of
    # 256; S = 6: 504 units, two rounds of 171; S = 9: 756 units, three
    # rounds of 114; S = 12: 1008 units, four rounds of 86.
    m = aj.attn_jvp_mask_rects(1560, 32760, [0, 1560], [0, 1], [0], [32760])
    assert aj.attn_jvp_split_choose(bf(1560), bf(32760), m, 256) == 3
    # a grid of many tiles per compute unit is never split
    tf = aj.attn_jvp_mask_tf(21, 1560, 3)
    assert aj.attn_jvp_split_choose(bf(65520), bf(65520), tf, 256) == 1
    assert aj.attn_jvp_split_choose(bf(1560), bf(32760), m, 8) == 1
    L = _lib.lib()
    a = _args(m, sp=1 << 26, n_q=1560, n_k=32760)
    out = ctypes.c_int32()
    assert L.attn_jvp_split_choose(ctypes.byref(a), m.handle, 0, ctypes.byref(out)) == \
        _lib.ATTN_JVP_ERR_SHAPE
    assert L.attn_jvp_split_choose(ctypes.byref(a), m.handle, 256, None) == _lib.ATTN_JVP_ERR_NULL
    assert L.attn_jvp_split_choose(ctypes.byref(_args(m, sp=1 << 26, n_q=1560, n_k=32760, D=96)),
                                   m.handle,
                                   256, ctypes.byref(out)) == _lib.ATTN_JVP_ERR_UNSUPPORTED


def test_plain_c_caller(tmp_path):
    """The header compiles as C99 and a C program linked against the library
    exercises the host-side entry points (no GPU needed)."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    src = os.path.join(ROOT, "tests", "c_abi", "host_calls.c")
    exe = str(tmp_path / "host_calls")
    libdir = os.path.dirname(_lib.LIB_PATH)
    r = subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-I",
                        os.path.join(ROOT, "include"), src, "-o", exe, "-L", libdir,
                        "-lattn_jvp", f"-Wl,-rpath,{libdir}"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr


def _workspace_query(a, mask):
    """attn_jvp_fwd_split_workspace: the forward's argument checks and host
    work only (nothing is launched), so placeholder addresses are safe."""
    need = ctypes.c_uint64(0)
    return _lib.lib().attn_jvp_fwd_split_workspace(ctypes.byref(a), mask.handle, 1,
                                                  ctypes.byref(need))


def test_interleaved_views_of_fused_buffers_are_accepted():
    # q, dq, o, d_o as the four slots of one [B, N, 4, H, D] buffer and k, v,
    # dk, dv of another: they interleave row by row but share no byte
    mask = aj.attn_jvp_mask_tf(4, 16, 1)
    N, H, D = 128, 2, 128
    row = 4 * H * D                      # elements per token row of a fused buffer
    qb, kb = 1 << 30, 2 << 30
    slot = H * D * 2                     # bytes of one slot
    kw = dict(q=qb, dq=qb + slot, o=qb + 2 * slot, d_o=qb + 3 * slot,
              k=kb, v=kb + slot, dk=kb + 2 * slot, dv=kb + 3 * slot, lse=3 << 30,
              q_stride_b=N * row, q_stride_n=row, q_stride_h=D,
              k_stride_b=N * row, k_stride_n=row, k_stride_h=D)
    assert _workspace_query(_args(mask, **kw), mask) == _lib.ATTN_JVP_OK
    # shifting o by one element makes it share bytes with dq and d_o
    kw["o"] += 16
    assert _workspace_query(_args(mask, **kw), mask) == _lib.ATTN_JVP_ERR_UNSUPPORTED


def test_output_overlap_check_matches_byte_sets():
    """The library's verdict on an output view o against the input view q
    (same strides, o at an offset) equals brute force over the bytes each
    covers: refused exactly when they share a byte or o covers a byte twice."""
    import numpy as np
    rng = np.random.default_rng(2024)
    D, es = 64, 2
    masks = {}
    seen = {True: 0, False: 0}
    for trial in range(600):
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
        N = int(rng.choice([1, 2, 3, 5, 8]))
        sb = 8 * int(rng.integers(0, 90))
        sn = 8 * int(rng.integers(0, 50))
        sh = 8 * int(rng.integers(8, 40)) if H > 1 else 8 * int(rng.integers(0, 40))
        if N not in masks:
            masks[N] = aj.attn_jvp_mask_dense(N, N)
        q = 1 << 32
        off = 16 * int(rng.integers(-400, 400))

        def covered(base):
            b, n, h = np.meshgrid(np.arange(B), np.arange(N), np.arange(H), indexing="ij")
            start = base + es * (b * sb + n * sn + h * sh)
            return (start.reshape(-1, 1) + np.arange(D * es)).reshape(-1)

        qs, os_ = covered(q), covered(q + off)
        expect = bool(np.intersect1d(qs, os_).size) or len(np.unique(os_)) < len(os_)
        a = _args(masks[N], B=B, H=H, D=D, q=q, o=q + off, dq=None, dk=None, dv=None, d_o=None,
                  k=1 << 40, v=2 << 40, lse=3 << 40, q_stride_b=sb, q_stride_n=sn,
                  q_stride_h=sh, k_stride_b=N * H * D, k_stride_n=H * D, k_stride_h=D)
        st = _workspace_query(a, masks[N])
        assert st == (_lib.ATTN_JVP_ERR_UNSUPPORTED if expect else _lib.ATTN_JVP_OK), \
            (B, N, H, sb, sn, sh, off, st)
        seen[expect] += 1
    assert seen[True] > 50 and seen[False] > 50, seen


def _build_module():
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "_attn_jvp_build", os.path.join(ROOT, "attention_jvp_causal_attn_amd", "csrc", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_m0_invariant_check(tmp_path):
    """The build refuses device code in which compiled instructions (outside
    the kernels' inline-asm copies, which set M0 without a save) name M0 or
    read it implicitly; the kernels as built pass."""
    b = _build_module()
    ok = tmp_path / "ok.s"
    ok.write_text("k:\n\t;;#ASMSTART\n\ts_mov_b32 m0, s4\n\ts_nop 0\n"
                  "\tglobal_load_lds_dwordx4 v1, s[2:3]\n\t;;#ASMEND\n"
                  "\tds_read_b128 v[4:7], v2\n\ts_endpgm\n")
    assert b.check_m0(str(ok)) == 1
    for bad in ("\ts_mov_b32 m0, s5\n", "\ts_add_i32 m0, s38, 0x2000\n",
                "\tglobal_load_lds_dwordx4 v6, s[4:5]\n", "\ts_sendmsg sendmsg(MSG_DEALLOC_VGPRS)\n",
                "\tv_readlane_b32 s0, v1, m0\n"):
        p = tmp_path / "bad.s"
        p.write_text("k:\n" + bad + "\ts_endpgm\n")
        with pytest.raises(RuntimeError):
            b.check_m0(str(p))
    built = [os.path.join(b.BUILD_DIR, os.path.splitext(s)[0] + ".gfx950.s")
             for s in b.M0_ASM_SOURCES]
    for path in built:
        if os.path.exists(path):
            assert b.check_m0(path) > 0
