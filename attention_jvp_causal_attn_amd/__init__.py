"""MI355X (gfx950) forward-mode JVP of masked scaled-dot-product attention.

Thin Python binding of ``libattn_jvp.so`` (C ABI in ``include/attn_jvp.h``).
The functions carry the C names and only marshal arguments: every step of the
computation runs in the library's HIP kernels on the GPU.  PyTorch supplies
device memory and the current stream.

    mask = attn_jvp_mask_tf(n_frames=21, tokens_per_frame=1560, frames_per_chunk=3)
    o, d_o, lse = attn_jvp_fwd(q, k, v, dq, dk, dv, mask)   # [B, N, H, D] tensors
"""

import ctypes

import numpy as np

from . import _lib
from ._lib import ATTN_JVP_BF16, ATTN_JVP_F32  # noqa: F401

__all__ = [
    "AttnJvpError", "Mask", "attn_jvp_mask_tf", "attn_jvp_mask_rects", "attn_jvp_mask_dense",
    "attn_jvp_mask_info", "attn_jvp_mask_export", "attn_jvp_mask_schedule", "attn_jvp_mask_free",
    "attn_jvp_mask_block_causal", "attn_jvp_mask_transpose", "attn_jvp_mask_split_schedule",
    "attn_jvp_fwd", "attn_jvp_fwd_split_workspace", "attn_jvp_split_choose",
    "attn_jvp_fwd_split_noalloc", "attn_jvp_bwd", "attn_jvp_tile_shape",
    "attn_jvp_status_str", "attn_jvp_version",
]


class AttnJvpError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {attn_jvp_status_str(status)} (status {status})")


def _check(status, where):
    if status != _lib.ATTN_JVP_OK:
        raise AttnJvpError(status, where)


def attn_jvp_status_str(status):
    return _lib.lib().attn_jvp_status_str(int(status)).decode()


def attn_jvp_version():
    return _lib.lib().attn_jvp_version()


class Mask:
    """Owner of an ``attn_jvp_mask*``; freed with the object (or explicitly)."""

    def __init__(self, handle):
        self._h = ctypes.c_void_p(handle)

    @property
    def handle(self):
        if not self._h.value:
            raise ValueError("mask has been freed")
        return self._h

    def free(self):
        if self._h.value:
            _lib.lib().attn_jvp_mask_free(self._h)
            self._h = ctypes.c_void_p(None)

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass

    def info(self):
        return attn_jvp_mask_info(self)


def _new_mask(fn, *args):
    out = ctypes.c_void_p()
    st = fn(*args, ctypes.byref(out))
    _check(st, fn.__name__)
    return Mask(out.value)


def attn_jvp_mask_tf(n_frames, tokens_per_frame, frames_per_chunk=1):
    """Teacher-forcing mask over [clean | noisy] (see attn_jvp.h)."""
    L = _lib.lib()
    return _new_mask(L.attn_jvp_mask_tf, int(n_frames), int(tokens_per_frame),
                     int(frames_per_chunk))


def _i32arr(x):
    a = np.ascontiguousarray(np.asarray(x, dtype=np.int32))
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def attn_jvp_mask_rects(n_q, n_k, group_q_begin, range_ptr, k_begin, k_end):
    """Query groups with admissible key ranges in CSR form (see attn_jvp.h)."""
    L = _lib.lib()
    gq, gq_p = _i32arr(group_q_begin)
    rp, rp_p = _i32arr(range_ptr)
    kb, kb_p = _i32arr(k_begin)
    ke, ke_p = _i32arr(k_end)
    if len(rp) != len(gq) or len(kb) != len(ke):
        raise ValueError("group_q_begin/range_ptr and k_begin/k_end lengths must match")
    # the C builder reads k_begin/k_end[range_ptr[g] .. range_ptr[g + 1]) (after
    # checking that range_ptr starts at 0 and does not decrease): every pointer
    # must stay inside the arrays given here
    if len(rp) < 1 or np.any(rp < 0) or np.any(rp > len(kb)):
        raise ValueError(f"range_ptr entries must lie in [0, {len(kb)}] (len(k_begin))")
    return _new_mask(L.attn_jvp_mask_rects, int(n_q), int(n_k), len(gq) - 1, gq_p, rp_p,
                     kb_p if len(kb) else None, ke_p if len(ke) else None)


def attn_jvp_mask_block_causal(n_units, unit_tokens):
    """Block-causal (diffusion-forcing) mask over one stream (see attn_jvp.h)."""
    L = _lib.lib()
    return _new_mask(L.attn_jvp_mask_block_causal, int(n_units), int(unit_tokens))


def attn_jvp_mask_dense(n_q, n_k):
    L = _lib.lib()
    return _new_mask(L.attn_jvp_mask_dense, int(n_q), int(n_k))


def attn_jvp_mask_transpose(mask):
    """The mask with key and query roles swapped (see attn_jvp.h)."""
    L = _lib.lib()
    return _new_mask(L.attn_jvp_mask_transpose, mask.handle)


def attn_jvp_mask_info(mask):
    """dict(n_q, n_k, n_groups, n_ranges, n_visible_pairs)."""
    v = [ctypes.c_int32() for _ in range(4)]
    nv = ctypes.c_int64()
    _check(_lib.lib().attn_jvp_mask_info(mask.handle, *[ctypes.byref(x) for x in v],
                                         ctypes.byref(nv)), "attn_jvp_mask_info")
    return dict(n_q=v[0].value, n_k=v[1].value, n_groups=v[2].value, n_ranges=v[3].value,
                n_visible_pairs=nv.value)


def attn_jvp_mask_export(mask):
    """Canonical CSR form: (group_q_begin, range_ptr, k_begin, k_end) int32 arrays."""
    info = attn_jvp_mask_info(mask)
    g, r = info["n_groups"], info["n_ranges"]
    gq = np.zeros(g + 1, np.int32)
    rp = np.zeros(g + 1, np.int32)
    kb = np.zeros(max(r, 1), np.int32)
    ke = np.zeros(max(r, 1), np.int32)
    p = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    _check(_lib.lib().attn_jvp_mask_export(mask.handle, p(gq), p(rp), p(kb), p(ke)),
           "attn_jvp_mask_export")
    return gq, rp, kb[:r], ke[:r]


def attn_jvp_mask_schedule(mask, block_m, block_n):
    """Host copy of the kernels' block schedule for a tile shape (see attn_jvp.h)."""
    L = _lib.lib()
    nt, ne, npart = ctypes.c_int32(), ctypes.c_int64(), ctypes.c_int64()
    _check(L.attn_jvp_mask_schedule(mask.handle, int(block_m), int(block_n), ctypes.byref(nt),
                                    ctypes.byref(ne), ctypes.byref(npart), None, None, None,
                                    None, None), "attn_jvp_mask_schedule")
    words = block_n // 32
    off = np.zeros(nt.value + 1, np.int32)
    order = np.zeros(nt.value, np.int32)
    eb = np.zeros(max(ne.value, 1), np.int32)
    ep = np.zeros(max(ne.value, 1), np.int32)
    bits = np.zeros(max(npart.value * block_m * words, 1), np.uint32)
    p32 = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    _check(L.attn_jvp_mask_schedule(mask.handle, int(block_m), int(block_n), ctypes.byref(nt),
                                    ctypes.byref(ne), ctypes.byref(npart), p32(off), p32(order),
                                    p32(eb), p32(ep),
                                    bits.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32))),
           "attn_jvp_mask_schedule")
    n = ne.value
    return dict(tile_offsets=off, tile_order=order, entry_block=eb[:n], entry_partial=ep[:n],
                partial_bits=bits[:npart.value * block_m * words].reshape(
                    npart.value, block_m, words))


def attn_jvp_mask_free(mask):
    mask.free()


def attn_jvp_tile_shape(dtype, D, tangent=True):
    """(block_m, block_n) of the forward kernel for (dtype, D), with or
    without input tangents (see attn_jvp.h)."""
    bm, bn = ctypes.c_int32(), ctypes.c_int32()
    _check(_lib.lib().attn_jvp_tile_shape(int(dtype), int(D), int(bool(tangent)),
                                          ctypes.byref(bm), ctypes.byref(bn)),
           "attn_jvp_tile_shape")
    return bm.value, bn.value


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return _lib.ATTN_JVP_BF16
    if t.dtype == torch.float32:
        return _lib.ATTN_JVP_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def attn_jvp_fwd(q, k, v, dq, dk, dv, mask, scale=None, o=None, d_o=None, lse=None,
                 stream=None, lse_tangent=False, d_lse=None, max_splits=1, workspace=None):
    """Masked attention O, its tangent dO and the row log-sum-exp, in one pass.

    q, dq: [B, n_q, H, D]; k, v, dk, dv: [B, n_k, H, D] device tensors of one
    dtype (bfloat16 or float32), last dim contiguous; q-side tensors (q, dq
    and the outputs o, d_o) share strides, as do the k-side ones.  Any tangent
    may be None (zero); all three None gives the primal only (then d_o is
    None).  Outputs are allocated when not given.  The call is asynchronous on
    ``stream`` (default: torch's current stream).  Returns (o, d_o, lse) with
    lse [B, H, n_q] fp32, and d_lse (the tangent of lse, same shape) as a
    fourth element when ``lse_tangent`` is set or ``d_lse`` is given.

    max_splits > 1 selects the split-key launch (attn_jvp_fwd_split): long
    key lists are cut into up to max_splits pieces run in parallel and merged;
    its scratch ``workspace`` (a uint8 device tensor) is allocated when not
    given.  max_splits="auto" lets attn_jvp_split_choose pick the count for
    this device.
    """
    import torch
    tangent = dq is not None or dk is not None or dv is not None
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("tensors must be [B, N, H, D]")
    qshape, kshape = q.shape, k.shape
    B, n_q, H, D = qshape
    n_k = kshape[1]
    if kshape != (B, n_k, H, D):
        raise ValueError(f"k has shape {tuple(kshape)}, expected {(B, n_k, H, D)}")
    qdt, qdev = q.dtype, q.device
    for name, t, want in (("k", k, kshape), ("v", v, kshape), ("dq", dq, qshape), ("dk", dk, kshape),
                          ("dv", dv, kshape)):
        if t is None:
            continue
        if t.shape != want:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(want)}")
        if t.dtype != qdt or t.device != qdev:
            raise ValueError(f"{name} differs from q in dtype or device")
    if not q.is_cuda:
        raise ValueError("tensors must live on the GPU")
    code = _dtype_code(q)
    want_dlse = lse_tangent or d_lse is not None
    if want_dlse and not tangent:
        raise ValueError("the tangent of lse needs at least one input tangent")
    qs, ks = q.stride(), k.stride()
    if o is None:
        o = torch.empty_strided(qshape, qs, dtype=qdt, device=qdev)
    if tangent and d_o is None:
        d_o = torch.empty_strided(qshape, qs, dtype=qdt, device=qdev)
    if lse is None:
        lse = torch.empty((B, H, n_q), dtype=torch.float32, device=qdev)
    if want_dlse and d_lse is None:
        d_lse = torch.empty((B, H, n_q), dtype=torch.float32, device=qdev)
    for name, t in (("dq", dq), ("o", o), ("d_o", d_o)):
        if t is not None and (t.shape != qshape or t.stride() != qs or t.dtype != qdt):
            raise ValueError(f"{name} must match q in shape, strides and dtype")
    for name, t in (("v", v), ("dk", dk), ("dv", dv)):
        if t is not None and t.stride() != ks:
            raise ValueError(f"{name} must have the strides of k")
    if qs[3] != 1 or ks[3] != 1:
        raise ValueError("the last dimension must be contiguous")
    for name, t in (("lse", lse), ("d_lse", d_lse)):
        if t is not None and (t.shape != (B, H, n_q) or t.dtype != torch.float32
                              or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous float32 [B, H, n_q] tensor")
    ptr = lambda t: t.data_ptr() if t is not None else None
    a = _lib.AttnJvpArgs(code, B, H, n_q, n_k, D,
                         q.data_ptr(), k.data_ptr(), v.data_ptr(), ptr(dq), ptr(dk), ptr(dv),
                         o.data_ptr(), d_o.data_ptr() if tangent else None, lse.data_ptr(),
                         qs[0], qs[1], qs[2], ks[0], ks[1], ks[2],
                         float(scale) if scale is not None else 0.0, ptr(d_lse))
    if stream is None:
        stream = torch.cuda.current_stream(qdev)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    L = _lib.lib()
    if max_splits == "auto":
        n_cu = torch.cuda.get_device_properties(q.device).multi_processor_count
        chosen = ctypes.c_int32(1)
        _check(L.attn_jvp_split_choose(ctypes.byref(a), mask.handle, n_cu, ctypes.byref(chosen)),
               "attn_jvp_split_choose")
        max_splits = chosen.value
    if max_splits == 1 and workspace is None and torch.cuda.current_device() == qdev.index:
        # the common case: q's device is already current (no device switch)
        _check(L.attn_jvp_fwd(ctypes.byref(a), mask.handle, ctypes.c_void_p(handle)), "attn_jvp_fwd")
        return (o, (d_o if tangent else None), lse, d_lse) if want_dlse else \
            (o, (d_o if tangent else None), lse)
    with torch.cuda.device(qdev):
        if max_splits == 1 and workspace is None:
            st = L.attn_jvp_fwd(ctypes.byref(a), mask.handle, ctypes.c_void_p(handle))
            _check(st, "attn_jvp_fwd")
        else:
            need = ctypes.c_uint64(0)
            _check(L.attn_jvp_fwd_split_workspace(ctypes.byref(a), mask.handle, int(max_splits),
                                                  ctypes.byref(need)),
                   "attn_jvp_fwd_split_workspace")
            if workspace is None:
                workspace = torch.empty(max(int(need.value), 16), dtype=torch.uint8,
                                        device=qdev)
            if not workspace.is_cuda or workspace.device != qdev:
                raise ValueError("workspace must live on the device of q")
            nbytes = workspace.numel() * workspace.element_size()
            st = L.attn_jvp_fwd_split(ctypes.byref(a), mask.handle, int(max_splits),
                                      ctypes.c_void_p(workspace.data_ptr()),
                                      ctypes.c_uint64(nbytes), ctypes.c_void_p(handle))
            _check(st, "attn_jvp_fwd_split")
    if want_dlse:
        return o, (d_o if tangent else None), lse, d_lse
    return o, (d_o if tangent else None), lse


def attn_jvp_fwd_split_noalloc(q, k, v, dq, dk, dv, mask, o, lse, d_o=None, d_lse=None,
                               max_splits=2, scale=None, stream=None):
    """The split-key forward with the library's fixed scratch array in place
    of a workspace (see attn_jvp.h): allocates nothing, so the outputs o, lse
    (and d_o with any tangent, d_lse if wanted) must be given.  The mask's
    schedule for this device and max_splits must be resident (one earlier
    attn_jvp_fwd with the same max_splits makes it so).  Layout rules as for
    attn_jvp_fwd.  Returns (o, d_o, lse), plus d_lse when given."""
    import torch
    tangent = dq is not None or dk is not None or dv is not None
    if not q.is_cuda:
        raise ValueError("tensors must live on the GPU")
    for name, t in (("o", o), ("lse", lse)) + ((("d_o", d_o),) if tangent else ()):
        if t is None:
            raise ValueError(f"{name} must be given: this call allocates nothing")
    B, n_q, H, D = q.shape
    ptr = lambda t: t.data_ptr() if t is not None else None
    a = _lib.AttnJvpArgs(
        dtype=_dtype_code(q), B=B, H=H, n_q=n_q, n_k=k.shape[1], D=D,
        q=ptr(q), k=ptr(k), v=ptr(v), dq=ptr(dq), dk=ptr(dk), dv=ptr(dv),
        o=ptr(o), d_o=ptr(d_o) if tangent else None, lse=ptr(lse),
        q_stride_b=q.stride(0), q_stride_n=q.stride(1), q_stride_h=q.stride(2),
        k_stride_b=k.stride(0), k_stride_n=k.stride(1), k_stride_h=k.stride(2),
        scale=float(scale) if scale is not None else 0.0, d_lse=ptr(d_lse))
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    with torch.cuda.device(q.device):
        st = _lib.lib().attn_jvp_fwd_split_noalloc(ctypes.byref(a), mask.handle, int(max_splits),
                                                   ctypes.c_void_p(handle))
    _check(st, "attn_jvp_fwd_split_noalloc")
    if d_lse is not None:
        return o, (d_o if tangent else None), lse, d_lse
    return o, (d_o if tangent else None), lse


def _shape_args(q, k, tangent):
    """Arguments carrying only the shapes and strides of q and k (for the
    host-only queries: the pointers are placeholders, never dereferenced)."""
    B, n_q, H, D = q.shape
    n_k = k.shape[1]
    es = q.element_size()

    def span(t, rows):  # bytes from the first to past the last element of a view
        return ((B - 1) * abs(t.stride(0)) + (rows - 1) * abs(t.stride(1)) +
                (H - 1) * abs(t.stride(2)) + D) * es
    # placeholders far enough apart that no two of them share a byte
    fake = (max(span(q, n_q), span(k, n_k), B * H * n_q * 4) + 0xfff) & ~0xfff
    return _lib.AttnJvpArgs(
        dtype=_dtype_code(q), B=B, H=H, n_q=n_q, n_k=n_k, D=D,
        q=fake, k=2 * fake, v=3 * fake, dq=4 * fake if tangent else None,
        o=5 * fake, d_o=6 * fake, lse=7 * fake,
        q_stride_b=q.stride(0), q_stride_n=q.stride(1), q_stride_h=q.stride(2),
        k_stride_b=k.stride(0), k_stride_n=k.stride(1), k_stride_h=k.stride(2), scale=0.0)


def attn_jvp_split_choose(q, k, mask, n_cu, tangent=True):
    """The max_splits attn_jvp_split_choose picks for tensors shaped like q
    and k on a device with ``n_cu`` compute units (host-only)."""
    chosen = ctypes.c_int32(0)
    _check(_lib.lib().attn_jvp_split_choose(ctypes.byref(_shape_args(q, k, tangent)), mask.handle,
                                            int(n_cu), ctypes.byref(chosen)),
           "attn_jvp_split_choose")
    return chosen.value


def attn_jvp_fwd_split_workspace(q, k, mask, max_splits, tangent=True):
    """Bytes of workspace attn_jvp_fwd with ``max_splits`` needs for tensors
    shaped like q [B, n_q, H, D] and k [B, n_k, H, D] (host-only query: the
    tensors may live on any device; nothing is launched)."""
    a = _shape_args(q, k, tangent)
    need = ctypes.c_uint64(0)
    _check(_lib.lib().attn_jvp_fwd_split_workspace(ctypes.byref(a), mask.handle, int(max_splits),
                                                   ctypes.byref(need)),
           "attn_jvp_fwd_split_workspace")
    return int(need.value)


def attn_jvp_mask_split_schedule(mask, block_m, block_n, max_splits):
    """Host copy of the unit list of a split-key launch (see the C header):
    dict with unit_offsets, unit_order, unit_tile, unit_part (numpy int32)
    and n_parts."""
    import numpy as np
    L = _lib.lib()
    nu, npart = ctypes.c_int32(), ctypes.c_int32()
    _check(L.attn_jvp_mask_split_schedule(mask.handle, block_m, block_n, max_splits,
                                          ctypes.byref(nu), ctypes.byref(npart),
                                          None, None, None, None),
           "attn_jvp_mask_split_schedule")
    arrs = {"unit_offsets": np.zeros(nu.value + 1, np.int32),
            "unit_order": np.zeros(max(nu.value, 1), np.int32),
            "unit_tile": np.zeros(max(nu.value, 1), np.int32),
            "unit_part": np.zeros(max(nu.value, 1), np.int32)}
    P = lambda x: x.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    _check(L.attn_jvp_mask_split_schedule(mask.handle, block_m, block_n, max_splits,
                                          ctypes.byref(nu), ctypes.byref(npart),
                                          P(arrs["unit_offsets"]), P(arrs["unit_order"]),
                                          P(arrs["unit_tile"]), P(arrs["unit_part"])),
           "attn_jvp_mask_split_schedule")
    out = {k_: v_[:nu.value + 1] if k_ == "unit_offsets" else v_[:nu.value]
           for k_, v_ in arrs.items()}
    out["n_parts"] = npart.value
    return out


def attn_jvp_bwd(q, k, v, o, g_o, lse, mask, scale=None, g_q=None, g_k=None, g_v=None,
                 delta=None, stream=None):
    """Gradients of sum(g_o * O) w.r.t. q, k, v for O = masked attention(q, k, v).

    q, o, g_o: [B, n_q, H, D]; k, v: [B, n_k, H, D] device tensors of one dtype
    (bfloat16 or float32) with the layout rules of attn_jvp_fwd; o and lse are
    the forward's outputs.
    Outputs (allocated when not given): g_q like q, g_k and g_v like k, and
    delta [B, H, n_q] fp32 (the row sums <g_o, o>).  Asynchronous on
    ``stream``.  Returns (g_q, g_k, g_v, delta).
    """
    import torch
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("tensors must be [B, N, H, D]")
    B, n_q, H, D = q.shape
    n_k = k.shape[1]
    for name, t, rows in (("k", k, n_k), ("v", v, n_k), ("o", o, n_q), ("g_o", g_o, n_q)):
        if tuple(t.shape) != (B, rows, H, D):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {(B, rows, H, D)}")
        if t.dtype != q.dtype or t.device != q.device:
            raise ValueError(f"{name} differs from q in dtype or device")
    if not q.is_cuda:
        raise ValueError("tensors must live on the GPU")
    for name, t in (("o", o), ("g_o", g_o)):
        if t.stride() != q.stride():
            raise ValueError(f"{name} must have the strides of q")
    if v.stride() != k.stride():
        raise ValueError("v must have the strides of k")
    if tuple(lse.shape) != (B, H, n_q) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, n_q] tensor")
    code = _dtype_code(q)
    if g_q is None:
        g_q = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
    if g_k is None:
        g_k = torch.empty_strided(k.shape, k.stride(), dtype=k.dtype, device=k.device)
    if g_v is None:
        g_v = torch.empty_strided(k.shape, k.stride(), dtype=k.dtype, device=k.device)
    if delta is None:
        delta = torch.empty((B, H, n_q), dtype=torch.float32, device=q.device)
    if g_q.stride() != q.stride() or g_k.stride() != k.stride() or g_v.stride() != k.stride():
        raise ValueError("g_q must have the strides of q, g_k and g_v those of k")
    ptr = lambda t: t.data_ptr()
    a = _lib.AttnJvpBwdArgs(
        dtype=code, B=B, H=H, n_q=n_q, n_k=n_k, D=D,
        q=ptr(q), k=ptr(k), v=ptr(v), o=ptr(o), g_o=ptr(g_o), lse=ptr(lse),
        g_q=ptr(g_q), g_k=ptr(g_k), g_v=ptr(g_v), delta=ptr(delta),
        q_stride_b=q.stride(0), q_stride_n=q.stride(1), q_stride_h=q.stride(2),
        k_stride_b=k.stride(0), k_stride_n=k.stride(1), k_stride_h=k.stride(2),
        scale=float(scale) if scale is not None else 0.0)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    with torch.cuda.device(q.device):
        st = _lib.lib().attn_jvp_bwd(ctypes.byref(a), mask.handle, ctypes.c_void_p(handle))
    _check(st, "attn_jvp_bwd")
    return g_q, g_k, g_v, delta
