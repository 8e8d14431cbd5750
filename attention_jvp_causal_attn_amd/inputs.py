"""Seeded synthetic workloads for the attention JVP under teacher-forcing masks.

This module generates inputs only; it holds none of the method's arithmetic, so
both the HIP path's tests/bench and the CPU oracle can be fed from it.

Workloads: synthetic Gaussian tensors at the attention shapes of a causal
Wan2.1-1.3B DiT (12 heads of width 128, 1560 latent tokens per frame), packed
as [clean | noisy] teacher-forcing sequences.  Real activations and the video
data the pages train on are not available; these stand in for them.

Recipe (fixed, so every run and every box sees the same values):
  * layout [B, N, H, D], sequence-major, contiguous;
  * tensor t of workload w (t = 0..5 for Q, K, V, dQ, dK, dV) is drawn with a
    torch CPU generator seeded ``1000 * w + t``: ``torch.randn`` in fp32, times
    the tensor's std, then cast to the workload dtype (bf16 casts round to
    nearest even);
  * the batched workload (w = 4) scales 5 % of the token rows of Q and of K by
    8: for every (b, h), ``round(0.05 * N)`` distinct rows chosen by
    ``torch.randperm`` from generators seeded ``1000 * w + 6`` (Q) and
    ``1000 * w + 7`` (K), drawn in (b, h) order.
"""

from dataclasses import dataclass
from typing import Optional

import torch


@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    B: int
    H: int
    D: int
    dtype: str                 # "f32" or "bf16"
    n_frames: int              # frames per stream (clean and noisy each)
    tokens_per_frame: int
    frames_per_chunk: int      # 1 = frame-wise mask
    qkv_std: float = 1.0
    tangent_std: float = 1.0
    outlier_frac: float = 0.0  # fraction of Q and K rows scaled by outlier_scale
    outlier_scale: float = 1.0

    @property
    def N(self) -> int:
        return 2 * self.n_frames * self.tokens_per_frame

    @property
    def n_units(self) -> int:
        return self.n_frames // self.frames_per_chunk

    @property
    def unit_tokens(self) -> int:
        return self.tokens_per_frame * self.frames_per_chunk

    def describe(self) -> str:
        kind = "frame-wise" if self.frames_per_chunk == 1 else \
            f"chunk-wise ({self.frames_per_chunk} frames per chunk)"
        return (f"{kind} teacher-forcing mask, {self.dtype}, B={self.B} H={self.H} "
                f"D={self.D}, {self.n_frames} clean + {self.n_frames} noisy frames x "
                f"{self.tokens_per_frame} tokens (N={self.N})")


WORKLOADS = {
    1: Workload(1, "tiny-tf-fp32", B=1, H=2, D=64, dtype="f32", n_frames=4,
                tokens_per_frame=16, frames_per_chunk=1, tangent_std=1.0),
    2: Workload(2, "wan1.3b-framewise-65k", B=1, H=12, D=128, dtype="bf16",
                n_frames=21, tokens_per_frame=1560, frames_per_chunk=1,
                tangent_std=0.1),
    3: Workload(3, "wan1.3b-chunkwise-65k", B=1, H=12, D=128, dtype="bf16",
                n_frames=21, tokens_per_frame=1560, frames_per_chunk=3,
                tangent_std=0.1),
    4: Workload(4, "wan1.3b-batched-22k-outliers", B=4, H=12, D=128,
                dtype="bf16", n_frames=7, tokens_per_frame=1560,
                frames_per_chunk=1, tangent_std=0.05, outlier_frac=0.05,
                outlier_scale=8.0),
    5: Workload(5, "wan1.3b-long-103k", B=1, H=16, D=128, dtype="bf16",
                n_frames=33, tokens_per_frame=1560, frames_per_chunk=3,
                tangent_std=0.1),
}

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}
NAMES = ("q", "k", "v", "dq", "dk", "dv")


def _randn(shape, seed, std):
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    x = torch.randn(shape, generator=g, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x


def _scale_rows(x, seed, frac, factor):
    """Scale round(frac * N) distinct token rows of every (b, h) by ``factor``."""
    B, N, H, _ = x.shape
    n_sel = int(round(frac * N))
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    for b in range(B):
        for h in range(H):
            rows = torch.randperm(N, generator=g)[:n_sel]
            x[b, rows, h, :] *= factor
    return x


def make_inputs(w: Workload, device: str = "cpu", seed_base: Optional[int] = None):
    """Q, K, V, dQ, dK, dV of workload ``w`` as a dict of [B, N, H, D] tensors."""
    base = 1000 * w.wid if seed_base is None else seed_base
    shape = (w.B, w.N, w.H, w.D)
    out = {}
    for t, name in enumerate(NAMES):
        std = w.qkv_std if t < 3 else w.tangent_std
        x = _randn(shape, base + t, std)
        if name in ("q", "k") and w.outlier_frac > 0:
            x = _scale_rows(x, base + (6 if name == "q" else 7), w.outlier_frac,
                            w.outlier_scale)
        out[name] = x.to(TORCH_DTYPE[w.dtype]).to(device)
    return out


def make_random(B, N, H, D, dtype="bf16", seed=0, std=1.0, tangent_std=1.0,
                device="cpu"):
    """Generic seeded inputs of any shape (tensor t seeded ``seed + t``)."""
    shape = (B, N, H, D)
    out = {}
    for t, name in enumerate(NAMES):
        x = _randn(shape, seed + t, std if t < 3 else tangent_std)
        out[name] = x.to(TORCH_DTYPE[dtype]).to(device)
    return out
