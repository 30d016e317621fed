"""Seeded synthetic Q/K/V for dynamic block-sparse attention.

The one module that both the GPU path's tests/bench and the CPU oracle's tests draw
inputs from. It holds none of the method's arithmetic: it only draws random numbers and
rounds them to bf16.

Workloads follow the pages' video-DiT shapes (480p and 720p latents, and the ~120K-token
sequence at which self-attention exceeds 80 % of a DiT pass, per the knowledge card
"600倍加速，720p视频实时生成！单卡也能带的动14B模型", section 事件概述/研究问题). No dataset
is involved; these tensors stand in for a real model's activations.

Recipe (stated as a reading, since the pages give no activation statistics):
  G1  token s <-> grid point (t, h, w) in row-major order over (T, Hg, Wg);
  G2  phi(s) = [sin 2pi t/T, cos 2pi t/T, sin 2pi h/Hg, cos 2pi h/Hg, sin 2pi w/Wg,
      cos 2pi w/Wg];
  G3  one seeded matrix M in R^{6 x D} with N(0, 1/3) entries, shared by Q, K, V and all
      heads, so each smooth entry has unit variance and Q/K block means agree where the
      (t, h, w) phases agree -- the spatial locality that makes block selection useful;
  G4  X = N(0,1) noise (independent per tensor) + alpha * phi(s) M, rounded to bf16
      (round to nearest even). The tiny configuration is pure noise.
  G5  the inputs of the fused RMSNorm + 3D RoPE call are Q and K projections before the
      head split: X_q and X_k of G4 laid out token-major [B, S, H, D] (a linear layer's
      output viewed per head), and RMSNorm weights 1 + 0.1 * N(0, 1) per channel, rounded
      to bf16, from their own seed.
Streams: numpy SeedSequence(seed) spawns 1 + 3*B*H child seeds; child 0 draws M (when a
grid is given), child 1 + t*B*H + (b*H + h) draws the [S, D] noise of tensor t (Q, K, V in
that order) for batch b, head h. The streams are independent of how many threads fill
them, so the bytes depend on the seed only.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CONFIGS = {
    # Tiny dense-checkable case: 16 blocks of 64, keep 4.
    "tiny": dict(B=1, H=2, S=1024, D=64, block=64, keep_ratio=0.25, grid=None, alpha=0.0, seed=1),
    # 480p latent 21x30x52, keep 20 %.
    "480p": dict(B=1, H=40, S=32760, D=128, block=128, keep_ratio=0.20, grid=(21, 30, 52),
                 alpha=0.5, seed=2),
    # 720p latent 21x45x80, keep 15 %.
    "720p": dict(B=1, H=40, S=75600, D=128, block=128, keep_ratio=0.15, grid=(21, 45, 80),
                 alpha=0.5, seed=3),
    # ~120K-token sequence 30x64x64, keep 10 %, locality term scaled 1.0.
    "long": dict(B=1, H=40, S=122880, D=128, block=128, keep_ratio=0.10, grid=(30, 64, 64),
                 alpha=1.0, seed=4),
    # FP8-QK variant on the 720p tensors (same seed); Q and K quantised per 128-token block.
    "fp8": dict(B=1, H=40, S=75600, D=128, block=128, keep_ratio=0.15, grid=(21, 45, 80),
                alpha=0.5, seed=3, fp8=True),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); returns the uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.reshape(-1).view(np.uint32)
    out = np.empty(u.size, dtype=np.uint16)
    step = 1 << 24
    for a in range(0, u.size, step):  # chunked: full-size tensors hold ~10^9 values
        c = u[a:a + step]
        # finite inputs cannot overflow 32 bits here (largest is 0xFF7FFFFF + 0x8000)
        out[a:a + step] = ((c + np.uint32(0x7FFF) + ((c >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    return out.reshape(x.shape)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def smooth_features(grid, S: int) -> np.ndarray:
    """phi(s) for s in [0, S): [S, 6] float64 (G1, G2)."""
    T, Hg, Wg = grid
    if T * Hg * Wg != S:
        raise ValueError("grid %r does not have %d points" % (grid, S))
    s = np.arange(S)
    t, h, w = s // (Hg * Wg), (s // Wg) % Hg, s % Wg
    cols = []
    for c, period in ((t, T), (h, Hg), (w, Wg)):
        a = 2.0 * np.pi * c / period
        cols += [np.sin(a), np.cos(a)]
    return np.stack(cols, axis=1)


def make_qkv(B: int, H: int, S: int, D: int, seed: int, grid=None, alpha: float = 0.0):
    """Seeded bf16 Q, K, V as uint16 bit arrays of shape [B, H, S, D]."""
    children = np.random.SeedSequence(seed).spawn(1 + 3 * B * H)
    smooth = None
    if grid is not None:
        M = np.random.default_rng(children[0]).normal(0.0, np.sqrt(1.0 / 3.0), size=(6, D))
        smooth = (alpha * (smooth_features(grid, S) @ M)).astype(np.float32)  # [S, D]
    out = [np.empty((B, H, S, D), dtype=np.uint16) for _ in range(3)]

    def fill(job):
        t, bh = divmod(job, B * H)
        x = np.random.default_rng(children[1 + job]).standard_normal(size=(S, D), dtype=np.float32)
        if smooth is not None:
            x += smooth
        out[t][bh // H, bh % H] = f32_to_bf16_bits(x)

    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(fill, range(3 * B * H)))
    return tuple(out)


def make_config(name: str, seed=None):
    """(q, k, v, cfg) for one of CONFIGS, optionally with another seed."""
    cfg = dict(CONFIGS[name])
    if seed is not None:
        cfg["seed"] = int(seed)
    q, k, v = make_qkv(cfg["B"], cfg["H"], cfg["S"], cfg["D"], cfg["seed"], cfg["grid"], cfg["alpha"])
    return q, k, v, cfg


def make_projections(B: int, S: int, H: int, D: int, seed: int, grid=None, alpha: float = 0.0):
    """(x_q, x_k): G4's Q and K, token-major uint16 bf16 bits [B, S, H, D] (G5)."""
    q, k, _ = make_qkv(B, H, S, D, seed, grid, alpha)
    return np.ascontiguousarray(q.transpose(0, 2, 1, 3)), np.ascontiguousarray(k.transpose(0, 2, 1, 3))


def make_norm_weight(C: int, seed: int) -> np.ndarray:
    """RMSNorm weights 1 + 0.1 * N(0, 1), bf16 bits [C] (G5)."""
    w = 1.0 + 0.1 * np.random.default_rng(seed).standard_normal(C)
    return f32_to_bf16_bits(w.astype(np.float32))
