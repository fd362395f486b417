"""Seeded synthetic workloads for packed full attention (inputs only).

This module is the one piece of code that both the fp64 oracle side (tests,
CPU baseline) and the HIP side consume.  It draws random numbers, rounds them
to bfloat16 and lays out the packed text + video + audio positions.  It holds
none of the method's arithmetic: no normalisation, no rotary embedding, no
softmax.  It imports numpy only.

Shapes follow the MiniMax-H3 WS1/WS2 kernel roadmap RFC (section 2,
"Omni-Transformer fingerprint": 56 heads of width 128; "Input, output and
conditioning fingerprint": packed text, video and audio rows in one document,
video tokens compressed 32x spatially and 4x temporally).  The five workloads
below are the packed documents the attention path is measured and checked on;
their video grids are (ceil(frames/4), height/32, width/32).

Position convention (the pages give only the three axes; this is the reading
used throughout): rows are packed text first, then video, then audio.  Text row
i gets (i, i, i); video row (t, h, w) in raster order (t slowest) gets (t, h, w);
audio row t gets (t, 0, 0).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Tuple

import numpy as np

HEAD_DIM = 128


@dataclass(frozen=True)
class Workload:
    """One packed document: heads, text rows, video grid (T, Hg, Wg), audio rows."""

    index: int
    name: str
    heads: int
    n_text: int
    video_grid: Tuple[int, int, int]
    n_audio: int
    # Fraction of K token rows scaled by 8 to stress the softmax range (0 = none).
    k_stress_rows: int = 0

    @property
    def n_video(self) -> int:
        t, h, w = self.video_grid
        return t * h * w

    @property
    def seq_len(self) -> int:
        return self.n_text + self.n_video + self.n_audio

    def describe(self) -> str:
        t, h, w = self.video_grid
        return (f"L={self.seq_len} H={self.heads} D={HEAD_DIM} "
                f"(text {self.n_text} + video {t}x{h}x{w}={self.n_video} "
                f"+ audio {self.n_audio})")


WORKLOADS = (
    # Tiny CPU-checkable document (fp32 draws, rounded to bf16).
    Workload(0, "tiny", 4, 24, (2, 6, 10), 16),
    # 320x192, 22 frames.
    Workload(1, "320x192x22", 56, 64, (6, 6, 10), 88),
    # 512x512, 22 frames, 5% of K token rows (96 of 1920) scaled by 8.
    Workload(2, "512x512x22", 56, 128, (6, 16, 16), 256, k_stress_rows=96),
    # 864x480, 141 frames: the long single-GPU block shape.
    Workload(3, "864x480x141", 56, 256, (36, 15, 27), 1664),
    # One GPU's 7-head share of the 56 heads at 1280x704, 121 frames.
    Workload(4, "1280x704x121-h7", 7, 256, (31, 22, 40), 1440),
)


def packed_positions(n_text: int, video_grid: Tuple[int, int, int],
                     n_audio: int) -> np.ndarray:
    """int32 [L, 3] (t, h, w) positions of a packed text+video+audio document."""
    t, h, w = video_grid
    text = np.repeat(np.arange(n_text, dtype=np.int32)[:, None], 3, axis=1)
    tt, hh, ww = np.meshgrid(np.arange(t, dtype=np.int32),
                             np.arange(h, dtype=np.int32),
                             np.arange(w, dtype=np.int32), indexing="ij")
    video = np.stack([tt.ravel(), hh.ravel(), ww.ravel()], axis=1)
    audio = np.zeros((n_audio, 3), dtype=np.int32)
    audio[:, 0] = np.arange(n_audio, dtype=np.int32)
    return np.ascontiguousarray(np.concatenate([text, video, audio], axis=0))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest even) -> uint16 bit patterns.

    NaN stays NaN (quiet); finite values round by the usual carry on bit 16.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    nan = np.isnan(x)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    if nan.any():
        out[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 array holding the bf16-rounded values of x."""
    return bf16_bits_to_f32(bf16_bits(x))


@dataclass
class Inputs:
    """Host copies of one workload's inputs.

    q, k, v: uint16 bf16 bit patterns, [L, H, 128], token-major.
    gamma_q, gamma_k: float32 [128] holding bf16-representable values.
    pos: int32 [L, 3] (t, h, w).
    stress_rows: sorted int64 token rows whose K is scaled by 8 (may be empty).
    """

    workload: Workload
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    gamma_q: np.ndarray
    gamma_k: np.ndarray
    pos: np.ndarray
    stress_rows: np.ndarray

    def as_f64(self, name: str) -> np.ndarray:
        return bf16_bits_to_f32(getattr(self, name)).astype(np.float64)


def _draw_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    return bf16_bits(rng.standard_normal(shape, dtype=np.float32))


def make_inputs(workload: Workload | int, seed: Optional[int] = None,
                heads: Optional[int] = None) -> Inputs:
    """Draw one workload's inputs from numpy's PCG64 with seed 1000 + index.

    Draw order: q, k, v (each standard normal float32 [L, H, 128]), then
    gamma_q and gamma_k (1 + 0.1 * standard normal [128]), then, for the
    stressed workload, the K rows to scale.  Every value is rounded to bf16.
    `heads` overrides the head count (for small parity cases on a big L).
    """
    if isinstance(workload, int):
        workload = WORKLOADS[workload]
    if seed is None:
        seed = 1000 + workload.index
    rng = np.random.default_rng(seed)
    H = workload.heads if heads is None else heads
    L = workload.seq_len
    shape = (L, H, HEAD_DIM)
    q = _draw_bf16(rng, shape)
    k = _draw_bf16(rng, shape)
    v = _draw_bf16(rng, shape)
    gq = round_to_bf16(1.0 + 0.1 * rng.standard_normal(HEAD_DIM, dtype=np.float32))
    gk = round_to_bf16(1.0 + 0.1 * rng.standard_normal(HEAD_DIM, dtype=np.float32))
    if workload.k_stress_rows:
        rows = np.sort(rng.choice(L, workload.k_stress_rows, replace=False)).astype(np.int64)
    else:
        rows = np.zeros(0, dtype=np.int64)
    pos = packed_positions(workload.n_text, workload.video_grid, workload.n_audio)
    return Inputs(workload, q, k, v, gq, gk, pos, rows)


def random_document(L: int, H: int, seed: int, *, pos_max: int = 64) -> Inputs:
    """A free-form document of L rows and H heads for edge-case tests.

    Positions are drawn uniformly in [0, pos_max) per axis.
    """
    rng = np.random.default_rng(seed)
    shape = (L, H, HEAD_DIM)
    q = _draw_bf16(rng, shape)
    k = _draw_bf16(rng, shape)
    v = _draw_bf16(rng, shape)
    gq = round_to_bf16(1.0 + 0.1 * rng.standard_normal(HEAD_DIM, dtype=np.float32))
    gk = round_to_bf16(1.0 + 0.1 * rng.standard_normal(HEAD_DIM, dtype=np.float32))
    pos = rng.integers(0, pos_max, size=(L, 3), dtype=np.int32)
    wl = Workload(-1, f"random-L{L}-H{H}", H, L, (0, 0, 0), 0)
    return Inputs(wl, q, k, v, gq, gk, np.ascontiguousarray(pos),
                  np.zeros(0, dtype=np.int64))


def scale_rows_bf16(bits: np.ndarray, rows: np.ndarray, factor_log2: int) -> np.ndarray:
    """Multiply the given token rows of a bf16 [L, H, D] array by 2**factor_log2.

    A power-of-two scale is exact in bf16 for normal values away from overflow;
    the result is produced by widening, scaling in float32 and re-rounding, so
    it is exact whenever the product is representable.
    """
    out = bits.copy()
    if len(rows):
        f = bf16_bits_to_f32(out[rows]) * np.float32(2.0 ** factor_log2)
        out[rows] = bf16_bits(f)
    return out


def with_tiny_norm_rows(inp: Inputs, every: int = 3, factor_log2: int = -10) -> Inputs:
    """The same document with every `every`-th token row of q and k (all heads,
    rows 0, every, 2 every, ...) multiplied by 2**factor_log2 (exact in bf16).

    At 2**-10 an N(0, 1) row has mean(x^2) ~ 1e-6, below the RMSNorm epsilon
    of 1e-5, so these rows make the epsilon (its value and where it enters)
    visible in the prologue's output; on N(0, 1) rows it changes the result by
    far less than a bf16 rounding.
    """
    rows = np.arange(0, inp.workload.seq_len, every, dtype=np.int64)
    return Inputs(inp.workload, scale_rows_bf16(inp.q, rows, factor_log2), scale_rows_bf16(inp.k, rows, factor_log2),
                  inp.v, inp.gamma_q, inp.gamma_k, inp.pos, inp.stress_rows)
