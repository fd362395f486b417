"""Plain fp64 CPU oracle for the MiniMax-H3 Q/K prologue and packed full attention.

TEST INFRASTRUCTURE.  Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import or run this module.  The product path
(the HIP kernels behind the C ABI and their Python binding) never calls it and
shares no code with it: no kernels, helpers, tables or constants.

What it computes, with the passages it follows (page titles as published):

* Per-head Q/K RMSNorm, epsilon 1e-5, over the 128 channels of one head --
  "MiniMax-H3 WS1/WS2 kernel roadmap" RFC, section 2 ("Omni-Transformer
  fingerprint": Q/K preprocessing), section 5 (work item h3_qk_rmsnorm_d128).
* Three-axis (t, h, w) MM-RoPE, 16 frequencies per axis, theta 10000,
  rotate-half on 96 of the 128 channels, the other 32 passed through -- same
  RFC, section 2 fingerprint rows "Position encoding", "RoPE frequencies",
  "Rotary channels"; section 5 work item h3_mm_rope_3axis_partial; the
  "split-half RoPE" operator named in the H3 Parity Evidence Ledger
  ("Current Runtime Scope" table, H3 DiT backbone row).
* Norm before RoPE, V untouched -- same RFC, section 4 ("H3-specific
  arithmetic rules").
* Full, non-causal, unmasked softmax(Q K^T * scale) V over the whole packed
  document, per head -- same RFC, section 2 ("Attention" row) and section 4
  ("Full attention is non-causal and unmasked over one packed document").

Readings taken where the pages leave a step open:

* Rotated channels are 0..95, pass-through 96..127.  The rotation is a single
  rotate-half over the 96 channels, so channel c (c < 48) pairs with c + 48.
  The 48 angles are laid out axis-major: [t * w_0..15, h * w_0..15, w * w_0..15]
  and the same 48 angles drive both halves.
* Frequencies w_j = 10000 ** (-j / 16), j = 0..15, the same for all three axes
  (16 frequencies per axis over a 32-channel rotary span per axis).
* RMSNorm: y = x / sqrt(mean(x^2) + eps) * gamma, with gamma a [128] weight
  shared by the heads of Q (gamma_q) and of K (gamma_k).
* Everything is evaluated in float64 with no intermediate rounding; the
  attention uses an exact two-pass softmax (subtract the row maximum,
  exponentiate, divide by the row sum).

Pinned by tests/test_oracle_pins.py against closed forms, invariants, brute
force and independent library routines; see that file for the list.
"""
from __future__ import annotations

import numpy as np

HEAD_DIM = 128
ROTARY_DIM = 96          # channels rotated; the remaining 32 pass through
HALF = ROTARY_DIM // 2   # 48: partner offset of the rotate-half pairing
FREQS_PER_AXIS = 16
ROPE_THETA = 10000.0
RMS_EPS = 1e-5


def rope_inverse_frequencies() -> np.ndarray:
    """w_j = theta ** (-2j / 32) = 10000 ** (-j / 16), j = 0..15, float64."""
    j = np.arange(FREQS_PER_AXIS, dtype=np.float64)
    return ROPE_THETA ** (-2.0 * j / (2 * FREQS_PER_AXIS))


def rope_angles(pos: np.ndarray) -> np.ndarray:
    """[L, 48] angles: for axis a in (t, h, w), 16 angles pos_a * w_j, axis-major."""
    pos = np.asarray(pos, dtype=np.float64)
    inv = rope_inverse_frequencies()
    return np.concatenate([pos[:, a:a + 1] * inv[None, :] for a in range(3)], axis=1)


def rms_norm(x: np.ndarray, gamma: np.ndarray, eps: float = RMS_EPS) -> np.ndarray:
    """Per-row RMSNorm over the last axis (one head's 128 channels)."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(gamma, dtype=np.float64)


def rotate_half(u: np.ndarray) -> np.ndarray:
    """(u_a, u_b) -> (-u_b, u_a) on the two halves of the last axis."""
    h = u.shape[-1] // 2
    return np.concatenate([-u[..., h:], u[..., :h]], axis=-1)


def mm_rope(y: np.ndarray, pos: np.ndarray) -> np.ndarray:
    """Partial three-axis MM-RoPE on [L, H, 128] (or [L, 128]) with per-row pos [L, 3]."""
    y = np.asarray(y, dtype=np.float64)
    phi = rope_angles(pos)                                   # [L, 48]
    cos = np.concatenate([np.cos(phi), np.cos(phi)], axis=1)  # [L, 96]
    sin = np.concatenate([np.sin(phi), np.sin(phi)], axis=1)
    if y.ndim == 3:
        cos, sin = cos[:, None, :], sin[:, None, :]
    out = y.copy()
    rot = y[..., :ROTARY_DIM]
    out[..., :ROTARY_DIM] = rot * cos + rotate_half(rot) * sin
    return out


def qk_prologue(q, k, gamma_q, gamma_k, pos, eps: float = RMS_EPS):
    """(RoPE(RMSNorm(q)), RoPE(RMSNorm(k))): norm first, then rotation."""
    return (mm_rope(rms_norm(q, gamma_q, eps), pos),
            mm_rope(rms_norm(k, gamma_k, eps), pos))


def softmax_rows(s: np.ndarray) -> np.ndarray:
    """Exact two-pass softmax along the last axis."""
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def attention_head(qh: np.ndarray, kh: np.ndarray, vh: np.ndarray, scale: float,
                   block: int = 1024) -> np.ndarray:
    """softmax(qh kh^T * scale) vh for one head; qh [Lq, D], kh/vh [L, D]."""
    qh = np.asarray(qh, dtype=np.float64)
    kh = np.asarray(kh, dtype=np.float64)
    vh = np.asarray(vh, dtype=np.float64)
    out = np.empty((qh.shape[0], vh.shape[1]), dtype=np.float64)
    for r0 in range(0, qh.shape[0], block):
        s = (qh[r0:r0 + block] @ kh.T) * scale
        out[r0:r0 + block] = softmax_rows(s) @ vh
    return out


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """Full bidirectional attention over [L, H, D] inputs -> [L, H, D] float64."""
    L, H, D = q.shape
    out = np.empty((L, H, D), dtype=np.float64)
    for h in range(H):
        out[:, h, :] = attention_head(q[:, h, :], k[:, h, :], v[:, h, :], scale)
    return out


def packed_attention(q, k, v, gamma_q, gamma_k, pos, scale: float,
                     eps: float = RMS_EPS) -> np.ndarray:
    """The whole path: Q/K RMSNorm -> MM-RoPE -> attention.  V is used raw."""
    qr, kr = qk_prologue(q, k, gamma_q, gamma_k, pos, eps)
    return attention(qr, kr, v, scale)


def packed_attention_sampled(q, k, v, gamma_q, gamma_k, pos, scale: float,
                             rows: np.ndarray, heads: np.ndarray,
                             k_row_scale: dict | None = None) -> np.ndarray:
    """Output rows o[rows[i], heads[i], :] of the whole path, one by one.

    Each sampled (row, head) needs Q' of that row and K' of every row of that
    head; K' is built per head, so memory stays O(L * D).  q, k, v may be any
    array-like indexable as [L, H, D] (e.g. a lazy bf16 view).
    k_row_scale optionally maps token rows to a factor applied to K' after the
    prologue (the stressed workload's key rows).
    """
    rows = np.asarray(rows)
    heads = np.asarray(heads)
    out = np.empty((len(rows), HEAD_DIM), dtype=np.float64)
    for h in np.unique(heads):
        sel = np.nonzero(heads == h)[0]
        kh = mm_rope(rms_norm(k(h) if callable(k) else k[:, h, :], gamma_k), pos)
        if k_row_scale:
            for r, f in k_row_scale.items():
                kh[r] *= f
        vh = np.asarray(v(h) if callable(v) else v[:, h, :], dtype=np.float64)
        qsrc = q(h) if callable(q) else q[:, h, :]
        qh = mm_rope(rms_norm(np.asarray(qsrc)[rows[sel]], gamma_q), pos[rows[sel]])
        out[sel] = attention_head(qh, kh, vh, scale)
    return out


def attention_bruteforce(q, k, v, scale: float) -> np.ndarray:
    """Scalar-loop attention for tiny inputs: every score, max, exp and sum by hand."""
    import math
    L, H, D = len(q), len(q[0]), len(q[0][0])
    out = [[[0.0] * D for _ in range(H)] for _ in range(L)]
    for h in range(H):
        for i in range(L):
            scores = []
            for j in range(L):
                acc = 0.0
                for c in range(D):
                    acc += float(q[i][h][c]) * float(k[j][h][c])
                scores.append(acc * scale)
            m = max(scores)
            w = [math.exp(s - m) for s in scores]
            tot = sum(w)
            for c in range(D):
                acc = 0.0
                for j in range(L):
                    acc += w[j] * float(v[j][h][c])
                out[i][h][c] = acc / tot
    return np.array(out, dtype=np.float64)
