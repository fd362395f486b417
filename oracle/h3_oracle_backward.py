"""Plain fp64 CPU oracle for the backward pass of the packed H3 attention path.

TEST INFRASTRUCTURE, like h3_oracle.py: only the test suite, the package smoke
check and the benchmark's CPU-baseline leg may import or run it, and it shares
no code with the HIP path.

Why a backward: the "MiniMax-H3 WS1/WS2 kernel roadmap" RFC, section 7
("Acceptance gates", per-operator gate) requires forward and backward of each
operator to match an independent reference; the operators are its section 5
work items h3_qk_rmsnorm_d128, h3_mm_rope_3axis_partial and h3_full_attention,
whose forward definitions h3_oracle.py writes out.

What it computes: the gradients of a scalar loss with respect to the path's
inputs, given dO = dLoss/dO for the attention output, by the chain rule through
the forward steps in reverse order, every step in float64 with no rounding:

* attention (per head, scores S = scale Q' K'^T, P = softmax rows of S,
  O = P V):  dV = P^T dO;  dP = dO V^T;  delta_i = sum_d dO_id O_id
  (= sum_j P_ij dP_ij);  dS = P * (dP - delta);  dQ' = scale dS K';
  dK' = scale dS^T Q'.
* MM-RoPE (an orthogonal rotation of each channel pair (c, c + 48) by the
  row's angle phi_c, channels 96..127 untouched): the gradient is the inverse
  rotation, dy = cos(phi) dout - rotate_half(sin(phi) dout) on the 96 rotated
  channels and dy = dout on the rest.
* RMSNorm (y = x r gamma, r = (mean(x^2) + eps)^(-1/2) over one head's 128
  channels):  dx = r (gamma dy) - x r^3 mean(gamma dy x);
  dgamma = sum over all rows (every token and head) of dy x r.

Pinned by tests/test_oracle_backward_pins.py against central finite
differences of the forward oracle, an independent autograd library, and
invariants of the definitions.
"""
from __future__ import annotations

import numpy as np

from .h3_oracle import (RMS_EPS, ROTARY_DIM, mm_rope, rms_norm, rope_angles, rotate_half,
                        softmax_rows)


def attention_head_backward(qh, kh, vh, doh, scale: float, block: int = 1024):
    """(dq, dk, dv) of o = softmax(qh kh^T scale) vh for one head, given do."""
    qh, kh, vh, doh = (np.asarray(a, dtype=np.float64) for a in (qh, kh, vh, doh))
    dq = np.empty_like(qh)
    dk = np.zeros_like(kh)
    dv = np.zeros_like(vh)
    for r0 in range(0, qh.shape[0], block):
        qb, dob = qh[r0:r0 + block], doh[r0:r0 + block]
        p = softmax_rows((qb @ kh.T) * scale)
        o = p @ vh
        dv += p.T @ dob
        dp = dob @ vh.T
        delta = np.sum(dob * o, axis=1, keepdims=True)
        ds = p * (dp - delta)
        dq[r0:r0 + block] = (ds @ kh) * scale
        dk += (ds.T @ qb) * scale
    return dq, dk, dv


def attention_backward(q, k, v, do, scale: float):
    """(dq, dk, dv) of full bidirectional attention over [L, H, D] inputs."""
    L, H, D = np.shape(q)
    dq, dk, dv = (np.empty((L, H, D), dtype=np.float64) for _ in range(3))
    for h in range(H):
        dq[:, h], dk[:, h], dv[:, h] = attention_head_backward(q[:, h], k[:, h], v[:, h], do[:, h], scale)
    return dq, dk, dv


def log_sum_exp_rows(q, k, scale: float) -> np.ndarray:
    """[H, L] natural log of sum_j exp(scale q_i . k_j) for every row of every head."""
    L, H, _ = np.shape(q)
    out = np.empty((H, L), dtype=np.float64)
    for h in range(H):
        s = (np.asarray(q[:, h], dtype=np.float64) @ np.asarray(k[:, h], dtype=np.float64).T) * scale
        m = np.max(s, axis=1, keepdims=True)
        out[h] = (m + np.log(np.sum(np.exp(s - m), axis=1, keepdims=True)))[:, 0]
    return out


def mm_rope_backward(dout, pos) -> np.ndarray:
    """Gradient of mm_rope with respect to its input: the inverse rotation."""
    dout = np.asarray(dout, dtype=np.float64)
    phi = rope_angles(pos)
    cos = np.concatenate([np.cos(phi), np.cos(phi)], axis=1)
    sin = np.concatenate([np.sin(phi), np.sin(phi)], axis=1)
    if dout.ndim == 3:
        cos, sin = cos[:, None, :], sin[:, None, :]
    dy = dout.copy()
    d = dout[..., :ROTARY_DIM]
    dy[..., :ROTARY_DIM] = d * cos - rotate_half(d * sin)
    return dy


def rms_norm_backward(x, gamma, dy, eps: float = RMS_EPS):
    """(dx, dgamma) of y = rms_norm(x, gamma); dgamma sums over every row."""
    x = np.asarray(x, dtype=np.float64)
    gamma = np.asarray(gamma, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    g = gamma * dy
    dx = r * g - x * r ** 3 * np.mean(g * x, axis=-1, keepdims=True)
    dgamma = np.sum((dy * x * r).reshape(-1, x.shape[-1]), axis=0)
    return dx, dgamma


def qk_prologue_backward(q, k, gamma_q, gamma_k, pos, dqr, dkr, eps: float = RMS_EPS):
    """(dq, dk, dgamma_q, dgamma_k) given the gradients dqr, dkr of the prologue outputs."""
    dq, dgq = rms_norm_backward(q, gamma_q, mm_rope_backward(dqr, pos), eps)
    dk, dgk = rms_norm_backward(k, gamma_k, mm_rope_backward(dkr, pos), eps)
    return dq, dk, dgq, dgk


def packed_attention_backward(q, k, v, gamma_q, gamma_k, pos, do, scale: float,
                              eps: float = RMS_EPS):
    """Gradients of the whole path (prologue, then attention) given do:
    (dq, dk, dv, dgamma_q, dgamma_k), all float64."""
    qr = mm_rope(rms_norm(q, gamma_q, eps), pos)
    kr = mm_rope(rms_norm(k, gamma_k, eps), pos)
    dqr, dkr, dv = attention_backward(qr, kr, v, do, scale)
    dq, dk, dgq, dgk = qk_prologue_backward(q, k, gamma_q, gamma_k, pos, dqr, dkr, eps)
    return dq, dk, dv, dgq, dgk
