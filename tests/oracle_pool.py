"""The fp64 oracle over every head (and query-row block) of a long workload, on
all of the host's cores.

TEST INFRASTRUCTURE.  Calls only functions of `oracle/` and adds no arithmetic
of its own: tasks run on a thread pool, each task one oracle call on one head
(or on one block of a head's query rows, which the oracle's attention treats
independently), with the BLAS library held to one thread so that the tasks, not
the matrix products, fill the cores.  numpy releases the interpreter lock inside
matrix products and elementwise loops, so the threads run in parallel.
"""
from __future__ import annotations

import contextlib
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle
from oracle import h3_oracle_backward as ob
from packed_full_attention_amd import workloads as wl


def workers() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _one_blas_thread():
    try:
        from threadpoolctl import threadpool_limits
        return threadpool_limits(limits=1, user_api="blas")
    except Exception:  # pragma: no cover
        return contextlib.nullcontext()


def _head(bits: np.ndarray, h: int) -> np.ndarray:
    return wl.bf16_bits_to_f32(np.ascontiguousarray(bits[:, h, :])).astype(np.float64)


def _run(fn, tasks):
    with _one_blas_thread(), ThreadPoolExecutor(workers()) as ex:
        return list(ex.map(fn, tasks))


def packed_attention_full(q_bits, k_bits, v_bits, gamma_q, gamma_k, pos, scale: float, block: int = 512):
    """Every output of the whole path (oracle.rms_norm -> oracle.mm_rope ->
    oracle.attention_head) for bf16 [L, H, 128] q, k, v; returns float64
    (out, q', k'), each [L, H, 128]."""
    L, H, D = q_bits.shape
    qr, kr, vh = [None] * H, [None] * H, [None] * H

    def prologue(h):
        qr[h] = oracle.mm_rope(oracle.rms_norm(_head(q_bits, h), gamma_q), pos)
        kr[h] = oracle.mm_rope(oracle.rms_norm(_head(k_bits, h), gamma_k), pos)
        vh[h] = _head(v_bits, h)

    _run(prologue, range(H))
    out = np.empty((L, H, D), dtype=np.float64)

    def attend(task):
        h, r0 = task
        out[r0:r0 + block, h] = oracle.attention_head(qr[h][r0:r0 + block], kr[h], vh[h], scale)

    _run(attend, [(h, r0) for h in range(H) for r0 in range(0, L, block)])
    return out, np.stack(qr, axis=1), np.stack(kr, axis=1)


def attention_backward_heads(q, k, v, do, scale: float, heads):
    """oracle attention_head_backward for the listed heads of float64 [L, H, 128]
    q, k, v, do; returns {head: (dq, dk, dv)}, each [L, 128]."""
    heads = [int(h) for h in heads]
    res = _run(lambda h: ob.attention_head_backward(q[:, h], k[:, h], v[:, h], do[:, h], scale), heads)
    return dict(zip(heads, res))


def packed_attention_fp8_full(q_bits, k_bits, v_bits, gamma_q, gamma_k, pos, q_scale: float, heads=None,
                              exact_scale=None, block: int = 512):
    """The quantized-score path (oracle.rms_norm -> oracle.mm_rope ->
    oracle.quantized_operands -> oracle.quantized_attention_head) for the listed
    heads (all by default) of bf16 [L, H, 128] q, k, v.  Returns float64
    (out_fp8, k', out_exact): [L, n_heads, 128] each; out_exact (the exact path's
    oracle.attention_head at `exact_scale`) is None unless exact_scale is given."""
    L, H, D = q_bits.shape
    heads = list(range(H)) if heads is None else [int(h) for h in heads]
    n = len(heads)
    qr, kr, q8, k8, vh = [None] * n, [None] * n, [None] * n, [None] * n, [None] * n

    def prologue(i):
        h = heads[i]
        qr[i] = oracle.mm_rope(oracle.rms_norm(_head(q_bits, h), gamma_q), pos)
        kr[i] = oracle.mm_rope(oracle.rms_norm(_head(k_bits, h), gamma_k), pos)
        q8[i], k8[i] = oracle.quantized_operands(qr[i], kr[i], q_scale)
        vh[i] = _head(v_bits, h)

    _run(prologue, range(n))
    out = np.empty((L, n, D), dtype=np.float64)
    exact = None if exact_scale is None else np.empty((L, n, D), dtype=np.float64)

    def attend(task):
        i, r0 = task
        out[r0:r0 + block, i] = oracle.quantized_attention_head(q8[i][r0:r0 + block], k8[i], vh[i])
        if exact is not None:
            exact[r0:r0 + block, i] = oracle.attention_head(qr[i][r0:r0 + block], kr[i], vh[i], exact_scale)

    _run(attend, [(i, r0) for i in range(n) for r0 in range(0, L, block)])
    return out, np.stack(kr, axis=1), exact
