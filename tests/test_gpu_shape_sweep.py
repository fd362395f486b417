"""GPU parity over seeded random shapes (L up to 6000, H up to 9) and a few
chosen ones: the fused forward (h3attn_kv_prologue + h3attn_forward_log2_qprologue)
and the plain path (h3attn_qk_prologue + h3attn_forward) against the fp64
oracle under the attention gate, and on the smaller shapes the attention
backward against the backward oracle under the gradient gate.

Random (L, H) pairs give grids of every kind the launch can form: one sparse
round in which every full query tile runs as two halves, several rounds with a
last round of partial tiles only, partial and half tiles together, ragged key
tails of every length.  The shapes and inputs are fixed by the seeds below.
"""
import math

import numpy as np
import pytest

import oracle
from gates import attention_ok, gradient_ok
from gpu_util import dev_bf16, dev_inputs, host_f64
from oracle import h3_oracle_backward as ob
from packed_full_attention_amd import (h3attn_attention_backward, h3attn_forward, h3attn_forward_log2_qprologue,
                                       h3attn_forward_lse, h3attn_kv_prologue, h3attn_qk_prologue)
from packed_full_attention_amd import workloads as wl

pytestmark = pytest.mark.gpu
SCALE = 1.0 / math.sqrt(128.0)
Q_SCALE = float(np.float32(SCALE * math.log2(math.e)))

_rng = np.random.default_rng(2026)
SHAPES = ([(int(_rng.integers(1, 6000)), int(_rng.integers(1, 10))) for _ in range(24)]
          + [(5120, 4), (4097, 3), (2816, 9)])


@pytest.mark.parametrize("i", range(len(SHAPES)), ids=[f"L{L}-H{H}" for L, H in SHAPES])
def test_random_shape_parity(i):
    L, H = SHAPES[i]
    print(f"shape sweep {i}: L={L} H={H}", flush=True)
    inp = wl.random_document(L, H, seed=900 + i, pos_max=3000)
    ref = oracle.packed_attention(inp.as_f64("q"), inp.as_f64("k"), inp.as_f64("v"), inp.gamma_q, inp.gamma_k,
                                  inp.pos, SCALE)
    q, k, v, gq, gk, pos = dev_inputs(inp)
    cs, vt = h3attn_kv_prologue(k, v, gk, pos)
    ok, e = attention_ok(host_f64(h3attn_forward_log2_qprologue(q, k, vt, gq, cs, Q_SCALE)), ref)
    assert ok, ("fused", e)

    q, k, v, gq, gk, pos = dev_inputs(inp)
    h3attn_qk_prologue(q, k, gq, gk, pos)
    ok, e = attention_ok(host_f64(h3attn_forward(q, k, v)), ref)
    assert ok, ("plain", e)

    if L * H <= 20000:
        out, lse = h3attn_forward_lse(q, k, v)
        dout = dev_bf16(wl.random_document(L, H, seed=950 + i).q)
        grads = h3attn_attention_backward(q, k, v, out, dout, lse)
        want = ob.attention_backward(host_f64(q), host_f64(k), inp.as_f64("v"), host_f64(dout), SCALE)
        for name, got, w in zip(("dq", "dk", "dv"), grads, want):
            ok, e = gradient_ok(host_f64(got), w)
            assert ok, (name, e)
