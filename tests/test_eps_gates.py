"""The RMSNorm epsilon is visible to the parity gates on tiny-norm rows.

The GPU eps tests (test_gpu_eps.py) feed every third token row of q and k scaled
by 2^-10, where mean(x^2) ~ 1e-6 is below the epsilon of 1e-5 ("MiniMax-H3
WS1/WS2 kernel roadmap" RFC, section 2 fingerprint: per-head RMSNorm, epsilon
1e-5).  Here, on the CPU and on exactly those inputs, two plausible slips are
planted in copies of the oracle's RMSNorm -- epsilon 1e-6, and epsilon added
outside the square root -- and every comparison those GPU tests make must
reject them: the prologue gate on Q' and K' (also Q' times the softmax-scale
factor of the scale-folded path), the attention gate on the whole path's
output, and the gradient gates on the prologue backward.
"""
import math

import numpy as np
import pytest

import oracle
from gates import attention_ok, dgamma_ok, gradient_ok, prologue_ok
from packed_full_attention_amd import workloads as wl

SCALE = 1.0 / math.sqrt(128.0)
Q_SCALE = float(np.float32(SCALE * math.log2(math.e)))


def norm_eps_small(x, gamma):
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + 1e-6) * gamma


def norm_eps_outside(x, gamma):
    x = np.asarray(x, np.float64)
    return x / (np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) + 1e-5) * gamma


MUTANTS = {"eps 1e-6": norm_eps_small, "eps outside the root": norm_eps_outside}


def norm_backward_eps_small(x, gamma, dy):
    # The chain rule of y = x r gamma with r = (mean(x^2) + 1e-6)^(-1/2).
    x = np.asarray(x, np.float64)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + 1e-6)
    g = gamma * dy
    dx = r * g - x * r ** 3 * np.mean(g * x, axis=-1, keepdims=True)
    dgamma = (dy * x * r).reshape(-1, x.shape[-1]).sum(axis=0)
    return dx, dgamma


@pytest.fixture(scope="module", params=[0, 1])
def case(request):
    inp = wl.with_tiny_norm_rows(wl.make_inputs(request.param))
    q, k, v = inp.as_f64("q"), inp.as_f64("k"), inp.as_f64("v")
    return inp, q, k, v


def test_tiny_norm_rows_are_below_eps(case):
    inp, q, _, _ = case
    ms = np.mean(q[::3] ** 2, axis=-1)
    assert np.all(ms < 1e-5) and np.all(np.mean(q[1::3] ** 2, axis=-1) > 0.3)


@pytest.mark.parametrize("mutant", list(MUTANTS))
def test_prologue_gate_rejects_eps_slips(case, mutant):
    inp, q, k, _ = case
    norm = MUTANTS[mutant]
    rq, rk = oracle.qk_prologue(q, k, inp.gamma_q, inp.gamma_k, inp.pos)
    bq = oracle.mm_rope(norm(q, inp.gamma_q), inp.pos)
    bk = oracle.mm_rope(norm(k, inp.gamma_k), inp.pos)
    for name, bad, ref in (("q", bq, rq), ("k", bk, rk), ("scaled q", bq * Q_SCALE, rq * Q_SCALE)):
        ok, e = prologue_ok(bad, ref)
        assert not ok, (mutant, name, e)
    # The gate still accepts the correct values rounded to bf16.
    assert prologue_ok(wl.round_to_bf16(rq.astype(np.float32)), rq)[0]


@pytest.mark.parametrize("mutant", list(MUTANTS))
def test_attention_gate_rejects_eps_slips(case, mutant):
    inp, q, k, v = case
    norm = MUTANTS[mutant]
    ref = oracle.packed_attention(q, k, v, inp.gamma_q, inp.gamma_k, inp.pos, SCALE)
    bq = oracle.mm_rope(norm(q, inp.gamma_q), inp.pos)
    bk = oracle.mm_rope(norm(k, inp.gamma_k), inp.pos)
    ok, e = attention_ok(oracle.attention(bq, bk, v, SCALE), ref)
    assert not ok, (mutant, e)
    assert e["max_abs"] > 4 * 2e-2, e  # a wide margin, not a borderline miss


def test_gradient_gates_reject_eps_slip(case):
    inp, q, k, _ = case
    rng = np.random.default_rng(17)
    dqr = wl.bf16_bits_to_f32(wl.bf16_bits(rng.standard_normal(q.shape).astype(np.float32))).astype(np.float64)
    dkr = wl.bf16_bits_to_f32(wl.bf16_bits(rng.standard_normal(k.shape).astype(np.float32))).astype(np.float64)
    import oracle.h3_oracle_backward as ob
    dq, dk, dgq, dgk = ob.qk_prologue_backward(q, k, inp.gamma_q, inp.gamma_k, inp.pos, dqr, dkr)
    bdq, bdgq = norm_backward_eps_small(q, inp.gamma_q, ob.mm_rope_backward(dqr, inp.pos))
    bdk, bdgk = norm_backward_eps_small(k, inp.gamma_k, ob.mm_rope_backward(dkr, inp.pos))
    for name, bad, ref in (("dq", bdq, dq), ("dk", bdk, dk)):
        ok, e = gradient_ok(bad, ref)
        assert not ok, (name, e)
    for name, bad, ref in (("dgamma_q", bdgq, dgq), ("dgamma_k", bdgk, dgk)):
        ok, e = dgamma_ok(bad, ref)
        assert not ok, (name, e)


def test_planted_backward_matches_oracle_at_the_right_eps(case):
    # The copy used above is the oracle's backward when its epsilon is right.
    inp, q, _, _ = case
    import oracle.h3_oracle_backward as ob
    dy = np.random.default_rng(3).standard_normal(q.shape)
    r = 1.0 / np.sqrt(np.mean(q * q, axis=-1, keepdims=True) + 1e-5)
    g = inp.gamma_q * dy
    dx = r * g - q * r ** 3 * np.mean(g * q, axis=-1, keepdims=True)
    want, _ = ob.rms_norm_backward(q, inp.gamma_q, dy)
    assert np.allclose(dx, want, rtol=1e-12, atol=1e-12 * np.abs(want).max())
