"""GPU parity of the backward pass (log-sum-exp forward, attention backward,
prologue backward) against the fp64 backward oracle, called through the C ABI.

Gates (tests/gates.py): dq, dk, dv relative L2 <= 1e-2 and max-abs <= 2^-6 of
the tensor's largest magnitude; gamma gradients max-abs <= 1e-3 of theirs; the
log-sum-exp within 2^-9 (a relative 2^-9 error in the row sum of bf16 weights).
Both sides take the same bf16 inputs: the oracle reads the bf16 values the GPU
reads, as float64.  dO is a seeded standard normal rounded to bf16.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import oracle_pool
from gates import dgamma_ok, gradient_ok
from gpu_util import dev_bf16, dev_inputs, host_bits, host_f64
from packed_full_attention_amd import (h3attn_forward_log2, h3attn_forward_log2_lse, h3attn_qk_prologue_backward_scaled,
                                       h3attn_qk_prologue_scaled, h3attn_v_transpose)
from packed_full_attention_amd import (h3attn_attention_backward, h3attn_forward, h3attn_forward_lse,
                                       h3attn_qk_prologue, h3attn_qk_prologue_backward)
from packed_full_attention_amd import workloads as wl

pytestmark = pytest.mark.gpu
SCALE = 1.0 / math.sqrt(128.0)
LSE_TOL = 2.0 ** -9


def _bf16_normal(shape, seed):
    return wl.bf16_bits(np.random.default_rng(seed).standard_normal(shape).astype(np.float32))


def _as_f64(bits):
    return wl.bf16_bits_to_f32(bits).astype(np.float64)


@pytest.fixture(scope="module")
def inputs():
    cache = {}

    def get(i):
        if i not in cache:
            cache[i] = wl.make_inputs(i)
        return cache[i]
    return get


def _prologue_outputs(inp):
    q, k, v, gq, gk, pos = dev_inputs(inp)
    h3attn_qk_prologue(q, k, gq, gk, pos)
    return q, k, v


def _check(name, ok_e):
    ok, e = ok_e
    print(f"{name}: {e}")
    assert ok, (name, e)


# ------------------------------------------------------------------ log-sum-exp forward

@pytest.mark.parametrize("idx", (0, 1, 2))
def test_forward_lse(inputs, idx):
    inp = inputs(idx)
    q, k, v = _prologue_outputs(inp)
    out, lse = h3attn_forward_lse(q, k, v, scale=SCALE)
    plain = h3attn_forward(q, k, v, scale=SCALE)
    torch.cuda.synchronize()
    # the same kernel with and without the extra output: identical bits
    assert torch.equal(out.view(torch.int16), plain.view(torch.int16))
    ref = oracle.log_sum_exp_rows(host_f64(q), host_f64(k), SCALE)
    err = float(np.abs(lse.cpu().numpy().astype(np.float64) - ref).max())
    print(f"lse workload {idx}: max-abs {err:.3e}")
    assert err <= LSE_TOL


# ------------------------------------------------------------------ attention backward

def _attention_case(q, k, v, seed, scale=SCALE):
    """GPU forward (with lse) and backward on device q, k, v; returns the
    device gradients and the bf16 dO bits."""
    L, H, _ = q.shape
    do_bits = _bf16_normal((L, H, 128), seed)
    do = dev_bf16(do_bits)
    out, lse = h3attn_forward_lse(q, k, v, scale=scale)
    dq, dk, dv = h3attn_attention_backward(q, k, v, out, do, lse, scale=scale)
    torch.cuda.synchronize()
    return dq, dk, dv, do_bits


def _compare_attention(tag, q, k, v, grads, do_bits, heads=None, scale=SCALE):
    dq, dk, dv = grads
    qf, kf, vf = host_f64(q), host_f64(k), host_f64(v)
    dof = _as_f64(do_bits)
    gq, gk, gv = host_f64(dq), host_f64(dk), host_f64(dv)
    hs = range(q.shape[1]) if heads is None else heads
    for h in hs:
        rq, rk, rv = oracle.attention_head_backward(qf[:, h], kf[:, h], vf[:, h], dof[:, h], scale)
        for name, got, ref in (("dq", gq[:, h], rq), ("dk", gk[:, h], rk), ("dv", gv[:, h], rv)):
            if heads is not None or h == 0:
                _check(f"{tag} head {h} {name}", gradient_ok(got, ref))
            else:
                assert gradient_ok(got, ref)[0], (tag, h, name, gradient_ok(got, ref)[1])


@pytest.mark.parametrize("idx", (0, 1, 2))
def test_attention_backward_full(inputs, idx):
    inp = inputs(idx)
    q, k, v = _prologue_outputs(inp)
    dq, dk, dv, do_bits = _attention_case(q, k, v, 500 + idx)
    _compare_attention(f"workload {idx}", q, k, v, (dq, dk, dv), do_bits)


@pytest.mark.parametrize("L", [1, 2, 63, 64, 65, 130, 255, 256, 257, 600])
def test_attention_backward_ragged_lengths(L):
    H = 2
    q = dev_bf16(_bf16_normal((L, H, 128), 10 + L))
    k = dev_bf16(_bf16_normal((L, H, 128), 20 + L))
    v = dev_bf16(_bf16_normal((L, H, 128), 30 + L))
    dq, dk, dv, do_bits = _attention_case(q, k, v, 40 + L)
    _compare_attention(f"L={L}", q, k, v, (dq, dk, dv), do_bits)


@pytest.mark.parametrize("scale", [SCALE, math.log(2.0)], ids=["scale_1_over_sqrt128", "scale_ln2"])
def test_attention_backward_very_negative_scores(scale):
    """Query rows whose every score is far below zero (log-sum-exp near -100),
    with keys past L in the last tile (L = 200): the weight those absent keys
    would get, exp(-lse), overflows fp32, so the dq kernel must keep it out of
    dQ.  The keys share a direction u, but each also has a random part as large
    (nearly equal keys would make dQ = scale sum_j dS_j k_j cancel down to the
    bf16 rounding of dS for any kernel).  At scale ln 2 (scale log2(e) = 1, the
    scale-folded layout) the dK/dV kernel starts its score chains from the
    rows' -lse log2(e), which is -inf on the padded rows."""
    L, H = 200, 1
    rng = np.random.default_rng(77)
    u = 1.0 + 0.05 * rng.standard_normal(128)
    k_f = (u[None, :] + rng.standard_normal((L, 128)))[:, None, :]
    q_f = rng.standard_normal((L, H, 128))
    q_f[::7] = -12.0 * (SCALE / scale) * u  # every 7th query row: scores between about -165 and -100
    q = dev_bf16(wl.bf16_bits(q_f.astype(np.float32)))
    k = dev_bf16(wl.bf16_bits(k_f.astype(np.float32)))
    v = dev_bf16(_bf16_normal((L, H, 128), 78))
    dq, dk, dv, do_bits = _attention_case(q, k, v, 79, scale=scale)
    for t in (dq, dk, dv):
        assert bool(torch.isfinite(t.float()).all())
    _compare_attention("very negative scores", q, k, v, (dq, dk, dv), do_bits, scale=scale)


@pytest.mark.parametrize("idx", (0, 1, 2))
def test_attention_backward_unit_scale_full(inputs, idx):
    """The scale-folded layout's backward (q' = c q, scale ln 2, so scale log2(e)
    is exactly 1 in fp32): the dK/dV kernel's unit-scale form, every head against
    the oracle at scale ln 2."""
    inp = inputs(idx)
    q, k, v, gq, gk, pos = dev_inputs(inp)
    h3attn_qk_prologue_scaled(q, k, gq, gk, pos, Q_SCALE)
    dq, dk, dv, do_bits = _attention_case(q, k, v, 700 + idx, scale=math.log(2.0))
    _compare_attention(f"unit scale workload {idx}", q, k, v, (dq, dk, dv), do_bits, scale=math.log(2.0))


@pytest.mark.parametrize("L", [2, 63, 65, 130, 257, 600])
def test_attention_backward_unit_scale_ragged(L):
    H = 2
    q = dev_bf16(_bf16_normal((L, H, 128), 110 + L))
    k = dev_bf16(_bf16_normal((L, H, 128), 120 + L))
    v = dev_bf16(_bf16_normal((L, H, 128), 130 + L))
    dq, dk, dv, do_bits = _attention_case(q, k, v, 140 + L, scale=math.log(2.0) / 8)
    # scale ln 2 / 8 leaves scale log2(e) at 1/8, the general form; ln 2 the unit form
    _compare_attention(f"L={L} scale ln2/8", q, k, v, (dq, dk, dv), do_bits, scale=math.log(2.0) / 8)
    qs = dev_bf16(wl.bf16_bits((host_f64(q) / 8).astype(np.float32)))
    dq, dk, dv, do_bits = _attention_case(qs, k, v, 140 + L, scale=math.log(2.0))
    _compare_attention(f"L={L} scale ln2", qs, k, v, (dq, dk, dv), do_bits, scale=math.log(2.0))


@pytest.mark.parametrize("scale", [math.log(2.0) / 8, math.log(2.0)], ids=["general", "unit"])
def test_attention_backward_single_token(scale):
    """L = 1: the one weight is 1, so dV = dO and dQ = dK = 0 exactly; dS = P (dP -
    delta) is then the fp32 difference of two evaluations of <dO, V> (one on the
    matrix core, one in the vector units), a rounding-level value, so dK and dQ are
    held to an absolute bound instead of the gradient gate's relative one."""
    H = 3
    q = dev_bf16(_bf16_normal((1, H, 128), 150))
    k = dev_bf16(_bf16_normal((1, H, 128), 151))
    v = dev_bf16(_bf16_normal((1, H, 128), 152))
    dq, dk, dv, do_bits = _attention_case(q, k, v, 153, scale=scale)
    assert np.array_equal(host_f64(dv), _as_f64(do_bits))
    for t in (dq, dk):
        assert float(np.abs(host_f64(t)).max()) <= 2.0 ** -14


def _compare_attention_pooled(tag, q, k, v, grads, do_bits, heads):
    """As _compare_attention, with the oracle's heads computed in parallel on the host cores."""
    qf, kf, vf = host_f64(q), host_f64(k), host_f64(v)
    refs = oracle_pool.attention_backward_heads(qf, kf, vf, _as_f64(do_bits), SCALE, heads)
    del qf, kf, vf
    got = [host_f64(t) for t in grads]
    for h in heads:
        for name, g, r in zip(("dq", "dk", "dv"), got, refs[h]):
            _check(f"{tag} head {h} {name}", gradient_ok(g[:, h], r))


def test_attention_backward_long_heads(inputs):
    """L = 16500, H = 56, the whole grid on the GPU; compared in full on one head
    from each run of seven heads (the forward and backward grids give each of
    the 8 XCDs a contiguous run of about seven heads' work) and the last head."""
    inp = inputs(3)
    q, k, v = _prologue_outputs(inp)
    dq, dk, dv, do_bits = _attention_case(q, k, v, 503)
    _compare_attention_pooled("workload 3", q, k, v, (dq, dk, dv), do_bits, heads=list(range(0, 56, 7)) + [55])


def test_attention_backward_stressed(inputs):
    """Workload 2 with its stress applied after the prologue: 96 token rows of K'
    (all heads) times 8 (exact in bf16), which makes a few keys dominate."""
    inp = inputs(2)
    q, k, v = _prologue_outputs(inp)
    k[torch.from_numpy(inp.stress_rows).to(k.device)] *= 8
    dq, dk, dv, do_bits = _attention_case(q, k, v, 520)
    _compare_attention("workload 2 stressed", q, k, v, (dq, dk, dv), do_bits, heads=[0, 29, 55])


def test_attention_backward_longest(inputs):
    """L = 28976, H = 7 (one 8-way head share of the 1280x704 video), every head in full."""
    inp = inputs(4)
    q, k, v = _prologue_outputs(inp)
    dq, dk, dv, do_bits = _attention_case(q, k, v, 504)
    _compare_attention_pooled("workload 4", q, k, v, (dq, dk, dv), do_bits, heads=list(range(7)))


def test_attention_backward_deterministic(inputs):
    inp = inputs(1)
    q, k, v = _prologue_outputs(inp)
    a = _attention_case(q, k, v, 77)[:3]
    b = _attention_case(q, k, v, 77)[:3]
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


# ------------------------------------------------------------------ prologue backward

def _prologue_backward_case(inp, seed):
    q, k, v, gq, gk, pos = dev_inputs(inp)
    L, H = inp.workload.seq_len, inp.workload.heads
    dqr_bits, dkr_bits = _bf16_normal((L, H, 128), seed), _bf16_normal((L, H, 128), seed + 1)
    dq, dk = dev_bf16(dqr_bits), dev_bf16(dkr_bits)
    dgq, dgk = h3attn_qk_prologue_backward(q, k, gq, gk, pos, dq, dk)
    torch.cuda.synchronize()
    return dq, dk, dgq.cpu().numpy(), dgk.cpu().numpy(), dqr_bits, dkr_bits


@pytest.mark.parametrize("idx", (0, 1, 2, 3))
def test_prologue_backward(inputs, idx):
    inp = inputs(idx)
    dq, dk, dgq, dgk, dqr_bits, dkr_bits = _prologue_backward_case(inp, 900 + idx)
    rq, rk, rgq, rgk = oracle.qk_prologue_backward(inp.as_f64("q"), inp.as_f64("k"), inp.gamma_q, inp.gamma_k,
                                                   inp.pos, _as_f64(dqr_bits), _as_f64(dkr_bits))
    _check(f"prologue workload {idx} dq", gradient_ok(host_f64(dq), rq))
    _check(f"prologue workload {idx} dk", gradient_ok(host_f64(dk), rk))
    _check(f"prologue workload {idx} dgamma_q", dgamma_ok(dgq, rgq))
    _check(f"prologue workload {idx} dgamma_k", dgamma_ok(dgk, rgk))


def test_prologue_backward_rows_independent(inputs):
    """Per-row locality: the gradient of one token's rows depends on that token
    only (a bf16 bit check of a token computed alone against the whole grid)."""
    inp = inputs(1)
    dq, dk, *_ = _prologue_backward_case(inp, 950)
    t = 123
    sub = wl.Inputs(workload=inp.workload, q=inp.q[t:t + 1], k=inp.k[t:t + 1], v=inp.v[t:t + 1],
                    gamma_q=inp.gamma_q, gamma_k=inp.gamma_k, pos=inp.pos[t:t + 1],
                    stress_rows=np.zeros(0, dtype=np.int64))
    q1, k1, v1, gq, gk, pos1 = dev_inputs(sub)
    L, H = inp.workload.seq_len, inp.workload.heads
    dqr = dev_bf16(_bf16_normal((L, H, 128), 950)[t:t + 1])
    dkr = dev_bf16(_bf16_normal((L, H, 128), 951)[t:t + 1])
    h3attn_qk_prologue_backward(q1, k1, gq, gk, pos1, dqr, dkr)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(dqr), host_bits(dq)[t:t + 1])
    assert np.array_equal(host_bits(dkr), host_bits(dk)[t:t + 1])


# ------------------------------------------------------------------ whole path

def test_whole_path_backward(inputs):
    """Raw inputs -> prologue -> forward (lse) -> attention backward -> prologue
    backward, against the oracle's gradients of the whole path."""
    inp = inputs(1)
    q, k, v, gq, gk, pos = dev_inputs(inp)
    q_raw, k_raw = q.clone(), k.clone()
    h3attn_qk_prologue(q, k, gq, gk, pos)
    L, H = inp.workload.seq_len, inp.workload.heads
    do_bits = _bf16_normal((L, H, 128), 4242)
    out, lse = h3attn_forward_lse(q, k, v, scale=SCALE)
    dq, dk, dv = h3attn_attention_backward(q, k, v, out, dev_bf16(do_bits), lse, scale=SCALE)
    dgq, dgk = h3attn_qk_prologue_backward(q_raw, k_raw, gq, gk, pos, dq, dk)
    torch.cuda.synchronize()
    rq, rk, rv, rgq, rgk = oracle.packed_attention_backward(inp.as_f64("q"), inp.as_f64("k"), inp.as_f64("v"),
                                                            inp.gamma_q, inp.gamma_k, inp.pos, _as_f64(do_bits),
                                                            SCALE)
    _check("whole path dq", gradient_ok(host_f64(dq), rq))
    _check("whole path dk", gradient_ok(host_f64(dk), rk))
    _check("whole path dv", gradient_ok(host_f64(dv), rv))
    # Here the gamma gradients are sums over the bf16 dq', dk' that the attention
    # backward hands on, so they carry that gradient's error (the fp32-only
    # dgamma gate applies when both sides start from the same dq', dk', as in
    # test_prologue_backward): they take the gradient gate.
    _check("whole path dgamma_q", gradient_ok(dgq.cpu().numpy(), rgq))
    _check("whole path dgamma_k", gradient_ok(dgk.cpu().numpy(), rgk))


# ------------------------------------------------------------------ the scale-folded training step

Q_SCALE = float(np.float32(SCALE * math.log2(math.e)))
LN2 = math.log(2.0)


@pytest.mark.parametrize("idx", (0, 1, 2))
def test_forward_log2_lse(inputs, idx):
    """The log2 kernel's log-sum-exp: ln sum_j 2^<q', k_j> = ln sum_j exp(ln 2 <q', k_j>); out
    is the plain log2 forward's, bit for bit."""
    inp = inputs(idx)
    q, k, v, gq, gk, pos = dev_inputs(inp)
    h3attn_qk_prologue_scaled(q, k, gq, gk, pos, Q_SCALE)
    vt = h3attn_v_transpose(v)
    out, lse = h3attn_forward_log2_lse(q, k, vt)
    plain = h3attn_forward_log2(q, k, vt)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), plain.view(torch.int16))
    ref = oracle.log_sum_exp_rows(host_f64(q), host_f64(k), LN2)
    err = float(np.abs(lse.cpu().numpy().astype(np.float64) - ref).max())
    print(f"log2 lse workload {idx}: max-abs {err:.3e}")
    assert err <= LSE_TOL


def test_prologue_backward_scale_one_is_plain(inputs):
    inp = inputs(1)
    L, H = inp.workload.seq_len, inp.workload.heads
    q, k, _, gq, gk, pos = dev_inputs(inp)
    res = []
    for scaled in (False, True):
        dq, dk = dev_bf16(_bf16_normal((L, H, 128), 60)), dev_bf16(_bf16_normal((L, H, 128), 61))
        if scaled:
            g = h3attn_qk_prologue_backward_scaled(q, k, gq, gk, pos, dq, dk, 1.0)
        else:
            g = h3attn_qk_prologue_backward(q, k, gq, gk, pos, dq, dk)
        torch.cuda.synchronize()
        res.append([host_bits(dq), host_bits(dk), g[0].cpu().numpy(), g[1].cpu().numpy()])
    for a, b in zip(*res):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("idx", (1, 2))
def test_whole_path_backward_scale_folded(inputs, idx):
    """Raw inputs -> scaled prologue (q' = c q) -> log2 forward with lse -> attention
    backward on q' at scale ln 2 -> scaled prologue backward, against the oracle's
    gradients of the plain path at scale 1/sqrt(128)."""
    inp = inputs(idx)
    q, k, v, gq, gk, pos = dev_inputs(inp)
    q_raw, k_raw = q.clone(), k.clone()
    h3attn_qk_prologue_scaled(q, k, gq, gk, pos, Q_SCALE)
    L, H = inp.workload.seq_len, inp.workload.heads
    do_bits = _bf16_normal((L, H, 128), 4343 + idx)
    out, lse = h3attn_forward_log2_lse(q, k, h3attn_v_transpose(v))
    dq, dk, dv = h3attn_attention_backward(q, k, v, out, dev_bf16(do_bits), lse, scale=LN2)
    dgq, dgk = h3attn_qk_prologue_backward_scaled(q_raw, k_raw, gq, gk, pos, dq, dk, Q_SCALE)
    torch.cuda.synchronize()
    rq, rk, rv, rgq, rgk = oracle.packed_attention_backward(inp.as_f64("q"), inp.as_f64("k"), inp.as_f64("v"),
                                                            inp.gamma_q, inp.gamma_k, inp.pos, _as_f64(do_bits),
                                                            SCALE)
    _check(f"scale-folded path {idx} dq", gradient_ok(host_f64(dq), rq))
    _check(f"scale-folded path {idx} dk", gradient_ok(host_f64(dk), rk))
    _check(f"scale-folded path {idx} dv", gradient_ok(host_f64(dv), rv))
    _check(f"scale-folded path {idx} dgamma_q", gradient_ok(dgq.cpu().numpy(), rgq))
    _check(f"scale-folded path {idx} dgamma_k", gradient_ok(dgk.cpu().numpy(), rgk))
