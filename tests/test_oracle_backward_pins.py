"""Pins for the fp64 backward oracle (oracle/h3_oracle_backward.py).

Each test fixes the backward oracle to something other than itself:

* central finite differences of the forward oracle (h3_oracle.py, itself pinned
  in test_oracle_pins.py) -- per coordinate and along random directions over
  every input at once, so a dropped term, a wrong sign, a transposed operand or
  a missing scale anywhere in the chain rule fails;
* torch float64 autograd through a forward written with torch operations, a
  library that differentiates on its own;
* invariants the definitions fix: the gradients of a softmax row sum to zero,
  so dK' summed over the keys of a head vanishes; the RoPE gradient is a
  rotation (pair norms kept); the RMSNorm gradient has a closed-form component
  along x; uniform attention gives dV = column mean of dO;
* planted mistakes (copies of the backward with one slip each) fail the
  finite-difference gate.
"""
import math

import numpy as np
import pytest
import torch

import oracle

SCALE = 1.0 / math.sqrt(128.0)


def _case(seed, L=6, H=2):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((L, H, 128))
    k = rng.standard_normal((L, H, 128))
    v = rng.standard_normal((L, H, 128))
    gq = 1.0 + 0.1 * rng.standard_normal(128)
    gk = 1.0 + 0.1 * rng.standard_normal(128)
    pos = rng.integers(0, 40, size=(L, 3)).astype(np.int32)
    do = rng.standard_normal((L, H, 128))
    # a few tiny-norm rows, where eps matters in the RMSNorm gradient
    q[1] *= 1e-3
    k[2] *= 1e-3
    return q, k, v, gq, gk, pos, do


def _loss(q, k, v, gq, gk, pos, do):
    return float(np.sum(do * oracle.packed_attention(q, k, v, gq, gk, pos, SCALE)))


def _grads(case, backward=oracle.packed_attention_backward):
    q, k, v, gq, gk, pos, do = case
    return backward(q, k, v, gq, gk, pos, do, SCALE)


def _fd_directional(case, which, direction, h=1e-5):
    """Central difference along direction, Richardson-extrapolated from steps h and
    h/2 (truncation error O(h^4): the tiny-norm rows have large curvature)."""
    def central(step):
        args = list(case)
        base = args[which]
        args[which] = base + step * direction
        lp = _loss(*args)
        args[which] = base - step * direction
        lm = _loss(*args)
        return (lp - lm) / (2 * step)
    return (4.0 * central(h / 2) - central(h)) / 3.0


@pytest.mark.parametrize("which,name", [(0, "q"), (1, "k"), (2, "v"), (3, "gamma_q"), (4, "gamma_k")])
def test_directional_derivatives_match_finite_differences(which, name):
    case = _case(1)
    g = _grads(case)[which]
    rng = np.random.default_rng(100 + which)
    for _ in range(3):
        u = rng.standard_normal(np.shape(case[which]))
        fd = _fd_directional(case, which, u)
        an = float(np.sum(g * u))
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (name, fd, an)


@pytest.mark.parametrize("which", [0, 1, 2])
def test_coordinate_derivatives_match_finite_differences(which):
    case = _case(2)
    g = _grads(case)[which]
    rng = np.random.default_rng(7 + which)
    shape = np.shape(case[which])
    for _ in range(12):
        idx = tuple(int(rng.integers(0, n)) for n in shape)
        e = np.zeros(shape)
        e[idx] = 1.0
        fd = _fd_directional(case, which, e)
        assert abs(fd - g[idx]) <= 1e-7 * max(1.0, abs(g[idx])), (which, idx, fd, g[idx])


def _torch_path(q, k, v, gq, gk, pos):
    """The forward written with torch operations (differentiated by autograd)."""
    j = torch.arange(16, dtype=torch.float64)
    inv = torch.pow(torch.tensor(10000.0, dtype=torch.float64), -j / 16.0)
    phi = torch.cat([pos[:, a:a + 1].double() * inv[None, :] for a in range(3)], dim=1)  # [L, 48]
    cos, sin = torch.cos(phi)[:, None, :], torch.sin(phi)[:, None, :]

    def prologue(x, g):
        y = x * torch.rsqrt(torch.mean(x * x, dim=-1, keepdim=True) + 1e-5) * g
        a, b, rest = y[..., :48], y[..., 48:96], y[..., 96:]
        return torch.cat([a * cos - b * sin, b * cos + a * sin, rest], dim=-1)

    qr, kr = prologue(q, gq), prologue(k, gk)
    s = torch.einsum("ihd,jhd->hij", qr, kr) * SCALE
    return torch.einsum("hij,jhd->ihd", torch.softmax(s, dim=-1), v)


def test_matches_torch_float64_autograd():
    case = _case(3, L=9, H=3)
    q, k, v, gq, gk, pos, do = case
    ts = [torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v, gq, gk)]
    out = _torch_path(*ts, torch.tensor(pos))
    (out * torch.tensor(do)).sum().backward()
    for a, g in zip(ts, _grads(case)):
        np.testing.assert_allclose(g, a.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_key_gradients_sum_to_zero_per_head():
    # dS has zero row sums (softmax gradient), so sum_j dK'_j = scale sum_i q_i sum_j dS_ij = 0.
    rng = np.random.default_rng(4)
    q, k, v, do = (rng.standard_normal((7, 2, 128)) for _ in range(4))
    dq, dk, dv = oracle.attention_backward(q, k, v, do, SCALE)
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-12)
    # and dV summed over keys is the sum of dO over queries (softmax rows sum to 1)
    np.testing.assert_allclose(dv.sum(axis=0), do.sum(axis=0), rtol=1e-12, atol=1e-12)


def test_uniform_attention_closed_forms():
    # q = 0: every row attends uniformly; dV_j = mean_i dO_i for every key j, and
    # dK' = 0 (dS_ij = p (dP_ij - delta_i) is multiplied by q_i = 0).
    rng = np.random.default_rng(5)
    L = 6
    q = np.zeros((L, 1, 128))
    k, v, do = (rng.standard_normal((L, 1, 128)) for _ in range(3))
    dq, dk, dv = oracle.attention_backward(q, k, v, do, SCALE)
    np.testing.assert_allclose(dv, np.broadcast_to(do.mean(axis=0), dv.shape), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(dk, 0.0, atol=0)


def test_rope_backward_is_a_rotation():
    rng = np.random.default_rng(6)
    d = rng.standard_normal((5, 3, 128))
    pos = rng.integers(-50, 50, size=(5, 3))
    dy = oracle.mm_rope_backward(d, pos)
    # pair norms are kept, pass-through channels are copied, and rotating back gives d
    np.testing.assert_allclose(dy[..., :48] ** 2 + dy[..., 48:96] ** 2, d[..., :48] ** 2 + d[..., 48:96] ** 2,
                               rtol=1e-13)
    assert np.array_equal(dy[..., 96:], d[..., 96:])
    np.testing.assert_allclose(oracle.mm_rope(dy, pos), d, rtol=1e-12, atol=1e-13)


def test_rmsnorm_backward_component_along_x():
    # x . dx = r (sum_c gamma_c dy_c x_c) eps / (ms + eps): zero without eps (scale invariance).
    rng = np.random.default_rng(8)
    x = rng.standard_normal((10, 128))
    x[::3] *= 1e-3
    g = 1.0 + 0.1 * rng.standard_normal(128)
    dy = rng.standard_normal((10, 128))
    dx, dg = oracle.rms_norm_backward(x, g, dy)
    ms = np.mean(x * x, axis=1)
    r = 1.0 / np.sqrt(ms + 1e-5)
    expect = r * np.sum(g * dy * x, axis=1) * 1e-5 / (ms + 1e-5)
    np.testing.assert_allclose(np.sum(x * dx, axis=1), expect, rtol=1e-9, atol=1e-15)
    np.testing.assert_allclose(dg, np.sum(dy * x * r[:, None], axis=0), rtol=1e-13)


def test_lse_rows_match_direct_sum():
    rng = np.random.default_rng(9)
    q, k = (rng.standard_normal((5, 2, 128)) for _ in range(2))
    lse = oracle.log_sum_exp_rows(q, k, SCALE)
    for h in range(2):
        for i in range(5):
            direct = math.log(sum(math.exp(SCALE * float(q[i, h] @ k[j, h])) for j in range(5)))
            assert abs(lse[h, i] - direct) < 1e-12


# ---------------------------------------------------------------- planted mistakes

def _mutant(slip):
    def attn_bwd(q, k, v, do, scale):
        L, H, D = q.shape
        dq, dk, dv = (np.empty((L, H, D)) for _ in range(3))
        for h in range(H):
            qh, kh, vh, doh = q[:, h], k[:, h], v[:, h], do[:, h]
            p = oracle.softmax_rows(qh @ kh.T * scale)
            o = p @ vh
            dp = doh @ vh.T
            delta = 0.0 if slip == "no_delta" else np.sum(doh * o, axis=1, keepdims=True)
            ds = p * (dp - delta)
            dv[:, h] = p.T @ doh
            dq[:, h] = ds @ kh * scale
            dk[:, h] = ds.T @ qh * (1.0 if slip == "dk_no_scale" else scale)
        return dq, dk, dv

    def rope_bwd(d, pos):
        if slip == "rope_forward_rotation":
            return oracle.mm_rope(d, pos)
        return oracle.mm_rope_backward(d, pos)

    def norm_bwd(x, g, dy):
        if slip != "norm_no_r3":
            return oracle.rms_norm_backward(x, g, dy)
        r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + 1e-5)
        return r * g * dy, np.sum((dy * x * r).reshape(-1, 128), axis=0)

    def backward(q, k, v, gq, gk, pos, do, scale):
        qr = oracle.mm_rope(oracle.rms_norm(q, gq), pos)
        kr = oracle.mm_rope(oracle.rms_norm(k, gk), pos)
        dqr, dkr, dv = attn_bwd(qr, kr, v, do, scale)
        dq, dgq = norm_bwd(q, gq, rope_bwd(dqr, pos))
        dk, dgk = norm_bwd(k, gk, rope_bwd(dkr, pos))
        return dq, dk, dv, dgq, dgk
    return backward


def test_mutant_harness_without_slip_matches_oracle():
    case = _case(10)
    for a, b in zip(_grads(case, _mutant(None)), _grads(case)):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("slip", ["no_delta", "dk_no_scale", "rope_forward_rotation", "norm_no_r3"])
def test_planted_mistakes_fail_finite_differences(slip):
    case = _case(11)
    grads = _grads(case, _mutant(slip))
    rng = np.random.default_rng(12)
    worst = 0.0
    for which in range(5):
        u = rng.standard_normal(np.shape(case[which]))
        fd = _fd_directional(case, which, u)
        an = float(np.sum(grads[which] * u))
        worst = max(worst, abs(fd - an) / max(1.0, abs(an)))
    assert worst > 1e-3, (slip, worst)
