"""Pins for the fp64 oracle: closed forms, invariants, brute force, library cross-checks.

Each test fixes the oracle to something other than itself: a value the
mathematics or the definition fixes (closed forms, textbook constants), an
invariant of the method, an independent formulation written here from the
definition, or an independent library routine (torch CPU float64).  The
pins are chosen so that a plausible slip in the oracle (a dropped term, a
wrong sign or index, a transposed operand, a wrong frequency exponent, a wrong
pairing) fails at least one of them.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from packed_full_attention_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
SCALE = 1.0 / math.sqrt(128.0)


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- RMSNorm

def test_rmsnorm_constant_row_closed_form():
    g = 1.0 + 0.1 * _rng(1).standard_normal(128)
    for c in (3.0, -0.5, 1e-3, 1e-4):
        x = np.full(128, c)
        y = oracle.rms_norm(x, g)
        expect = c / math.sqrt(c * c + 1e-5) * g
        np.testing.assert_allclose(y, expect, rtol=1e-14, atol=0)


def test_rmsnorm_zero_row_is_zero():
    y = oracle.rms_norm(np.zeros((3, 128)), np.ones(128))
    assert np.all(y == 0.0)


def test_rmsnorm_mean_square_identity_and_eps_visible():
    # mean((y/g)^2) = ms / (ms + eps); tiny-norm rows make eps matter.
    rng = _rng(2)
    x = rng.standard_normal((64, 128))
    x[::4] *= 1e-3
    g = 1.0 + 0.1 * rng.standard_normal(128)
    y = oracle.rms_norm(x, g)
    ms = np.mean(x * x, axis=1)
    np.testing.assert_allclose(np.mean((y / g) ** 2, axis=1), ms / (ms + 1e-5), rtol=1e-12)
    # eps is not negligible on the tiny rows: dropping it changes them by > 10 %.
    y_noeps = x / np.sqrt(ms)[:, None] * g
    assert np.max(np.abs(y[::4] - y_noeps[::4]) / np.abs(y_noeps[::4]).max()) > 0.1


def test_rmsnorm_matches_torch_float64():
    rng = _rng(3)
    x = rng.standard_normal((5, 7, 128))
    x[1] *= 1e-3
    g = 1.0 + 0.1 * rng.standard_normal(128)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (128,), weight=torch.from_numpy(g),
                                       eps=1e-5).numpy()
    np.testing.assert_allclose(oracle.rms_norm(x, g), ref, rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------- MM-RoPE

def test_rope_frequencies_closed_form():
    w = oracle.rope_inverse_frequencies()
    assert w.shape == (16,)
    # 10000 ** (-j/16): j=0 -> 1, 4 -> 0.1, 8 -> 0.01, 12 -> 0.001
    np.testing.assert_allclose(w[[0, 4, 8, 12]], [1.0, 0.1, 0.01, 0.001], rtol=1e-15)
    np.testing.assert_allclose(w[1:] / w[:-1], np.full(15, 10.0 ** -0.25), rtol=1e-14)


def _golden_rows():
    rows = []
    with open(os.path.join(GOLDEN, "rope_unit_rotations.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            a, j, p, ang, c, s = line.split()
            rows.append(("thw".index(a), int(j), int(p), float(c), float(s)))
    return rows


@pytest.mark.parametrize("row", _golden_rows())
def test_rope_unit_vector_golden(row):
    axis, j, p, c_ref, s_ref = row
    ch = 16 * axis + j
    pos = np.zeros((1, 3), dtype=np.int32)
    pos[0, axis] = p
    e = np.zeros((1, 128))
    e[0, ch] = 1.0
    out = oracle.mm_rope(e, pos)[0]
    assert abs(out[ch] - c_ref) < 1e-12 and abs(out[ch + 48] - s_ref) < 1e-12
    others = np.delete(out, [ch, ch + 48])
    assert np.all(others == 0.0)
    e2 = np.zeros((1, 128))
    e2[0, ch + 48] = 1.0
    out2 = oracle.mm_rope(e2, pos)[0]
    assert abs(out2[ch] + s_ref) < 1e-12 and abs(out2[ch + 48] - c_ref) < 1e-12


def test_rope_preserves_pair_and_row_norms():
    rng = _rng(4)
    y = rng.standard_normal((40, 3, 128))
    pos = rng.integers(0, 2000, size=(40, 3)).astype(np.int32)
    out = oracle.mm_rope(y, pos)
    pair_in = y[..., :48] ** 2 + y[..., 48:96] ** 2
    pair_out = out[..., :48] ** 2 + out[..., 48:96] ** 2
    np.testing.assert_allclose(pair_out, pair_in, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(np.linalg.norm(out, axis=-1), np.linalg.norm(y, axis=-1), rtol=1e-13)


def test_rope_passthrough_bit_identical():
    rng = _rng(5)
    y = rng.standard_normal((30, 2, 128))
    pos = rng.integers(0, 500, size=(30, 3)).astype(np.int32)
    out = oracle.mm_rope(y, pos)
    assert np.array_equal(out[..., 96:], y[..., 96:])


def test_rope_origin_is_identity():
    y = _rng(6).standard_normal((4, 5, 128))
    out = oracle.mm_rope(y, np.zeros((4, 3), dtype=np.int32))
    assert np.array_equal(out, y)


def test_rope_complex_formulation():
    # z_c = y_c + i y_{c+48} turns into z_c * exp(i phi_c): written independently here.
    rng = _rng(7)
    y = rng.standard_normal((25, 128))
    pos = rng.integers(0, 3000, size=(25, 3)).astype(np.int32)
    freq = np.array([10000.0 ** (-k / 16.0) for k in range(16)])
    phi = np.empty((25, 48))
    for c in range(48):
        phi[:, c] = pos[:, c // 16] * freq[c % 16]
    z = (y[:, :48] + 1j * y[:, 48:96]) * np.exp(1j * phi)
    out = oracle.mm_rope(y, pos)
    np.testing.assert_allclose(out[:, :48], z.real, rtol=0, atol=1e-12)
    np.testing.assert_allclose(out[:, 48:96], z.imag, rtol=0, atol=1e-12)


def test_rope_axis_reduces_to_textbook_1d_rope():
    # A row at (t, 0, 0) only rotates its t block.  Collect that block's 32 channels
    # (0..15 and 48..63) into one vector: textbook rotate-half RoPE of width 32,
    # theta 10000, inv_freq = theta ** (-arange(0, 32, 2) / 32).
    rng = _rng(8)
    y = rng.standard_normal((6, 128))
    t = np.array([0, 1, 7, 100, 999, 1663])
    pos = np.zeros((6, 3), dtype=np.int32)
    pos[:, 0] = t
    out = oracle.mm_rope(y, pos)
    u = np.concatenate([y[:, 0:16], y[:, 48:64]], axis=1)
    inv = 10000.0 ** (-np.arange(0, 32, 2) / 32.0)
    ang = np.outer(t, inv)
    emb = np.concatenate([ang, ang], axis=1)
    rot = np.concatenate([-u[:, 16:], u[:, :16]], axis=1)
    u_ref = u * np.cos(emb) + rot * np.sin(emb)
    np.testing.assert_allclose(np.concatenate([out[:, 0:16], out[:, 48:64]], axis=1), u_ref,
                               rtol=0, atol=1e-12)
    untouched = [c for c in range(128) if not (c < 16 or 48 <= c < 64)]
    assert np.array_equal(out[:, untouched], y[:, untouched])


def test_rope_relative_position_identity():
    # <R(p) q, R(p') k> = <q, R(p' - p) k>
    rng = _rng(9)
    q = rng.standard_normal((20, 128))
    k = rng.standard_normal((20, 128))
    p = rng.integers(0, 1000, size=(20, 3)).astype(np.int32)
    p2 = rng.integers(0, 1000, size=(20, 3)).astype(np.int32)
    lhs = np.sum(oracle.mm_rope(q, p) * oracle.mm_rope(k, p2), axis=1)
    rhs = np.sum(q * oracle.mm_rope(k, p2 - p), axis=1)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-11, atol=1e-10)


# ---------------------------------------------------------------- softmax / attention

def test_softmax_rows_sum_to_one_and_shift_invariant():
    s = _rng(10).standard_normal((30, 50)) * 20
    p = oracle.softmax_rows(s)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.all(p >= 0)
    np.testing.assert_allclose(oracle.softmax_rows(s + 123.25), p, rtol=1e-12, atol=1e-15)


def test_attention_matches_bruteforce_tiny():
    rng = _rng(11)
    for L, H in ((1, 1), (2, 2), (7, 1), (5, 3)):
        q = rng.standard_normal((L, H, 128))
        k = rng.standard_normal((L, H, 128))
        v = rng.standard_normal((L, H, 128))
        ref = oracle.attention_bruteforce(q.tolist(), k.tolist(), v.tolist(), SCALE)
        np.testing.assert_allclose(oracle.attention(q, k, v, SCALE), ref, rtol=1e-12, atol=1e-12)


def test_attention_block_split_equals_unsplit():
    rng = _rng(12)
    q, k, v = (rng.standard_normal((150, 128)) for _ in range(3))
    a = oracle.attention_head(q, k, v, SCALE, block=1024)
    b = oracle.attention_head(q, k, v, SCALE, block=7)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-14)


def test_attention_closed_forms():
    rng = _rng(13)
    L = 33
    k = rng.standard_normal((L, 1, 128))
    v = rng.standard_normal((L, 1, 128))
    # Q = 0: uniform weights -> column mean of V.
    out = oracle.attention(np.zeros((L, 1, 128)), k, v, SCALE)
    np.testing.assert_allclose(out, np.broadcast_to(v.mean(axis=0), out.shape), rtol=0, atol=1e-13)
    # Identical K rows -> mean of V for any Q.
    q = rng.standard_normal((L, 1, 128))
    ksame = np.broadcast_to(k[:1], k.shape).copy()
    out = oracle.attention(q, ksame, v, SCALE)
    np.testing.assert_allclose(out, np.broadcast_to(v.mean(axis=0), out.shape), rtol=0, atol=1e-13)
    # L = 1 -> the single V row.
    out = oracle.attention(q[:1], k[:1], v[:1], SCALE)
    np.testing.assert_allclose(out, v[:1], rtol=0, atol=1e-15)
    # Positive queries and one key of all-large positive entries: its score
    # dominates every row, so each output row is that key's V row.
    kbig = k.copy()
    kbig[5, 0] = 1e3
    out = oracle.attention(np.abs(q), kbig, v, SCALE)
    np.testing.assert_allclose(out[:, 0], np.broadcast_to(v[5, 0], (L, 128)), rtol=0, atol=1e-12)


def test_attention_matches_torch_float64_sdpa():
    rng = _rng(14)
    L, H = 45, 3
    q, k, v = (rng.standard_normal((L, H, 128)) for _ in range(3))
    t = lambda a: torch.from_numpy(a).permute(1, 0, 2).contiguous()  # [H, L, D]
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), scale=SCALE)
    ref = ref.permute(1, 0, 2).numpy()
    np.testing.assert_allclose(oracle.attention(q, k, v, SCALE), ref, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- whole path

def _tiny_inputs(seed=15, L=40, H=2):
    d = wl.random_document(L, H, seed, pos_max=300)
    return (d.as_f64("q"), d.as_f64("k"), d.as_f64("v"), d.gamma_q.astype(np.float64),
            d.gamma_k.astype(np.float64), d.pos)


def test_path_matches_torch_composition():
    # Prologue and attention rebuilt from torch float64 library calls plus the
    # complex-number rotation; shares nothing with the oracle's code.
    q, k, v, gq, gk, pos = _tiny_inputs()
    freq = torch.tensor([10000.0 ** (-j / 16.0) for j in range(16)], dtype=torch.float64)
    p = torch.from_numpy(pos.astype(np.float64))
    phi = torch.cat([p[:, a:a + 1] * freq for a in range(3)], dim=1)  # [L, 48]

    def pro(x, g):
        y = torch.nn.functional.rms_norm(torch.from_numpy(x), (128,), weight=torch.from_numpy(g), eps=1e-5)
        z = torch.complex(y[..., :48], y[..., 48:96]) * torch.polar(torch.ones_like(phi), phi)[:, None, :]
        return torch.cat([z.real, z.imag, y[..., 96:]], dim=-1)

    qr, kr = pro(q, gq), pro(k, gk)
    t = lambda a: a.permute(1, 0, 2).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(t(qr), t(kr), t(torch.from_numpy(v)),
                                                           scale=SCALE).permute(1, 0, 2).numpy()
    out = oracle.packed_attention(q, k, v, gq, gk, pos, SCALE)
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-12)


def test_path_permutation_equivariance():
    q, k, v, gq, gk, pos = _tiny_inputs(16)
    perm = _rng(16).permutation(len(pos))
    out = oracle.packed_attention(q, k, v, gq, gk, pos, SCALE)
    outp = oracle.packed_attention(q[perm], k[perm], v[perm], gq, gk, pos[perm], SCALE)
    np.testing.assert_allclose(outp, out[perm], rtol=1e-12, atol=1e-13)


def test_path_head_independence():
    q, k, v, gq, gk, pos = _tiny_inputs(17, H=3)
    out = oracle.packed_attention(q, k, v, gq, gk, pos, SCALE)
    one = oracle.packed_attention(q[:, 1:2], k[:, 1:2], v[:, 1:2], gq, gk, pos, SCALE)
    np.testing.assert_allclose(one[:, 0], out[:, 1], rtol=1e-14, atol=1e-15)


def test_path_global_position_shift_invariance():
    q, k, v, gq, gk, pos = _tiny_inputs(18)
    out = oracle.packed_attention(q, k, v, gq, gk, pos, SCALE)
    out2 = oracle.packed_attention(q, k, v, gq, gk, pos + np.array([5, 3, 2], dtype=np.int32), SCALE)
    np.testing.assert_allclose(out2, out, rtol=1e-10, atol=1e-11)


def test_sampled_path_equals_full_path():
    d = wl.make_inputs(0)
    q, k, v = d.as_f64("q"), d.as_f64("k"), d.as_f64("v")
    full = oracle.packed_attention(q, k, v, d.gamma_q, d.gamma_k, d.pos, SCALE)
    rows = np.array([0, 5, 23, 24, 100, 143, 144, 159])
    heads = np.array([0, 3, 1, 2, 0, 3, 1, 2])
    s = oracle.packed_attention_sampled(q, k, v, d.gamma_q, d.gamma_k, d.pos, SCALE, rows, heads)
    np.testing.assert_allclose(s, full[rows, heads], rtol=1e-13, atol=1e-14)
    # Per-head accessors give the same answer.
    s2 = oracle.packed_attention_sampled(lambda h: q[:, h], lambda h: k[:, h], lambda h: v[:, h],
                                         d.gamma_q, d.gamma_k, d.pos, SCALE, rows, heads)
    np.testing.assert_array_equal(s, s2)
