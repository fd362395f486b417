"""Pins for the quantized-score oracle (oracle/h3_oracle_fp8.py).

The e4m3 cast is pinned to values the OCP OFP8 specification fixes (largest and
smallest normal and subnormal magnitudes, the NaN pattern, the spacing of each
binade), to brute-force nearest-value search over the format's whole table with
ties to the even code, and to an independent library conversion (torch's CPU
float8_e4m3fn).  The attention of the cast operands is pinned to the exact
oracle (itself pinned in test_oracle_pins.py): with the casts replaced by the
identity the variant must be the path's own attention, and the base-2 softmax
must be the natural softmax with the scale ln 2.  Hand-worked operand values pin
where the factors 4 and 1/4 sit.  CPU only.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import h3_oracle_fp8 as fp8
from packed_full_attention_amd import workloads as wl

SCALE = 1.0 / math.sqrt(128.0)
Q_SCALE = SCALE * math.log2(math.e)


# ---------------------------------------------------------------- the format

@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6), (0x38, 1.0), (0x39, 1.125),
    (0x3F, 1.875), (0x40, 2.0), (0x77, 240.0), (0x7E, 448.0), (0xC0, -2.0), (0xFE, -448.0), (0x81, -2.0 ** -9),
])
def test_decode_spec_values(code, value):
    assert fp8.e4m3_decode(np.array([code]))[0] == value


def test_nan_patterns_and_negative_zero():
    d = fp8.e4m3_decode(np.array([0x7F, 0xFF, 0x80]))
    assert np.isnan(d[0]) and np.isnan(d[1])
    assert d[2] == 0.0 and np.signbit(d[2])


def test_table_is_increasing_with_binade_spacing():
    vals = fp8.e4m3_decode(np.arange(0x7F))  # every finite non-negative code
    assert np.all(np.diff(vals) > 0)
    assert len(np.unique(vals)) == 127
    # codes 0..15: subnormals and the first normal binade share the quantum 2^-9;
    # binade with exponent field E >= 1 has quantum 2^(E - 10)
    for c in range(0x7E):
        E = max(c >> 3, 1)
        assert vals[c + 1] - vals[c] == 2.0 ** (E - 10), c


def test_encode_decode_round_trip_every_finite_code():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    assert np.array_equal(fp8.e4m3_encode(fp8.e4m3_decode(codes)), codes)


def _nearest_even(x, table):
    """Brute force: the non-negative code whose value is nearest |x|; on a tie the even code."""
    d = np.abs(table[None, :] - np.abs(x)[:, None])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    codes = np.empty(len(x), dtype=np.int64)
    for i in range(len(x)):
        c = np.flatnonzero(cand[i])
        codes[i] = c[0] if len(c) == 1 else c[c % 2 == 0][0]
    return codes


def test_encode_is_nearest_ties_to_even_brute_force():
    table = fp8.e4m3_decode(np.arange(0x7F))
    rng = np.random.default_rng(7)
    mags = np.concatenate([
        2.0 ** rng.uniform(-12, math.log2(448.0), 6000),
        rng.uniform(0, 448.0, 2000),
        (table[:-1] + table[1:]) / 2,                       # every midpoint: a tie
        (table[:-1] + table[1:]) / 2 * (1 + 1e-12),
        (table[:-1] + table[1:]) / 2 * (1 - 1e-12),
    ])
    signs = np.where(rng.random(len(mags)) < 0.5, -1.0, 1.0)
    x = signs * mags
    got = fp8.e4m3_encode(x).astype(np.int64)
    want = _nearest_even(x, table)
    assert np.array_equal(got & 0x7F, want)
    assert np.array_equal(got >> 7, np.signbit(x).astype(np.int64))


@pytest.mark.parametrize("x,code", [
    (1.0 + 1 / 16, 0x38), (1.0 + 3 / 16, 0x3A), (17.0, 0x58), (19.0, 0x5A), (0.3, 0x2A),
    (1.5 * 2.0 ** -9, 0x02), (0.5 * 2.0 ** -9, 0x00), (15.5 * 2.0 ** -10, 0x08), (432.0, 0x7E), (440.0, 0x7E),
])
def test_encode_hand_worked(x, code):
    assert int(fp8.e4m3_encode(np.array([x]))[0]) == code


def test_encode_agrees_with_torch_float8_e4m3fn():
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.standard_normal(20000) * 8, rng.standard_normal(5000) * 2.0 ** -7,
                        rng.uniform(-448, 448, 5000)]).astype(np.float32)
    t = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = fp8.e4m3_encode(x.astype(np.float64))
    zero = (t & 0x7F) == 0
    assert np.array_equal(got[~zero], t[~zero])
    assert np.all((got[zero] & 0x7F) == 0)  # signed zeros may differ in sign only


def test_relative_error_bound():
    rng = np.random.default_rng(3)
    x = np.concatenate([2.0 ** rng.uniform(-6, 8.8, 10000), -(2.0 ** rng.uniform(-6, 8.8, 10000))])
    x = x[np.abs(x) <= 448.0]
    r = fp8.e4m3_round(x)
    assert np.all(np.abs(r - x) <= 2.0 ** -4 * np.abs(x))
    s = rng.uniform(-2.0 ** -6, 2.0 ** -6, 5000)
    assert np.all(np.abs(fp8.e4m3_round(s) - s) <= 2.0 ** -10)


@pytest.mark.parametrize("bad", [449.0, -1000.0, np.inf, np.nan])
def test_out_of_domain_raises(bad):
    with pytest.raises(ValueError):
        fp8.e4m3_encode(np.array([1.0, bad]))


# ---------------------------------------------------------------- the attention

def test_operand_factors_hand_worked():
    # q' times 4 q_scale (q_scale = 1/4 here) is q' itself: 0.3 -> 0.3125, 1.0 -> 1.0.
    # k' / 4: 4 * 1.3 * 2^-7 / 4 = 5.2 * 2^-9, a subnormal, -> 5 * 2^-9; 100 / 4 = 25 -> 24 (quantum 2, tie to even).
    q8, k8 = fp8.quantized_operands(np.array([0.3, 1.0]), np.array([4 * 1.3 * 2.0 ** -7, 100.0]), 0.25)
    assert list(q8) == [0.3125, 1.0]
    assert list(k8) == [5 * 2.0 ** -9, 24.0]


def test_base2_softmax_is_natural_softmax_at_scale_ln2():
    rng = np.random.default_rng(5)
    q8 = fp8.e4m3_round(rng.standard_normal((40, 128)))
    k8 = fp8.e4m3_round(rng.standard_normal((70, 128)) / 4)
    v = rng.standard_normal((70, 128))
    got = fp8.quantized_attention_head(q8, k8, v, block=16)
    want = oracle.attention_head(q8, k8, v, math.log(2.0))
    np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-12)


def test_identity_cast_reduces_to_the_exact_path(monkeypatch):
    d = wl.make_inputs(0)
    q, k, v = d.as_f64("q"), d.as_f64("k"), d.as_f64("v")
    want = oracle.packed_attention(q, k, v, d.gamma_q, d.gamma_k, d.pos, SCALE)
    monkeypatch.setattr(fp8, "e4m3_round", lambda x: np.asarray(x, dtype=np.float64))
    got = fp8.packed_attention_fp8(q, k, v, d.gamma_q, d.gamma_k, d.pos, Q_SCALE)
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12)


def test_quantized_path_is_the_cast_operands_attention():
    """With the casts in place the output differs from the exact path by about
    e4m3's relative precision and is the attention of the cast operands."""
    d = wl.make_inputs(0)
    q, k, v = d.as_f64("q"), d.as_f64("k"), d.as_f64("v")
    exact = oracle.packed_attention(q, k, v, d.gamma_q, d.gamma_k, d.pos, SCALE)
    got = fp8.packed_attention_fp8(q, k, v, d.gamma_q, d.gamma_k, d.pos, Q_SCALE)
    rel = np.linalg.norm(got - exact) / np.linalg.norm(exact)
    assert 1e-3 < rel < 0.1, rel
    qr, kr = oracle.qk_prologue(q, k, d.gamma_q, d.gamma_k, d.pos)
    q8, k8 = fp8.quantized_operands(qr, kr, Q_SCALE)
    assert np.all(np.abs(q8 - 4 * Q_SCALE * qr) <= 2.0 ** -4 * np.abs(4 * Q_SCALE * qr) + 2.0 ** -10)
    assert np.all(np.abs(k8 - kr / 4) <= 2.0 ** -4 * np.abs(kr / 4) + 2.0 ** -10)
    h = 2
    np.testing.assert_allclose(got[:, h], oracle.attention_head(q8[:, h], k8[:, h], v[:, h], math.log(2.0)),
                               rtol=1e-10, atol=1e-12)


def test_token_permutation_equivariance():
    d = wl.make_inputs(0)
    q, k, v = d.as_f64("q"), d.as_f64("k"), d.as_f64("v")
    perm = np.random.default_rng(9).permutation(q.shape[0])
    a = fp8.packed_attention_fp8(q, k, v, d.gamma_q, d.gamma_k, d.pos, Q_SCALE)
    b = fp8.packed_attention_fp8(q[perm], k[perm], v[perm], d.gamma_q, d.gamma_k, d.pos[perm], Q_SCALE)
    np.testing.assert_allclose(b, a[perm], rtol=1e-12, atol=1e-13)
