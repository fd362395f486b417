"""Seeded input generator: determinism, shapes, positions, bf16 rounding."""
import numpy as np
import pytest
import torch

from packed_full_attention_amd import workloads as wl


@pytest.mark.parametrize("w", wl.WORKLOADS, ids=lambda w: w.name)
def test_row_counts_and_lengths(w):
    expect_L = {0: 160, 1: 512, 2: 1920, 3: 16500, 4: 28976}[w.index]
    expect_H = {0: 4, 1: 56, 2: 56, 3: 56, 4: 7}[w.index]
    assert w.seq_len == expect_L and w.heads == expect_H
    pos = wl.packed_positions(w.n_text, w.video_grid, w.n_audio)
    assert pos.shape == (expect_L, 3) and pos.dtype == np.int32
    # (0, 0, 0) opens each modality.
    for r in (0, w.n_text, w.n_text + w.n_video):
        assert tuple(pos[r]) == (0, 0, 0)
    # text (i, i, i); video raster (t slowest); audio (t, 0, 0)
    i = np.arange(w.n_text)
    assert np.array_equal(pos[:w.n_text], np.stack([i, i, i], 1))
    T, Hg, Wg = w.video_grid
    vid = pos[w.n_text:w.n_text + w.n_video]
    assert np.array_equal(vid[:, 0] * Hg * Wg + vid[:, 1] * Wg + vid[:, 2], np.arange(w.n_video))
    aud = pos[w.n_text + w.n_video:]
    assert np.array_equal(aud[:, 0], np.arange(w.n_audio)) and not aud[:, 1:].any()


def test_generator_is_deterministic_and_seeded():
    a = wl.make_inputs(0)
    b = wl.make_inputs(0)
    c = wl.make_inputs(0, seed=7)
    for n in ("q", "k", "v", "gamma_q", "gamma_k", "pos"):
        assert np.array_equal(getattr(a, n), getattr(b, n))
    assert not np.array_equal(a.q, c.q)
    assert a.q.shape == (160, 4, 128) and a.q.dtype == np.uint16


def test_stress_rows_only_on_the_stressed_workload():
    a = wl.make_inputs(1, heads=1)
    assert len(a.stress_rows) == 0
    b = wl.make_inputs(2, heads=1)
    assert len(b.stress_rows) == 96 and len(np.unique(b.stress_rows)) == 96
    assert b.stress_rows.min() >= 0 and b.stress_rows.max() < 1920


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(100000) * 10.0 ** rng.integers(-5, 5, 100000),
                        np.array([1.0, -1.0, 0.0, 1.00390625, 1.01171875, 3.4e38, 1e-40], np.float32)])
    x = x.astype(np.float32)
    ours = wl.bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)
    # Ties to even: 1 + 2^-8 is halfway between 1 and 1 + 2^-7 -> 1.
    assert wl.bf16_bits(np.array([1.00390625], np.float32))[0] == 0x3F80
    assert wl.bf16_bits(np.array([1.01171875], np.float32))[0] == 0x3F82


def test_gammas_are_bf16_values_near_one():
    a = wl.make_inputs(0)
    for g in (a.gamma_q, a.gamma_k):
        assert g.dtype == np.float32 and g.shape == (128,)
        assert np.array_equal(wl.round_to_bf16(g), g)
        assert 0.5 < g.min() and g.max() < 1.5


def test_scale_rows_by_power_of_two_is_exact():
    a = wl.make_inputs(2, heads=2)
    s = wl.scale_rows_bf16(a.k, a.stress_rows, 3)
    f0 = wl.bf16_bits_to_f32(a.k[a.stress_rows])
    f1 = wl.bf16_bits_to_f32(s[a.stress_rows])
    assert np.array_equal(f1, f0 * 8)
    other = np.setdiff1d(np.arange(a.k.shape[0]), a.stress_rows)
    assert np.array_equal(s[other], a.k[other])
