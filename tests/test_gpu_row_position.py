"""GPU tests: a row's result does not depend on where the launch puts it.

The "MiniMax-H3 WS1/WS2 kernel roadmap" RFC, section 4 ("Numerical contract",
item 2), requires reduction and addition order to be independent of packed-row
count and launch geometry.  The attention kernels give each wave 32 query rows
of one head and stream every key in the same order, so the arithmetic of a
query row is the same whether its row falls in a full 256-row query tile or in
a head's last, partial one.  With the keys held fixed, permuting only the query
rows (and what belongs to them: their rotation-table rows for the fused
forms; their out, dout and log-sum-exp rows for dq) must therefore permute the
output rows bit for bit.  The permutations move rows between full tiles, the
partial tile and both halves of a tile.  dk and dv sum over the query rows, in
row order, so for them a permutation of the queries changes only the summation
order: they are held to the gradient gate there, and tested bit for bit under a
permutation of the key rows with the queries fixed.
"""
import math

import numpy as np
import pytest
import torch

from gates import gradient_ok
from gpu_util import dev_bf16, dev_inputs, host_bits, host_f64
from packed_full_attention_amd import (h3attn_attention_backward, h3attn_forward, h3attn_forward_fp8_qprologue,
                                       h3attn_forward_log2_qprologue, h3attn_forward_lse, h3attn_kv_prologue,
                                       h3attn_kv_prologue_fp8, h3attn_qk_prologue, h3attn_qk_prologue_scaled)
from packed_full_attention_amd import workloads as wl

pytestmark = pytest.mark.gpu
SCALE = 1.0 / math.sqrt(128.0)
Q_SCALE = float(np.float32(SCALE * math.log2(math.e)))

# (L, H): a partial tile of 88 rows after two full ones; one of 232 rows; a
# single row past one full tile; several heads with a partial tile of 100 rows.
# In those the grid is one sparse round, so every full tile runs as two
# 128-row halves; at L = 35890, H = 2 it holds 282 tiles, and 256 run whole, 24
# as halves and 2 as partial tiles, so rows move between all three kinds.
SHAPES = [(600, 3), (1000, 2), (257, 1), (1380, 5), (35890, 2)]


def perms(L: int, seed: int):
    rng = np.random.default_rng(seed)
    return [np.arange(L)[::-1].copy(), rng.permutation(L), np.roll(np.arange(L), L // 2 + 7)]


def take_rows(t: torch.Tensor, perm: np.ndarray) -> torch.Tensor:
    return t[torch.from_numpy(perm).to(t.device)].contiguous()


@pytest.mark.parametrize("L,H", SHAPES)
def test_plain_forward_rows_keep_their_bits(L, H):
    inp = wl.random_document(L, H, seed=700 + L, pos_max=2000)
    q, k, v, gq, gk, pos = dev_inputs(inp)
    h3attn_qk_prologue(q, k, gq, gk, pos)
    ref = host_bits(h3attn_forward(q, k, v))
    for i, perm in enumerate(perms(L, L)):
        print(f"plain forward L={L} H={H} permutation {i}", flush=True)
        got = host_bits(h3attn_forward(take_rows(q, perm), k, v))
        assert np.array_equal(got, ref[perm])


@pytest.mark.parametrize("L,H", SHAPES)
def test_fused_forward_rows_keep_their_bits(L, H):
    inp = wl.random_document(L, H, seed=710 + L, pos_max=2000)
    q, k, v, gq, gk, pos = dev_inputs(inp)
    cs, vt = h3attn_kv_prologue(k, v, gk, pos)
    ref = host_bits(h3attn_forward_log2_qprologue(q, k, vt, gq, cs, Q_SCALE))
    for i, perm in enumerate(perms(L, L + 1)):
        print(f"fused forward L={L} H={H} permutation {i}", flush=True)
        got = host_bits(h3attn_forward_log2_qprologue(take_rows(q, perm), k, vt, gq, take_rows(cs, perm), Q_SCALE))
        assert np.array_equal(got, ref[perm])


@pytest.mark.parametrize("L,H", SHAPES[:2] + SHAPES[-1:])
def test_quantized_score_forward_rows_keep_their_bits(L, H):
    inp = wl.random_document(L, H, seed=720 + L, pos_max=2000)
    q, k, v, gq, gk, pos = dev_inputs(inp)
    cs, k8, vt = h3attn_kv_prologue_fp8(k, v, gk, pos)
    ref = host_bits(h3attn_forward_fp8_qprologue(q, k8, vt, gq, cs, Q_SCALE))
    for i, perm in enumerate(perms(L, L + 2)):
        print(f"quantized-score forward L={L} H={H} permutation {i}", flush=True)
        got = host_bits(h3attn_forward_fp8_qprologue(take_rows(q, perm), k8, vt, gq, take_rows(cs, perm), Q_SCALE))
        assert np.array_equal(got, ref[perm])


@pytest.mark.parametrize("L,H", SHAPES)
@pytest.mark.parametrize("unit", [False, True], ids=["scale", "unit_scale"])
def test_backward_dq_rows_keep_their_bits(L, H, unit):
    inp = wl.random_document(L, H, seed=730 + L, pos_max=2000)
    q, k, v, gq, gk, pos = dev_inputs(inp)
    if unit:  # the scale-folded layout: q' = c q, attention at scale ln 2
        h3attn_qk_prologue_scaled(q, k, gq, gk, pos, Q_SCALE)
        scale = math.log(2.0)
    else:
        h3attn_qk_prologue(q, k, gq, gk, pos)
        scale = SCALE
    out, lse = h3attn_forward_lse(q, k, v, scale=scale)
    dout = dev_bf16(wl.random_document(L, H, seed=740 + L).q)
    dq, dk, dv = h3attn_attention_backward(q, k, v, out, dout, lse, scale=scale)
    ref_dq = host_bits(dq)
    ref_dk, ref_dv = host_f64(dk), host_f64(dv)
    for i, perm in enumerate(perms(L, L + 3)):
        print(f"backward L={L} H={H} unit={unit} permutation {i}", flush=True)
        p = torch.from_numpy(perm).to("cuda")
        dq2, dk2, dv2 = h3attn_attention_backward(take_rows(q, perm), k, v, take_rows(out, perm),
                                                  take_rows(dout, perm), lse[:, p].contiguous(), scale=scale)
        assert np.array_equal(host_bits(dq2), ref_dq[perm])
        for name, got, ref in (("dk", host_f64(dk2), ref_dk), ("dv", host_f64(dv2), ref_dv)):
            ok, e = gradient_ok(got, ref)
            assert ok, (name, e)


@pytest.mark.parametrize("L,H", SHAPES)
@pytest.mark.parametrize("unit", [False, True], ids=["scale", "unit_scale"])
def test_backward_dk_dv_rows_keep_their_bits(L, H, unit):
    # The key side: the dk/dv kernel gives each wave 32 keys and streams the
    # queries in one order, so with q, out, dout and lse held fixed, permuting
    # the key rows (k and v together) permutes dk and dv bit for bit.
    inp = wl.random_document(L, H, seed=750 + L, pos_max=2000)
    q, k, v, gq, gk, pos = dev_inputs(inp)
    if unit:
        h3attn_qk_prologue_scaled(q, k, gq, gk, pos, Q_SCALE)
        scale = math.log(2.0)
    else:
        h3attn_qk_prologue(q, k, gq, gk, pos)
        scale = SCALE
    out, lse = h3attn_forward_lse(q, k, v, scale=scale)
    dout = dev_bf16(wl.random_document(L, H, seed=760 + L).q)
    _, dk, dv = h3attn_attention_backward(q, k, v, out, dout, lse, scale=scale)
    ref_dk, ref_dv = host_bits(dk), host_bits(dv)
    for i, perm in enumerate(perms(L, L + 4)):
        print(f"backward keys L={L} H={H} unit={unit} permutation {i}", flush=True)
        _, dk2, dv2 = h3attn_attention_backward(q, take_rows(k, perm), take_rows(v, perm), out, dout, lse,
                                                scale=scale)
        assert np.array_equal(host_bits(dk2), ref_dk[perm])
        assert np.array_equal(host_bits(dv2), ref_dv[perm])
