"""GPU tests of the Q-prologue fusion: h3attn_k_prologue_table (K's prologue and
the per-token rotation table) + h3attn_v_transpose + h3attn_forward_log2_qprologue
(attention with Q's RMSNorm and MM-RoPE applied at its Q load), through the C ABI.

The fusion is exact by design (the "h3-metal" README, "Implementation and
performance notes", "Profiling and diagnostic paths", keeps its fused Q/K
normalization and RoPE byte-identical): its output must equal, bit for bit, the
unfused path h3attn_qk_prologue_scaled + h3attn_v_transpose + h3attn_forward_log2
on the same inputs, and K must equal the plain prologue's K.  Those unfused
kernels are checked against the fp64 oracle elsewhere; here the fused output is
also checked against the oracle directly, and the table against the fp64
cosines and sines of the oracle's angles.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from gates import attention_ok
from gpu_util import dev_bf16, dev_inputs, host_bits, host_f64
from packed_full_attention_amd import (h3attn_forward_log2, h3attn_forward_log2_qprologue, h3attn_k_prologue_table,
                                       h3attn_kv_prologue, h3attn_qk_prologue_scaled, h3attn_v_transpose)
from packed_full_attention_amd import workloads as wl

pytestmark = pytest.mark.gpu
SCALE = 1.0 / math.sqrt(128.0)
Q_SCALE = float(np.float32(SCALE * math.log2(math.e)))


def unfused(inp, q_scale=Q_SCALE):
    q, k, v, gq, gk, pos = dev_inputs(inp)
    h3attn_qk_prologue_scaled(q, k, gq, gk, pos, q_scale)
    out = h3attn_forward_log2(q, k, h3attn_v_transpose(v))
    torch.cuda.synchronize()
    return host_bits(out), host_bits(k)


def fused(inp, q_scale=Q_SCALE):
    q, k, v, gq, gk, pos = dev_inputs(inp)
    cs = h3attn_k_prologue_table(k, gk, pos)
    out = h3attn_forward_log2_qprologue(q, k, h3attn_v_transpose(v), gq, cs, q_scale)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(q), inp.q), "the fused path must not modify q"
    return host_bits(out), host_bits(k), cs.cpu().numpy()


def with_stress(inp):
    """The stressed workload's chosen K rows x 8 before the prologue (as the
    whole-path tests apply them)."""
    if not len(inp.stress_rows):
        return inp
    return wl.Inputs(inp.workload, inp.q, wl.scale_rows_bf16(inp.k, inp.stress_rows, 3), inp.v, inp.gamma_q,
                     inp.gamma_k, inp.pos, inp.stress_rows)


@pytest.mark.parametrize("idx", [0, 1, 2, 3, 4])
def test_fused_path_bit_identical_to_unfused(idx):
    inp = with_stress(wl.make_inputs(idx))
    print(f"fused vs unfused, workload {idx}: {inp.workload.describe()}", flush=True)
    out_u, k_u = unfused(inp)
    out_f, k_f, _ = fused(inp)
    assert np.array_equal(k_f, k_u)
    diff = int(np.count_nonzero(out_f != out_u))
    assert diff == 0, f"{diff} of {out_u.size} output values differ"


@pytest.mark.parametrize("L,H", [(1, 1), (2, 3), (31, 2), (32, 1), (33, 1), (64, 2), (65, 1), (255, 1),
                                 (256, 2), (257, 1), (600, 3), (1000, 5)])
def test_fused_path_bit_identical_edge_lengths(L, H):
    inp = wl.random_document(L, H, seed=300 + L + H, pos_max=5000)
    print(f"fused vs unfused, L={L} H={H}", flush=True)
    out_u, k_u = unfused(inp)
    out_f, k_f, _ = fused(inp)
    assert np.array_equal(k_f, k_u) and np.array_equal(out_f, out_u)


@pytest.mark.parametrize("q_scale", [1.0, 0.5, 3.0])
def test_fused_path_bit_identical_other_q_scales(q_scale):
    inp = wl.make_inputs(1)
    out_u, _ = unfused(inp, q_scale)
    out_f, _, _ = fused(inp, q_scale)
    assert np.array_equal(out_f, out_u)


def test_fused_path_bit_identical_on_extreme_rows():
    # Rows of zeros (norm 0: the eps alone), huge rows (sum of squares overflows
    # to inf, r = 0), tiny rows (subnormal sum of squares) and signed zeros.
    L, H = 300, 4
    inp = wl.random_document(L, H, seed=17, pos_max=3000)
    q = inp.q.copy()
    f = lambda x: wl.bf16_bits(np.full((H, 128), x, np.float32))
    q[3] = f(0.0)
    q[4] = f(-0.0)
    q[5] = f(1e30)
    q[6] = f(-3e-20)
    q[7, :, ::2] = f(2e-38)[:, ::2]
    q[8] = wl.bf16_bits(wl.bf16_bits_to_f32(q[8]) * np.float32(1e25))
    inp = wl.Inputs(inp.workload, q, inp.k, inp.v, inp.gamma_q, inp.gamma_k, inp.pos, inp.stress_rows)
    out_u, _ = unfused(inp)
    out_f, _, _ = fused(inp)
    assert np.array_equal(out_f, out_u)


@pytest.mark.parametrize("idx", [0, 1, 2])
def test_fused_path_oracle_parity(idx):
    inp = with_stress(wl.make_inputs(idx))
    out, _, _ = fused(inp)
    kf = wl.bf16_bits_to_f32(inp.k).astype(np.float64)
    ref = oracle.packed_attention(inp.as_f64("q"), kf, inp.as_f64("v"), inp.gamma_q, inp.gamma_k, inp.pos, SCALE)
    ok, e = attention_ok(wl.bf16_bits_to_f32(out).astype(np.float64), ref)
    print(f"fused path workload {idx}: {e}")
    assert ok, e


@pytest.mark.parametrize("idx", [1, 3])
def test_rope_table_matches_oracle_angles(idx):
    # The table holds fp32 cos and sin of fp32 angles pos * w_j; against the
    # fp64 values the error is the angle's rounding (about 2^-22 relative, from
    # w_j and the product) plus the sine's own (a few 2^-24).
    inp = wl.make_inputs(idx)
    _, _, cs = fused(inp)
    phi = oracle.rope_angles(inp.pos)
    tol = 5e-7 * np.abs(phi) + 5e-7
    assert np.all(np.abs(cs[:, :48] - np.cos(phi)) <= tol)
    assert np.all(np.abs(cs[:, 48:] - np.sin(phi)) <= tol)


def test_k_prologue_table_writes_only_its_buffers():
    L, H = 130, 3
    inp = wl.random_document(L, H, seed=23)
    n, guard = L * H * 128, 4096
    kfull = dev_bf16(np.full(n + 2 * guard, 0x7FC1, np.uint16))
    k = kfull[guard:guard + n].view(L, H, 128)
    k.copy_(dev_bf16(inp.k))
    tfull = torch.full((L * 96 + 2 * guard,), float("nan"), dtype=torch.float32, device="cuda")
    cs = tfull[guard:guard + L * 96].view(L, 96)
    _, _, _, _, gk, pos = dev_inputs(inp)
    h3attn_k_prologue_table(k, gk, pos, cs)
    torch.cuda.synchronize()
    kh, th = host_bits(kfull), tfull.cpu().numpy()
    assert np.all(kh[:guard] == 0x7FC1) and np.all(kh[-guard:] == 0x7FC1)
    assert np.all(np.isnan(th[:guard])) and np.all(np.isnan(th[-guard:]))
    assert not np.any(np.isnan(th[guard:guard + L * 96]))
    out_u, k_u = unfused(inp)
    assert np.array_equal(kh[guard:guard + n].reshape(L, H, 128), k_u)


# ------------------------------------------------------------------ h3attn_kv_prologue

def _kv_pair(inp):
    """(k', rope_cs, vt) from h3attn_k_prologue_table + h3attn_v_transpose and from
    h3attn_kv_prologue, on the same inputs."""
    _, k1, v, _, gk, pos = dev_inputs(inp)
    cs1 = h3attn_k_prologue_table(k1, gk, pos)
    vt1 = h3attn_v_transpose(v)
    k2 = dev_bf16(inp.k)
    cs2, vt2 = h3attn_kv_prologue(k2, v, gk, pos)
    torch.cuda.synchronize()
    return (host_bits(k1), cs1.cpu().numpy(), host_bits(vt1)), (host_bits(k2), cs2.cpu().numpy(), host_bits(vt2))


@pytest.mark.parametrize("idx", [0, 1, 2, 3, 4])
def test_kv_prologue_bit_identical_to_the_two_passes(idx):
    inp = with_stress(wl.make_inputs(idx))
    print(f"kv prologue vs two passes, workload {idx}: {inp.workload.describe()}", flush=True)
    (k1, cs1, vt1), (k2, cs2, vt2) = _kv_pair(inp)
    assert np.array_equal(k1, k2)
    assert np.array_equal(cs1.view(np.uint32), cs2.view(np.uint32))
    assert np.array_equal(vt1, vt2)


@pytest.mark.parametrize("L,H", [(1, 1), (2, 3), (63, 2), (64, 1), (65, 3), (255, 1), (257, 2), (1000, 5),
                                 (777, 57)])
def test_kv_prologue_bit_identical_edge_lengths(L, H):
    inp = wl.random_document(L, H, seed=700 + L + H, pos_max=5000)
    print(f"kv prologue vs two passes, L={L} H={H}", flush=True)
    (k1, cs1, vt1), (k2, cs2, vt2) = _kv_pair(inp)
    assert np.array_equal(k1, k2) and np.array_equal(vt1, vt2)
    assert np.array_equal(cs1.view(np.uint32), cs2.view(np.uint32))
    # V^T is an exact copy with zero padding.
    Lp = (L + 63) // 64 * 64
    want = np.zeros((H, 128, Lp), np.uint16)
    want[:, :, :L] = inp.v.transpose(1, 2, 0)
    assert np.array_equal(vt2, want)


def test_kv_prologue_writes_only_its_buffers():
    L, H = 130, 3
    inp = wl.random_document(L, H, seed=29)
    n, guard, Lp = L * H * 128, 4096, 192
    kfull = dev_bf16(np.full(n + 2 * guard, 0x7FC1, np.uint16))
    k = kfull[guard:guard + n].view(L, H, 128)
    k.copy_(dev_bf16(inp.k))
    tfull = torch.full((L * 96 + 2 * guard,), float("nan"), dtype=torch.float32, device="cuda")
    cs = tfull[guard:guard + L * 96].view(L, 96)
    nv = H * 128 * Lp
    vfull = dev_bf16(np.full(nv + 2 * guard, 0x7FC1, np.uint16))
    vt = vfull[guard:guard + nv].view(H, 128, Lp)
    _, _, v, _, gk, pos = dev_inputs(inp)
    h3attn_kv_prologue(k, v, gk, pos, cs, vt)
    torch.cuda.synchronize()
    kh, th, vh = host_bits(kfull), tfull.cpu().numpy(), host_bits(vfull)
    for a in (kh, vh):
        assert np.all(a[:guard] == 0x7FC1) and np.all(a[-guard:] == 0x7FC1)
    assert np.all(np.isnan(th[:guard])) and np.all(np.isnan(th[-guard:]))
    assert not np.any(np.isnan(th[guard:guard + L * 96]))
    assert not np.any(vh[guard:guard + nv] == 0x7FC1)
