"""GPU parity of the scale-folded path: h3attn_qk_prologue_scaled (Q output
times scale * log2(e) before its bf16 rounding), h3attn_v_transpose (V^T, bit
exact) and h3attn_forward_log2 (base-2 softmax on V^T), called through the C
ABI, against the fp64 oracle.

h3attn_forward_log2(q', k, v) is the oracle's attention with scale ln 2 on
the same bf16 q', k, v; the whole path equals the oracle's packed attention
of the raw inputs at scale 1/sqrt(128).  Same gates as the plain path
(tests/gates.py).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from gates import attention_ok, prologue_ok
from gpu_util import dev_bf16, dev_inputs, head_f64, host_bits, host_f64, sample_heads, sample_rows
from packed_full_attention_amd import (h3attn_forward_log2, h3attn_qk_prologue, h3attn_qk_prologue_scaled,
                                       h3attn_v_transpose, padded_length)
from packed_full_attention_amd import workloads as wl

pytestmark = pytest.mark.gpu
SCALE = 1.0 / math.sqrt(128.0)
Q_SCALE = float(np.float32(SCALE * math.log2(math.e)))  # what a caller passes, as fp32
LN2 = math.log(2.0)
SMALL = (0, 1, 2)
LONG = (3, 4)


@pytest.fixture(scope="module")
def inputs():
    cache = {}

    def get(i):
        if i not in cache:
            cache[i] = wl.make_inputs(i)
        return cache[i]
    return get


def run_prologue(inp, kbits=None):
    q, k, v, gq, gk, pos = dev_inputs(inp)
    if kbits is not None:
        k = dev_bf16(kbits)
    h3attn_qk_prologue_scaled(q, k, gq, gk, pos, Q_SCALE)
    torch.cuda.synchronize()
    return q, k, v


def bf16_of(x: np.ndarray) -> np.ndarray:
    return wl.bf16_bits(x.astype(np.float32))


# ------------------------------------------------------------------ V transpose (bit exact)

def transpose_ref(vbits: np.ndarray) -> np.ndarray:
    L, H, D = vbits.shape
    ref = np.zeros((H, D, padded_length(L)), np.uint16)
    ref[:, :, :L] = vbits.transpose(1, 2, 0)
    return ref


@pytest.mark.parametrize("L,H", [(1, 1), (63, 2), (64, 1), (65, 3), (160, 4), (1920, 56), (16500, 56)])
def test_v_transpose_bit_exact(L, H):
    vbits = wl.random_document(L, H, seed=40 + L).v
    vt = h3attn_v_transpose(dev_bf16(vbits))
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(vt), transpose_ref(vbits))


def test_v_transpose_overwrites_padding_and_stays_in_bounds():
    # vt starts as NaN patterns in a guarded buffer: padding becomes zero, guards stay.
    L, H = 70, 2
    vbits = wl.random_document(L, H, seed=41).v
    n, guard = H * 128 * padded_length(L), 2048
    full = dev_bf16(np.full(n + 2 * guard, 0x7FC1, np.uint16))
    vt = full[guard:guard + n].view(H, 128, padded_length(L))
    h3attn_v_transpose(dev_bf16(vbits), vt)
    torch.cuda.synchronize()
    h = host_bits(full)
    assert np.all(h[:guard] == 0x7FC1) and np.all(h[-guard:] == 0x7FC1)
    assert np.array_equal(h[guard:guard + n].reshape(H, 128, -1), transpose_ref(vbits))


# ------------------------------------------------------------------ prologue

@pytest.mark.parametrize("idx", SMALL)
def test_prologue_scaled_parity_full(inputs, idx):
    inp = inputs(idx)
    q, k, _ = run_prologue(inp)
    rq, rk = oracle.qk_prologue(inp.as_f64("q"), inp.as_f64("k"), inp.gamma_q, inp.gamma_k, inp.pos)
    for name, got, ref in (("q", host_f64(q), rq * Q_SCALE), ("k", host_f64(k), rk)):
        ok, e = prologue_ok(got, ref)
        print(f"scaled prologue workload {idx} {name}: {e}")
        assert ok, (name, e)


def test_prologue_scale_one_is_the_plain_prologue(inputs):
    # q_scale = 1 reproduces h3attn_qk_prologue bit for bit; K never depends on q_scale.
    inp = inputs(1)
    outs = []
    for fn in (lambda *a: h3attn_qk_prologue(*a), lambda *a: h3attn_qk_prologue_scaled(*a, 1.0),
               lambda *a: h3attn_qk_prologue_scaled(*a, Q_SCALE)):
        q, k, v, gq, gk, pos = dev_inputs(inp)
        fn(q, k, gq, gk, pos)
        torch.cuda.synchronize()
        outs.append((host_bits(q), host_bits(k)))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
    assert np.array_equal(outs[0][1], outs[2][1])


@pytest.mark.parametrize("idx", LONG)
def test_prologue_scaled_parity_sampled_long(inputs, idx):
    inp = inputs(idx)
    q, _, _ = run_prologue(inp)
    toks = sample_rows(inp.workload, 1500, 7 + idx)
    x = wl.bf16_bits_to_f32(inp.q[toks]).astype(np.float64)
    ref = oracle.mm_rope(oracle.rms_norm(x, inp.gamma_q), inp.pos[toks]) * Q_SCALE
    ok, e = prologue_ok(wl.bf16_bits_to_f32(host_bits(q)[toks]), ref)
    print(f"scaled prologue workload {idx} q ({len(toks)} tokens): {e}")
    assert ok, e


# ------------------------------------------------------------------ attention alone

@pytest.mark.parametrize("idx", SMALL)
def test_forward_log2_parity_full(inputs, idx):
    # q' = bf16(oracle q * Q_SCALE), k' = bf16(oracle k) with the stressed
    # workload's chosen K rows x 8 after the prologue: the large scores that
    # drive the offset rebase.
    inp = inputs(idx)
    rq, rk = oracle.qk_prologue(inp.as_f64("q"), inp.as_f64("k"), inp.gamma_q, inp.gamma_k, inp.pos)
    qb, kb = bf16_of(rq * Q_SCALE), bf16_of(rk)
    kb = wl.scale_rows_bf16(kb, inp.stress_rows, 3)
    out = h3attn_forward_log2(dev_bf16(qb), dev_bf16(kb), h3attn_v_transpose(dev_bf16(inp.v)))
    torch.cuda.synchronize()
    f = lambda b: wl.bf16_bits_to_f32(b).astype(np.float64)
    ref = oracle.attention(f(qb), f(kb), inp.as_f64("v"), LN2)
    ok, e = attention_ok(host_f64(out), ref)
    print(f"forward_log2 workload {idx} (stress rows {len(inp.stress_rows)}): {e}")
    assert ok, e


@pytest.mark.parametrize("idx", LONG)
def test_forward_log2_parity_sampled_long(inputs, idx):
    # The generated bf16 q (times Q_SCALE, rounded), k, v straight into the kernel.
    inp = inputs(idx)
    qb = bf16_of(wl.bf16_bits_to_f32(inp.q).astype(np.float64) * Q_SCALE)
    out = h3attn_forward_log2(dev_bf16(qb), dev_bf16(inp.k), h3attn_v_transpose(dev_bf16(inp.v)))
    torch.cuda.synchronize()
    rows, heads = sample_rows(inp.workload, 96, 11 + idx), sample_heads(inp.workload)
    got_all = host_bits(out)
    qh, kh, vh = head_f64(qb), head_f64(inp.k), head_f64(inp.v)
    got, ref = [], []
    for h in heads:
        ref.append(oracle.attention_head(qh(h)[rows], kh(h), vh(h), LN2))
        got.append(wl.bf16_bits_to_f32(got_all[rows, h]).astype(np.float64))
    ok, e = attention_ok(np.stack(got), np.stack(ref))
    print(f"forward_log2 workload {idx} ({len(rows)} rows x {len(heads)} heads): {e}")
    assert ok, e


# ------------------------------------------------------------------ whole path

@pytest.mark.parametrize("idx", SMALL)
def test_scaled_path_parity_full(inputs, idx):
    inp = inputs(idx)
    kbits = wl.scale_rows_bf16(inp.k, inp.stress_rows, 3)  # literal reading: before the prologue
    q, k, v = run_prologue(inp, kbits)
    out = h3attn_forward_log2(q, k, h3attn_v_transpose(v))
    torch.cuda.synchronize()
    kf = wl.bf16_bits_to_f32(kbits).astype(np.float64)
    ref = oracle.packed_attention(inp.as_f64("q"), kf, inp.as_f64("v"), inp.gamma_q, inp.gamma_k,
                                  inp.pos, SCALE)
    ok, e = attention_ok(host_f64(out), ref)
    print(f"scaled path workload {idx}: {e}")
    assert ok, e


@pytest.mark.parametrize("idx", LONG)
def test_scaled_path_parity_sampled_long(inputs, idx):
    inp = inputs(idx)
    q, k, v = run_prologue(inp)
    out = h3attn_forward_log2(q, k, h3attn_v_transpose(v))
    torch.cuda.synchronize()
    rows, heads = sample_rows(inp.workload, 96, 21 + idx), sample_heads(inp.workload)
    rr = np.repeat(rows[None, :], len(heads), 0).ravel()
    hh = np.repeat(heads[:, None], len(rows), 1).ravel()
    ref = oracle.packed_attention_sampled(head_f64(inp.q), head_f64(inp.k), head_f64(inp.v),
                                          inp.gamma_q, inp.gamma_k, inp.pos, SCALE, rr, hh)
    got = wl.bf16_bits_to_f32(host_bits(out)[rr, hh]).astype(np.float64)
    ok, e = attention_ok(got, ref)
    print(f"scaled path workload {idx} ({len(rows)} rows x {len(heads)} heads): {e}")
    assert ok, e


# ------------------------------------------------------------------ edge cases and invariants

@pytest.mark.parametrize("L,H", [(1, 1), (2, 3), (3, 1), (31, 2), (32, 1), (33, 1), (63, 1), (64, 2),
                                 (65, 1), (127, 1), (128, 2), (129, 1), (200, 3), (1000, 2)])
def test_scaled_path_edge_lengths(L, H):
    inp = wl.random_document(L, H, seed=100 + L + H, pos_max=2000)
    q, k, v = run_prologue(inp)
    out = h3attn_forward_log2(q, k, h3attn_v_transpose(v))
    torch.cuda.synchronize()
    ref = oracle.packed_attention(inp.as_f64("q"), inp.as_f64("k"), inp.as_f64("v"), inp.gamma_q,
                                  inp.gamma_k, inp.pos, SCALE)
    ok, e = attention_ok(host_f64(out), ref)
    assert ok, (L, H, e)


def test_log2_zero_queries_give_column_mean_of_v():
    inp = wl.random_document(300, 2, seed=5)
    qz = torch.zeros(300, 2, 128, dtype=torch.bfloat16, device="cuda")
    out = h3attn_forward_log2(qz, dev_bf16(inp.k), h3attn_v_transpose(dev_bf16(inp.v)))
    torch.cuda.synchronize()
    ref = np.broadcast_to(inp.as_f64("v").mean(axis=0), (300, 2, 128))
    ok, e = attention_ok(host_f64(out), ref)
    assert ok, e


def test_scaled_path_repeat_and_head_subset_bit_identical(inputs):
    inp = inputs(1)
    outs = []
    for _ in range(2):
        q, k, v = run_prologue(inp)
        outs.append(host_bits(h3attn_forward_log2(q, k, h3attn_v_transpose(v))))
        torch.cuda.synchronize()
    assert np.array_equal(outs[0], outs[1])
    sub = wl.Inputs(inp.workload, np.ascontiguousarray(inp.q[:, 7:14]), np.ascontiguousarray(inp.k[:, 7:14]),
                    np.ascontiguousarray(inp.v[:, 7:14]), inp.gamma_q, inp.gamma_k, inp.pos, inp.stress_rows)
    q2, k2, v2 = run_prologue(sub)
    out2 = host_bits(h3attn_forward_log2(q2, k2, h3attn_v_transpose(v2)))
    torch.cuda.synchronize()
    assert np.array_equal(outs[0][:, 7:14], out2)


def test_scaled_path_permutation_equivariance(inputs):
    inp = inputs(0)
    perm = np.random.default_rng(3).permutation(inp.workload.seq_len)
    pinp = wl.Inputs(inp.workload, inp.q[perm], inp.k[perm], inp.v[perm], inp.gamma_q, inp.gamma_k,
                     np.ascontiguousarray(inp.pos[perm]), inp.stress_rows)
    outs = []
    for x in (inp, pinp):
        q, k, v = run_prologue(x)
        outs.append(host_f64(h3attn_forward_log2(q, k, h3attn_v_transpose(v))))
    torch.cuda.synchronize()
    ok, e = attention_ok(outs[1], outs[0][perm])
    assert ok, e


def test_scaled_path_no_writes_outside_buffers():
    L, H = 1000, 3
    n = L * H * 128
    guard = 4096
    inp = wl.random_document(L, H, seed=9)
    sentinel = 0x7FC1  # a bf16 NaN pattern no kernel produces from finite inputs
    bufs = []
    for bits in (inp.q, inp.k):
        full = np.full(n + 2 * guard, sentinel, np.uint16)
        full[guard:guard + n] = bits.ravel()
        bufs.append(dev_bf16(full))
    q = bufs[0][guard:guard + n].view(L, H, 128)
    k = bufs[1][guard:guard + n].view(L, H, 128)
    out_full = dev_bf16(np.full(n + 2 * guard, sentinel, np.uint16))
    out = out_full[guard:guard + n].view(L, H, 128)
    h3attn_qk_prologue_scaled(q, k, torch.from_numpy(inp.gamma_q).cuda(), torch.from_numpy(inp.gamma_k).cuda(),
                              torch.from_numpy(inp.pos).cuda(), Q_SCALE)
    h3attn_forward_log2(q, k, h3attn_v_transpose(dev_bf16(inp.v)), out)
    torch.cuda.synchronize()
    for t in (bufs[0], bufs[1], out_full):
        h = host_bits(t)
        assert np.all(h[:guard] == sentinel) and np.all(h[-guard:] == sentinel)
    assert not np.any(host_bits(out_full)[guard:guard + n] == sentinel)


# ------------------------------------------------------------------ one long head

def test_long_single_head_scaled_and_fused_paths():
    """L = 70001 tokens of one head (1094 key tiles, L mod 256 = 113, L mod 64 = 49,
    positions up to 5000): sampled rows of the scale-folded path against the
    oracle, and the fused path bit-identical to it."""
    from packed_full_attention_amd import h3attn_forward_log2_qprologue, h3attn_k_prologue_table
    L, H = 70001, 1
    inp = wl.random_document(L, H, seed=7001, pos_max=5000)
    print(f"long single head: L={L} H={H}", flush=True)
    q, k, v = run_prologue(inp)
    vt = h3attn_v_transpose(v)
    out = h3attn_forward_log2(q, k, vt)
    q2, k2, _, gq, gk, pos = dev_inputs(inp)
    cs = h3attn_k_prologue_table(k2, gk, pos)
    out2 = h3attn_forward_log2_qprologue(q2, k2, vt, gq, cs, Q_SCALE)
    torch.cuda.synchronize()
    got_all = host_bits(out)
    assert np.array_equal(host_bits(out2), got_all)
    rng = np.random.default_rng(7002)
    rows = np.unique(np.concatenate([[0, 1, L - 50, L - 49, L - 2, L - 1], rng.choice(L, 40, replace=False)]))
    heads = np.zeros_like(rows)
    ref = oracle.packed_attention_sampled(head_f64(inp.q), head_f64(inp.k), head_f64(inp.v), inp.gamma_q,
                                          inp.gamma_k, inp.pos, SCALE, rows, heads)
    got = wl.bf16_bits_to_f32(got_all[rows, 0]).astype(np.float64)
    ok, e = attention_ok(got, ref)
    print(f"long single head ({len(rows)} rows): {e}")
    assert ok, e


# ------------------------------------------------------------------ extreme score ranges

@pytest.mark.parametrize("alpha", [3.0, 8.0])
def test_dominant_keys_and_overflowing_weights(alpha):
    """Query i = alpha * k[j(i)] for a random key j(i): that key's score exceeds the
    others by about 30 (alpha 3) or 80 (alpha 8) in natural units, so the output is
    nearly v[j(i)].  The dominant key usually sits in a later tile than the first,
    so the exponent offset must move mid-row; at alpha 8 a tile's base-2 weights
    reach 2^130 and overflow fp32, which must also lead to a rebase, not to inf or
    NaN.  Plain and scale-folded kernels against the oracle."""
    from packed_full_attention_amd import h3attn_forward
    L, H = 700, 2
    rng = np.random.default_rng(int(alpha * 10))
    k = rng.standard_normal((L, H, 128)).astype(np.float32)
    v = rng.standard_normal((L, H, 128)).astype(np.float32)
    j = rng.integers(0, L, size=(L, H))
    q = alpha * k[j, np.arange(H)[None, :], :]
    qb, kb, vb = bf16_of(q), bf16_of(k), bf16_of(v)
    f = lambda b: wl.bf16_bits_to_f32(b).astype(np.float64)
    out_plain = h3attn_forward(dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), scale=SCALE)
    q2 = bf16_of(f(qb) * Q_SCALE)
    out_log2 = h3attn_forward_log2(dev_bf16(q2), dev_bf16(kb), h3attn_v_transpose(dev_bf16(vb)))
    torch.cuda.synchronize()
    for name, got, ref in (("plain", host_f64(out_plain), oracle.attention(f(qb), f(kb), f(vb), SCALE)),
                           ("log2", host_f64(out_log2), oracle.attention(f(q2), f(kb), f(vb), LN2))):
        ok, e = attention_ok(got, ref)
        print(f"alpha {alpha} {name}: {e}")
        assert ok, (name, e)
