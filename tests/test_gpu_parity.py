"""GPU parity: the HIP path, called through the C ABI, against the fp64 oracle.

Gates (tests/gates.py): attention output max-abs <= 2e-2, mean-abs <= 2e-3,
rel-L2 <= 1e-2; prologue output |gpu - ref| <= 2^-8 (|ref| + 1) per element and
mean-abs <= 2e-3.  The three small workloads are compared on every element;
for the two long ones (L = 16500, H = 56 and L = 28976, H = 7) the attention
kernel alone, on the raw generated inputs, is compared on sampled outputs the
oracle computes one by one (the whole path at those sizes is compared on every
output in test_gpu_parity_full.py).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from gates import attention_ok, prologue_ok
from gpu_util import dev_bf16, dev_inputs, head_f64, host_bits, host_f64, sample_heads, sample_rows
from packed_full_attention_amd import h3attn_forward, h3attn_qk_prologue
from packed_full_attention_amd import workloads as wl

pytestmark = pytest.mark.gpu
SCALE = 1.0 / math.sqrt(128.0)
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


def run_prologue(inp):
    q, k, v, gq, gk, pos = dev_inputs(inp)
    h3attn_qk_prologue(q, k, gq, gk, pos)
    torch.cuda.synchronize()
    return q, k, v


# ------------------------------------------------------------------ prologue

@pytest.mark.parametrize("idx", SMALL)
def test_prologue_parity_full(inputs, idx):
    inp = inputs(idx)
    q, k, _ = run_prologue(inp)
    rq, rk = oracle.qk_prologue(inp.as_f64("q"), inp.as_f64("k"), inp.gamma_q, inp.gamma_k, inp.pos)
    for name, got, ref in (("q", host_f64(q), rq), ("k", host_f64(k), rk)):
        ok, e = prologue_ok(got, ref)
        print(f"prologue workload {idx} {name}: {e}")
        assert ok, (name, e)


# ------------------------------------------------------------------ attention alone

def bf16_of(x: np.ndarray) -> np.ndarray:
    return wl.bf16_bits(x.astype(np.float32))


@pytest.mark.parametrize("idx", SMALL)
def test_forward_parity_full(inputs, idx):
    # Inputs: the oracle's prologue output rounded to bf16 (and, for the
    # stressed workload, its chosen K token rows multiplied by 8 after the
    # prologue); both sides attend over exactly these bf16 values.
    inp = inputs(idx)
    rq, rk = oracle.qk_prologue(inp.as_f64("q"), inp.as_f64("k"), inp.gamma_q, inp.gamma_k, inp.pos)
    qb, kb = bf16_of(rq), bf16_of(rk)
    kb = wl.scale_rows_bf16(kb, inp.stress_rows, 3)
    out = h3attn_forward(dev_bf16(qb), dev_bf16(kb), dev_bf16(inp.v))
    torch.cuda.synchronize()
    f = lambda b: wl.bf16_bits_to_f32(b).astype(np.float64)
    ref = oracle.attention(f(qb), f(kb), inp.as_f64("v"), SCALE)
    ok, e = attention_ok(host_f64(out), ref)
    print(f"forward workload {idx} (stress rows {len(inp.stress_rows)}): {e}")
    assert ok, e


@pytest.mark.parametrize("idx", LONG)
def test_forward_parity_sampled_long(inputs, idx):
    # The generated bf16 q, k, v go straight into the attention kernel.
    inp = inputs(idx)
    out = h3attn_forward(dev_bf16(inp.q), dev_bf16(inp.k), dev_bf16(inp.v))
    torch.cuda.synchronize()
    rows, heads = sample_rows(inp.workload, 96, 11 + idx), sample_heads(inp.workload)
    got_all = host_bits(out)
    qh, kh, vh = head_f64(inp.q), head_f64(inp.k), head_f64(inp.v)
    got, ref = [], []
    for h in heads:
        ref.append(oracle.attention_head(qh(h)[rows], kh(h), vh(h), SCALE))
        got.append(wl.bf16_bits_to_f32(got_all[rows, h]).astype(np.float64))
    ok, e = attention_ok(np.stack(got), np.stack(ref))
    print(f"forward workload {idx} ({len(rows)} rows x {len(heads)} heads): {e}")
    assert ok, e


# ------------------------------------------------------------------ whole path

@pytest.mark.parametrize("idx", SMALL)
def test_path_parity_full(inputs, idx):
    # For the stressed workload this is the literal reading: K rows x 8 before
    # the prologue (the RMSNorm then removes the scale up to eps).
    inp = inputs(idx)
    kbits = wl.scale_rows_bf16(inp.k, inp.stress_rows, 3)
    q, k, v, gq, gk, pos = dev_inputs(inp)
    k = dev_bf16(kbits)
    h3attn_qk_prologue(q, k, gq, gk, pos)
    out = h3attn_forward(q, k, v)
    torch.cuda.synchronize()
    kf = wl.bf16_bits_to_f32(kbits).astype(np.float64)
    ref = oracle.packed_attention(inp.as_f64("q"), kf, inp.as_f64("v"), inp.gamma_q, inp.gamma_k,
                                  inp.pos, SCALE)
    ok, e = attention_ok(host_f64(out), ref)
    print(f"path workload {idx}: {e}")
    assert ok, e


# ------------------------------------------------------------------ edge cases

@pytest.mark.parametrize("L,H", [(1, 1), (2, 3), (3, 1), (31, 2), (32, 1), (33, 1), (63, 1), (64, 2),
                                 (65, 1), (127, 1), (128, 2), (129, 1), (200, 3), (1000, 2),
                                 (300, 128), (513, 97)])
def test_path_edge_lengths(L, H):
    inp = wl.random_document(L, H, seed=100 + L + H, pos_max=2000)
    q, k, v, gq, gk, pos = dev_inputs(inp)
    h3attn_qk_prologue(q, k, gq, gk, pos)
    pro_q, pro_k = host_f64(q), host_f64(k)
    out = h3attn_forward(q, k, v)
    torch.cuda.synchronize()
    rq, rk = oracle.qk_prologue(inp.as_f64("q"), inp.as_f64("k"), inp.gamma_q, inp.gamma_k, inp.pos)
    assert prologue_ok(pro_q, rq)[0] and prologue_ok(pro_k, rk)[0]
    ref = oracle.attention(rq, rk, inp.as_f64("v"), SCALE)
    ok, e = attention_ok(host_f64(out), ref)
    assert ok, (L, H, e)


def test_zero_queries_give_column_mean_of_v():
    inp = wl.random_document(300, 2, seed=5)
    qz = torch.zeros(300, 2, 128, dtype=torch.bfloat16, device="cuda")
    out = h3attn_forward(qz, dev_bf16(inp.k), dev_bf16(inp.v))
    torch.cuda.synchronize()
    ref = np.broadcast_to(inp.as_f64("v").mean(axis=0), (300, 2, 128))
    ok, e = attention_ok(host_f64(out), ref)
    assert ok, e


def test_other_scales():
    inp = wl.random_document(257, 2, seed=6)
    for scale in (0.02, 0.25):
        out = h3attn_forward(dev_bf16(inp.q), dev_bf16(inp.k), dev_bf16(inp.v), scale=scale)
        torch.cuda.synchronize()
        ref = oracle.attention(inp.as_f64("q"), inp.as_f64("k"), inp.as_f64("v"), scale)
        ok, e = attention_ok(host_f64(out), ref)
        assert ok, (scale, e)


# ------------------------------------------------------------------ invariants

def test_repeat_runs_are_bit_identical(inputs):
    # Repeat identical calls: zero drift (RFC section 6.3, control H-C0).
    inp = inputs(1)
    outs = []
    for _ in range(2):
        q, k, v = run_prologue(inp)
        outs.append((host_bits(q), host_bits(k), host_bits(h3attn_forward(q, k, v))))
        torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


def test_head_subset_is_bit_identical(inputs):
    # Heads are independent: heads 7..13 of the 56-head run equal an H = 7 run.
    inp = inputs(1)
    q, k, v = run_prologue(inp)
    out = host_bits(h3attn_forward(q, k, v))
    sub = wl.Inputs(inp.workload, np.ascontiguousarray(inp.q[:, 7:14]), np.ascontiguousarray(inp.k[:, 7:14]),
                    np.ascontiguousarray(inp.v[:, 7:14]), inp.gamma_q, inp.gamma_k, inp.pos, inp.stress_rows)
    q2, k2, v2 = run_prologue(sub)
    out2 = host_bits(h3attn_forward(q2, k2, v2))
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(q)[:, 7:14], host_bits(q2))
    assert np.array_equal(out[:, 7:14], out2)


def test_permutation_equivariance(inputs):
    # Permute packed rows together with their positions (RFC section 6.3, H-C3).
    inp = inputs(0)
    perm = np.random.default_rng(3).permutation(inp.workload.seq_len)
    pinp = wl.Inputs(inp.workload, inp.q[perm], inp.k[perm], inp.v[perm], inp.gamma_q, inp.gamma_k,
                     np.ascontiguousarray(inp.pos[perm]), inp.stress_rows)
    outs = []
    for x in (inp, pinp):
        q, k, v = run_prologue(x)
        outs.append(host_f64(h3attn_forward(q, k, v)))
    torch.cuda.synchronize()
    ok, e = attention_ok(outs[1], outs[0][perm])
    assert ok, e


def test_global_position_shift_invariance(inputs):
    inp = inputs(0)
    sh = wl.Inputs(inp.workload, inp.q, inp.k, inp.v, inp.gamma_q, inp.gamma_k,
                   inp.pos + np.array([5, 3, 2], np.int32), inp.stress_rows)
    q, k, v = run_prologue(sh)
    out = host_f64(h3attn_forward(q, k, v))
    torch.cuda.synchronize()
    ref = oracle.packed_attention(inp.as_f64("q"), inp.as_f64("k"), inp.as_f64("v"), inp.gamma_q,
                                  inp.gamma_k, inp.pos, SCALE)
    ok, e = attention_ok(out, ref)
    assert ok, e


# ------------------------------------------------------------------ memory safety

def test_no_writes_outside_buffers():
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
    h3attn_qk_prologue(q, k, torch.from_numpy(inp.gamma_q).cuda(), torch.from_numpy(inp.gamma_k).cuda(),
                       torch.from_numpy(inp.pos).cuda())
    h3attn_forward(q, k, dev_bf16(inp.v), out)
    torch.cuda.synchronize()
    for t in (bufs[0], bufs[1], out_full):
        h = host_bits(t)
        assert np.all(h[:guard] == sentinel) and np.all(h[-guard:] == sentinel)
    assert not np.any(host_bits(out_full)[guard:guard + n] == sentinel)


def test_side_stream_and_binding_errors():
    inp = wl.random_document(130, 2, seed=10)
    q, k, v = dev_bf16(inp.q), dev_bf16(inp.k), dev_bf16(inp.v)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out = h3attn_forward(q, k, v)
    s.synchronize()
    ref = oracle.attention(inp.as_f64("q"), inp.as_f64("k"), inp.as_f64("v"), SCALE)
    assert attention_ok(host_f64(out), ref)[0]
    with pytest.raises(ValueError, match="contiguous"):
        h3attn_forward(q.transpose(0, 1).contiguous().transpose(0, 1), k, v)
    with pytest.raises(TypeError):
        h3attn_forward(q.half(), k, v)
    with pytest.raises(RuntimeError, match="overlap"):
        h3attn_forward(q, k, v, out=q)
    with pytest.raises(ValueError):
        h3attn_qk_prologue(q, k, torch.ones(128, device="cuda"), torch.ones(128, device="cuda"),
                           torch.zeros(129, 3, dtype=torch.int32, device="cuda"))
