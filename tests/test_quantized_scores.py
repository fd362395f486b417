"""Why the score product stays bf16: quantized Q'K^T measured against the gate.

A quantized score product in the spirit of the SageAttention baseline that the
"H3 Parity Evidence Ledger" page names -- Q' and K' rounded to 8-bit values with
a per-row scale (OCP FP8 e4m3, or symmetric INT8), the P V product unchanged --
is evaluated here in float64 against the oracle on the workloads' own inputs.
It misses the attention gate (tests/gates.py: relative L2 <= 1e-2, max-abs
<= 2e-2): e4m3 keeps 3 mantissa bits, so the scores carry a relative error of
about 2^-4 per term; INT8 sits at the relative-L2 limit on ordinary rows and
both fail on the stressed workload (K' rows x8), whose large scores turn small
relative score errors into large weight errors.  The bf16 path passes the same
gate with a wide margin (the last test).  CPU only.
"""
import math

import numpy as np
import pytest

import oracle
from gates import attention_ok
from packed_full_attention_amd import workloads as wl

SCALE = 1.0 / math.sqrt(128.0)


def e4m3(x):
    """Round to OCP FP8 e4m3 (round half to even, saturating at 448)."""
    a = np.abs(x)
    e = np.maximum(np.floor(np.log2(np.maximum(a, 1e-300))), -6.0)  # subnormal step 2^-9
    step = 2.0 ** (e - 3.0)
    return np.sign(x) * np.minimum(np.round(a / step) * step, 448.0)


def fp8_rows(x):
    s = 448.0 / np.maximum(np.abs(x).max(axis=1, keepdims=True), 1e-300)
    return e4m3(x * s) / s


def int8_rows(x):
    s = 127.0 / np.maximum(np.abs(x).max(axis=1, keepdims=True), 1e-300)
    return np.clip(np.round(x * s), -127, 127) / s


def _head(idx, h=0):
    inp = wl.make_inputs(idx)
    f = lambda bits: wl.bf16_bits_to_f32(np.ascontiguousarray(bits[:, h])).astype(np.float64)
    q = wl.round_to_bf16(oracle.mm_rope(oracle.rms_norm(f(inp.q), inp.gamma_q), inp.pos).astype(np.float32))
    k = wl.round_to_bf16(oracle.mm_rope(oracle.rms_norm(f(inp.k), inp.gamma_k), inp.pos).astype(np.float32))
    q, k = q.astype(np.float64), k.astype(np.float64)
    if len(inp.stress_rows):
        k[inp.stress_rows] *= 8.0
    return q, k, f(inp.v)


@pytest.mark.parametrize("quant", [fp8_rows, int8_rows], ids=["fp8_e4m3", "int8"])
def test_quantized_scores_fail_the_gate_on_the_stressed_workload(quant):
    q, k, v = _head(2)
    ref = oracle.attention_head(q, k, v, SCALE)
    ok, e = attention_ok(oracle.attention_head(quant(q), quant(k), v, SCALE), ref)
    print(quant.__name__, e)
    assert not ok and e["max_abs"] > 10 * 2e-2


def test_fp8_scores_fail_relative_l2_on_an_ordinary_workload():
    q, k, v = _head(1)
    ref = oracle.attention_head(q, k, v, SCALE)
    ok, e = attention_ok(oracle.attention_head(fp8_rows(q), fp8_rows(k), v, SCALE), ref)
    print(e)
    assert not ok and e["rel_l2"] > 2e-2


def test_bf16_scores_pass_with_margin():
    q, k, v = _head(2)
    ref = oracle.attention_head(q, k, v, SCALE)
    # the inputs are already bf16; round P to bf16 as the kernel does
    s = (q @ k.T) * SCALE
    p = np.exp(s - s.max(axis=1, keepdims=True))
    pb = wl.round_to_bf16(p.astype(np.float32)).astype(np.float64)
    out = (pb @ v) / pb.sum(axis=1, keepdims=True)
    ok, e = attention_ok(out, ref)
    print(e)
    assert ok and e["max_abs"] < 2e-2 / 4
