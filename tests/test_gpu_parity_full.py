"""GPU parity on every output of all five workloads: the three forms of the whole
path, called through the C ABI, against the fp64 oracle on every (row, head,
channel) -- including the two long workloads (L = 16500, H = 56 and L = 28976,
H = 7), run in the launch configuration the benchmark times.

The forms ("MiniMax-H3 WS1/WS2 kernel roadmap" RFC, section 5 items
h3_qk_rmsnorm_d128, h3_mm_rope_3axis_partial, h3_full_attention):
  plain         h3attn_qk_prologue + h3attn_forward
  scale-folded  h3attn_qk_prologue_scaled (q' carries scale log2 e) +
                h3attn_v_transpose + h3attn_forward_log2
  fused         h3attn_kv_prologue (K's prologue, the rotation table and V^T
                in one launch) + h3attn_forward_log2_qprologue (Q's prologue
                inside attention), the form the benchmark times
Gates (tests/gates.py): attention output max-abs <= 2e-2, mean-abs <= 2e-3 and
rel-L2 <= 1e-2 over all outputs; the prologue outputs that leave the GPU (Q'
and K', or K' alone for the fused form) |gpu - ref| <= 2^-8 (|ref| + 1) per
element.  The stressed workload runs its literal reading (K rows x 8 before the
prologue).  The oracle runs head by head on all host cores (tests/oracle_pool.py).
"""
import math
import time

import numpy as np
import pytest
import torch

import oracle_pool
from gates import attention_ok, prologue_ok
from gpu_util import dev_bf16, dev_inputs, host_f64
from packed_full_attention_amd import (h3attn_forward, h3attn_forward_log2, h3attn_forward_log2_qprologue,
                                       h3attn_kv_prologue, h3attn_qk_prologue, h3attn_qk_prologue_scaled,
                                       h3attn_v_transpose)
from packed_full_attention_amd import workloads as wl

pytestmark = pytest.mark.gpu
SCALE = 1.0 / math.sqrt(128.0)
Q_SCALE = float(np.float32(SCALE * math.log2(math.e)))
PATHS = ("plain", "scale_folded", "fused")


@pytest.fixture(scope="module")
def reference():
    cache = {}

    def get(idx):
        if idx not in cache:
            cache.clear()  # one workload's reference in memory at a time
            inp = wl.make_inputs(idx)
            if len(inp.stress_rows):
                inp = wl.Inputs(inp.workload, inp.q, wl.scale_rows_bf16(inp.k, inp.stress_rows, 3), inp.v,
                                inp.gamma_q, inp.gamma_k, inp.pos, inp.stress_rows)
            t0 = time.perf_counter()
            out, qr, kr = oracle_pool.packed_attention_full(inp.q, inp.k, inp.v, inp.gamma_q, inp.gamma_k, inp.pos,
                                                            SCALE)
            print(f"oracle, workload {idx} ({inp.workload.describe()}): {time.perf_counter() - t0:.1f} s "
                  f"on {oracle_pool.workers()} threads", flush=True)
            cache[idx] = (inp, out, qr, kr)
        return cache[idx]
    return get


def _check(tag, ok_e):
    ok, e = ok_e
    print(f"{tag}: {e}", flush=True)
    assert ok, (tag, e)


@pytest.mark.parametrize("idx,path", [(i, p) for i in range(5) for p in PATHS])
def test_path_parity_full(reference, idx, path):
    inp, ref, qr, kr = reference(idx)
    q, k, v, gq, gk, pos = dev_inputs(inp)
    print(f"workload {idx}, {path} path, L={inp.workload.seq_len} H={q.shape[1]}", flush=True)
    if path == "plain":
        h3attn_qk_prologue(q, k, gq, gk, pos)
        out = h3attn_forward(q, k, v, scale=SCALE)
        checks = (("q'", q, qr), ("k'", k, kr))
    elif path == "scale_folded":
        h3attn_qk_prologue_scaled(q, k, gq, gk, pos, Q_SCALE)
        out = h3attn_forward_log2(q, k, h3attn_v_transpose(v))
        checks = (("q' (scaled)", q, qr * Q_SCALE), ("k'", k, kr))
    else:
        cs, vt = h3attn_kv_prologue(k, v, gk, pos)
        out = h3attn_forward_log2_qprologue(q, k, vt, gq, cs, Q_SCALE)
        checks = (("k'", k, kr),)
    torch.cuda.synchronize()
    for name, got, want in checks:
        _check(f"workload {idx} {path} {name}", prologue_ok(host_f64(got), want))
    _check(f"workload {idx} {path} out", attention_ok(host_f64(out), ref))
