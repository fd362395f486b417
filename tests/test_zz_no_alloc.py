"""h3attn_attention_backward_noalloc (the attention backward with its per-row
statistics in the library's own device array, for callers that cannot
allocate) against h3attn_attention_backward with a caller workspace: the same
kernels, so the gradients must agree bit for bit.  Two calls in a row, the
second on a smaller (L, H), so the second reads nothing the first left behind
in the shared array; the workspace form's gradients are themselves compared
with the fp64 oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
from gates import gradient_ok
from gpu_util import dev_bf16, host_f64
from packed_full_attention_amd import (h3attn_attention_backward, h3attn_attention_backward_noalloc,
                                       h3attn_forward_lse)
from packed_full_attention_amd import workloads as wl

pytestmark = pytest.mark.gpu
SCALE = 1.0 / math.sqrt(128.0)


def _bits(shape, seed):
    return wl.bf16_bits(np.random.default_rng(seed).standard_normal(shape).astype(np.float32))


def test_noalloc_backward_matches_workspace_form():
    for L, H, seed in ((2000, 8, 1), (700, 3, 2)):
        print(f"no-alloc backward, L={L} H={H}", flush=True)
        qb, kb, vb, db = (_bits((L, H, 128), 10 * seed + i) for i in range(4))
        q, k, v, do = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb), dev_bf16(db)
        out, lse = h3attn_forward_lse(q, k, v, scale=SCALE)
        ref = h3attn_attention_backward(q, k, v, out, do, lse, scale=SCALE)
        got = tuple(torch.full_like(q, float("nan")) for _ in range(3))
        h3attn_attention_backward_noalloc(q, k, v, out, do, lse, *got, scale=SCALE)
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), got, ref):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), (L, H, name)
        f = lambda x: wl.bf16_bits_to_f32(x).astype(np.float64)
        want = oracle.attention_backward(host_f64(q), host_f64(k), host_f64(v), f(db), SCALE)
        for name, a, w in zip(("dq", "dk", "dv"), got, want):
            ok, e = gradient_ok(host_f64(a), w)
            assert ok, (L, H, name, e)
