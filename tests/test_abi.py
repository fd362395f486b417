"""C ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects invalid arguments before any HIP call.

Only calls that validation rejects are made here (with fake device addresses);
nothing is ever launched.
"""
import ctypes
import os
import re

import pytest

from packed_full_attention_amd import _binding as b

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "h3attn.h")


@pytest.fixture(scope="module")
def lib():
    return b.load_library()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(h3attn_\w+)\s*\(", src)))


def test_header_declares_the_expected_entry_points():
    assert declared_functions() == sorted(b.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert lib.h3attn_abi_version() == 8


def test_strerror_strings(lib):
    assert lib.h3attn_strerror(0) == b"success"
    assert lib.h3attn_strerror(1) == b"invalid argument"
    assert lib.h3attn_strerror(2) == b"unsupported geometry"
    assert lib.h3attn_strerror(3) == b"HIP launch error"
    assert lib.h3attn_strerror(99) == b"unknown status"


A = 0x7F0000000000            # fake, 256-byte aligned device addresses, far apart
B = 0x7F1000000000
C = 0x7F2000000000
O = 0x7F3000000000
G = 0x7F4000000000
P = 0x7F5000000000


def prologue(lib, q=A, k=B, gq=G, gk=G + 512, pos=P, L=160, H=4):
    return lib.h3attn_qk_prologue(q, k, gq, gk, pos, L, H, None)


def forward(lib, q=A, k=B, v=C, out=O, L=160, H=4, scale=0.08838834764831845):
    return lib.h3attn_forward(q, k, v, out, L, H, scale, None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(q=None), 1, "null"), (dict(k=None), 1, "null"), (dict(gq=None), 1, "null"),
    (dict(gk=None), 1, "null"), (dict(pos=None), 1, "null"),
    (dict(L=0), 1, "empty"), (dict(L=-5), 1, "L must"), (dict(H=0), 1, "H must"), (dict(H=-1), 1, "H must"),
    (dict(q=A + 8), 1, "aligned"), (dict(k=B + 2), 1, "aligned"), (dict(gq=G + 2), 1, "aligned"),
    (dict(pos=P + 1), 1, "aligned"),
    (dict(k=A + 160 * 4 * 128 * 2 - 256), 1, "overlap"), (dict(q=B - 256), 1, "overlap"),
    (dict(L=1 << 31), 2, "2^31"), (dict(L=(1 << 31) - 1, H=1 << 30), 2, "too large"),
    (dict(L=(1 << 30), H=1, k=A + (1 << 42)), 2, "grid"),
])
def test_prologue_rejects(lib, kw, code, msg):
    assert prologue(lib, **kw) == code
    assert msg in lib.h3attn_last_error().decode()


@pytest.mark.parametrize("kw,code,msg", [
    (dict(q=None), 1, "null"), (dict(k=None), 1, "null"), (dict(v=None), 1, "null"), (dict(out=None), 1, "null"),
    (dict(L=0), 1, "empty"), (dict(H=0), 1, "H must"),
    (dict(v=C + 8), 1, "aligned"), (dict(out=O + 4), 1, "aligned"),
    (dict(scale=0.0), 1, "scale"), (dict(scale=-1.0), 1, "scale"), (dict(scale=float("nan")), 1, "scale"),
    (dict(scale=float("inf")), 1, "scale"),
    (dict(out=A), 1, "overlap"), (dict(out=B + 1024), 1, "overlap"), (dict(out=C - 1024), 1, "overlap"),
    (dict(L=1 << 31), 2, "2^31"),
    (dict(L=(1 << 31) - 1, H=56, q=1 << 46, k=2 << 46, v=3 << 46, out=4 << 46), 2, "grid"),
])
def test_forward_rejects(lib, kw, code, msg):
    assert forward(lib, **kw) == code
    assert msg in lib.h3attn_last_error().decode()


def test_prologue_rejects_weights_or_positions_inside_q_or_k(lib):
    # q = A, k = B, each 160 * 4 * 128 * 2 bytes: gammas or positions inside either are rejected.
    for kw in (dict(gq=A + 1024), dict(gk=B + 4096), dict(pos=A + 256), dict(pos=B)):
        assert prologue(lib, **kw) == 1 and "overlaps" in lib.h3attn_last_error().decode()
    assert lib.h3attn_k_prologue_table(B, B + 512, P, C, 160, 4, None) == 1
    assert "k overlaps" in lib.h3attn_last_error().decode()
    assert lib.h3attn_k_prologue_table(B, G, B + 2048, C, 160, 4, None) == 1


def test_scaled_entry_points_reject(lib):
    f = lambda **kw: lib.h3attn_qk_prologue_scaled(kw.get("q", A), B, G, G + 512, P, kw.get("L", 160), 4,
                                                     kw.get("s", 0.1275), None)
    for s_ in (0.0, -1.0, float("nan"), float("inf")):
        assert f(s=s_) == 1 and "q_scale" in lib.h3attn_last_error().decode()
    assert f(q=None) == 1 and f(L=0) == 1 and f(q=A + 8) == 1
    g = lambda **kw: lib.h3attn_forward_log2(kw.get("q", A), B, kw.get("vt", C), kw.get("out", O), kw.get("L", 160),
                                             4, None)
    assert g(q=None) == 1 and g(L=-1) == 1 and g(vt=C + 8) == 1
    assert g(out=A) == 1 and "overlap" in lib.h3attn_last_error().decode()
    # vt is H * 128 * Lp * 2 bytes long, more than v: an out just past v's size still overlaps vt.
    assert g(out=C + 4 * 128 * 160 * 2) == 1 and "vt" in lib.h3attn_last_error().decode()
    t = lambda **kw: lib.h3attn_v_transpose(kw.get("v", A), kw.get("vt", B), kw.get("L", 160), 4, None)
    assert t(v=None) == 1 and t(vt=None) == 1 and t(L=0) == 1 and t(vt=B + 4) == 1
    assert t(vt=A + 1024) == 1 and "overlap" in lib.h3attn_last_error().decode()


def test_fused_entry_points_reject(lib):
    kp = lambda **kw: lib.h3attn_k_prologue_table(kw.get("k", B), kw.get("gk", G), kw.get("pos", P),
                                                  kw.get("cs", C), kw.get("L", 160), kw.get("H", 4), None)
    for kw in (dict(k=None), dict(gk=None), dict(pos=None), dict(cs=None)):
        assert kp(**kw) == 1 and "null" in lib.h3attn_last_error().decode()
    assert kp(L=0) == 1 and kp(H=0) == 1
    assert kp(cs=C + 4) == 1 and "aligned" in lib.h3attn_last_error().decode()
    assert kp(k=B + 8) == 1 and kp(pos=P + 2) == 1
    assert kp(cs=B + 1024) == 1 and "overlap" in lib.h3attn_last_error().decode()
    assert kp(cs=P - 256) == 1 and "overlap" in lib.h3attn_last_error().decode()
    fq = lambda **kw: lib.h3attn_forward_log2_qprologue(kw.get("q", A), B, kw.get("vt", C), kw.get("out", O),
                                                        kw.get("gq", G), kw.get("cs", P), kw.get("L", 160), 4,
                                                        kw.get("s", 0.1275), None)
    for kw in (dict(q=None), dict(vt=None), dict(out=None), dict(gq=None), dict(cs=None)):
        assert fq(**kw) == 1 and "null" in lib.h3attn_last_error().decode()
    assert fq(gq=G + 4) == 1 and "aligned" in lib.h3attn_last_error().decode()
    assert fq(cs=P + 8) == 1 and "aligned" in lib.h3attn_last_error().decode()
    for s_ in (0.0, -1.0, float("nan"), float("inf")):
        assert fq(s=s_) == 1 and "q_scale" in lib.h3attn_last_error().decode()
    for out in (A, B + 256, C + 1024, G - 256, P + 4096):
        assert fq(out=out) == 1 and "overlap" in lib.h3attn_last_error().decode()
    assert fq(L=1 << 31) == 2


def test_fp8_entry_points_reject(lib):
    kv = lambda **kw: lib.h3attn_kv_prologue_fp8(kw.get("k", A), kw.get("v", B), kw.get("gk", G), kw.get("pos", P),
                                                 kw.get("cs", C), kw.get("k8", O), kw.get("vt", O + (1 << 30)),
                                                 kw.get("L", 160), kw.get("H", 4), None)
    for kw in (dict(k=None), dict(v=None), dict(gk=None), dict(pos=None), dict(cs=None), dict(k8=None),
               dict(vt=None)):
        assert kv(**kw) == 1 and "null" in lib.h3attn_last_error().decode()
    assert kv(L=0) == 1 and kv(H=0) == 1 and kv(L=-5) == 1
    assert kv(k8=O + 8) == 1 and "aligned" in lib.h3attn_last_error().decode()
    assert kv(gk=G + 2) == 1 and "aligned" in lib.h3attn_last_error().decode()
    # k8 is L * H * 128 bytes; it may not overlap k (read) or vt (written)
    for k8 in (A + 1024, B, C + 64, P - 256):
        assert kv(k8=k8) == 1 and "overlap" in lib.h3attn_last_error().decode()
    assert kv(vt=O + 160 * 4 * 128 - 256) == 1 and "overlap" in lib.h3attn_last_error().decode()
    ff = lambda **kw: lib.h3attn_forward_fp8_qprologue(kw.get("q", A), kw.get("k8", B), kw.get("vt", C),
                                                       kw.get("out", O), kw.get("gq", G), kw.get("cs", P),
                                                       kw.get("L", 160), kw.get("H", 4), kw.get("s", 0.1275), None)
    for kw in (dict(q=None), dict(k8=None), dict(vt=None), dict(out=None), dict(gq=None), dict(cs=None)):
        assert ff(**kw) == 1 and "null" in lib.h3attn_last_error().decode()
    assert ff(k8=B + 8) == 1 and "aligned" in lib.h3attn_last_error().decode()
    for s_ in (0.0, -1.0, float("nan"), float("inf")):
        assert ff(s=s_) == 1 and "q_scale" in lib.h3attn_last_error().decode()
    for out in (A, B + 128, C + 1024, G - 256, P + 4096):
        assert ff(out=out) == 1 and "overlap" in lib.h3attn_last_error().decode()
    assert ff(L=1 << 31) == 2
    big = FAR
    assert lib.h3attn_forward_fp8_qprologue(big[0], big[1], big[2], big[3], big[4], big[5], 64, H_WRAP, 0.1275,
                                            None) == 2
    assert "2^32" in lib.h3attn_last_error().decode()
    assert lib.h3attn_forward_fp8_qprologue(big[0], big[1], big[2], big[3], big[4], big[5], L_VT_WRAP, 1, 0.1275,
                                            None) == 2
    assert "vt" in lib.h3attn_last_error().decode()
    assert lib.h3attn_kv_prologue_fp8(big[0], big[1], big[2], big[3], big[4], big[5], big[6], 1, (1 << 30) - 31,
                                      None) == 2


def test_training_entry_points_reject(lib):
    fl = lambda **kw: lib.h3attn_forward_log2_lse(kw.get("q", A), B, kw.get("vt", C), kw.get("out", O),
                                                  kw.get("lse", G), kw.get("L", 160), 4, None)
    for kw in (dict(q=None), dict(vt=None), dict(out=None), dict(lse=None)):
        assert fl(**kw) == 1 and "null" in lib.h3attn_last_error().decode()
    assert fl(lse=G + 2) == 1 and "aligned" in lib.h3attn_last_error().decode()
    assert fl(lse=A + 512) == 1 and "overlap" in lib.h3attn_last_error().decode()
    assert fl(L=0) == 1
    pb = lambda **kw: lib.h3attn_qk_prologue_backward_scaled(A, B, G, G + 512, P, C, O, G + 1024, G + 1536,
                                                             kw.get("ws", G + 4096), kw.get("L", 160), 4,
                                                             kw.get("s", 0.1275), None)
    for s_ in (0.0, -2.0, float("nan"), float("inf")):
        assert pb(s=s_) == 1 and "q_scale" in lib.h3attn_last_error().decode()
    assert pb(ws=None) == 1 and pb(L=-3) == 1
    assert pb(ws=C + 64) == 1 and "overlap" in lib.h3attn_last_error().decode()


@pytest.mark.parametrize("L,H,want", [(160, 4, 160 * 384), (1, 56, 384), (16500, 56, 16500 * 384), (0, 4, -1),
                                      (8, 0, -1)])
def test_rope_table_bytes(lib, L, H, want):
    assert lib.h3attn_rope_table_bytes(L, H) == want


@pytest.mark.parametrize("L,H,want", [
    (160, 4, 4 * 128 * 192 * 2), (64, 1, 128 * 64 * 2), (65, 1, 128 * 128 * 2), (1, 56, 56 * 128 * 64 * 2),
    (16500, 56, 56 * 128 * 16512 * 2), (0, 4, -1), (160, 0, -1), (1 << 31, 1, -1),
])
def test_vt_bytes(lib, L, H, want):
    assert lib.h3attn_vt_bytes(L, H) == want


def test_binding_rejects_bad_tensors_on_cpu():
    import torch
    q = torch.zeros(8, 2, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        b.h3attn_forward(q, q, q)
    with pytest.raises(TypeError, match="bfloat16"):
        b.h3attn_forward(q.float(), q, q)
    with pytest.raises(ValueError, match=r"\[L, H, 128\]"):
        b.h3attn_forward(torch.zeros(8, 2, 64, dtype=torch.bfloat16), q, q)
    with pytest.raises(ValueError, match="GPU"):
        b.h3attn_qk_prologue(q, q.clone(), torch.ones(128), torch.ones(128),
                             torch.zeros(8, 3, dtype=torch.int32))


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError, match="no fallback"):
        b.load_library(str(tmp_path / "libh3attn.so"))


# Geometries whose tile DMA offsets would pass 2^32 bytes (the kernels address a
# tile through a buffer resource with 32-bit offsets): rejected, never launched.
# Fake addresses 2^44 apart, so no size overlaps another range.
FAR = [(i + 1) << 44 for i in range(12)]
H_WRAP = 266305        # 63 * H * 256 + 256 > 2^32 - 1 (H = 266304 still fits)
L_VT_WRAP = 16909313   # Lp = 16909376: 127 * 2 * Lp + 128 > 2^32 - 1


def test_row_tile_span_rejected_on_every_attention_entry_point(lib):
    L, H = 64, H_WRAP
    q, k, v, out, lse, vt, gq, cs, dout, dq, dk, dv = FAR
    ws = FAR[11] + (1 << 43)
    calls = {
        "forward": lambda: lib.h3attn_forward(q, k, v, out, L, H, 0.088, None),
        "forward_lse": lambda: lib.h3attn_forward_lse(q, k, v, out, lse, L, H, 0.088, None),
        "forward_log2": lambda: lib.h3attn_forward_log2(q, k, vt, out, L, H, None),
        "forward_log2_lse": lambda: lib.h3attn_forward_log2_lse(q, k, vt, out, lse, L, H, None),
        "forward_log2_qprologue": lambda: lib.h3attn_forward_log2_qprologue(q, k, vt, out, gq, cs, L, H, 0.1275,
                                                                            None),
        "attention_backward": lambda: lib.h3attn_attention_backward(q, k, v, out, dout, lse, dq, dk, dv, ws, L, H,
                                                                    0.088, None),
    }
    for name, call in calls.items():
        assert call() == 2, name
        assert "2^32" in lib.h3attn_last_error().decode(), name


def test_vt_tile_span_rejected_on_the_vt_entry_points(lib):
    L, H = L_VT_WRAP, 1
    q, k, out, lse, vt, gq, cs = FAR[:7]
    for name, call in {
        "forward_log2": lambda: lib.h3attn_forward_log2(q, k, vt, out, L, H, None),
        "forward_log2_lse": lambda: lib.h3attn_forward_log2_lse(q, k, vt, out, lse, L, H, None),
        "forward_log2_qprologue": lambda: lib.h3attn_forward_log2_qprologue(q, k, vt, out, gq, cs, L, H, 0.1275,
                                                                            None),
    }.items():
        assert call() == 2, name
        msg = lib.h3attn_last_error().decode()
        assert "vt" in msg and "2^32" in msg, (name, msg)


def test_prologue_row_count_overflow_rejected(lib):
    L, H = 1, (1 << 30) - 31  # 2H + 64 > 2^31 - 1
    q, k, gq, gk, pos, cs, dq, dk, dgq, dgk, ws = FAR[:11]
    for name, call in {
        "qk_prologue": lambda: lib.h3attn_qk_prologue(q, k, gq, gk, pos, L, H, None),
        "qk_prologue_scaled": lambda: lib.h3attn_qk_prologue_scaled(q, k, gq, gk, pos, L, H, 0.5, None),
        "k_prologue_table": lambda: lib.h3attn_k_prologue_table(k, gk, pos, cs, L, H, None),
        "qk_prologue_backward": lambda: lib.h3attn_qk_prologue_backward(q, k, gq, gk, pos, dq, dk, dgq, dgk, ws, L,
                                                                        H, None),
        "qk_prologue_backward_scaled": lambda: lib.h3attn_qk_prologue_backward_scaled(
            q, k, gq, gk, pos, dq, dk, dgq, dgk, ws, L, H, 0.5, None),
    }.items():
        assert call() == 2, name
        assert "prologue" in lib.h3attn_last_error().decode(), name


def test_noalloc_backward_rejects_before_any_hip_call(lib):
    # Beyond the library's 16 MiB of statistics (H * Lp <= 2^21): rejected.
    q, k, v, out, dout, lse, dq, dk, dv = FAR[:9]
    f = lambda L, H, **kw: lib.h3attn_attention_backward_noalloc(kw.get("q", q), k, v, out, dout, lse, dq, dk, dv,
                                                                 L, H, kw.get("s", 0.088), None)
    assert f(37504, 56) == 2 and "scratch" in lib.h3attn_last_error().decode()
    assert f((1 << 21) + 1, 1) == 2  # Lp = 2^21 + 64 at H = 1 (2^21 itself is the limit)
    assert f(64, 1, q=None) == 1 and "null" in lib.h3attn_last_error().decode()
    assert f(0, 1) == 1 and f(64, 1, s=0.0) == 1 and f(64, 1, q=FAR[0] + 8) == 1
    assert f(64, H_WRAP) == 2
