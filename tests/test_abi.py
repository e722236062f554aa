"""The C ABI: library loads, exports what include/dfs.h declares, and rejects bad
arguments on the host before touching any device (CPU only; no compute calls)."""
import ctypes
import os
import re

import pytest

import draft_selection_position_amd as dfs

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "dfs.h")
P = 0x10000  # a fake, 256-byte-aligned device address; never dereferenced by these calls
OK, E_NULL, E_SHAPE, E_UNSUP, E_WS, E_ALIGN, E_HIP, E_ARCH, E_ARG, E_TOO_LARGE = range(10)


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dfs_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(dfs.lib_path()):
        pytest.skip("libdfs.so not built")
    return dfs.lib()


def test_every_declared_symbol_is_exported(L):
    names = _declared()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), n


def test_abi_version_and_status_strings(L):
    assert L.dfs_abi_version() == 105
    for code in range(10):
        s = dfs.status_str(code)
        assert s.startswith("DFS_")
    assert dfs.status_str(12345) == "unknown dfs status"


def test_workspace_queries_are_host_only(L):
    assert dfs.topk_workspace_bytes(4096, 151936, __import__("torch").bfloat16) == 0  # one chunk per row
    assert dfs.topk_workspace_bytes(16, 151936, __import__("torch").bfloat16) > 0  # split rows
    assert L.dfs_topk_workspace_bytes(0, 100, 1) == 0
    assert dfs.gate_workspace_bytes(16, 5120, __import__("torch").bfloat16) > 0
    nb = dfs.select_workspace_bytes(256, 16, 151936, 5120)
    assert 4 << 20 < nb < 64 << 20
    assert dfs.select_workspace_bytes(1, 17, 1000, 64) == 0  # L > 16 is rejected


def _topk(L, logits=P, dt=1, rows=8, V=1000, k=16, idx=P, val=P, ws=P, wsb=1 << 20):
    return L.dfs_topk(logits, dt, rows, V, k, idx, val, ws, wsb, None)


def test_topk_validation(L):
    assert _topk(L, logits=None) == E_NULL
    assert _topk(L, idx=None) == E_NULL
    assert _topk(L, k=8) == E_UNSUP
    assert _topk(L, dt=7) == E_UNSUP
    assert _topk(L, rows=0) == E_SHAPE
    assert _topk(L, V=15) == E_SHAPE
    assert _topk(L, V=2**31) == E_SHAPE
    assert _topk(L, logits=P + 1) == E_ALIGN
    assert _topk(L, dt=0, logits=P + 2) == E_ALIGN
    assert _topk(L, val=P + 2) == E_ALIGN
    assert _topk(L, rows=8, V=151936, ws=None, wsb=0) == E_WS  # split rows need scratch


def test_gate_validation(L):
    def g(h=P, w=P, dt=1, rows=4, d=64, E=256, out=P, ws=P, wsb=1 << 24):
        return L.dfs_gate(h, w, dt, rows, d, E, out, ws, wsb, None)

    assert g(h=None) == E_NULL
    assert g(E=128) == E_UNSUP
    assert g(d=60) == E_UNSUP
    assert g(rows=0) == E_SHAPE
    assert g(d=(1 << 20) + 8) == E_SHAPE  # wider than DFS_MAX_D
    assert L.dfs_gate_workspace_bytes(4, (1 << 20) + 8, 1) == 0
    assert g(h=P + 8) == E_ALIGN
    assert g(ws=None, wsb=0) == E_WS


def test_pair_and_walk_validation(L):
    def p(ci=P, cv=P, pt=P, g=P, A=P, B=P, dt=1, b=2, Lp=4, V=100, E=256, k=16, out=P):
        return L.dfs_pair_scores(ci, cv, pt, g, A, B, dt, b, Lp, V, E, k, out, None)

    assert p(A=None) == E_NULL
    assert p(k=4) == E_UNSUP
    assert p(E=64) == E_UNSUP
    assert p(Lp=17) == E_SHAPE
    assert p(Lp=0) == E_SHAPE
    assert p(V=10) == E_SHAPE
    assert p(g=P + 4) == E_ALIGN

    def w(pair=P, ci=P, b=2, Lw=4, k=16, mode=0, T=1.0, seed=0, path=P, sc=P):
        return L.dfs_walk(pair, ci, b, Lw, k, mode, T, seed, path, sc, None)

    assert w(pair=None) == E_NULL
    assert w(mode=3) == E_UNSUP
    assert w(mode=1, T=0.0) == E_ARG
    assert w(mode=1, T=float("nan")) == E_ARG
    assert w(mode=1, T=float("inf")) == E_ARG
    assert w(Lw=0) == E_SHAPE
    assert w(path=P + 2) == E_ALIGN


def test_select_validation(L):
    shape = dfs._Shape(2, 4, 1000, 64, 1, 1, 1)

    def s(lg=P, h=P, pt=P, A=P, B=P, W=P, k=16, sh=ctypes.byref(shape), mode=0, T=1.0, ws=P, wsb=1 << 26,
          path=P, sc=P):
        return L.dfs_select(lg, h, pt, A, B, W, k, sh, mode, T, 0, ws, wsb, path, sc, None)

    assert s(lg=None) == E_NULL
    assert s(sh=None) == E_NULL
    assert s(k=32) == E_UNSUP
    assert s(mode=1, T=-1.0) == E_ARG
    assert s(h=P + 2) == E_ALIGN
    assert s(ws=P + 64) == E_ALIGN
    assert s(wsb=16) == E_WS
    assert s(ws=None) == E_WS
    for bad in [dict(batch=0), dict(L=17), dict(V=3), dict(d=0), dict(d=(1 << 20) + 8)]:
        sh = dfs._Shape(2, 4, 1000, 64, 1, 1, 1)
        for k_, v_ in bad.items():
            setattr(sh, k_, v_)
        assert s(sh=ctypes.byref(sh)) == E_SHAPE
    sh = dfs._Shape(2, 4, 1000, 60, 1, 1, 1)
    assert s(sh=ctypes.byref(sh)) == E_UNSUP
    sh = dfs._Shape(2, 4, 1000, 64, 1, 5, 1)
    assert s(sh=ctypes.byref(sh)) == E_UNSUP


def test_packed_weight_validation(L):
    # W_h packed once: bf16 [ceil(d/32)][256][32] (zero-padded), fp32 a plain copy
    assert L.dfs_gate_pack_bytes(5120, 1) == 160 * 256 * 32 * 2
    assert L.dfs_gate_pack_bytes(72, 1) == 3 * 256 * 32 * 2
    assert L.dfs_gate_pack_bytes(1024, 0) == 1024 * 256 * 4
    assert L.dfs_gate_pack_bytes(60, 1) == 0
    assert L.dfs_gate_pack_bytes(0, 1) == 0
    assert L.dfs_gate_pack_bytes(64, 9) == 0
    nb = L.dfs_gate_pack_bytes(64, 1)

    def pk(W=P, dt=1, d=64, out=P + 0x100000, ob=nb):
        return L.dfs_gate_pack(W, dt, d, out, ob, None)

    assert pk(W=None) == E_NULL
    assert pk(out=None) == E_NULL
    assert pk(dt=5) == E_UNSUP
    assert pk(d=0) == E_SHAPE
    assert pk(d=60) == E_UNSUP
    assert pk(W=P + 8) == E_ALIGN
    assert pk(ob=nb - 1) == E_WS
    assert pk(out=P + 0x100) == E_ARG  # overlaps W_h
    assert L.dfs_gate_packed(None, P, 1, 4, 64, 256, P, P, 1 << 24, None) == E_NULL
    assert L.dfs_gate_packed(P, P, 1, 4, 60, 256, P, P, 1 << 24, None) == E_UNSUP
    shape = dfs._Shape(2, 4, 1000, 64, 1, 1, 1)
    assert L.dfs_select_packed(P, P, P, P, P, None, 16, ctypes.byref(shape), 0, 1.0, 0, P, 1 << 26, P, P,
                               None) == E_NULL
    assert L.dfs_select_packed(P, P, P, P, P, P, 16, ctypes.byref(shape), 0, 1.0, 0, P, 16, P, P, None) == E_WS
    assert L.dfs_select_draft_packed(P, P, P, P, P, P, 16, ctypes.byref(shape), 0, 0.0, 0, P, 1 << 26, P, P,
                                     P, P, None) == E_ARG
    assert L.dfs_select_draft_packed(P, P, P, P, P, P, 16, ctypes.byref(shape), 0, 1.0, 0, P, 1 << 26, P, P,
                                     None, P, None) == E_NULL


def test_static_scratch_validation(L):
    # dfs_select_packed_static: the same checks as dfs_select_packed, plus the size of its
    # static scratch (32 MiB), all on the host before anything is launched
    def st(sh, lg=P, W=P, T=1.0, mode=0):
        return L.dfs_select_packed_static(lg, P, P, P, P, W, 16, ctypes.byref(sh) if sh is not None else None, mode,
                                          T, 0, P, P, None)

    assert st(None) == E_NULL
    assert st(dfs._Shape(2, 4, 1000, 64, 1, 1, 1), lg=None) == E_NULL
    assert st(dfs._Shape(2, 4, 1000, 64, 1, 1, 1), mode=1, T=0.0) == E_ARG
    assert st(dfs._Shape(0, 4, 1000, 64, 1, 1, 1)) == E_SHAPE
    big = dfs._Shape(4096, 16, 151936, 5120, 1, 1, 1)  # 65536 rows: 64 MB of gate rows alone
    assert L.dfs_select_workspace_bytes(ctypes.byref(big)) > 32 << 20
    assert st(big) == E_TOO_LARGE
    for name in ("throughput", "sampled", "small_batch", "single_stream", "tiny"):
        from workloads import config_by_name
        c = config_by_name(name)
        dt = 1 if c.dtype == "bf16" else 0
        sh = dfs._Shape(c.batch, c.L, c.V, c.d, dt, dt, dt)
        assert L.dfs_select_workspace_bytes(ctypes.byref(sh)) <= 32 << 20, name


def test_select_draft_and_verify_validation(L):
    shape = dfs._Shape(2, 4, 1000, 64, 1, 1, 1)

    def sd(q=P, c=P, T=1.0, mode=0):
        return L.dfs_select_draft(P, P, P, P, P, P, 16, ctypes.byref(shape), mode, T, 0, P, 1 << 26, P, P,
                                  q, c, None)

    assert sd(q=None) == E_NULL
    assert sd(c=None) == E_NULL
    assert sd(q=P + 2) == E_ALIGN
    assert sd(T=0.0) == E_ARG  # the draft rows need a temperature in every mode
    assert sd(T=float("inf")) == E_ARG

    def v(tl=P, dt=1, b=2, Lv=4, V=1000, path=P, cand=P, q=P, k=16, T=1.0, ws=P, wsb=1 << 20, acc=P, tok=P):
        return L.dfs_verify(tl, dt, b, Lv, V, path, cand, q, k, T, 0, ws, wsb, acc, tok, None)

    assert v(tl=None) == E_NULL
    assert v(ws=None) == E_NULL
    assert v(tok=None) == E_NULL
    assert v(k=8) == E_UNSUP
    assert v(dt=3) == E_UNSUP
    assert v(b=0) == E_SHAPE
    assert v(Lv=0) == E_SHAPE
    assert v(Lv=17) == E_SHAPE
    assert v(V=15) == E_SHAPE
    assert v(V=4190209) == E_SHAPE  # the draw keeps at most 1023 segments of 4096 tokens
    assert v(T=0.0) == E_ARG
    assert v(T=float("nan")) == E_ARG
    assert v(tl=P + 1) == E_ALIGN
    assert v(ws=P + 64) == E_ALIGN
    assert v(wsb=16) == E_WS
    assert L.dfs_verify_workspace_bytes(2, 4, 1000, 1) >= 16
    assert L.dfs_verify_workspace_bytes(2, 0, 1000, 1) == 0


def test_valid_arguments_without_a_device_report_hip_error(L):
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert _topk(L, rows=4096, V=151936) == E_HIP


def _conv(L, x=P, xp=P + 0x100000, base=P + 0x200000, W=P + 0x300000, dt=1, batch=2, Lp=4, D=512,
          y=P + 0x1000000, ws=None, wsb=0):
    return L.dfs_conv2(x, xp, base, W, dt, batch, Lp, D, y, ws, wsb, None)


def test_conv2_validation(L):
    assert _conv(L, x=None) == E_NULL
    assert _conv(L, y=None) == E_NULL
    assert _conv(L, dt=7) == E_UNSUP
    assert _conv(L, D=128) == E_SHAPE
    assert _conv(L, D=768 + 16) == E_UNSUP  # not a multiple of 256
    assert _conv(L, Lp=0) == E_SHAPE
    assert _conv(L, batch=0) == E_SHAPE
    assert _conv(L, x=P + 8) == E_ALIGN
    assert _conv(L, y=P + 64) == E_ARG  # overlaps x
    assert _conv(L, y=P + 0x100000) == E_ARG  # overlaps x_prev
    # fp32 needs no workspace; bf16 needs one only when K is split (512 rows of 5120:
    # 20 tiles, too few for the chip), for the split partial sums of the correction
    assert L.dfs_conv2_workspace_bytes(2, 4, 512, 0) == 0
    assert L.dfs_conv2_workspace_bytes(2, 4, 512, 1) == 0
    nb = L.dfs_conv2_workspace_bytes(32, 16, 5120, 1)
    assert nb >= 2 * 512 * 640 * 4
    assert _conv(L, batch=32, Lp=16, D=5120, ws=None, wsb=0) == E_WS
    assert _conv(L, batch=32, Lp=16, D=5120, ws=P + 0x3000000, wsb=nb - 1) == E_WS
    assert _conv(L, dt=0, ws=P + 0x3000000 + 1, wsb=64) == E_ALIGN
    assert L.dfs_conv2_workspace_bytes(2, 4, 500, 0) == 0
    # fp32: at most 2^32 elements of x (the grid's work-item count)
    assert _conv(L, dt=0, batch=1 << 13, Lp=64, D=8192 + 256) == E_SHAPE


def test_lmhead_validation(L):
    f = lambda **kw: L.dfs_lmhead_topk(kw.get("h", P), kw.get("W", P + 0x100000), kw.get("dt", 1),  # noqa: E731
                                       kw.get("rows", 16), kw.get("V", 1000), kw.get("d", 512), kw.get("k", 16),
                                       kw.get("idx", P), kw.get("val", P), kw.get("ws", P), kw.get("wsb", 1 << 30),
                                       None)
    assert f(h=None) == E_NULL
    assert f(ws=None) == E_NULL
    assert f(dt=0) == E_UNSUP
    assert f(d=100) == E_SHAPE or f(d=100) == E_UNSUP
    assert f(d=96) == E_UNSUP
    assert f(V=15) == E_SHAPE
    assert f(rows=0) == E_SHAPE
    assert f(k=8) == E_UNSUP
    assert f(h=P + 4) == E_ALIGN
    assert f(wsb=16) == E_WS
    nb = L.dfs_lmhead_topk_workspace_bytes(16, 151936, 5120)
    assert 0 < nb < 1 << 24
    assert L.dfs_lmhead_topk_workspace_bytes(16, 151936, 5100) == 0
    assert L.dfs_lmhead_logits(P, P, 0, 16, 1000, 512, P, None) == E_UNSUP


def test_row_limit(L):
    # DFS_MAX_ROWS rows per call: one more is a shape error before any launch, so that no
    # launch grid passes 2^31 work-items; at the limit validation goes on to the next check
    M = 1 << 22
    assert _topk(L, rows=M + 1, V=16) == E_SHAPE
    assert L.dfs_topk_workspace_bytes(M + 1, 16, 1) == 0
    assert _topk(L, rows=M, V=16, ws=None, wsb=0) != E_SHAPE
    assert L.dfs_gate(P, P, 1, M + 1, 64, 256, P, P, 1 << 20, None) == E_SHAPE
    assert L.dfs_gate_workspace_bytes(M + 1, 64, 1) == 0
    assert L.dfs_pair_scores(P, P, P, P, P, P, 1, M // 16 + 1, 16, 100, 256, 16, P, None) == E_SHAPE
    assert L.dfs_walk(P, P, M // 4 + 1, 4, 16, 0, 1.0, 0, P, P, None) == E_SHAPE
    assert L.dfs_walk(P, P, M + 1, 1, 16, 0, 1.0, 0, P, P, None) == E_SHAPE
    sh = dfs._Shape(M // 16 + 1, 16, 1000, 64, 1, 1, 1)
    assert L.dfs_select_workspace_bytes(ctypes.byref(sh)) == 0
    assert L.dfs_select(P, P, P, P, P, P, 16, ctypes.byref(sh), 0, 1.0, 0, P, 1 << 26, P, P, None) == E_SHAPE
    assert L.dfs_verify_workspace_bytes(M // 17 + 1, 16, 1000, 1) == 0
    assert L.dfs_verify_workspace_bytes(M // 17, 16, 1000, 1) > 0
    assert L.dfs_conv2_workspace_bytes(M // 16 + 1, 16, 256, 1) == 0
    assert L.dfs_conv2_workspace_bytes(M // 16, 16, 256, 1) >= 0
    assert _conv(L, batch=1 << 16, Lp=64, D=1 << 20) == E_SHAPE  # 2^22 rows x 2^20 channels
    assert L.dfs_lmhead_topk_workspace_bytes(M + 1, 1000, 512) == 0
    assert L.dfs_lmhead_topk_workspace_bytes(1 << 16, 1 << 24, 512) == 0  # 2^9 x 2^17 tiles
    assert L.dfs_lmhead_topk_workspace_bytes(4096, 151936, 5120) > 0


EXTREMES = [-1, 0, 1, 2, 7, 8, 15, 16, 17, 31, 32, 33, 255, 256, 257, 4095, 4096, 4097, 151936, 262144,
            (1 << 20) - 1, 1 << 20, (1 << 20) + 1, (1 << 22) - 1, 1 << 22, (1 << 22) + 1, (1 << 31) - 1, 1 << 31,
            (1 << 62), -(1 << 62)]


def test_planners_over_extreme_sizes(L):
    # every workspace query plans the launches it would make; none may crash, overflow or
    # report an absurd size for any int64 it is given (run under the host-sanitized build too)
    import itertools

    cap = 1 << 46
    for a, b in itertools.product(EXTREMES, EXTREMES):
        for dt in (0, 1, 5):
            for q in (L.dfs_topk_workspace_bytes, L.dfs_gate_workspace_bytes, L.dfs_lmhead_topk_workspace_bytes):
                args = (a, b, dt) if q is not L.dfs_lmhead_topk_workspace_bytes else (a, b, 4096)
                assert q(*args) < cap
        assert L.dfs_gate_pack_bytes(a, b & 1) < cap
    for bsz, Ln, V, d in itertools.product([-1, 0, 1, 256, 1 << 22, 1 << 40], [0, 1, 16, 17],
                                           [0, 16, 151936, (1 << 31) - 1, 1 << 31], [0, 8, 5120, 1 << 20, 1 << 21]):
        for dt in (0, 1, 9):
            s = dfs._shape(bsz, Ln, V, d, dt, dt, dt)
            assert L.dfs_select_workspace_bytes(ctypes.byref(s)) < cap
            assert L.dfs_verify_workspace_bytes(bsz, Ln, V, dt) < cap
            assert L.dfs_conv2_workspace_bytes(bsz, Ln, d, dt) < cap
