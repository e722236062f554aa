"""DFlash 2 draft-path selector for AMD Instinct MI355X (gfx950).

Thin Python binding of ``libdfs.so`` (C ABI declared in ``include/dfs.h``).  It
only checks and marshals arguments: every step of the selector runs in the
library's HIP kernels.  PyTorch supplies device memory and the current stream.
The library is required; there is no other code path.

    import draft_selection_position_amd as dfs
    path, scores = dfs.select(logits, hidden, prev_token, A, B, W_h)

The selector (blog post "DFlash 2: Keep Drafting Parallel", section "A
Lightweight Path Selector"): keep the 16 best candidates per block position,
score every adjacent pair with S_t(a,b) = U_t(b) + <A(a) * sigmoid(h_t W_h), B(b)>,
then walk the scores once from the last verified token.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

__all__ = [
    "DfsError", "K", "E", "MAX_L", "lib", "lib_path", "topk", "gate", "pair_scores", "walk",
    "select", "Selector", "select_workspace_bytes", "topk_workspace_bytes", "PackedWeight", "gate_pack",
    "gate_workspace_bytes", "status_str", "conv2", "conv2_workspace_bytes", "Conv2", "lmhead_topk", "lmhead_logits",
    "lmhead_topk_workspace_bytes",
]

K = 16
E = 256
MAX_L = 16
F32, BF16 = 0, 1
GREEDY, GUMBEL, VITERBI = 0, 1, 2
_MODES = {"greedy": GREEDY, "gumbel": GUMBEL, "sampled": GUMBEL, "viterbi": VITERBI}

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None
_lock = threading.Lock()


def lib_path() -> str:
    """libdfs.so next to this file, or the build that DFS_LIBRARY names (another build of the
    same sources, e.g. the host-sanitized one the ABI tests run against)."""
    return os.environ.get("DFS_LIBRARY") or os.path.join(_HERE, "libdfs.so")


class _Shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("L", ctypes.c_int64), ("V", ctypes.c_int64),
                ("d", ctypes.c_int64), ("logits_dtype", ctypes.c_int), ("act_dtype", ctypes.c_int),
                ("table_dtype", ctypes.c_int)]


def lib() -> ctypes.CDLL:
    """Load libdfs.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with `python -m draft_selection_position_amd.build`")
        L = ctypes.CDLL(path)
        vp, i64, sz, i32p, f32p = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p
        c_int, c_double, u64 = ctypes.c_int, ctypes.c_double, ctypes.c_uint64
        L.dfs_status_str.argtypes, L.dfs_status_str.restype = [c_int], ctypes.c_char_p
        L.dfs_abi_version.argtypes, L.dfs_abi_version.restype = [], c_int
        L.dfs_topk_workspace_bytes.argtypes, L.dfs_topk_workspace_bytes.restype = [i64, i64, c_int], sz
        L.dfs_topk.argtypes = [vp, c_int, i64, i64, c_int, i32p, f32p, vp, sz, vp]
        L.dfs_topk.restype = c_int
        L.dfs_gate_workspace_bytes.argtypes, L.dfs_gate_workspace_bytes.restype = [i64, i64, c_int], sz
        L.dfs_gate.argtypes = [vp, vp, c_int, i64, i64, i64, f32p, vp, sz, vp]
        L.dfs_gate.restype = c_int
        L.dfs_gate_packed.argtypes = [vp, vp, c_int, i64, i64, i64, f32p, vp, sz, vp]
        L.dfs_gate_packed.restype = c_int
        L.dfs_gate_pack_bytes.argtypes, L.dfs_gate_pack_bytes.restype = [i64, c_int], sz
        L.dfs_gate_pack.argtypes = [vp, c_int, i64, vp, sz, vp]
        L.dfs_gate_pack.restype = c_int
        L.dfs_pair_scores.argtypes = [i32p, f32p, i32p, f32p, vp, vp, c_int, i64, i64, i64, i64, c_int,
                                      f32p, vp]
        L.dfs_pair_scores.restype = c_int
        L.dfs_walk.argtypes = [f32p, i32p, i64, i64, c_int, c_int, c_double, u64, i32p, f32p, vp]
        L.dfs_walk.restype = c_int
        L.dfs_select_workspace_bytes.argtypes = [ctypes.POINTER(_Shape)]
        L.dfs_select_workspace_bytes.restype = sz
        L.dfs_select.argtypes = [vp, vp, i32p, vp, vp, vp, c_int, ctypes.POINTER(_Shape), c_int, c_double,
                                 u64, vp, sz, i32p, f32p, vp]
        L.dfs_select.restype = c_int
        L.dfs_select_packed.argtypes = L.dfs_select.argtypes
        L.dfs_select_packed.restype = c_int
        L.dfs_select_packed_static.argtypes = [vp, vp, i32p, vp, vp, vp, c_int, ctypes.POINTER(_Shape), c_int,
                                               c_double, u64, i32p, f32p, vp]
        L.dfs_select_packed_static.restype = c_int
        L.dfs_select_draft.argtypes = [vp, vp, i32p, vp, vp, vp, c_int, ctypes.POINTER(_Shape), c_int,
                                       c_double, u64, vp, sz, i32p, f32p, f32p, i32p, vp]
        L.dfs_select_draft.restype = c_int
        L.dfs_select_draft_packed.argtypes = L.dfs_select_draft.argtypes
        L.dfs_select_draft_packed.restype = c_int
        L.dfs_verify_workspace_bytes.argtypes, L.dfs_verify_workspace_bytes.restype = [i64, i64, i64, c_int], sz
        L.dfs_verify.argtypes = [vp, c_int, i64, i64, i64, i32p, i32p, f32p, c_int, c_double, u64, vp, sz,
                                 i32p, i32p, vp]
        L.dfs_verify.restype = c_int
        L.dfs_conv2_workspace_bytes.argtypes, L.dfs_conv2_workspace_bytes.restype = [i64, i64, i64, c_int], sz
        L.dfs_conv2.argtypes = [vp, vp, vp, vp, c_int, i64, i64, i64, vp, vp, sz, vp]
        L.dfs_conv2.restype = c_int
        L.dfs_lmhead_topk_workspace_bytes.argtypes = [i64, i64, i64]
        L.dfs_lmhead_topk_workspace_bytes.restype = sz
        L.dfs_lmhead_topk.argtypes = [vp, vp, c_int, i64, i64, i64, c_int, i32p, f32p, vp, sz, vp]
        L.dfs_lmhead_topk.restype = c_int
        L.dfs_lmhead_logits.argtypes = [vp, vp, c_int, i64, i64, i64, f32p, vp]
        L.dfs_lmhead_logits.restype = c_int
        _lib = L
    return _lib


class DfsError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {status_str(code)}")


def status_str(code: int) -> str:
    return lib().dfs_status_str(int(code)).decode()


def _check(rc: int, where: str) -> None:
    if rc != 0:
        raise DfsError(rc, where)


def _dtype_code(t: torch.Tensor, what: str) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise ValueError(f"{what} must be float32 or bfloat16, got {t.dtype}")


def _dev(t: torch.Tensor, what: str, dtype=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{what} must be on a HIP device, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{what} must be {dtype}, got {t.dtype}")
    return t


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


class _Workspace:
    """Cached scratch buffers, one per (device, stream), grown on demand, never shrunk.

    A call without an explicit workspace uses the buffer of the stream it is enqueued
    on, so calls on different streams never share scratch memory.  Each buffer is
    allocated while its own stream is current, so when a grown buffer replaces it, the
    caching allocator hands the old block out again only to later work on that same
    stream (after everything already enqueued there).
    """

    def __init__(self):
        self._bufs: dict[tuple, torch.Tensor] = {}

    @staticmethod
    def key(device: torch.device) -> tuple:
        return (device, torch.cuda.current_stream(device).cuda_stream)

    def get(self, device: torch.device, nbytes: int) -> torch.Tensor | None:
        if nbytes == 0:
            return None
        key = self.key(device)
        buf = self._bufs.get(key)
        if buf is None or buf.numel() < nbytes:
            with torch.cuda.device(device):
                buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
            self._bufs[key] = buf
        return buf


_WS = _Workspace()


def _ws_arg(ws, device, nbytes):
    if ws is None:
        ws = _WS.get(device, nbytes)
    elif nbytes and (ws.device != device or ws.numel() * ws.element_size() < nbytes):
        raise ValueError(f"workspace must hold {nbytes} bytes on {device}")
    return ws


# ---------------------------------------------------------------- step entry points


def topk_workspace_bytes(rows: int, V: int, dtype: torch.dtype) -> int:
    return int(lib().dfs_topk_workspace_bytes(rows, V, BF16 if dtype == torch.bfloat16 else F32))


def topk(logits: torch.Tensor, k: int = K, workspace: torch.Tensor | None = None):
    """Top-16 of each row of ``logits`` [..., V]: (ids int32 [..., 16], values fp32 [..., 16]).

    Order: value descending, then id ascending.
    """
    _dev(logits, "logits")
    dt = _dtype_code(logits, "logits")
    V = logits.shape[-1]
    rows = logits.numel() // V if V else 0
    lead = tuple(logits.shape[:-1])
    idx = torch.empty(lead + (K,), dtype=torch.int32, device=logits.device)
    val = torch.empty(lead + (K,), dtype=torch.float32, device=logits.device)
    nb = int(lib().dfs_topk_workspace_bytes(rows, V, dt))
    ws = _ws_arg(workspace, logits.device, nb)
    _check(lib().dfs_topk(logits.data_ptr(), dt, rows, V, k, idx.data_ptr(), val.data_ptr(), _ptr(ws), nb,
                          _stream(logits.device)), "dfs_topk")
    return idx, val


def gate_workspace_bytes(rows: int, d: int, dtype: torch.dtype) -> int:
    return int(lib().dfs_gate_workspace_bytes(rows, d, BF16 if dtype == torch.bfloat16 else F32))


class PackedWeight:
    """W_h [d, 256] packed once for the gate's matrix cores (dfs_gate_pack).

    Pass it wherever W_h is taken (``gate``, ``select``, ``Selector``): the results are
    bitwise those of the unpacked weight, without repacking it on every call.  It holds
    its own device bytes; ``d`` and ``dtype`` are those of the weight it came from.
    """

    def __init__(self, data: torch.Tensor, d: int, dtype: torch.dtype):
        self.data, self.d, self.dtype = data, int(d), dtype
        self.device = data.device
        self.shape = (int(d), E)

    def data_ptr(self) -> int:
        return self.data.data_ptr()


def gate_pack(W_h: torch.Tensor) -> PackedWeight:
    """Pack the gate weight W_h [d, 256] (bf16 or fp32) for the matrix cores, once."""
    _dev(W_h, "W_h")
    dt = _dtype_code(W_h, "W_h")
    if W_h.dim() != 2 or W_h.shape[1] != E:
        raise ValueError(f"W_h must be [d, 256], got {tuple(W_h.shape)}")
    d = W_h.shape[0]
    nb = int(lib().dfs_gate_pack_bytes(d, dt))
    if nb == 0:
        raise ValueError(f"unsupported gate width d = {d}")
    out = torch.empty(nb, dtype=torch.uint8, device=W_h.device)
    _check(lib().dfs_gate_pack(W_h.data_ptr(), dt, d, out.data_ptr(), nb, _stream(W_h.device)), "dfs_gate_pack")
    return PackedWeight(out, d, W_h.dtype)


def _weight(W_h, d: int, dtype: torch.dtype, what: str = "W_h"):
    """(pointer, packed?) of a W_h argument: a [d, 256] tensor of `dtype` or a PackedWeight."""
    if isinstance(W_h, PackedWeight):
        if W_h.d != d or W_h.dtype != dtype:
            raise ValueError(f"{what} was packed for d = {W_h.d}, {W_h.dtype}; need d = {d}, {dtype}")
        if W_h.device.type != "cuda":
            raise ValueError(f"{what} must be on a HIP device")
        return W_h.data_ptr(), True
    _dev(W_h, what, dtype)
    if W_h.dim() != 2 or tuple(W_h.shape) != (d, E):
        raise ValueError(f"{what} must be [{d}, 256], got {tuple(W_h.shape)}")
    return W_h.data_ptr(), False


def gate(hidden: torch.Tensor, W_h, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """sigmoid(hidden @ W_h) in fp32: hidden [..., d], W_h [d, 256] (same dtype, or a
    PackedWeight) -> [..., 256]."""
    _dev(hidden, "hidden")
    dt = _dtype_code(hidden, "hidden")
    d = hidden.shape[-1]
    wptr, packed = _weight(W_h, d, hidden.dtype)
    rows = hidden.numel() // d if d else 0
    out = torch.empty(tuple(hidden.shape[:-1]) + (E,), dtype=torch.float32, device=hidden.device)
    nb = int(lib().dfs_gate_workspace_bytes(rows, d, dt))
    ws = _ws_arg(workspace, hidden.device, nb)
    fn = lib().dfs_gate_packed if packed else lib().dfs_gate
    _check(fn(hidden.data_ptr(), wptr, dt, rows, d, E, out.data_ptr(), _ptr(ws), nb, _stream(hidden.device)),
           "dfs_gate_packed" if packed else "dfs_gate")
    return out


def pair_scores(cand_idx: torch.Tensor, cand_val: torch.Tensor, prev_token: torch.Tensor,
                gate_: torch.Tensor, A: torch.Tensor, B: torch.Tensor) -> torch.Tensor:
    """S[b, t, i, j] for all adjacent candidate pairs: fp32 [batch, L, 16, 16]."""
    _dev(cand_idx, "cand_idx", torch.int32)
    _dev(cand_val, "cand_val", torch.float32)
    _dev(prev_token, "prev_token", torch.int32)
    _dev(gate_, "gate", torch.float32)
    _dev(A, "A")
    _dev(B, "B", A.dtype)
    if cand_idx.dim() != 3 or cand_idx.shape[-1] != K or cand_val.shape != cand_idx.shape:
        raise ValueError("cand_idx and cand_val must both be [batch, L, 16]")
    batch, L = cand_idx.shape[0], cand_idx.shape[1]
    if prev_token.shape != (batch,) or gate_.numel() != batch * L * E:
        raise ValueError("prev_token must be [batch] and gate [batch*L, 256]")
    if A.dim() != 2 or A.shape != B.shape:
        raise ValueError("A and B must both be [V, 256]")
    out = torch.empty((batch, L, K, K), dtype=torch.float32, device=cand_idx.device)
    _check(lib().dfs_pair_scores(cand_idx.data_ptr(), cand_val.data_ptr(), prev_token.data_ptr(),
                                 gate_.data_ptr(), A.data_ptr(), B.data_ptr(), _dtype_code(A, "A"), batch, L,
                                 A.shape[0], A.shape[1], K, out.data_ptr(), _stream(A.device)),
           "dfs_pair_scores")
    return out


def walk(pair: torch.Tensor, cand_idx: torch.Tensor, mode: str = "greedy", temperature: float = 1.0,
         seed: int = 0):
    """One walk per sequence over pair [batch, L, 16, 16]: (path int32 [batch, L], scores fp32)."""
    _dev(pair, "pair", torch.float32)
    _dev(cand_idx, "cand_idx", torch.int32)
    if pair.dim() != 4 or pair.shape[2:] != (K, K) or cand_idx.shape != pair.shape[:3]:
        raise ValueError("pair must be [batch, L, 16, 16] and cand_idx [batch, L, 16]")
    batch, L = pair.shape[0], pair.shape[1]
    path = torch.empty((batch, L), dtype=torch.int32, device=pair.device)
    scores = torch.empty((batch, L), dtype=torch.float32, device=pair.device)
    _check(lib().dfs_walk(pair.data_ptr(), cand_idx.data_ptr(), batch, L, K, _MODES[mode], float(temperature),
                          int(seed) & (2**64 - 1), path.data_ptr(), scores.data_ptr(), _stream(pair.device)),
           "dfs_walk")
    return path, scores


# ---------------------------------------------------------------- fused selector


def _shape(batch, L, V, d, logits_dt, act_dt, table_dt) -> _Shape:
    return _Shape(batch, L, V, d, logits_dt, act_dt, table_dt)


def select_workspace_bytes(batch: int, L: int, V: int, d: int, logits_dtype=torch.bfloat16,
                           act_dtype=torch.bfloat16, table_dtype=torch.bfloat16) -> int:
    c = lambda t: BF16 if t == torch.bfloat16 else F32  # noqa: E731
    s = _shape(batch, L, V, d, c(logits_dtype), c(act_dtype), c(table_dtype))
    return int(lib().dfs_select_workspace_bytes(ctypes.byref(s)))


def select(logits: torch.Tensor, hidden: torch.Tensor, prev_token: torch.Tensor, A: torch.Tensor,
           B: torch.Tensor, W_h, k: int = K, mode: str = "greedy", temperature: float = 1.0,
           seed: int = 0, workspace: torch.Tensor | None = None, out=None, draft: bool = False):
    """The whole selector on one draft block per sequence.

    logits [batch, L, V]; hidden [batch, L, d]; prev_token [batch] int32 (last
    verified token); A, B [V, 256]; W_h [d, 256] or a PackedWeight (gate_pack).
    Returns (path int32 [batch, L], scores fp32 [batch, L]).  ``out`` may pass
    preallocated (path, scores).  With ``draft=True`` also the draft distributions q
    fp32 [batch, L, 16] and the candidate ids int32 [batch, L, 16] (dfs_select_draft).
    """
    _dev(logits, "logits")
    _dev(hidden, "hidden")
    _dev(prev_token, "prev_token", torch.int32)
    _dev(A, "A")
    _dev(B, "B", A.dtype)
    if logits.dim() != 3 or hidden.dim() != 3 or hidden.shape[:2] != logits.shape[:2]:
        raise ValueError("logits must be [batch, L, V] and hidden [batch, L, d]")
    batch, L, V = logits.shape
    d = hidden.shape[2]
    wptr, packed = _weight(W_h, d, hidden.dtype)
    if A.shape != (V, E) or B.shape != (V, E) or prev_token.shape != (batch,):
        raise ValueError("A, B must be [V, 256] and prev_token [batch]")
    s = _shape(batch, L, V, d, _dtype_code(logits, "logits"), _dtype_code(hidden, "hidden"),
               _dtype_code(A, "A"))
    nb = int(lib().dfs_select_workspace_bytes(ctypes.byref(s)))
    ws = _ws_arg(workspace, logits.device, nb)
    if out is None:
        path = torch.empty((batch, L), dtype=torch.int32, device=logits.device)
        scores = torch.empty((batch, L), dtype=torch.float32, device=logits.device)
    else:
        path, scores = out
    if not draft:
        fn = lib().dfs_select_packed if packed else lib().dfs_select
        _check(fn(logits.data_ptr(), hidden.data_ptr(), prev_token.data_ptr(), A.data_ptr(), B.data_ptr(), wptr,
                  k, ctypes.byref(s), _MODES[mode], float(temperature), int(seed) & (2**64 - 1), _ptr(ws), nb,
                  path.data_ptr(), scores.data_ptr(), _stream(logits.device)),
               "dfs_select_packed" if packed else "dfs_select")
        return path, scores
    q = torch.empty((batch, L, K), dtype=torch.float32, device=logits.device)
    cand = torch.empty((batch, L, K), dtype=torch.int32, device=logits.device)
    fn = lib().dfs_select_draft_packed if packed else lib().dfs_select_draft
    _check(fn(logits.data_ptr(), hidden.data_ptr(), prev_token.data_ptr(), A.data_ptr(), B.data_ptr(), wptr, k,
              ctypes.byref(s), _MODES[mode], float(temperature), int(seed) & (2**64 - 1), _ptr(ws), nb,
              path.data_ptr(), scores.data_ptr(), q.data_ptr(), cand.data_ptr(), _stream(logits.device)),
           "dfs_select_draft_packed" if packed else "dfs_select_draft")
    return path, scores, q, cand


def verify_workspace_bytes(batch: int, L: int, V: int, dtype: torch.dtype) -> int:
    code = F32 if dtype == torch.float32 else BF16 if dtype == torch.bfloat16 else -1
    return int(lib().dfs_verify_workspace_bytes(batch, L, V, code))


def verify(target_logits: torch.Tensor, path: torch.Tensor, cand: torch.Tensor, q: torch.Tensor,
           temperature: float = 1.0, seed: int = 0, workspace: torch.Tensor | None = None):
    """Speculative-sampling verification of drafted blocks (see dfs_verify).

    target_logits [batch, L + 1, V]; path [batch, L] int32; cand [batch, L, 16] int32 and
    q [batch, L, 16] fp32 (``select(..., draft=True)``).  Returns (accepted int32 [batch],
    token int32 [batch]): the number of draft tokens kept and the token drawn after them.
    """
    _dev(target_logits, "target_logits")
    _dev(path, "path", torch.int32)
    _dev(cand, "cand", torch.int32)
    _dev(q, "q", torch.float32)
    if target_logits.dim() != 3:
        raise ValueError("target_logits must be [batch, L + 1, V]")
    batch, L1, V = target_logits.shape
    L = L1 - 1
    if path.shape != (batch, L) or cand.shape != (batch, L, K) or q.shape != (batch, L, K):
        raise ValueError("path must be [batch, L], cand and q [batch, L, 16] with L + 1 target rows")
    dt = _dtype_code(target_logits, "target_logits")
    nb = int(lib().dfs_verify_workspace_bytes(batch, L, V, dt))
    ws = _ws_arg(workspace, target_logits.device, nb)
    accepted = torch.empty(batch, dtype=torch.int32, device=target_logits.device)
    token = torch.empty(batch, dtype=torch.int32, device=target_logits.device)
    _check(lib().dfs_verify(target_logits.data_ptr(), dt, batch, L, V, path.data_ptr(), cand.data_ptr(),
                            q.data_ptr(), K, float(temperature), int(seed) & (2**64 - 1), _ptr(ws), nb,
                            accepted.data_ptr(), token.data_ptr(), _stream(target_logits.device)), "dfs_verify")
    return accepted, token


def conv2_workspace_bytes(batch: int, L: int, D: int, dtype: torch.dtype) -> int:
    code = F32 if dtype == torch.float32 else BF16 if dtype == torch.bfloat16 else -1
    return int(lib().dfs_conv2_workspace_bytes(batch, L, D, code))


def conv2(x: torch.Tensor, x_prev: torch.Tensor, base: torch.Tensor, W_c: torch.Tensor,
          out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Two-tap dynamic depthwise convolution across block positions (see dfs_conv2).

    x [batch, L, D], x_prev [batch, D], base [2, D], W_c [D/16, 2, D], all of one dtype
    (bf16 or fp32).  Returns y [batch, L, D] (written into ``out`` when given)."""
    _dev(x, "x")
    dt = _dtype_code(x, "x")
    _dev(x_prev, "x_prev", x.dtype)
    _dev(base, "base", x.dtype)
    _dev(W_c, "W_c", x.dtype)
    if x.dim() != 3:
        raise ValueError("x must be [batch, L, D]")
    batch, L, D = x.shape
    if x_prev.shape != (batch, D) or base.shape != (2, D) or W_c.shape != (D // 16, 2, D):
        raise ValueError(f"x_prev must be [{batch}, {D}], base [2, {D}] and W_c [{D // 16}, 2, {D}]")
    if out is None:
        out = torch.empty_like(x)
    else:
        _dev(out, "out", x.dtype)
        if out.shape != x.shape:
            raise ValueError("out must have the shape of x")
    nb = int(lib().dfs_conv2_workspace_bytes(batch, L, D, dt))
    ws = _ws_arg(workspace, x.device, nb)
    _check(lib().dfs_conv2(x.data_ptr(), x_prev.data_ptr(), base.data_ptr(), W_c.data_ptr(), dt, batch, L, D,
                           out.data_ptr(), _ptr(ws), nb, _stream(x.device)), "dfs_conv2")
    return out


def _lmhead_args(hidden, W_lm):
    _dev(hidden, "hidden", torch.bfloat16)
    _dev(W_lm, "W_lm", torch.bfloat16)
    d = hidden.shape[-1]
    if W_lm.dim() != 2 or W_lm.shape[1] != d:
        raise ValueError(f"W_lm must be [V, {d}], got {tuple(W_lm.shape)}")
    return hidden.numel() // d, W_lm.shape[0], d


def lmhead_topk_workspace_bytes(rows: int, V: int, d: int) -> int:
    return int(lib().dfs_lmhead_topk_workspace_bytes(rows, V, d))


def lmhead_topk(hidden: torch.Tensor, W_lm: torch.Tensor, workspace: torch.Tensor | None = None):
    """Top-16 of U = hidden @ W_lm.T per row without writing U (see dfs_lmhead_topk).

    hidden [..., d] and W_lm [V, d], bf16.  Returns (ids int32 [..., 16], values fp32 [..., 16])."""
    rows, V, d = _lmhead_args(hidden, W_lm)
    lead = tuple(hidden.shape[:-1])
    idx = torch.empty(lead + (K,), dtype=torch.int32, device=hidden.device)
    val = torch.empty(lead + (K,), dtype=torch.float32, device=hidden.device)
    nb = lmhead_topk_workspace_bytes(rows, V, d)
    ws = _ws_arg(workspace, hidden.device, nb)
    _check(lib().dfs_lmhead_topk(hidden.data_ptr(), W_lm.data_ptr(), BF16, rows, V, d, K, idx.data_ptr(),
                                 val.data_ptr(), _ptr(ws), nb, _stream(hidden.device)), "dfs_lmhead_topk")
    return idx, val


def lmhead_logits(hidden: torch.Tensor, W_lm: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """U = hidden @ W_lm.T in fp32 by the same product as lmhead_topk: [..., V]."""
    rows, V, d = _lmhead_args(hidden, W_lm)
    if out is None:
        out = torch.empty(tuple(hidden.shape[:-1]) + (V,), dtype=torch.float32, device=hidden.device)
    _dev(out, "out", torch.float32)
    _check(lib().dfs_lmhead_logits(hidden.data_ptr(), W_lm.data_ptr(), BF16, rows, V, d, out.data_ptr(),
                                   _stream(hidden.device)), "dfs_lmhead_logits")
    return out


class Selector:
    """Fixed-shape selector with its own workspace and output buffers (no per-call allocation).

    Tensor shapes, dtypes and devices are checked against the construction-time
    shape on every call, but with one tuple comparison each; the call then goes
    straight to dfs_select.  The path and scores buffers are reused by every call.
    """

    def __init__(self, batch: int, L: int, V: int, d: int, device="cuda", logits_dtype=torch.bfloat16,
                 act_dtype=torch.bfloat16, table_dtype=torch.bfloat16, mode: str = "greedy",
                 temperature: float = 1.0, seed: int = 0):
        self.device = torch.device(device)
        if self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        self.mode, self.temperature, self.seed = _MODES[mode], float(temperature), int(seed) & (2**64 - 1)
        c = lambda t: BF16 if t == torch.bfloat16 else F32  # noqa: E731
        self._shape = _Shape(batch, L, V, d, c(logits_dtype), c(act_dtype), c(table_dtype))
        nb = int(lib().dfs_select_workspace_bytes(ctypes.byref(self._shape)))
        if nb == 0:
            raise ValueError("unsupported selector shape")
        self._ws_bytes = nb
        self.workspace = torch.empty(nb, dtype=torch.uint8, device=self.device)
        self.path = torch.empty((batch, L), dtype=torch.int32, device=self.device)
        self.scores = torch.empty((batch, L), dtype=torch.float32, device=self.device)
        self._expect = (
            ((batch, L, V), logits_dtype), ((batch, L, d), act_dtype), ((batch,), torch.int32),
            ((V, E), table_dtype), ((V, E), table_dtype), ((d, E), act_dtype),
        )
        self._fn = lib().dfs_select
        self._fn_packed = lib().dfs_select_packed

    def __call__(self, logits, hidden, prev_token, A, B, W_h):
        """W_h: the [d, 256] weight, or a PackedWeight of it (then dfs_select_packed)."""
        packed = isinstance(W_h, PackedWeight)
        args = (logits, hidden, prev_token, A, B) if packed else (logits, hidden, prev_token, A, B, W_h)
        for t, (shape, dtype) in zip(args, self._expect):
            if t.shape != shape or t.dtype != dtype or t.device != self.device or not t.is_contiguous():
                raise ValueError(f"selector input must be a contiguous {dtype} tensor of shape {shape} "
                                 f"on {self.device}")
        if packed and (W_h.d, W_h.dtype, W_h.device) != (self._expect[5][0][0], self._expect[5][1], self.device):
            raise ValueError("packed W_h does not match the selector's d, dtype or device")
        fn = self._fn_packed if packed else self._fn
        rc = fn(logits.data_ptr(), hidden.data_ptr(), prev_token.data_ptr(), A.data_ptr(), B.data_ptr(),
                W_h.data_ptr(), K, ctypes.byref(self._shape), self.mode, self.temperature, self.seed,
                self.workspace.data_ptr(), self._ws_bytes, self.path.data_ptr(), self.scores.data_ptr(),
                torch.cuda.current_stream(self.device).cuda_stream)
        _check(rc, "dfs_select_packed" if packed else "dfs_select")
        return self.path, self.scores


class Conv2:
    """Fixed-shape two-tap convolution (dfs_conv2) with its own workspace and output.

    Inputs are checked against the construction-time shape with one tuple
    comparison each; the call then goes straight to dfs_conv2 and writes ``self.y``.
    """

    def __init__(self, batch: int, L: int, D: int, device="cuda", dtype=torch.bfloat16):
        self.device = torch.device(device)
        if self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        self._dt = BF16 if dtype == torch.bfloat16 else F32
        if dtype not in (torch.bfloat16, torch.float32):
            raise ValueError("dtype must be bfloat16 or float32")
        self._dims = (batch, L, D)
        self._ws_bytes = int(lib().dfs_conv2_workspace_bytes(batch, L, D, self._dt))
        if D % 256 or D < 256 or batch < 1 or L < 1:
            raise ValueError("unsupported convolution shape")
        self.workspace = torch.empty(max(1, self._ws_bytes), dtype=torch.uint8, device=self.device)
        self.y = torch.empty((batch, L, D), dtype=dtype, device=self.device)
        self._expect = (((batch, L, D), dtype), ((batch, D), dtype), ((2, D), dtype), ((D // 16, 2, D), dtype))
        self._fn = lib().dfs_conv2

    def __call__(self, x, x_prev, base, W_c):
        args = (x, x_prev, base, W_c)
        for t, (shape, dtype) in zip(args, self._expect):
            if t.shape != shape or t.dtype != dtype or t.device != self.device or not t.is_contiguous():
                raise ValueError(f"convolution input must be a contiguous {dtype} tensor of shape {shape} "
                                 f"on {self.device}")
        rc = self._fn(x.data_ptr(), x_prev.data_ptr(), base.data_ptr(), W_c.data_ptr(), self._dt, *self._dims,
                      self.y.data_ptr(), self.workspace.data_ptr(), self._ws_bytes,
                      torch.cuda.current_stream(self.device).cuda_stream)
        _check(rc, "dfs_conv2")
        return self.y
