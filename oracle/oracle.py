"""CPU oracle for the zero-copy MoE dispatch -> expert -> combine path.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The product package never imports
this module, and this module imports nothing from the product package.

The arithmetic lives in ``oracle.c`` (plain C, compiled with gcc); this file
marshals numpy arrays into it and composes the steps in the order the
"MORI CCO: Next-Generation Collective Communication Object for GPUs" article
gives them in its section "Zero-copy MoE dispatch -> expert -> combine":
dispatch into the receive region, expert from the receive region into the
combine staging region (row i to row i), combine from the staging region.

bf16 tensors are carried as ``numpy.uint16`` bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

OK = 0
BAD_EXPERT = 1
CAPACITY = 2


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so (gcc, no fast-math, no FP contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
               "-shared", "-fPIC", "-o", tmp, _SRC, "-lm", "-lpthread"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64 = ctypes.c_int32, ctypes.c_int64
        L.orc_plan.argtypes = [P, i64, i32, i32, i32, i64, P, P, P, P]
        L.orc_plan.restype = ctypes.c_int
        L.orc_dispatch.argtypes = [P, P, P, P, i64, i32, i64, i32, i32, i64, P, P, P, P]
        L.orc_dispatch.restype = None
        L.orc_dispatch_fp8.argtypes = [P, P, i32, P, P, P, i64, i32, i64, i32, i32, i64, P, P, P, P]
        L.orc_dispatch_fp8.restype = None
        L.orc_swiglu_rows.argtypes = [P, i64, i64, i64, P, P, P, ctypes.c_int]
        L.orc_swiglu_rows.restype = None
        L.orc_combine_tokens.argtypes = [P, P, P, P, P, i64, i32, i64, i32, i32, i64, P]
        L.orc_combine_tokens.restype = None
        L.orc_combine_rows.argtypes = [P, P, i64, i32, i64, P]
        L.orc_combine_rows.restype = None
        L.orc_f32_to_bf16.argtypes = [ctypes.c_float]
        L.orc_f32_to_bf16.restype = ctypes.c_uint16
        L.orc_dequant_e4m3_rows.argtypes = [P, i64, i64, i32, P]
        L.orc_dequant_e4m3_rows.restype = None
        L.orc_f64_to_bf16.argtypes = [ctypes.c_double]
        L.orc_f64_to_bf16.restype = ctypes.c_uint16
        _lib = L
    return _lib


def _p(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def capacity(T: int, K: int, E: int, S: int) -> int:
    """Rows each slot must be able to receive: every token may send min(K, E/S)
    distinct-expert rows to one slot (duplicates beyond that are a capacity
    error, not extra room)."""
    return T * min(K, E // S)


@dataclass
class Plan:
    status: int
    counts: np.ndarray      # int32 [E]
    expert_off: np.ndarray  # int32 [E], slot-local
    slot_total: np.ndarray  # int32 [S]
    pos: np.ndarray         # int32 [T, K]


def plan(idx: np.ndarray, E: int, S: int, cap: int) -> Plan:
    idx = _c(idx, np.int32)
    T, K = idx.shape
    counts = np.zeros(E, np.int32)
    off = np.zeros(E, np.int32)
    tot = np.zeros(S, np.int32)
    pos = np.zeros((T, K), np.int32)
    st = lib().orc_plan(_p(idx), T, K, E, S, cap, _p(counts), _p(off), _p(tot), _p(pos))
    return Plan(st, counts, off, tot, pos)


@dataclass
class Dispatched:
    disp_x: np.ndarray    # uint16 [S, cap, H]
    meta_src: np.ndarray  # int32  [S, cap]
    meta_w: np.ndarray    # float32 [S, cap]
    meta_e: np.ndarray    # int32  [S, cap]


def dispatch(x: np.ndarray, w: np.ndarray, idx: np.ndarray, pos: np.ndarray,
             E: int, S: int, cap: int) -> Dispatched:
    x = _c(x, np.uint16)
    w = _c(w, np.float32)
    idx = _c(idx, np.int32)
    pos = _c(pos, np.int32)
    T, H = x.shape
    K = idx.shape[1]
    dx = np.zeros((S, cap, H), np.uint16)
    ms = np.full((S, cap), -1, np.int32)
    mw = np.zeros((S, cap), np.float32)
    me = np.full((S, cap), -1, np.int32)
    lib().orc_dispatch(_p(x), _p(w), _p(idx), _p(pos), T, K, H, E, S, cap,
                       _p(dx), _p(ms), _p(mw), _p(me))
    return Dispatched(dx, ms, mw, me)


def dispatch_fp8(x8: np.ndarray, scales: np.ndarray, w: np.ndarray, idx: np.ndarray,
                 pos: np.ndarray, E: int, S: int, cap: int) -> Dispatched:
    """Dispatch of 8-bit tokens x8 [T, H] (raw bytes) with fp32 scales
    [T, ns]: returns the receive rows as bytes [S, cap, 2H] (token bytes,
    then the scales' bytes, then zeros) and the per-row metadata."""
    x8 = _c(x8, np.uint8)
    scales = _c(scales, np.float32)
    w = _c(w, np.float32)
    idx = _c(idx, np.int32)
    pos = _c(pos, np.int32)
    T, H = x8.shape
    ns = scales.shape[1]
    assert scales.shape[0] == T and 4 * ns <= H
    K = idx.shape[1]
    rows = np.zeros((S, cap, 2 * H), np.uint8)
    ms = np.full((S, cap), -1, np.int32)
    mw = np.zeros((S, cap), np.float32)
    me = np.full((S, cap), -1, np.int32)
    lib().orc_dispatch_fp8(_p(x8), _p(scales), ns, _p(w), _p(idx), _p(pos), T, K, H, E, S, cap,
                           _p(rows), _p(ms), _p(mw), _p(me))
    return Dispatched(rows, ms, mw, me)


def dequant_e4m3_rows(rows: np.ndarray, ns: int) -> np.ndarray:
    """The bf16 expert input of 8-bit receive rows: rows [..., 2H] bytes
    (H e4m3 values, then ns fp32 scales) -> bf16 bits [..., H]; each value
    decoded, times its block's scale in binary32, rounded to bf16."""
    rows = _c(rows, np.uint8)
    shape = rows.shape
    H = shape[-1] // 2
    assert shape[-1] == 2 * H and ns >= 0 and 4 * ns <= H and (ns == 0 or H % ns == 0)
    n = int(np.prod(shape[:-1]))
    out = np.zeros(shape[:-1] + (H,), np.uint16)
    lib().orc_dequant_e4m3_rows(_p(rows), n, H, ns, _p(out))
    return out


def swiglu_rows(X: np.ndarray, w13_e: np.ndarray, w2_e: np.ndarray,
                nthreads: int | None = None) -> np.ndarray:
    """SwiGLU of one expert on the rows X [n, H]; w13_e [2I, H], w2_e [H, I]."""
    X = _c(X, np.uint16)
    w13_e = _c(w13_e, np.uint16)
    w2_e = _c(w2_e, np.uint16)
    n, H = X.shape
    I2, H2 = w13_e.shape
    assert H2 == H and I2 % 2 == 0 and w2_e.shape == (H, I2 // 2)
    Y = np.zeros((n, H), np.uint16)
    lib().orc_swiglu_rows(_p(X), n, H, I2 // 2, _p(w13_e), _p(w2_e), _p(Y),
                          nthreads or default_threads())
    return Y


def expert_all(disp_x: np.ndarray, counts: np.ndarray, expert_off: np.ndarray,
               w13: np.ndarray, w2: np.ndarray, E: int, S: int,
               nthreads: int | None = None) -> np.ndarray:
    """Run every expert on its rows of the receive region; returns the
    combine staging region [S, cap, H] (rows past slot_total stay 0)."""
    eps = E // S
    cap = disp_x.shape[1]
    out = np.zeros_like(disp_x)
    for e in range(E):
        s, o = e // eps, int(expert_off[e])
        n = min(int(counts[e]), cap - o)  # rows past the slot were dropped
        if n <= 0:
            continue
        out[s, o:o + n] = swiglu_rows(disp_x[s, o:o + n], w13[e], w2[e], nthreads)
    return out


def combine_tokens(src: np.ndarray, w: np.ndarray, idx: np.ndarray, pos: np.ndarray,
                   E: int, S: int, tokens: np.ndarray | None = None) -> np.ndarray:
    src = _c(src, np.uint16)
    w = _c(w, np.float32)
    idx = _c(idx, np.int32)
    pos = _c(pos, np.int32)
    Sx, cap, H = src.shape
    assert Sx == S
    T, K = idx.shape
    if tokens is None:
        tokens = np.arange(T, dtype=np.int64)
    tokens = _c(tokens, np.int64)
    out = np.zeros((tokens.shape[0], H), np.uint16)
    lib().orc_combine_tokens(_p(src), _p(w), _p(idx), _p(pos), _p(tokens),
                             tokens.shape[0], K, H, E, S, cap, _p(out))
    return out


def combine_rows(rows: list[np.ndarray], w: np.ndarray) -> np.ndarray:
    """rows[q*K + j] is the bf16 row [H] that token q's pair j contributes;
    w is [nt, K].  Returns [nt, H]."""
    w = _c(w, np.float32)
    nt, K = w.shape
    assert len(rows) == nt * K
    rows = [_c(r, np.uint16) for r in rows]
    H = rows[0].shape[-1]
    ptrs = (ctypes.c_void_p * len(rows))(*[r.ctypes.data for r in rows])
    out = np.zeros((nt, H), np.uint16)
    lib().orc_combine_rows(ctypes.cast(ptrs, ctypes.c_void_p), _p(w), nt, K, H, _p(out))
    return out


def f32_to_bf16(v: float) -> int:
    return int(lib().orc_f32_to_bf16(v))


def f64_to_bf16(v: float) -> int:
    return int(lib().orc_f64_to_bf16(v))


@dataclass
class PipelineResult:
    plan: Plan
    disp: Dispatched
    out_tok: np.ndarray | None  # [S, cap, H] (None for identity experts)
    out: np.ndarray             # [T, H]


def pipeline(x, w, idx, E, S, cap, w13=None, w2=None, nthreads=None,
             allow_overflow=False) -> PipelineResult:
    """The whole path on the CPU: plan, dispatch, expert (SwiGLU, or the
    identity when no weights are given), combine.  With allow_overflow a
    slot overflow is not an error: the pairs past a slot's capacity are
    dropped (pos -1) and the rest of the path runs without them."""
    pl = plan(idx, E, S, cap)
    if pl.status != OK and not (allow_overflow and pl.status == CAPACITY):
        raise ValueError("oracle plan failed with status %d" % pl.status)
    d = dispatch(x, w, idx, pl.pos, E, S, cap)
    if w13 is None:
        out_tok = None
        src = d.disp_x
    else:
        out_tok = expert_all(d.disp_x, pl.counts, pl.expert_off, w13, w2, E, S, nthreads)
        src = out_tok
    out = combine_tokens(src, w, idx, pl.pos, E, S)
    return PipelineResult(pl, d, out_tok, out)
