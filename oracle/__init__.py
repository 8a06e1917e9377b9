"""PISA CPU oracle (ctypes wrapper over ``pisa_oracle.c``) -- TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline``
leg may import this package.  It shares nothing with the GPU library and never
imports it.  Everything is computed in float64 from the exact input values.

Method source: "Block Sparse Attention with Log-Linear Complexity" (PISA), the
hyper.ai page, sections on block-sparse attention, the pyramid key-block
hierarchy, coarse-to-fine top-K selection and kernel implementation.  The C
file's header lists the readings taken where the page is silent.

Inputs are numpy arrays: ``uint16`` = bf16 bit patterns, ``float32`` = fp32.
Layouts: q [B][Hq][N][D], k and v [B][Hkv][N][D].
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pisa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libpisa_oracle.so")
_lib = None

CNT = {
    "queries": 0,
    "scored_blocks": 1,
    "child_dots": 2,
    "leaf_pairs": 3,
    "leaf_key_dots": 4,
    "max_candidates": 5,
    "max_kept": 6,
    "scored_levels": 7,
}
CNT_LEVEL_BASE = 16


def build(force: bool = False, src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the oracle with gcc (plain -O2, IEEE arithmetic, OpenMP)."""
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src):
        tmp = out + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", src, "-o", tmp, "-lm"])
        os.replace(tmp, out)
    return out


class _Problem(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("N", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
        ("D", ctypes.c_int32), ("C", ctypes.c_int32), ("K", ctypes.c_int32), ("causal", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("q_sampled", ctypes.c_int32), ("scale", ctypes.c_double),
    ]


def load(path: str = _LIB_PATH):
    """Load (building first if needed) an oracle shared library."""
    global _lib
    if path == _LIB_PATH and _lib is not None:
        return _lib
    if path == _LIB_PATH and not os.path.exists(path):
        build()
    lib = ctypes.CDLL(path)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    P = ctypes.POINTER(_Problem)
    lib.oracle_level_rows.argtypes, lib.oracle_level_rows.restype = [i64, i32, i32], i64
    lib.oracle_levels.argtypes, lib.oracle_levels.restype = [i64, i32], i32
    lib.oracle_pyramid_rows.argtypes, lib.oracle_pyramid_rows.restype = [i64, i32], i64
    lib.oracle_build_pyramid.argtypes, lib.oracle_build_pyramid.restype = [P, vp, vp], ctypes.c_int
    lib.oracle_select.argtypes = [P, vp, vp, vp, i64, vp, vp, vp, vp]
    lib.oracle_select.restype = ctypes.c_int
    lib.oracle_attention.argtypes = [P, vp, vp, vp, vp, i64, vp, vp, vp]
    lib.oracle_attention.restype = ctypes.c_int
    lib.oracle_flat_select.argtypes = [P, vp, vp, vp, i64, vp, vp]
    lib.oracle_flat_select.restype = ctypes.c_int
    lib.oracle_exact_topk.argtypes = [P, vp, vp, vp, i64, vp, vp]
    lib.oracle_exact_topk.restype = ctypes.c_int
    lib.oracle_leaf_scores.argtypes = [P, vp, vp, vp, i64, vp, i32, vp]
    lib.oracle_leaf_scores.restype = ctypes.c_int
    lib.oracle_attention_backward.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.oracle_attention_backward.restype = ctypes.c_int
    lib.oracle_counter_len.argtypes, lib.oracle_counter_len.restype = [], ctypes.c_int
    lib.oracle_threads.argtypes, lib.oracle_threads.restype = [], ctypes.c_int
    if path == _LIB_PATH:
        _lib = lib
    return lib


@dataclass
class Problem:
    B: int
    N: int
    Hq: int
    Hkv: int
    D: int
    C: int
    K: int
    causal: bool = False
    scale: float | None = None  # None -> 1/sqrt(D)

    def c_struct(self, dtype_code: int, q_sampled: bool = False) -> _Problem:
        s = self.scale if self.scale is not None else 1.0 / math.sqrt(self.D)
        return _Problem(self.B, self.N, self.Hq, self.Hkv, self.D, self.C, self.K, int(self.causal), dtype_code,
                        int(q_sampled), s)


def _dtype_code(*arrays) -> int:
    kinds = {a.dtype for a in arrays if a is not None}
    if kinds == {np.dtype(np.uint16)}:
        return 1
    if kinds == {np.dtype(np.float32)}:
        return 0
    raise TypeError(f"inputs must all be uint16 (bf16 bits) or all float32, got {kinds}")


def _c(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a)


def _ts(p: Problem, ts) -> np.ndarray:
    if ts is None:
        return np.arange(p.N, dtype=np.int32)
    return np.ascontiguousarray(np.asarray(ts, dtype=np.int32))


def threads(lib=None) -> int:
    """Host threads used by the oracle's parallel loops."""
    return (lib or load()).oracle_threads()


def levels(n: int, C: int, lib=None) -> int:
    return (lib or load()).oracle_levels(n, C)


def level_rows(n: int, C: int, level: int, lib=None) -> int:
    return (lib or load()).oracle_level_rows(n, C, level)


def pyramid(p: Problem, k: np.ndarray, lib=None) -> list:
    """List over levels 1..L of float64 arrays [B][Hkv][M_l][D]."""
    lib = lib or load()
    k = _c(k)
    rows = lib.oracle_pyramid_rows(p.N, p.C)
    out = np.empty((p.B, p.Hkv, rows, p.D), np.float64)
    lib.oracle_build_pyramid(ctypes.byref(p.c_struct(_dtype_code(k))), k.ctypes.data, out.ctypes.data)
    res, off = [], 0
    for l in range(1, lib.oracle_levels(p.N, p.C) + 1):
        m = lib.oracle_level_rows(p.N, p.C, l)
        res.append(out[:, :, off:off + m, :])
        off += m
    return res


def _check_q(p: Problem, q: np.ndarray, nt: int, q_sampled: bool) -> None:
    want = (p.B, p.Hq, nt if q_sampled else p.N, p.D)
    if q.shape != want:
        raise ValueError(f"q shape {q.shape} != {want}")


def select(p: Problem, q: np.ndarray, k: np.ndarray, ts=None, lib=None, q_sampled: bool = False):
    """PISA selection for the query positions ``ts`` (all positions by
    default).  With ``q_sampled`` q holds only those positions,
    [B][Hq][len(ts)][D].  Returns (idx int32 [B][Hkv][nt][K] ascending -1 padded,
    score float64 same shape (GQA-summed leaf LSE, -inf padded),
    min_gap float64 [B][Hkv][nt], counters dict)."""
    lib = lib or load()
    q, k, ts = _c(q), _c(k), _ts(p, ts)
    nt = len(ts)
    _check_q(p, q, nt, q_sampled)
    idx = np.empty((p.B, p.Hkv, nt, p.K), np.int32)
    score = np.empty((p.B, p.Hkv, nt, p.K), np.float64)
    gap = np.empty((p.B, p.Hkv, nt), np.float64)
    cnt = np.zeros(lib.oracle_counter_len(), np.int64)
    rc = lib.oracle_select(ctypes.byref(p.c_struct(_dtype_code(q, k), q_sampled)), q.ctypes.data, k.ctypes.data,
                           ts.ctypes.data, nt, idx.ctypes.data, score.ctypes.data, gap.ctypes.data, cnt.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle_select failed ({rc})")
    counters = {name: int(cnt[i]) for name, i in CNT.items()}
    counters["per_level_candidates"] = [int(c) for c in cnt[CNT_LEVEL_BASE:]]
    return idx, score, gap, counters


def attention(p: Problem, q, k, v, idx, ts=None, lib=None, q_sampled: bool = False):
    """Softmax attention of every query head over the keys of its KV head's
    selected leaves.  Returns (o float64 [B][Hq][nt][D], lse [B][Hq][nt])."""
    lib = lib or load()
    q, k, v, ts = _c(q), _c(k), _c(v), _ts(p, ts)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    nt = len(ts)
    _check_q(p, q, nt, q_sampled)
    if idx.shape != (p.B, p.Hkv, nt, p.K):
        raise ValueError(f"idx shape {idx.shape} != {(p.B, p.Hkv, nt, p.K)}")
    o = np.empty((p.B, p.Hq, nt, p.D), np.float64)
    lse = np.empty((p.B, p.Hq, nt), np.float64)
    rc = lib.oracle_attention(ctypes.byref(p.c_struct(_dtype_code(q, k, v), q_sampled)), q.ctypes.data, k.ctypes.data,
                              v.ctypes.data, ts.ctypes.data, nt, idx.ctypes.data, o.ctypes.data, lse.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle_attention failed ({rc})")
    return o, lse


def flat_select(p: Problem, q, k, ts=None, lib=None, q_sampled: bool = False):
    """Single-level selector over all leaf summaries.  Returns (idx, score)."""
    lib = lib or load()
    q, k, ts = _c(q), _c(k), _ts(p, ts)
    nt = len(ts)
    _check_q(p, q, nt, q_sampled)
    idx = np.empty((p.B, p.Hkv, nt, p.K), np.int32)
    score = np.empty((p.B, p.Hkv, nt, p.K), np.float64)
    rc = lib.oracle_flat_select(ctypes.byref(p.c_struct(_dtype_code(q, k), q_sampled)), q.ctypes.data, k.ctypes.data,
                                ts.ctypes.data, nt, idx.ctypes.data, score.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle_flat_select failed ({rc})")
    return idx, score


def attention_backward(p: Problem, q, k, v, idx, dout, lib=None):
    """Gradients of L = sum_t dout_t . o_t for attention over the fixed
    selection idx [B][Hkv][N][K] (every position).  Returns (dq, dk, dv) in
    float64, shaped like q, k, v."""
    lib = lib or load()
    q, k, v, dout = _c(q), _c(k), _c(v), _c(dout)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    if q.shape != (p.B, p.Hq, p.N, p.D) or dout.shape != q.shape:
        raise ValueError(f"q / dout shape {q.shape} / {dout.shape} != {(p.B, p.Hq, p.N, p.D)}")
    if idx.shape != (p.B, p.Hkv, p.N, p.K):
        raise ValueError(f"idx shape {idx.shape} != {(p.B, p.Hkv, p.N, p.K)}")
    dq = np.empty(q.shape, np.float64)
    dk = np.empty(k.shape, np.float64)
    dv = np.empty(v.shape, np.float64)
    rc = lib.oracle_attention_backward(ctypes.byref(p.c_struct(_dtype_code(q, k, v, dout))), q.ctypes.data,
                                       k.ctypes.data, v.ctypes.data, idx.ctypes.data, dout.ctypes.data,
                                       dq.ctypes.data, dk.ctypes.data, dv.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle_attention_backward failed ({rc})")
    return dq, dk, dv


def exact_topk(p: Problem, q, k, ts=None, lib=None, q_sampled: bool = False):
    """Top-K over every valid leaf by the exact level-1 block score (raw-key
    LSE summed over the group): what the descent returns when every leaf is a
    candidate.  Returns (idx, score) shaped like select()'s."""
    lib = lib or load()
    q, k, ts = _c(q), _c(k), _ts(p, ts)
    nt = len(ts)
    _check_q(p, q, nt, q_sampled)
    idx = np.empty((p.B, p.Hkv, nt, p.K), np.int32)
    score = np.empty((p.B, p.Hkv, nt, p.K), np.float64)
    rc = lib.oracle_exact_topk(ctypes.byref(p.c_struct(_dtype_code(q, k), q_sampled)), q.ctypes.data, k.ctypes.data,
                               ts.ctypes.data, nt, idx.ctypes.data, score.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle_exact_topk failed ({rc})")
    return idx, score


def leaf_scores(p: Problem, q, k, leaves, ts=None, lib=None, q_sampled: bool = False):
    """Level-1 block score (raw-key LSE, causally masked, summed over the GQA
    group) of every listed leaf.  leaves: int [B][Hkv][nt][nl] (entries < 0
    give -inf).  Returns float64 [B][Hkv][nt][nl]."""
    lib = lib or load()
    q, k, ts = _c(q), _c(k), _ts(p, ts)
    nt = len(ts)
    _check_q(p, q, nt, q_sampled)
    leaves = np.ascontiguousarray(leaves, dtype=np.int32)
    if leaves.ndim != 4 or leaves.shape[:3] != (p.B, p.Hkv, nt):
        raise ValueError(f"leaves shape {leaves.shape} != {(p.B, p.Hkv, nt)} + (nl,)")
    nl = leaves.shape[3]
    out = np.empty(leaves.shape, np.float64)
    rc = lib.oracle_leaf_scores(ctypes.byref(p.c_struct(_dtype_code(q, k), q_sampled)), q.ctypes.data, k.ctypes.data,
                                ts.ctypes.data, nt, leaves.ctypes.data, nl, out.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle_leaf_scores failed ({rc})")
    return out


def decode_reference(p: Problem, q_new, k_prefix, v_prefix, lib=None):
    """One decode step as the method defines it: the new token sits at
    position n-1 of an n-token prefix whose pyramid is that of the prefix, and
    every block of the prefix is valid for it.  q_new: [B][Hq][D];
    k_prefix, v_prefix: [B][Hkv][n][D] including the new token's k and v.
    Returns (idx [B][Hkv][K], score, min_gap [B][Hkv], o [B][Hq][D], lse)."""
    n = k_prefix.shape[2]
    pp = Problem(p.B, n, p.Hq, p.Hkv, p.D, p.C, p.K, causal=True, scale=p.scale)
    q1 = np.ascontiguousarray(q_new[:, :, None, :])
    ts = [n - 1]
    idx, score, gap, _ = select(pp, q1, k_prefix, ts=ts, lib=lib, q_sampled=True)
    o, lse = attention(pp, q1, k_prefix, v_prefix, idx, ts=ts, lib=lib, q_sampled=True)
    return idx[:, :, 0], score[:, :, 0], gap[:, :, 0], o[:, :, 0], lse[:, :, 0]
