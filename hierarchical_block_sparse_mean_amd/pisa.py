"""Thin ctypes binding of libpisa.so (the C ABI in include/pisa.h).

Argument marshalling only: every step of the hot path runs in the HIP
kernels of libpisa.so.  PyTorch supplies device memory (tensors on a ROCm
device) and the current HIP stream.  There is no CPU fallback: if the library
is missing, loading it raises.

Names follow the C entry points: build_pyramid, select, sparse_attn,
flat_select, decode_step.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpisa.so")
_lib = None

PISA_OK, PISA_ERR_INVALID_ARG, PISA_ERR_UNSUPPORTED, PISA_ERR_WORKSPACE, PISA_ERR_HIP = range(5)
PISA_F32, PISA_BF16 = 0, 1
SELECT_AUTO, SELECT_TWO_STAGE, SELECT_FUSED = 0, 1, 2
ATTN_AUTO, ATTN_LEAF_MAJOR, ATTN_QUERY_MAJOR = 0, 1, 2
STATUS_NAMES = {0: "PISA_OK", 1: "PISA_ERR_INVALID_ARG", 2: "PISA_ERR_UNSUPPORTED", 3: "PISA_ERR_WORKSPACE",
                4: "PISA_ERR_HIP"}

EXPORTS = [
    "pisa_pyramid_bytes", "pisa_levels", "pisa_level_rows", "pisa_level_offset", "pisa_build_pyramid",
    "pisa_select_workspace_bytes", "pisa_select", "pisa_attn_workspace_bytes", "pisa_sparse_attn",
    "pisa_attn_backward_workspace_bytes", "pisa_sparse_attn_backward", "pisa_flat_workspace_bytes", "pisa_flat_select", "pisa_decode_step", "pisa_timer_enable", "pisa_timer_report",
    "pisa_route_counts", "pisa_select_noalloc", "pisa_probe_gather", "pisa_probe_stream",
    "pisa_last_error", "pisa_version",
]


class PisaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class CProblem(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("N", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
        ("D", ctypes.c_int32), ("C", ctypes.c_int32), ("g", ctypes.c_int32), ("K", ctypes.c_int32),
        ("causal", ctypes.c_int32), ("dtype", ctypes.c_int32), ("scale", ctypes.c_float),
        ("q_tile", ctypes.c_int32), ("cap", ctypes.c_int32), ("select_algo", ctypes.c_int32),
        ("attn_algo", ctypes.c_int32),
    ]


class CDecodeProblem(ctypes.Structure):
    _fields_ = [
        ("S", ctypes.c_int32), ("cap", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
        ("D", ctypes.c_int32), ("C", ctypes.c_int32), ("g", ctypes.c_int32), ("K", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("scale", ctypes.c_float),
    ]


def load(path: str = LIB_PATH):
    """Loads libpisa.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m hierarchical_block_sparse_mean_amd.build`"
                           " (there is no CPU fallback)")
    lib = ctypes.CDLL(path)
    vp, sz, i32, i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64
    P, DP = ctypes.POINTER(CProblem), ctypes.POINTER(CDecodeProblem)
    sigs = {
        "pisa_pyramid_bytes": ([P], sz),
        "pisa_levels": ([i64, i32], i32),
        "pisa_level_rows": ([i64, i32, i32], i64),
        "pisa_level_offset": ([i64, i32, i32], i64),
        "pisa_build_pyramid": ([P, vp, vp, vp], ctypes.c_int),
        "pisa_select_workspace_bytes": ([P], sz),
        "pisa_select": ([P, vp, vp, vp, vp, vp, vp, sz, vp], ctypes.c_int),
        "pisa_select_noalloc": ([P, vp, vp, vp, vp, vp, vp], ctypes.c_int),
        "pisa_probe_gather": ([vp, i64, i32, i32, i32, i64, vp, vp], ctypes.c_int),
        "pisa_probe_stream": ([vp, vp, i64, i32, i32, vp, vp], ctypes.c_int),
        "pisa_attn_workspace_bytes": ([P], sz),
        "pisa_sparse_attn": ([P, vp, vp, vp, vp, vp, vp, vp, sz, vp], ctypes.c_int),
        "pisa_attn_backward_workspace_bytes": ([P], sz),
        "pisa_sparse_attn_backward": ([P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp], ctypes.c_int),
        "pisa_flat_workspace_bytes": ([P], sz),
        "pisa_flat_select": ([P, vp, vp, vp, vp, vp, sz, vp], ctypes.c_int),
        "pisa_decode_step": ([DP, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp], ctypes.c_int),
        "pisa_timer_enable": ([i32], None),
        "pisa_route_counts": ([P, vp, vp, vp, vp, vp, sz, vp], ctypes.c_int),
        "pisa_timer_report": ([ctypes.c_char_p, sz], i32),
        "pisa_last_error": ([], ctypes.c_char_p),
        "pisa_version": ([], ctypes.c_char_p),
    }
    for name, (args, res) in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes, fn.restype = args, res
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != PISA_OK:
        raise PisaError(status, load().pisa_last_error().decode())


@dataclass
class Problem:
    """Mirror of pisa_problem.  dtype: "f32" or "bf16"."""

    B: int
    N: int
    Hq: int
    Hkv: int
    D: int
    C: int
    K: int
    causal: bool = False
    dtype: str = "bf16"
    scale: float = 0.0  # 0 -> 1/sqrt(D)
    g: int = 2
    q_tile: int = 0
    cap: int = 0
    select_algo: int = SELECT_AUTO
    attn_algo: int = ATTN_AUTO

    def c(self) -> CProblem:
        return CProblem(self.B, self.N, self.Hq, self.Hkv, self.D, self.C, self.g, self.K, int(self.causal),
                        PISA_BF16 if self.dtype == "bf16" else PISA_F32, self.scale, self.q_tile, self.cap,
                        self.select_algo, self.attn_algo)

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    @property
    def cap_tokens(self) -> int:
        return self.cap or self.N


def _stream(stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, name: str, shape, dtype) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} shape {tuple(t.shape)} != {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} dtype {t.dtype} != {dtype}")


def levels(n: int, C: int) -> int:
    return load().pisa_levels(n, C)


def level_rows(n: int, C: int, l: int) -> int:
    return load().pisa_level_rows(n, C, l)


def level_offset(cap: int, C: int, l: int) -> int:
    return load().pisa_level_offset(cap, C, l)


def pyramid_rows(p: Problem) -> int:
    cap = p.cap_tokens
    return sum(level_rows(cap, p.C, l) for l in range(1, levels(cap, p.C) + 1))


def pyramid_bytes(p: Problem) -> int:
    n = load().pisa_pyramid_bytes(ctypes.byref(p.c()))
    if n == 0:
        _check(PISA_ERR_INVALID_ARG)
    return n


def alloc_pyramid(p: Problem, device="cuda") -> torch.Tensor:
    """Flat float32 buffer of pisa_pyramid_bytes: fp32 summaries, then their
    fp16 block-floating-point copy and per-row exponents."""
    return torch.empty((pyramid_bytes(p) + 3) // 4, dtype=torch.float32, device=device)


def pyramid_view(p: Problem, pyr: torch.Tensor) -> torch.Tensor:
    """fp32 summaries [B][Hkv][R][D] of a pyramid buffer."""
    return pyr[: p.B * p.Hkv * pyramid_rows(p) * p.D].view(p.B, p.Hkv, pyramid_rows(p), p.D)


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def build_pyramid(p: Problem, k: torch.Tensor, pyr: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    _need(k, "k", (p.B, p.Hkv, p.cap_tokens, p.D), p.torch_dtype)
    if pyr is None:
        pyr = alloc_pyramid(p, k.device)
    _need(pyr, "pyr", ((pyramid_bytes(p) + 3) // 4,), torch.float32)
    _check(load().pisa_build_pyramid(ctypes.byref(p.c()), k.data_ptr(), pyr.data_ptr(), _stream(stream)))
    return pyr


def pyramid_level(p: Problem, pyr: torch.Tensor, l: int, n: int | None = None) -> torch.Tensor:
    """View of level l (rows M_l(n)) of a pyramid tensor."""
    n = p.N if n is None else n
    off = level_offset(p.cap_tokens, p.C, l)
    return pyramid_view(p, pyr)[:, :, off:off + level_rows(n, p.C, l), :]


def pyramid_f16_level(p: Problem, pyr: torch.Tensor, l: int, n: int | None = None) -> torch.Tensor:
    """Level l of the fp16 block-floating-point copy, decoded to float32
    (f16 * 2^ex)."""
    n = p.N if n is None else n
    off = level_offset(p.cap_tokens, p.C, l)
    R = pyramid_rows(p)
    plane = p.B * p.Hkv * R * p.D
    raw = pyr.view(torch.int16)
    f16 = raw[2 * plane: 3 * plane].view(torch.float16).view(p.B, p.Hkv, R, p.D)
    ex = raw[3 * plane: 3 * plane + 2 * p.B * p.Hkv * R].view(torch.int32).view(p.B, p.Hkv, R)
    rows = slice(off, off + level_rows(n, p.C, l))
    return torch.ldexp(f16[:, :, rows, :].float(), ex[:, :, rows, None].float())


def select_workspace_bytes(p: Problem) -> int:
    return load().pisa_select_workspace_bytes(ctypes.byref(p.c()))


def select(p: Problem, q, k, pyr, idx=None, score=None, ws=None, with_score: bool = True, stream=None):
    """Returns (idx int32 [B][Hkv][N][K], score float32 or None)."""
    _need(q, "q", (p.B, p.Hq, p.N, p.D), p.torch_dtype)
    _need(k, "k", (p.B, p.Hkv, p.cap_tokens, p.D), p.torch_dtype)
    dev = q.device
    if idx is None:
        idx = torch.empty((p.B, p.Hkv, p.N, p.K), dtype=torch.int32, device=dev)
    if score is None and with_score:
        score = torch.empty((p.B, p.Hkv, p.N, p.K), dtype=torch.float32, device=dev)
    if ws is None:
        ws = workspace(select_workspace_bytes(p), dev)
    _check(load().pisa_select(ctypes.byref(p.c()), q.data_ptr(), k.data_ptr(), pyr.data_ptr(), idx.data_ptr(),
                              _ptr(score), ws.data_ptr(), ws.numel(), _stream(stream)))
    return idx, score


NOALLOC_SCRATCH_BYTES = 128 << 20  # PISA_NOALLOC_SCRATCH_BYTES


def select_noalloc(p: Problem, q, k, pyr, idx, score=None, stream=None):
    """pisa_select_noalloc: pisa_select with the library's own per-GPU
    scratch (no workspace argument, nothing allocated by the call).  idx (and
    score, if given) must be preallocated.  Returns (idx, score)."""
    _need(q, "q", (p.B, p.Hq, p.N, p.D), p.torch_dtype)
    _need(k, "k", (p.B, p.Hkv, p.cap_tokens, p.D), p.torch_dtype)
    _need(idx, "idx", (p.B, p.Hkv, p.N, p.K), torch.int32)
    if score is not None:
        _need(score, "score", (p.B, p.Hkv, p.N, p.K), torch.float32)
    _check(load().pisa_select_noalloc(ctypes.byref(p.c()), q.data_ptr(), k.data_ptr(), pyr.data_ptr(),
                                      idx.data_ptr(), _ptr(score), _stream(stream)))
    return idx, score


def select_level2(p: Problem, ws: torch.Tensor) -> torch.Tensor:
    """View of the stage-1 result a two-stage select left in its workspace:
    int32 [B][Hkv][N][K], the level-2 blocks kept per (b, h, t), -1 padded."""
    n = p.B * p.Hkv * p.N * p.K
    return ws[: 4 * n].view(torch.int32).view(p.B, p.Hkv, p.N, p.K)


def attn_workspace_bytes(p: Problem) -> int:
    return load().pisa_attn_workspace_bytes(ctypes.byref(p.c()))


def sparse_attn(p: Problem, q, k, v, idx, o=None, lse=None, ws=None, with_lse: bool = True, stream=None):
    """Returns (o [B][Hq][N][D] input dtype, lse float32 [B][Hq][N] or None)."""
    _need(q, "q", (p.B, p.Hq, p.N, p.D), p.torch_dtype)
    _need(k, "k", (p.B, p.Hkv, p.cap_tokens, p.D), p.torch_dtype)
    _need(v, "v", (p.B, p.Hkv, p.cap_tokens, p.D), p.torch_dtype)
    _need(idx, "idx", (p.B, p.Hkv, p.N, p.K), torch.int32)
    dev = q.device
    if o is None:
        o = torch.empty((p.B, p.Hq, p.N, p.D), dtype=p.torch_dtype, device=dev)
    if lse is None and with_lse:
        lse = torch.empty((p.B, p.Hq, p.N), dtype=torch.float32, device=dev)
    if ws is None:
        ws = workspace(attn_workspace_bytes(p), dev)
    _check(load().pisa_sparse_attn(ctypes.byref(p.c()), q.data_ptr(), k.data_ptr(), v.data_ptr(), idx.data_ptr(),
                                   o.data_ptr(), _ptr(lse), ws.data_ptr(), ws.numel(), _stream(stream)))
    return o, lse


def flat_workspace_bytes(p: Problem) -> int:
    return load().pisa_flat_workspace_bytes(ctypes.byref(p.c()))


def attn_backward_workspace_bytes(p: Problem) -> int:
    return load().pisa_attn_backward_workspace_bytes(ctypes.byref(p.c()))


def sparse_attn_backward(p: Problem, q, k, v, idx, o, lse, dout, dq=None, dk=None, dv=None, ws=None, stream=None):
    """Gradients (dq, dk, dv) of sum(dout * o) for the attention over the fixed
    selection idx; o and lse are the forward's outputs."""
    _need(q, "q", (p.B, p.Hq, p.N, p.D), p.torch_dtype)
    _need(k, "k", (p.B, p.Hkv, p.cap_tokens, p.D), p.torch_dtype)
    _need(v, "v", (p.B, p.Hkv, p.cap_tokens, p.D), p.torch_dtype)
    _need(idx, "idx", (p.B, p.Hkv, p.N, p.K), torch.int32)
    _need(o, "o", (p.B, p.Hq, p.N, p.D), p.torch_dtype)
    _need(lse, "lse", (p.B, p.Hq, p.N), torch.float32)
    _need(dout, "dout", (p.B, p.Hq, p.N, p.D), p.torch_dtype)
    dev = q.device
    if dq is None:
        dq = torch.empty_like(q)
    if dk is None:
        dk = torch.zeros_like(k)
    if dv is None:
        dv = torch.zeros_like(v)
    if ws is None:
        ws = workspace(attn_backward_workspace_bytes(p), dev)
    _check(load().pisa_sparse_attn_backward(ctypes.byref(p.c()), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                            idx.data_ptr(), o.data_ptr(), lse.data_ptr(), dout.data_ptr(),
                                            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws.data_ptr(), ws.numel(),
                                            _stream(stream)))
    return dq, dk, dv


def flat_select(p: Problem, q, pyr, idx=None, score=None, ws=None, with_score: bool = True, stream=None):
    _need(q, "q", (p.B, p.Hq, p.N, p.D), p.torch_dtype)
    dev = q.device
    if idx is None:
        idx = torch.empty((p.B, p.Hkv, p.N, p.K), dtype=torch.int32, device=dev)
    if score is None and with_score:
        score = torch.empty((p.B, p.Hkv, p.N, p.K), dtype=torch.float32, device=dev)
    if ws is None:
        ws = workspace(flat_workspace_bytes(p), dev)
    _check(load().pisa_flat_select(ctypes.byref(p.c()), q.data_ptr(), pyr.data_ptr(), idx.data_ptr(), _ptr(score),
                                   ws.data_ptr(), ws.numel(), _stream(stream)))
    return idx, score


@dataclass
class DecodeProblem:
    S: int
    cap: int
    Hq: int
    Hkv: int
    D: int
    C: int
    K: int
    dtype: str = "bf16"
    scale: float = 0.0
    g: int = 2

    def c(self) -> CDecodeProblem:
        return CDecodeProblem(self.S, self.cap, self.Hq, self.Hkv, self.D, self.C, self.g, self.K,
                              PISA_BF16 if self.dtype == "bf16" else PISA_F32, self.scale)

    def prefill_problem(self, n: int) -> Problem:
        """The problem that builds this cache's pyramid over its first n tokens."""
        return Problem(self.S, n, self.Hq, self.Hkv, self.D, self.C, self.K, causal=True, dtype=self.dtype,
                       scale=self.scale, g=self.g, cap=self.cap)


def decode_step(p: DecodeProblem, k_cache, v_cache, pyr, length, q_new, k_new, v_new, o=None, idx=None, score=None,
                err=None, stream=None):
    """One fused decode step; returns (o, idx, score)."""
    dt = torch.bfloat16 if p.dtype == "bf16" else torch.float32
    _need(k_cache, "k_cache", (p.S, p.Hkv, p.cap, p.D), dt)
    _need(v_cache, "v_cache", (p.S, p.Hkv, p.cap, p.D), dt)
    _need(length, "len", (p.S,), torch.int32)
    _need(q_new, "q_new", (p.S, p.Hq, p.D), dt)
    _need(k_new, "k_new", (p.S, p.Hkv, p.D), dt)
    _need(v_new, "v_new", (p.S, p.Hkv, p.D), dt)
    dev = q_new.device
    if o is None:
        o = torch.empty((p.S, p.Hq, p.D), dtype=dt, device=dev)
    _check(load().pisa_decode_step(ctypes.byref(p.c()), k_cache.data_ptr(), v_cache.data_ptr(), pyr.data_ptr(),
                                   length.data_ptr(), q_new.data_ptr(), k_new.data_ptr(), v_new.data_ptr(),
                                   o.data_ptr(), _ptr(idx), _ptr(score), _ptr(err), _stream(stream)))
    return o, idx, score


def timer_enable(on: bool) -> None:
    """Start (clearing earlier records) or stop per-kernel HIP event timing."""
    load().pisa_timer_enable(1 if on else 0)


def timer_report() -> dict:
    """{kernel: (launches, total_ms)} of the launches recorded since
    timer_enable(True); waits for their events and clears the records."""
    buf = ctypes.create_string_buffer(1 << 16)
    load().pisa_timer_report(buf, len(buf))
    out = {}
    for line in buf.value.decode().splitlines():
        name, n, ms = line.split("\t")
        out[name] = (int(n), float(ms))
    return out


def route_counts(p: Problem, q, k, pyr, ws=None, stream=None) -> dict:
    """Work counters of the stage-1 routing kernel (diagnostic run)."""
    counts = torch.zeros(6, dtype=torch.int64, device=q.device)
    if ws is None:
        ws = workspace(select_workspace_bytes(p), q.device)
    _check(load().pisa_route_counts(ctypes.byref(p.c()), q.data_ptr(), k.data_ptr(), pyr.data_ptr(),
                                    counts.data_ptr(), ws.data_ptr(), ws.numel(), _stream(stream)))
    c = counts.cpu().tolist()
    return {"queries": c[0], "scored_candidates": c[1], "child_rows": c[2], "scored_levels": c[3], "kept_level2": c[4],
            "child_rows_from_memory": c[5]}


def default_scale(D: int) -> float:
    return 1.0 / math.sqrt(D)


def probe_gather(table: torch.Tensor, rows_per_head: int, heads: int, D: int, workgroups: int, tiles_per_wave: int,
                 sink: torch.Tensor, stream=None) -> None:
    """Measurement probe: pisa_probe_gather over an fp16 table [heads][rows][D]."""
    _check(load().pisa_probe_gather(table.data_ptr(), rows_per_head, heads, D, workgroups, tiles_per_wave,
                                    sink.data_ptr(), _stream(stream)))


def probe_stream(src: torch.Tensor, dst: torch.Tensor | None, nbytes: int, mode: int, workgroups: int,
                 sink: torch.Tensor | None, stream=None) -> None:
    """Measurement probe: pisa_probe_stream (mode 0 reads src, mode 1 copies src to dst)."""
    _check(load().pisa_probe_stream(src.data_ptr(), _ptr(dst), nbytes, mode, workgroups, _ptr(sink),
                                    _stream(stream)))
