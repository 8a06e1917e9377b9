"""Seeded synthetic workloads for the PISA hot path.

This module only makes inputs: q, k, v tensors in the shapes, sizes and value
distributions of the workloads, plus planted "needle" structure.  It holds
none of the method's arithmetic and is shared by the CPU oracle's tests and
the GPU library's tests and benchmark, so both sides see bit-identical data.

Numbers come from the counter-based SplitMix64 + Box-Muller generator in
``pisa_gen.c`` (compiled next to this file): element ``i`` of tensor stream
``s`` under seed ``seed`` is a pure function of ``(seed, s, i)``, so any slice
can be regenerated alone.  bf16 tensors are returned as ``uint16`` bit
patterns, fp32 tensors as ``float32``.

Layouts (row-major): ``q[B][Hq][N][D]``, ``k, v[B][Hkv][N][D]``.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pisa_gen.c")
_LIB_PATH = os.path.join(_HERE, "libpisa_gen.so")
_lib = None

# tensor stream ids
STREAM_Q, STREAM_K, STREAM_V, STREAM_NEEDLE_IDX = 1, 2, 3, 4
STREAM_DEC_Q, STREAM_DEC_K, STREAM_DEC_V = 5, 6, 7
STREAM_NEEDLE_NOISE, STREAM_NEEDLE_DIR = 8, 9


def build_generator(force: bool = False) -> str:
    """Compile pisa_gen.c into libpisa_gen.so (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build_generator()
        lib = ctypes.CDLL(_LIB_PATH)
        u64, i64, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p
        for name in ("pisa_gen_normal_f64", "pisa_gen_normal_f32", "pisa_gen_normal_bf16", "pisa_gen_u64"):
            getattr(lib, name).argtypes = [u64, u64, i64, i64, vp]
            getattr(lib, name).restype = None
        lib.pisa_gen_f64_to_bf16.argtypes = [vp, i64, vp]
        lib.pisa_gen_f64_to_bf16.restype = None
        _lib = lib
    return _lib


def normal(seed: int, stream: int, n: int, start: int = 0, dtype: str = "f64") -> np.ndarray:
    """n standard-normal draws of (seed, stream) starting at element ``start``."""
    lib = _load()
    if dtype == "f64":
        out = np.empty(n, np.float64)
        lib.pisa_gen_normal_f64(seed, stream, start, n, out.ctypes.data)
    elif dtype == "f32":
        out = np.empty(n, np.float32)
        lib.pisa_gen_normal_f32(seed, stream, start, n, out.ctypes.data)
    elif dtype == "bf16":
        out = np.empty(n, np.uint16)
        lib.pisa_gen_normal_bf16(seed, stream, start, n, out.ctypes.data)
    else:
        raise ValueError(dtype)
    return out


def draws_u64(seed: int, stream: int, n: int, start: int = 0) -> np.ndarray:
    out = np.empty(n, np.uint64)
    _load().pisa_gen_u64(seed, stream, start, n, out.ctypes.data)
    return out


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """double -> float -> bf16, round to nearest even at each step."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, np.uint16)
    _load().pisa_gen_f64_to_bf16(x.ctypes.data, x.size, out.ctypes.data)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def widen(x: np.ndarray) -> np.ndarray:
    """Exact float64 values of a bf16 (uint16 bits) or float32 array."""
    if x.dtype == np.uint16:
        return bf16_bits_to_f32(x).astype(np.float64)
    return x.astype(np.float64)


@dataclass(frozen=True)
class Workload:
    """One synthetic workload.  Prefill: q [B][Hq][N][D], k/v [B][Hkv][N][D].
    Decode: B sequences with an N-token cached prefix, then ``steps`` new
    tokens, cache capacity N + steps."""

    name: str
    B: int
    N: int
    Hq: int
    Hkv: int
    D: int
    C: int
    K: int
    dtype: str  # "f32" or "bf16"
    causal: bool
    needles: str = "none"  # "none" | "leaf_per_query" | "shared_spans"
    seed: int = 0
    steps: int = 0
    g: int = 2

    @property
    def gq(self) -> int:
        return self.Hq // self.Hkv


WORKLOADS = {
    # tiny oracle case: 16 leaves (16 -> 8 -> 4 -> 2 -> 1), non-causal, fp32
    "tiny": Workload("tiny", 1, 1024, 4, 1, 64, 64, 4, "f32", False, "none", seed=0),
    "prefill_32k": Workload("prefill_32k", 1, 32768, 32, 8, 128, 64, 16, "bf16", True, "leaf_per_query", seed=1000),
    "prefill_128k": Workload("prefill_128k", 1, 131072, 32, 8, 128, 64, 16, "bf16", True, "leaf_per_query", seed=2000),
    "prefill_256k": Workload("prefill_256k", 1, 262144, 32, 8, 128, 128, 32, "bf16", True, "shared_spans", seed=3000),
    "decode_128k": Workload("decode_128k", 64, 131072, 32, 8, 128, 64, 16, "bf16", True, "none", seed=4000, steps=256),
}


def workload(name: str, **overrides) -> Workload:
    return replace(WORKLOADS[name], **overrides)


def _tensor(seed: int, stream: int, shape, dtype: str, start: int = 0) -> np.ndarray:
    n = int(np.prod(shape))
    return normal(seed, stream, n, start=start, dtype=dtype).reshape(shape)


def _distinct(seed: int, stream: int, start: int, pool: int, count: int) -> np.ndarray:
    """``count`` distinct integers from [0, pool), by ranking ``pool`` draws."""
    keys = draws_u64(seed, stream, pool, start=start)
    return np.sort(np.argsort(keys, kind="stable")[:count])


def _plant_leaf_per_query(w: Workload, q: np.ndarray, k: np.ndarray) -> dict:
    """Per (b, h): floor(M1/4) distinct host leaves j in [0, M1-2]; each host
    gets one needle query t in [(j+1)C, N) and all its keys become
    3 * unit(sum of the group's q_t) + 0.1 * N(0, 1) per component."""
    M1 = -(-w.N // w.C)
    P = M1 // 4
    meta = {"hosts": [], "queries": []}
    stride = 4 * M1 + 16
    for b in range(w.B):
        for h in range(w.Hkv):
            base = (b * w.Hkv + h) * stride
            hosts = _distinct(w.seed, STREAM_NEEDLE_IDX, base, M1 - 1, P)
            tdraw = draws_u64(w.seed, STREAM_NEEDLE_IDX, len(hosts), start=base + M1)
            ts = []
            for j, dr in zip(hosts, tdraw):
                lo = (int(j) + 1) * w.C
                t = lo + int(dr % np.uint64(w.N - lo))
                qsum = widen(q[b, h * w.gq:(h + 1) * w.gq, t, :]).sum(axis=0)
                unit = qsum / np.linalg.norm(qsum)
                kstart = ((b * w.Hkv + h) * w.N + int(j) * w.C) * w.D
                noise = normal(w.seed, STREAM_NEEDLE_NOISE, w.C * w.D, start=kstart).reshape(w.C, w.D)
                vals = 3.0 * unit[None, :] + 0.1 * noise
                k[b, h, int(j) * w.C:(int(j) + 1) * w.C, :] = _cast(vals, k.dtype)
                ts.append(t)
            meta["hosts"].append(hosts)
            meta["queries"].append(np.array(ts, np.int64))
    return meta


def _plant_shared_spans(w: Workload, q: np.ndarray, k: np.ndarray, n_hosts: int = 64, span: int = 1024) -> dict:
    """Per (b, h): 64 distinct host leaves j in [0, M1-2], each with a random
    unit direction u_j; host keys become 3 u_j + 0.1 N(0, 1); each host gets a
    disjoint span of ``span`` later queries whose vectors become
    (q + sqrt(D) u_j) / sqrt(2) in every query head of the group."""
    M1 = -(-w.N // w.C)
    meta = {"hosts": [], "spans": []}
    stride = 4 * M1 + 4096
    for b in range(w.B):
        for h in range(w.Hkv):
            base = (b * w.Hkv + h) * stride
            hosts = _distinct(w.seed, STREAM_NEEDLE_IDX, base, M1 - 1, min(n_hosts, M1 - 1))
            cursor = base + M1
            taken = []
            spans = []
            for n, j in enumerate(hosts):
                j = int(j)
                d = normal(w.seed, STREAM_NEEDLE_DIR, w.D, start=((b * w.Hkv + h) * n_hosts + n) * w.D)
                u = d / np.linalg.norm(d)
                kstart = ((b * w.Hkv + h) * w.N + j * w.C) * w.D
                noise = normal(w.seed, STREAM_NEEDLE_NOISE, w.C * w.D, start=kstart).reshape(w.C, w.D)
                hi = min((j + 1) * w.C, w.N)
                k[b, h, j * w.C:hi, :] = _cast((3.0 * u[None, :] + 0.1 * noise)[: hi - j * w.C], k.dtype)
                lo = (j + 1) * w.C
                if lo > w.N - span:
                    spans.append((j, -1))
                    continue
                start = -1
                for _ in range(256):
                    dr = draws_u64(w.seed, STREAM_NEEDLE_IDX, 1, start=cursor)[0]
                    cursor += 1
                    s = lo + int(dr % np.uint64(w.N - span - lo + 1))
                    if all(s + span <= a or s >= a + span for a in taken):
                        start = s
                        break
                spans.append((j, start))
                if start < 0:
                    continue
                taken.append(start)
                g0, g1 = h * w.gq, (h + 1) * w.gq
                block = widen(q[b, g0:g1, start:start + span, :])
                block = (block + math.sqrt(w.D) * u[None, None, :]) / math.sqrt(2.0)
                q[b, g0:g1, start:start + span, :] = _cast(block, q.dtype)
            meta["hosts"].append(hosts)
            meta["spans"].append(spans)
    return meta


def _cast(x: np.ndarray, dtype) -> np.ndarray:
    if dtype == np.uint16:
        return to_bf16_bits(x)
    return x.astype(np.float32)


def generate(w: Workload, with_v: bool = True) -> dict:
    """q, k, v (and needle metadata) of a prefill workload, or of a decode
    workload's cached prefix (q is then the prefix queries, rarely needed)."""
    qshape = (w.B, w.Hq, w.N, w.D)
    kshape = (w.B, w.Hkv, w.N, w.D)
    q = _tensor(w.seed, STREAM_Q, qshape, w.dtype)
    k = _tensor(w.seed, STREAM_K, kshape, w.dtype)
    v = _tensor(w.seed, STREAM_V, kshape, w.dtype) if with_v else None
    meta = {}
    if w.needles == "leaf_per_query":
        meta = _plant_leaf_per_query(w, q, k)
    elif w.needles == "shared_spans":
        meta = _plant_shared_spans(w, q, k)
    return {"q": q, "k": k, "v": v, "meta": meta}


def decode_cache(w: Workload, seqs=None) -> dict:
    """Cached prefix K/V of a decode workload laid out with capacity
    N + steps: k, v [S][Hkv][N + steps][D] (rows >= N are zero), for the
    sequences ``seqs`` (all by default).  Row s of the result is sequence
    seqs[s]; each is regenerated from its own element range."""
    seqs = list(range(w.B)) if seqs is None else list(seqs)
    cap = w.N + w.steps
    dt = np.uint16 if w.dtype == "bf16" else np.float32
    k = np.zeros((len(seqs), w.Hkv, cap, w.D), dt)
    v = np.zeros_like(k)
    per_seq = w.Hkv * w.N * w.D
    for r, s in enumerate(seqs):
        k[r, :, : w.N, :] = _tensor(w.seed, STREAM_K, (w.Hkv, w.N, w.D), w.dtype, start=s * per_seq)
        v[r, :, : w.N, :] = _tensor(w.seed, STREAM_V, (w.Hkv, w.N, w.D), w.dtype, start=s * per_seq)
    return {"k": k, "v": v, "cap": cap, "seqs": seqs}


def decode_prefix(w: Workload, s: int) -> tuple[np.ndarray, np.ndarray]:
    """Cached prefix k, v [Hkv][N][D] of decode sequence ``s`` alone (the
    same values decode_cache places in row s)."""
    per_seq = w.Hkv * w.N * w.D
    k = _tensor(w.seed, STREAM_K, (w.Hkv, w.N, w.D), w.dtype, start=s * per_seq)
    v = _tensor(w.seed, STREAM_V, (w.Hkv, w.N, w.D), w.dtype, start=s * per_seq)
    return k, v


def decode_token(w: Workload, step: int, seqs=None) -> dict:
    """New q [S][Hq][D], k, v [S][Hkv][D] of decode step ``step``."""
    out = {}
    for name, stream, H in (("q", STREAM_DEC_Q, w.Hq), ("k", STREAM_DEC_K, w.Hkv), ("v", STREAM_DEC_V, w.Hkv)):
        per = H * w.D
        if seqs is None:  # all sequences of a step are one contiguous element range
            out[name] = _tensor(w.seed, stream, (w.B, H, w.D), w.dtype, start=step * w.B * per)
        else:
            rows = [_tensor(w.seed, stream, (H, w.D), w.dtype, start=(step * w.B + s) * per) for s in seqs]
            out[name] = np.stack(rows)
    return out
