"""The prefill step (pyramid, two-stage selection, leaf-major attention) and
the fused decode step captured in a HIP graph.

The library enqueues kernels only (no memset, copy or allocation inside a
call), so a captured step must replay to the eager result.  Each replay runs
after eager work of the program itself (calls on other inputs that rewrite
the shared workspaces) and after the outputs were overwritten, and is
compared with the eager run: identical leaf indices, scores and outputs
within 1e-6 (each (query, leaf) pair is computed on its own, whatever work
chunk the clustering puts it in)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from gpu_util import log, to_dev
from hierarchical_block_sparse_mean_amd import inputs as I
from hierarchical_block_sparse_mean_amd import pisa

pytestmark = pytest.mark.gpu

REPLAYS = 3


def test_prefill_step_graph_replays():
    w = I.Workload("graph_bf16", 1, 2100, 16, 4, 128, 64, 8, "bf16", True, "leaf_per_query", seed=61)
    other = I.Workload("graph_bf16_other", 1, 2100, 16, 4, 128, 64, 8, "bf16", True, seed=62)
    log("[test_prefill_step_graph_replays]")
    d, d2 = I.generate(w), I.generate(other)
    q, k, v = (to_dev(d[x]) for x in ("q", "k", "v"))
    q2, k2, v2 = (to_dev(d2[x]) for x in ("q", "k", "v"))
    p = pisa.Problem(w.B, w.N, w.Hq, w.Hkv, w.D, w.C, w.K, causal=w.causal, dtype=w.dtype)
    pyr = pisa.alloc_pyramid(p)
    ws = pisa.workspace(pisa.select_workspace_bytes(p))
    aws = pisa.workspace(pisa.attn_workspace_bytes(p))
    idx = torch.empty((w.B, w.Hkv, w.N, w.K), dtype=torch.int32, device="cuda")
    score = torch.empty((w.B, w.Hkv, w.N, w.K), dtype=torch.float32, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device="cuda")

    def step(qq, kk, vv):
        pisa.build_pyramid(p, kk, pyr)
        pisa.select(p, qq, kk, pyr, idx=idx, score=score, ws=ws)
        pisa.sparse_attn(p, qq, kk, vv, idx, o=o, lse=lse, ws=aws)

    step(q, k, v)
    torch.cuda.synchronize()
    ref = [x.clone() for x in (idx, score, o, lse)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up on the capture stream
        step(q, k, v)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(q, k, v)
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        step(q2, k2, v2)  # eager work on other inputs: rewrites pyr, ws, aws and the outputs
        torch.cuda.synchronize()
        assert not torch.equal(idx, ref[0])
        idx.fill_(-7)
        score.fill_(float("nan"))
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, ref[0]), f"replay {r}: idx differs"
        for label, got, want in (("score", score, ref[1]), ("o", o, ref[2]), ("lse", lse, ref[3])):
            a, b = got.float(), want.float()
            fin = torch.isfinite(b)
            assert torch.equal(torch.isfinite(a), fin), f"replay {r}: {label} finiteness differs"
            err = (a[fin] - b[fin]).abs().max().item()
            assert err <= 1e-6 * max(1.0, b[fin].abs().max().item()), f"replay {r}: {label} error {err}"
        log(f"  replay {r} matches the eager step")


def test_decode_steps_graph_replays():
    """Four decode steps captured once; each replay starts from the same
    restored cache state and must reproduce the eager steps."""
    w = I.Workload("graph_dec", 2, 1021, 8, 2, 128, 64, 4, "bf16", True, seed=63, steps=4)
    log("[test_decode_steps_graph_replays]")
    cache = I.decode_cache(w)
    cap = cache["cap"]
    dp = pisa.DecodeProblem(w.B, cap, w.Hq, w.Hkv, w.D, w.C, w.K, dtype=w.dtype)
    kc, vc = to_dev(cache["k"]), to_dev(cache["v"])
    pp = dp.prefill_problem(w.N)
    pyr = pisa.build_pyramid(pp, kc, pisa.alloc_pyramid(pp))
    length = torch.full((w.B,), w.N, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    toks = [I.decode_token(w, s) for s in range(w.steps)]
    tq = [to_dev(t["q"]) for t in toks]
    tk = [to_dev(t["k"]) for t in toks]
    tv = [to_dev(t["v"]) for t in toks]
    outs = [torch.empty((w.B, w.Hq, w.D), dtype=torch.bfloat16, device="cuda") for _ in range(w.steps)]
    idxs = [torch.empty((w.B, w.Hkv, w.K), dtype=torch.int32, device="cuda") for _ in range(w.steps)]
    torch.cuda.synchronize()
    state0 = [x.clone() for x in (kc, vc, pyr, length)]

    def restore():
        for dst, src in zip((kc, vc, pyr, length), state0):
            dst.copy_(src)

    def steps():
        for s in range(w.steps):
            pisa.decode_step(dp, kc, vc, pyr, length, tq[s], tk[s], tv[s], o=outs[s], idx=idxs[s], err=err)

    steps()
    torch.cuda.synchronize()
    ref = [x.clone() for x in outs + idxs]
    ref_len = length.clone()
    restore()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        steps()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    restore()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        steps()
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        restore()
        for x in outs:
            x.fill_(float("nan"))
        for x in idxs:
            x.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(length, ref_len)
        for i, (got, want) in enumerate(zip(outs + idxs, ref)):
            if got.dtype == torch.int32:
                assert torch.equal(got, want), f"replay {r}: idx of step {i - w.steps} differs"
            else:
                e = (got.float() - want.float()).abs().max().item()
                assert e <= 1e-6, f"replay {r}: o of step {i} differs by {e}"
        log(f"  replay {r} matches the eager steps")
    assert int(err.item()) == 0
