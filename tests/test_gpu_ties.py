"""GPU path on exact ties, pinned by closed forms rather than by the oracle.

With every query zero, every logit is exactly 0 on both the fp16 stage-1
products and the bf16 / fp32 leaf and attention products, so
  * each block's routing score is G_Q log(#valid children) and each leaf's
    score G_Q log(#valid keys): every full block ties with every other;
  * the tie rule (score descending, then the lower block index) then keeps,
    at every level, the lowest-index full blocks, and the returned leaves of
    query t are the first min(K, #valid leaves of t), ascending, -1 padded;
  * attention weights every valid key of those leaves equally: o is the mean
    of their values and lse the log of their number.
The parity tests exempt near-ties (gaps below 1e-3), so the tie rule itself
is checked only here.  Both selection schedules, both attention schedules,
the fused decode step and the attention backward (whose dK vanishes and
whose dV and dQ reduce to sums over the uniform weights) are run; the inputs
are ragged (partial last leaf and blocks with one child)."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from gpu_util import ATTN_TOL, log, to_dev, to_host_f64
from hierarchical_block_sparse_mean_amd import inputs as I
from hierarchical_block_sparse_mean_amd import pisa

pytestmark = pytest.mark.gpu

CASES = {
    "bf16_g4_c64_k8_causal": I.Workload("ties_bf16_g4", 1, 1500, 8, 2, 128, 64, 8, "bf16", True, seed=71),
    "bf16_g16_c32_k4_b2": I.Workload("ties_bf16_g16", 2, 1100, 16, 1, 64, 32, 4, "bf16", False, seed=72),
    "f32_g2_c48_k16_causal": I.Workload("ties_f32_g2", 1, 900, 4, 2, 64, 48, 16, "f32", True, seed=73),
}


def expected(w: I.Workload):
    """idx [N][K] and per-slot key counts [N][K] of the closed form (the same
    for every batch and KV head)."""
    M1 = -(-w.N // w.C)
    idx = np.full((w.N, w.K), -1, np.int64)
    cnt = np.zeros((w.N, w.K), np.int64)
    for t in range(w.N):
        nvalid = min(M1, t // w.C + 1) if w.causal else M1
        last = t + 1 if w.causal else w.N  # keys < last are valid
        for s in range(min(w.K, nvalid)):
            idx[t, s] = s
            cnt[t, s] = min((s + 1) * w.C, last) - s * w.C
    return idx, cnt


@pytest.mark.parametrize("algo", [pisa.SELECT_AUTO, pisa.SELECT_FUSED], ids=["two_stage", "fused"])
@pytest.mark.parametrize("name", list(CASES))
def test_zero_queries_select_lowest_leaves(name, algo):
    w = CASES[name]
    log(f"[test_zero_queries_select_lowest_leaves {name} algo={algo}]")
    data = I.generate(w, with_v=False)
    q = np.zeros_like(data["q"])  # +0.0 in fp32 and in bf16 bits
    p = pisa.Problem(w.B, w.N, w.Hq, w.Hkv, w.D, w.C, w.K, causal=w.causal, dtype=w.dtype, select_algo=algo)
    k = to_dev(data["k"])
    pyr = pisa.build_pyramid(p, k)
    idx, score = pisa.select(p, to_dev(q), k, pyr)
    torch.cuda.synchronize()
    e_idx, e_cnt = expected(w)
    got = idx.cpu().numpy()
    for b in range(w.B):
        for h in range(w.Hkv):
            bad = np.argwhere((got[b, h] != e_idx).any(axis=-1))
            assert bad.size == 0, f"t={int(bad[0][0])}: got {got[b, h, bad[0][0]].tolist()} " \
                                  f"want {e_idx[bad[0][0]].tolist()}"
    if algo == pisa.SELECT_AUTO:
        g = score.cpu().numpy().astype(np.float64)
        want = np.where(e_idx >= 0, w.gq * np.log(np.maximum(e_cnt, 1)), -np.inf)
        for b in range(w.B):
            for h in range(w.Hkv):
                assert np.array_equal(np.isneginf(g[b, h]), e_idx < 0)
                m = e_idx >= 0
                err = np.abs(g[b, h][m] - want[m]).max()
                assert err <= 1e-5 * max(1.0, np.abs(want[m]).max()), err


@pytest.mark.parametrize("attn", [pisa.ATTN_LEAF_MAJOR, pisa.ATTN_QUERY_MAJOR], ids=["leaf_major", "query_major"])
@pytest.mark.parametrize("name", list(CASES))
def test_zero_queries_attention_is_mean(name, attn):
    w = CASES[name]
    log(f"[test_zero_queries_attention_is_mean {name} attn={attn}]")
    data = I.generate(w)
    q = np.zeros_like(data["q"])
    p = pisa.Problem(w.B, w.N, w.Hq, w.Hkv, w.D, w.C, w.K, causal=w.causal, dtype=w.dtype)
    p.attn_algo = attn
    e_idx, e_cnt = expected(w)
    idx = np.broadcast_to(e_idx.astype(np.int32), (w.B, w.Hkv, w.N, w.K))
    o, lse = pisa.sparse_attn(p, to_dev(q), to_dev(data["k"]), to_dev(data["v"]), to_dev(np.ascontiguousarray(idx)))
    torch.cuda.synchronize()
    v = I.widen(data["v"])  # [B][Hkv][N][D] float64
    got_o = to_host_f64(o)
    got_lse = lse.cpu().numpy().astype(np.float64)
    n_keys = e_cnt.sum(axis=1)  # valid keys per query
    # mean of the values of the keys [0, n_keys[t]) (the kept leaves are the
    # first ones and, under the causal mask, end at t): prefix sums over keys
    csum = np.cumsum(v, axis=2)
    worst = 0.0
    for b in range(w.B):
        for h in range(w.Hkv):
            ref = csum[b, h, n_keys - 1] / n_keys[:, None]  # [N][D]
            for g in range(w.gq):
                worst = max(worst, float(np.abs(got_o[b, h * w.gq + g] - ref).max()))
                lerr = np.abs(got_lse[b, h * w.gq + g] - np.log(n_keys)).max()
                assert lerr <= 1e-4 * max(1.0, math.log(n_keys.max())), lerr
    assert worst <= ATTN_TOL[w.dtype], worst
    log(f"  attention max-abs err {worst:.3g}")


DECODE_CASES = {
    # n0 = 1021 -> 1024: the new tokens fill the last leaf; K = 4 of 16 leaves
    "bf16_g4_c64_k4": I.Workload("ties_dec_bf16", 3, 1021, 8, 2, 128, 64, 4, "bf16", True, seed=74, steps=3),
    # K = 16 of 7 leaves: every leaf kept, the last one partial
    "f32_g1_c48_k16": I.Workload("ties_dec_f32", 2, 300, 2, 2, 64, 48, 16, "f32", True, seed=75, steps=2),
}


@pytest.mark.parametrize("name", list(DECODE_CASES))
def test_zero_queries_decode(name):
    """The fused decode step on zero queries: the first min(K, leaves) leaves,
    scores G_Q log(#keys), o the mean of their values (new token included)."""
    w = DECODE_CASES[name]
    log(f"[test_zero_queries_decode {name}]")
    cache = I.decode_cache(w)
    cap = cache["cap"]
    dp = pisa.DecodeProblem(w.B, cap, w.Hq, w.Hkv, w.D, w.C, w.K, dtype=w.dtype)
    kc, vc = to_dev(cache["k"]), to_dev(cache["v"])
    pp = dp.prefill_problem(w.N)
    pyr = pisa.build_pyramid(pp, kc, pisa.alloc_pyramid(pp))
    length = torch.full((w.B,), w.N, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    v_host = I.widen(cache["v"]).copy()
    for step in range(w.steps):
        n = w.N + step  # position of the new token; keys 0..n are valid
        tok = I.decode_token(w, step)
        q0 = np.zeros_like(tok["q"])
        idx = torch.empty((w.B, w.Hkv, w.K), dtype=torch.int32, device="cuda")
        score = torch.empty((w.B, w.Hkv, w.K), dtype=torch.float32, device="cuda")
        o, _, _ = pisa.decode_step(dp, kc, vc, pyr, length, to_dev(q0), to_dev(tok["k"]), to_dev(tok["v"]),
                                   idx=idx, score=score, err=err)
        torch.cuda.synchronize()
        v_host[:, :, n] = I.widen(tok["v"])
        M1 = n // w.C + 1
        keep = min(w.K, M1)
        e_idx = np.array([j if j < keep else -1 for j in range(w.K)])
        cnt = np.array([min((j + 1) * w.C, n + 1) - j * w.C if j < keep else 0 for j in range(w.K)])
        got = idx.cpu().numpy()
        assert (got == e_idx).all(), f"step {step}: got {got.reshape(-1, w.K)[0].tolist()} want {e_idx.tolist()}"
        g = score.cpu().numpy().astype(np.float64)
        want = w.gq * np.log(np.maximum(cnt, 1))
        m = e_idx >= 0
        assert np.isneginf(g[..., ~m]).all()
        assert np.abs(g[..., m] - want[m]).max() <= 1e-5 * max(1.0, np.abs(want[m]).max())
        nk = int(cnt.sum())
        ref = v_host[:, :, :nk].mean(axis=2)  # [B][Hkv][D]
        got_o = to_host_f64(o).reshape(w.B, w.Hkv, w.gq, w.D)
        err_o = np.abs(got_o - ref[:, :, None, :]).max()
        assert err_o <= ATTN_TOL[w.dtype], f"step {step}: attention error {err_o:.3g}"
    assert int(err.item()) == 0


BWD_CASES = {
    "f32_g2_c48_k4_causal": I.Workload("ties_bwd_f32", 1, 900, 4, 2, 64, 48, 4, "f32", True, seed=76),
    "bf16_g4_c32_k4_b2": I.Workload("ties_bwd_bf16", 2, 1100, 8, 2, 128, 32, 4, "bf16", False, seed=77),
}
BWD_TOL = {"f32": 1e-4, "bf16": 2e-2}


@pytest.mark.parametrize("name", list(BWD_CASES))
def test_zero_queries_backward(name):
    """Backward of sum(dO . o) on zero queries over the first leaves: every
    probability is 1/n_t, so dK = scale * sum_t dS q_t is exactly zero,
    dV_i = sum over the group's heads and the queries t with i < n_t of
    dO_t / n_t, and dQ_t = scale / n_t * sum_{i < n_t} (dO_t.v_i - dO_t.o_t) k_i."""
    w = BWD_CASES[name]
    log(f"[test_zero_queries_backward {name}]")
    data = I.generate(w)
    q = np.zeros_like(data["q"])
    dout = I.normal(w.seed, 11, w.B * w.Hq * w.N * w.D, dtype=w.dtype).reshape(w.B, w.Hq, w.N, w.D)
    p = pisa.Problem(w.B, w.N, w.Hq, w.Hkv, w.D, w.C, w.K, causal=w.causal, dtype=w.dtype)
    e_idx, e_cnt = expected(w)
    idx = to_dev(np.ascontiguousarray(np.broadcast_to(e_idx.astype(np.int32), (w.B, w.Hkv, w.N, w.K))))
    qd, kd, vd, gd = (to_dev(x) for x in (q, data["k"], data["v"], dout))
    o, lse = pisa.sparse_attn(p, qd, kd, vd, idx)
    dq, dk, dv = pisa.sparse_attn_backward(p, qd, kd, vd, idx, o, lse, gd)
    torch.cuda.synchronize()
    scale = 1.0 / math.sqrt(w.D)
    k64, v64, g64 = I.widen(data["k"]), I.widen(data["v"]), I.widen(dout)
    n_t = e_cnt.sum(axis=1)  # keys [0, n_t) for query t
    r_dv = np.zeros_like(v64)
    r_dq = np.zeros_like(g64)
    for b in range(w.B):
        for h in range(w.Hkv):
            for gg in range(w.gq):
                hq = h * w.gq + gg
                # dV: dO_t / n_t added to keys [0, n_t), by sums over the end n_t
                ends = np.zeros((w.N + 1, w.D))
                np.add.at(ends, n_t, g64[b, hq] / n_t[:, None])
                r_dv[b, h] += np.cumsum(ends[::-1], axis=0)[::-1][1:]
                for t in range(w.N):
                    kk, vv = k64[b, h, : n_t[t]], v64[b, h, : n_t[t]]
                    o_t = vv.mean(axis=0)
                    ds = vv @ g64[b, hq, t] - g64[b, hq, t] @ o_t
                    r_dq[b, hq, t] = scale / n_t[t] * (ds @ kk)
    got_dk = to_host_f64(dk)
    assert (got_dk == 0.0).all(), f"dk not zero: max |dk| {np.abs(got_dk).max():.3g}"
    for label, got, ref in (("dq", dq, r_dq), ("dv", dv, r_dv)):
        err = np.abs(to_host_f64(got) - ref).max()
        lim = BWD_TOL[w.dtype] * max(1.0, np.abs(ref).max())
        log(f"  {label}: max err {err:.3g} (limit {lim:.3g})")
        assert err <= lim, f"{name} {label}: {err} > {lim}"
