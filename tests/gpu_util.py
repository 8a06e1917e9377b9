"""Helpers of the GPU parity tests: upload of seeded host inputs and the
comparison rules (selection sets identical except where the oracle's K-th and
(K+1)-th scores at some scored level are closer than 1e-3; scores within
1e-4 * max(1, |u|); attention within 1e-3 (fp32) or 2e-2 (bf16) max-abs)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle

NEAR_TIE = 1e-3
SCORE_RTOL = 1e-4
ATTN_TOL = {"f32": 1e-3, "bf16": 2e-2}


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(x: np.ndarray) -> torch.Tensor:
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def to_host_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def check_selection(g_idx, g_score, o_idx, o_score, o_gap, label=""):
    """Returns (exempt_fraction, exact_match_rate); asserts the parity bar."""
    g_idx = np.asarray(g_idx)
    o_idx = np.asarray(o_idx)
    exempt = np.asarray(o_gap) < NEAR_TIE
    same = (g_idx == o_idx).all(axis=-1)
    bad = ~same & ~exempt
    if bad.any():
        where = np.argwhere(bad)[:5]
        msg = [f"{label}: {int(bad.sum())} non-exempt mismatches of {bad.size}"]
        for w in where:
            w = tuple(w)
            msg.append(f"  at {w}: gpu {g_idx[w].tolist()} oracle {o_idx[w].tolist()} gap {o_gap[w]:.3g}")
        raise AssertionError("\n".join(msg))
    if g_score is not None:
        g_score = np.asarray(g_score, dtype=np.float64)
        o_score = np.asarray(o_score, dtype=np.float64)
        m = same[..., None] & (o_idx >= 0)
        err = np.abs(g_score[m] - o_score[m])
        lim = (SCORE_RTOL * np.maximum(1.0, np.abs(o_score)))[m]
        assert (err <= lim).all(), f"{label}: score error {err.max():.3g} beyond {SCORE_RTOL} rel"
        assert np.isneginf(g_score[same[..., None] & (o_idx < 0)]).all()
    # every GPU set, exempt or not, is a valid ascending -1 padded set
    K = g_idx.shape[-1]
    rows = g_idx.reshape(-1, K)
    k = (rows >= 0).sum(axis=1)
    pos = np.arange(K)
    assert ((rows >= 0) == (pos[None, :] < k[:, None])).all(), f"{label}: -1 padding not at the end"
    inside = pos[None, 1:] < k[:, None]
    assert (np.diff(rows, axis=1)[inside] > 0).all(), f"{label}: kept set not strictly ascending"
    return float(exempt.mean()), float(same.mean())


def check_attention(g_o, o_ref, dtype, label=""):
    err = np.abs(np.asarray(g_o, np.float64) - o_ref).max()
    tol = ATTN_TOL[dtype]
    assert err <= tol, f"{label}: attention max-abs error {err:.3g} > {tol}"
    return float(err)


def check_gpu_sets(op, q, k, ts, g_idx, g_score, g_blk2=None, q_sampled=False, label=""):
    """Checks on the GPU's own selection that hold whichever member of a
    near-tie it kept (coarse-to-fine top-K section: per-level top-K, keep-all
    rule, LSE score; kernel-implementation section: GQA sum):

    (a) the reported score of every kept leaf equals the oracle's level-1
        score of that leaf (raw-key LSE summed over the group) within
        1e-4 * max(1, |u|); padding slots are -inf;
    (b) given the level-2 blocks stage 1 kept (g_blk2), the set is a top-K of
        their valid children by the oracle's leaf scores: it holds
        min(K, #valid children) of them, and no child left out scores more
        than the band above a kept one (band = the 1e-3 near-tie width plus
        the score tolerance on both sides).

    g_idx, g_score, g_blk2: [B][Hkv][nt][K] at positions ts (None = all).
    Returns counts for the log: rows checked by (a) and by (b), and the
    largest score error."""
    g_idx = np.asarray(g_idx)
    g_score = np.asarray(g_score, np.float64)
    B, Hkv, nt, K = g_idx.shape
    pos = np.arange(op.N) if ts is None else np.asarray(ts)
    sc = oracle.leaf_scores(op, q, k, g_idx, ts=pos, q_sampled=q_sampled)
    kept = g_idx >= 0
    assert np.isfinite(sc[kept]).all(), f"{label}: a kept leaf has no valid key"
    err = np.abs(g_score[kept] - sc[kept])
    lim = SCORE_RTOL * np.maximum(1.0, np.abs(sc[kept]))
    assert (err <= lim).all(), f"{label}: GPU score of its own leaf off by {err.max():.3g}"
    assert np.isneginf(g_score[~kept]).all(), f"{label}: padding score not -inf"
    out = {"rows": int(B * Hkv * nt), "score_err": float(err.max()) if err.size else 0.0, "topk_checked": 0}
    if g_blk2 is None:
        return out
    M1 = -(-op.N // op.C)
    j2 = np.asarray(g_blk2, np.int64)
    cand = np.stack([2 * j2, 2 * j2 + 1], axis=-1).reshape(B, Hkv, nt, 2 * K)
    has = np.repeat(j2 >= 0, 2, axis=-1)
    t = pos.reshape(1, 1, nt, 1)
    valid = has & (cand < M1) & ((not op.causal) | (cand * op.C <= t))
    cand = np.where(valid, cand, -1).astype(np.int32)
    csc = oracle.leaf_scores(op, q, k, cand, ts=pos, q_sampled=q_sampled)
    for b in range(B):
        for h in range(Hkv):
            for s in range(nt):
                v = cand[b, h, s][valid[b, h, s]]
                u = csc[b, h, s][valid[b, h, s]]
                gk = g_idx[b, h, s][kept[b, h, s]]
                where = f"{label}: (b={b}, h={h}, t={int(pos[s])})"
                assert set(gk.tolist()) <= set(v.tolist()), f"{where}: kept {gk} not among children {v}"
                assert len(gk) == min(K, len(v)), f"{where}: kept {len(gk)} of {len(v)} children (K={K})"
                if len(v) > K:
                    inside = np.isin(v, gk)
                    lo, hi = u[inside].min(), u[~inside].max()
                    band = NEAR_TIE + 2 * SCORE_RTOL * max(1.0, abs(lo), abs(hi))
                    assert lo >= hi - band, f"{where}: left-out child scores {hi:.6g} > kept {lo:.6g} + {band:.3g}"
    out["topk_checked"] = int(B * Hkv * nt)
    return out


def check_attention_on_gpu_idx(op, q, k, v, ts, g_idx, g_o, dtype, q_sampled=False, label=""):
    """pisa_sparse_attn's output on the GPU's own selection against the
    oracle's attention on that same selection, at every sampled position
    (block-sparse attention section, the o_t equation)."""
    pos = np.arange(op.N) if ts is None else np.asarray(ts)
    r_o, _ = oracle.attention(op, q, k, v, np.ascontiguousarray(g_idx, dtype=np.int32), ts=pos, q_sampled=q_sampled)
    return check_attention(g_o, r_o, dtype, label)
