"""Helpers of the GPU parity tests: upload of seeded host inputs and the
comparison rules (selection sets identical except where the oracle's K-th and
(K+1)-th scores at some scored level are closer than 1e-3; scores within
1e-4 * max(1, |u|); attention within 1e-3 (fp32) or 2e-2 (bf16) max-abs)."""
from __future__ import annotations

import sys

import numpy as np
import torch

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
