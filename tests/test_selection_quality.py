"""Selection quality of PISA's descent against the exact leaf top-K and the
flat selector, on the needle workloads (CPU oracle; the GPU path returns the
same sets up to near-ties, which the GPU parity tests check).

For sampled query positions and every KV head:
* exact: the top K over every valid leaf of the raw-key LSE summed over the
  group (the level-1 block score);
* recall of PISA's kept set and of the flat selector's set against it;
* mass: sum of exp(score) over the set divided by the same sum over the exact
  top K (the share of the best attainable block score mass; <= 1);
* needle recall: whether the planted host leaf of a needle query is kept.

Run as a script for the full report:
    python tests/test_selection_quality.py --workload prefill_128k --positions 64
"""
from __future__ import annotations

import argparse
import json
import os
import sys

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(_HERE)
for _p in (_ROOT, _HERE):
    if _p not in sys.path:
        sys.path.insert(0, _p)

import oracle  # noqa: E402
from hierarchical_block_sparse_mean_amd import inputs as I  # noqa: E402


def _sets(idx: np.ndarray) -> list:
    return [set(int(j) for j in row if j >= 0) for row in idx.reshape(-1, idx.shape[-1])]


def quality(w: I.Workload, n_pos: int, n_needle: int, seed: int = 7) -> dict:
    data = I.generate(w, with_v=False)
    rng = np.random.default_rng(seed)
    # evenly spread positions past the first leaf, plus needle queries
    pos = np.unique(np.linspace(w.C, w.N - 1, n_pos).astype(np.int64))
    needles = []
    if w.needles == "leaf_per_query":
        for b in range(w.B):
            for h in range(w.Hkv):
                hosts = np.asarray(data["meta"]["hosts"][b * w.Hkv + h])
                tq = np.asarray(data["meta"]["queries"][b * w.Hkv + h])
                pick = rng.choice(len(hosts), size=min(n_needle, len(hosts)), replace=False)
                needles += [(b, h, int(tq[i]), int(hosts[i])) for i in pick]
    ts = np.unique(np.concatenate([pos, np.array([n[2] for n in needles], np.int64)]))
    M1 = -(-w.N // w.C)
    p = oracle.Problem(w.B, w.N, w.Hq, w.Hkv, w.D, w.C, w.K, causal=w.causal)
    p_all = oracle.Problem(w.B, w.N, w.Hq, w.Hkv, w.D, w.C, M1, causal=w.causal)
    d_idx, d_score, _, _ = oracle.select(p, data["q"], data["k"], ts=ts)
    f_idx, _ = oracle.flat_select(p, data["q"], data["k"], ts=ts)
    a_idx, a_score = oracle.exact_topk(p_all, data["q"], data["k"], ts=ts)  # every valid leaf
    e_idx, e_score = oracle.exact_topk(p, data["q"], data["k"], ts=ts)
    # U[b, h, s, j]: exact level-1 score of leaf j (-inf when invalid)
    U = np.full(a_idx.shape[:3] + (M1,), -np.inf)
    valid = a_idx >= 0
    bb, hh, ss, kk = np.nonzero(valid)
    U[bb, hh, ss, a_idx[valid]] = a_score[valid]
    # consistency: the exact top K is the top K of all scores; PISA reports
    # the exact score of each kept leaf
    for s_ in range(len(ts)):
        for b in range(w.B):
            for h in range(w.Hkv):
                u = U[b, h, s_]
                n = int(np.isfinite(u).sum())
                order = sorted(range(n), key=lambda j: (-u[j], j))[: w.K]
                assert sorted(order) == [int(j) for j in e_idx[b, h, s_] if j >= 0]
    kept = d_idx >= 0
    np.testing.assert_allclose(d_score[kept], np.take_along_axis(U, np.maximum(d_idx, 0), -1)[kept], rtol=1e-12)

    def mass(idx):
        m = U.max(-1, keepdims=True)
        e = np.where(idx >= 0, np.exp(np.take_along_axis(U, np.maximum(idx, 0), -1) - m), 0.0).sum(-1)
        best = np.where(e_idx >= 0, np.exp(np.take_along_axis(U, np.maximum(e_idx, 0), -1) - m), 0.0).sum(-1)
        return e / best

    E, P, F = _sets(e_idx), _sets(d_idx), _sets(f_idx)
    rec = lambda S: np.array([len(a & e) / max(1, len(e)) for a, e in zip(S, E)])
    r_p, r_f = rec(P), rec(F)
    m_p, m_f = mass(d_idx), mass(f_idx)
    pos_of = {int(t): i for i, t in enumerate(ts)}
    nd = {"queries": len(needles), "pisa": 0, "flat": 0, "exact": 0}
    for b, h, t, j in needles:
        s_ = pos_of[t]
        nd["pisa"] += int(j in d_idx[b, h, s_])
        nd["flat"] += int(j in f_idx[b, h, s_])
        nd["exact"] += int(j in e_idx[b, h, s_])
    return {
        "workload": w.name, "N": w.N, "C": w.C, "K": w.K, "positions": int(len(ts)), "heads": w.B * w.Hkv,
        "recall_pisa_vs_exact": round(float(r_p.mean()), 4), "recall_flat_vs_exact": round(float(r_f.mean()), 4),
        "exact_set_rate_pisa": round(float((r_p == 1.0).mean()), 4),
        "exact_set_rate_flat": round(float((r_f == 1.0).mean()), 4),
        "mass_pisa": round(float(m_p.mean()), 4), "mass_flat": round(float(m_f.mean()), 4),
        "mass_pisa_p10": round(float(np.percentile(m_p, 10)), 4),
        "mass_flat_p10": round(float(np.percentile(m_f, 10)), 4),
        "needle_recall": nd, "_mass": (m_p, m_f),
    }


def test_selection_quality_small():
    """32K needle workload, a small sample: the exact top K bounds both
    selectors' score mass, PISA reports exact leaf scores, and recall is a
    fraction; the planted needles are found by the exact top K."""
    w = I.WORKLOADS["prefill_32k"]
    q = quality(w, n_pos=12, n_needle=2)
    m_p, m_f = q.pop("_mass")
    assert (m_p <= 1 + 1e-9).all() and (m_f <= 1 + 1e-9).all()
    assert 0.0 <= q["recall_pisa_vs_exact"] <= 1.0 and 0.0 <= q["recall_flat_vs_exact"] <= 1.0
    assert q["needle_recall"]["exact"] == q["needle_recall"]["queries"]
    print(json.dumps(q))


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="prefill_32k")
    ap.add_argument("--positions", type=int, default=64)
    ap.add_argument("--needles", type=int, default=4, help="needle queries per KV head")
    args = ap.parse_args()
    res = quality(I.workload(args.workload), args.positions, args.needles)
    res.pop("_mass")
    print(json.dumps(res))
