"""Selection quality of the GPU's own sets (pisa_select and the flat selector
as the benchmark runs them), on the needle workloads at 32K, 128K and 256K.

For sampled query positions and every KV head the oracle scores every valid
leaf by the level-1 block score (raw-key LSE summed over the group: the
coarse-to-fine top-K section's score at the leaf level) and takes the exact
top K.  Against it, for the GPU's PISA sets, the GPU's flat sets and the
oracle's own descent:
* recall: the fraction of the exact top K a set holds;
* mass: the sum of exp(score) over the set divided by the same over the exact
  top K (the share of the attainable block score mass, <= 1);
* needle recall: whether the planted host leaf of a needle query is kept
  (32K/128K: each host's needle query; 256K: queries inside a host's span).

Asserted: every mass <= 1; the exact top K keeps every sampled needle; the
GPU PISA sets keep the same needles as the oracle's descent (the descent is
a heuristic: at 128K it prunes one of the sampled needles at a coarse level,
GPU and oracle alike); the mean mass of the GPU's PISA sets is within 1% of
the oracle descent's (they differ only at near-ties); the GPU flat sets'
mean mass is within 1% of the oracle flat selector's."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from gpu_util import log, to_dev
from hierarchical_block_sparse_mean_amd import inputs as I
from hierarchical_block_sparse_mean_amd import pisa

pytestmark = pytest.mark.gpu


def _needles(w: I.Workload, meta: dict, rng, per_head: int) -> list:
    """(b, h, t, host leaf) needle queries, per_head of them per KV head."""
    out = []
    for b in range(w.B):
        for h in range(w.Hkv):
            i = b * w.Hkv + h
            if w.needles == "leaf_per_query":
                hosts = np.asarray(meta["hosts"][i])
                tq = np.asarray(meta["queries"][i])
                for k in rng.choice(len(hosts), size=min(per_head, len(hosts)), replace=False):
                    out.append((b, h, int(tq[k]), int(hosts[k])))
            elif w.needles == "shared_spans":
                spans = [(j, s) for j, s in meta["spans"][i] if s >= 0]
                for k in rng.choice(len(spans), size=min(per_head, len(spans)), replace=False):
                    j, s = spans[k]
                    out.append((b, h, int(s + rng.integers(0, 1024)), int(j)))
    return out


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,n_pos", [("prefill_32k", 48), ("prefill_128k", 40), ("prefill_256k", 24)])
def test_gpu_selection_quality(name, n_pos):
    w = I.WORKLOADS[name]
    log(f"[quality {name}] generating inputs")
    data = I.generate(w, with_v=False)
    q, k = to_dev(data["q"]), to_dev(data["k"])
    p = pisa.Problem(w.B, w.N, w.Hq, w.Hkv, w.D, w.C, w.K, causal=w.causal, dtype=w.dtype)
    pyr = pisa.build_pyramid(p, k)
    g_idx, _ = pisa.select(p, q, k, pyr)
    gf_idx, _ = pisa.flat_select(p, q, pyr)
    torch.cuda.synchronize()
    rng = np.random.default_rng(w.seed + 17)
    needles = _needles(w, data["meta"], rng, 2)
    pos = np.unique(np.linspace(w.C, w.N - 1, n_pos).astype(np.int64))
    ts = np.unique(np.concatenate([pos, np.array([n[2] for n in needles], np.int64)]))
    log(f"[quality {name}] oracle on {len(ts)} positions ({len(needles)} needle queries)")
    M1 = -(-w.N // w.C)
    op = oracle.Problem(w.B, w.N, w.Hq, w.Hkv, w.D, w.C, w.K, causal=w.causal)
    op_all = oracle.Problem(w.B, w.N, w.Hq, w.Hkv, w.D, w.C, M1, causal=w.causal)
    a_idx, a_score = oracle.exact_topk(op_all, data["q"], data["k"], ts=ts)  # every valid leaf, scored
    e_idx, _ = oracle.exact_topk(op, data["q"], data["k"], ts=ts)
    d_idx, _, _, _ = oracle.select(op, data["q"], data["k"], ts=ts)
    f_idx, _ = oracle.flat_select(op, data["q"], data["k"], ts=ts)
    gp = g_idx.cpu().numpy()[:, :, ts]
    gf = gf_idx.cpu().numpy()[:, :, ts]
    U = np.full(a_idx.shape[:3] + (M1,), -np.inf)
    ok = a_idx >= 0
    bb, hh, ss, _ = np.nonzero(ok)
    U[bb, hh, ss, a_idx[ok]] = a_score[ok]
    m = U.max(-1, keepdims=True)

    def mass(idx):
        e = np.where(idx >= 0, np.exp(np.take_along_axis(U, np.maximum(idx, 0), -1) - m), 0.0).sum(-1)
        best = np.where(e_idx >= 0, np.exp(np.take_along_axis(U, np.maximum(e_idx, 0), -1) - m), 0.0).sum(-1)
        return e / best

    def recall(idx):
        hit = (idx[..., :, None] == e_idx[..., None, :]) & (idx[..., :, None] >= 0)
        return hit.any(-2).sum(-1) / np.maximum(1, (e_idx >= 0).sum(-1))

    res = {}
    for label, idx in (("gpu_pisa", gp), ("oracle_pisa", d_idx), ("gpu_flat", gf), ("oracle_flat", f_idx)):
        ms = mass(idx)
        assert (ms <= 1 + 1e-9).all(), f"{name} {label}: mass above 1"
        res[label] = {"recall": round(float(recall(idx).mean()), 4), "mass": round(float(ms.mean()), 4),
                      "mass_p10": round(float(np.percentile(ms, 10)), 4)}
    pos_of = {int(t): i for i, t in enumerate(ts)}
    kept = {lab: [int(j in idx[b, h, pos_of[t]]) for b, h, t, j in needles]
            for lab, idx in (("gpu_pisa", gp), ("oracle_pisa", d_idx), ("gpu_flat", gf), ("exact", e_idx))}
    log(f"[quality {name}] {res}; needles kept " + str({lab: sum(v) for lab, v in kept.items()}) +
        f" of {len(needles)}")
    assert sum(kept["exact"]) == len(needles), kept
    assert kept["gpu_pisa"] == kept["oracle_pisa"], kept
    assert abs(res["gpu_pisa"]["mass"] - res["oracle_pisa"]["mass"]) <= 0.01, res
    assert abs(res["gpu_flat"]["mass"] - res["oracle_flat"]["mass"]) <= 0.01, res
