"""GPU parity where a head has more key blocks than the clustering's LDS
histogram holds (16384 bins), so the counting sort takes its global-atomic
path -- the path every head takes at long contexts (about 1M tokens and more
at C = 64).

* bf16, C = 4, N = 140000: 35000 leaves and 17500 level-2 blocks per head, so
  stage 2 (clusters of level-2 blocks), the attention (leaves and sibling
  pairs) and the backward all cluster through global atomics;
* fp32, C = 8, N = 140000, two KV heads, non-causal: 17500 leaves per head,
  so the attention and the backward take that path (stage 2 stays on the
  LDS histogram).

Checked against the oracle: selection on sampled positions (identical sets
except near-ties, the GPU's own sets as top-K of the children of its kept
level-2 blocks, scores), attention on the GPU's selection at every sampled
position, and the backward over the GPU's selection at every position."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from gpu_util import check_attention_on_gpu_idx, check_gpu_sets, check_selection, log, to_dev, to_host_f64
from hierarchical_block_sparse_mean_amd import inputs as I
from hierarchical_block_sparse_mean_amd import pisa

pytestmark = pytest.mark.gpu

LDS_BINS = 16384  # bins per head the clustering's LDS histogram holds
BWD_TOL = {"f32": 1e-4, "bf16": 2e-2}

CASES = {
    "bf16_c4_causal": I.Workload("bins_bf16_c4", 1, 140000, 4, 1, 64, 4, 16, "bf16", True, seed=101),
    "f32_c8_g2": I.Workload("bins_f32_c8", 1, 140000, 4, 2, 64, 8, 8, "f32", False, seed=102),
}


def _positions(w: I.Workload, n_mid: int) -> np.ndarray:
    rng = np.random.default_rng(w.seed)
    edge = np.concatenate([np.arange(0, 3), np.arange(w.C - 1, 4 * w.C + 1), np.arange(w.N - 3, w.N)])
    return np.unique(np.concatenate([edge, rng.integers(0, w.N, n_mid)]))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", list(CASES))
def test_large_bins(name):
    w = CASES[name]
    M1 = -(-w.N // w.C)
    assert M1 > LDS_BINS  # the attention clustering leaves the LDS histogram
    log(f"[largebins {name}] N={w.N} C={w.C} K={w.K} M1={M1} M2={-(-M1 // 2)}: generating inputs")
    data = I.generate(w)
    dout = I.normal(w.seed, 11, w.B * w.Hq * w.N * w.D, dtype=w.dtype).reshape(w.B, w.Hq, w.N, w.D)
    q, k, v, g = (to_dev(x) for x in (data["q"], data["k"], data["v"], dout))
    p = pisa.Problem(w.B, w.N, w.Hq, w.Hkv, w.D, w.C, w.K, causal=w.causal, dtype=w.dtype)
    log(f"[largebins {name}] GPU pyramid, select, attention, backward")
    pyr = pisa.build_pyramid(p, k)
    ws = pisa.workspace(pisa.select_workspace_bytes(p))
    idx, score = pisa.select(p, q, k, pyr, ws=ws)
    blk2 = pisa.select_level2(p, ws).clone()
    o, lse = pisa.sparse_attn(p, q, k, v, idx)
    dq, dk, dv = pisa.sparse_attn_backward(p, q, k, v, idx, o, lse, g)
    torch.cuda.synchronize()

    ts = _positions(w, 300)
    log(f"[largebins {name}] oracle selection and attention on {len(ts)} positions")
    op = oracle.Problem(w.B, w.N, w.Hq, w.Hkv, w.D, w.C, w.K, causal=w.causal)
    r_idx, r_score, r_gap, _ = oracle.select(op, data["q"], data["k"], ts=ts)
    full_idx = idx.cpu().numpy()
    g_idx, g_score = full_idx[:, :, ts], score.cpu().numpy()[:, :, ts]
    ex, rate = check_selection(g_idx, g_score, r_idx, r_score, r_gap, name)
    chk = check_gpu_sets(op, data["q"], data["k"], ts, g_idx, g_score, blk2.cpu().numpy()[:, :, ts], label=name)
    log(f"  exempt {ex:.4f}, exact-match {rate:.4f}, {int((~(g_idx == r_idx).all(-1)).sum())} rows differ; "
        f"GPU-set checks on {chk['rows']} rows (top-K within level-2 children on {chk['topk_checked']})")
    assert rate > 0.95
    err = check_attention_on_gpu_idx(op, data["q"], data["k"], data["v"], ts, g_idx, to_host_f64(o)[:, :, ts],
                                     w.dtype, label=name)
    log(f"  attention max-abs err {err:.3g}")

    log(f"[largebins {name}] oracle backward over the GPU's selection ({w.N} positions)")
    r_dq, r_dk, r_dv = oracle.attention_backward(op, data["q"], data["k"], data["v"], full_idx, dout)
    for label, got, ref in (("dq", dq, r_dq), ("dk", dk, r_dk), ("dv", dv, r_dv)):
        e = np.abs(to_host_f64(got) - ref).max()
        lim = BWD_TOL[w.dtype] * max(1.0, np.abs(ref).max())
        log(f"  {label}: max err {e:.3g} (limit {lim:.3g})")
        assert e <= lim, f"{name} {label}: {e} > {lim}"
