"""GPU parity of the leaf-major attention on selections rich in sibling pairs.

Where a query keeps both leaves 2j and 2j + 1 of a level-2 block (adjacent in
its ascending row) and C <= 64, the attention clusters the pair under that
block and attends its 2C keys in one tile, writing one partial for both
leaves.  These selections are crafted (seeded, ascending, -1 padded) so that
most kept leaves come in such pairs, including pairs in a row's last two
slots, a ragged last leaf as the odd sibling or as a lone even leaf, lone odd
leaves next to unrelated even ones, short rows and odd K.  Both attention
schedules are compared with the oracle's attention on the same idx, to the
attention bar (1e-3 fp32, 2e-2 bf16 max-abs; lse within 1e-4 relative)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from gpu_util import check_attention, log, to_dev, to_host_f64
from hierarchical_block_sparse_mean_amd import inputs as I
from hierarchical_block_sparse_mean_amd import pisa

pytestmark = pytest.mark.gpu

CASES = {
    # N = 1000, C = 64: the last leaf (15, 40 keys) is the odd sibling of 14
    "f32_c64_k6_causal": I.Workload("pairs_f32_c64", 1, 1000, 4, 1, 64, 64, 6, "f32", True, seed=91),
    # N = 1100, C = 48: 23 leaves, the last one (22) has no sibling
    "bf16_c48_k5_causal": I.Workload("pairs_bf16_c48", 1, 1100, 8, 2, 128, 48, 5, "bf16", True, seed=92),
    "bf16_c32_k8_b2": I.Workload("pairs_bf16_c32", 2, 700, 8, 2, 128, 32, 8, "bf16", False, seed=93),
    "bf16_c64_k16_g4": I.Workload("pairs_bf16_c64", 1, 2100, 16, 4, 128, 64, 16, "bf16", True, seed=94),
    # C = 128: 256-key pair tiles (bf16 only), ragged N
    "bf16_c128_k6_causal": I.Workload("pairs_bf16_c128", 1, 2000, 8, 2, 128, 128, 6, "bf16", True, seed=97),
    # the 256-key pair tile at d = 64, and with a 16-head group (one query per
    # 16-column MFMA tile)
    "bf16_c128_d64_k8": I.Workload("pairs_bf16_c128_d64", 1, 2300, 4, 2, 64, 128, 8, "bf16", True, seed=98),
    "bf16_c128_g16_k5": I.Workload("pairs_bf16_c128_g16", 1, 1900, 16, 1, 128, 128, 5, "bf16", False, seed=99),
    # fp32 rows of d = 128: pairs are attended leaf by leaf (a 2C-key tile
    # would leave LDS for two waves), and 128-key leaf tiles run with fewer
    # waves
    "f32_d128_c64_k6": I.Workload("pairs_f32_d128_c64", 1, 800, 4, 2, 128, 64, 6, "f32", True, seed=95),
    "f32_d128_c128_k4": I.Workload("pairs_f32_d128_c128", 1, 900, 4, 1, 128, 128, 4, "f32", False, seed=96),
}


def paired_selection(w: I.Workload, seed: int) -> np.ndarray:
    """idx [B][Hkv][N][K]: per row up to K valid leaves (causal: leaf j is
    valid for query t when j*C <= t), mostly whole sibling pairs."""
    rng = np.random.default_rng(seed)
    M1 = -(-w.N // w.C)
    idx = np.full((w.B, w.Hkv, w.N, w.K), -1, np.int32)
    for b in range(w.B):
        for h in range(w.Hkv):
            for t in range(w.N):
                nvalid = min(M1, t // w.C + 1) if w.causal else M1
                want = min(w.K, nvalid)
                if rng.random() < 0.2:  # a short row
                    want = int(rng.integers(1, want + 1))
                chosen: set = set()
                if rng.random() < 0.3 and nvalid >= 2:  # the row's two largest leaves as one pair
                    jb = (nvalid - 1) // 2
                    for j in (2 * jb, 2 * jb + 1):
                        if j < nvalid and len(chosen) < want:
                            chosen.add(j)
                while len(chosen) < want:
                    jb = int(rng.integers(0, (nvalid + 1) // 2))
                    r = rng.random()
                    pick = (2 * jb, 2 * jb + 1) if r < 0.7 else ((2 * jb + 1,) if r < 0.85 else (2 * jb,))
                    for j in pick:
                        if j < nvalid and len(chosen) < want:
                            chosen.add(j)
                row = sorted(chosen)
                idx[b, h, t, : len(row)] = row
    return idx


def pair_fraction(idx: np.ndarray) -> float:
    """Fraction of kept leaves that sit in a kept sibling pair."""
    j = idx.astype(np.int64)
    both = (j[..., :-1] >= 0) & (j[..., :-1] % 2 == 0) & (j[..., 1:] == j[..., :-1] + 1)
    return 2.0 * both.sum() / max(1, (j >= 0).sum())


@pytest.mark.parametrize("algo", [pisa.ATTN_LEAF_MAJOR, pisa.ATTN_QUERY_MAJOR], ids=["leaf_major", "query_major"])
@pytest.mark.parametrize("name", list(CASES))
def test_attention_sibling_pairs(name, algo):
    w = CASES[name]
    data = I.generate(w)
    idx = paired_selection(w, w.seed)
    frac = pair_fraction(idx)
    log(f"[test_attention_sibling_pairs {name} algo={algo}] {frac:.2f} of kept leaves in sibling pairs")
    assert frac > 0.5
    # the pair in the last two slots and a lone odd leaf both occur
    last_pair = (idx[..., -2] >= 0) & (idx[..., -2] % 2 == 0) & (idx[..., -1] == idx[..., -2] + 1)
    assert last_pair.any()
    p = pisa.Problem(w.B, w.N, w.Hq, w.Hkv, w.D, w.C, w.K, causal=w.causal, dtype=w.dtype)
    p.attn_algo = algo
    q, k, v = (to_dev(data[x]) for x in ("q", "k", "v"))
    o, lse = pisa.sparse_attn(p, q, k, v, to_dev(idx))
    torch.cuda.synchronize()
    op = oracle.Problem(w.B, w.N, w.Hq, w.Hkv, w.D, w.C, w.K, causal=w.causal)
    r_o, r_lse = oracle.attention(op, data["q"], data["k"], data["v"], idx)
    err = check_attention(to_host_f64(o), r_o, w.dtype, name)
    got_lse = lse.cpu().numpy().astype(np.float64)
    lse_err = np.abs(got_lse - r_lse).max()
    assert lse_err <= 1e-4 * max(1.0, np.abs(r_lse).max()), lse_err
    log(f"  attention max-abs err {err:.3g}, lse err {lse_err:.3g}")
