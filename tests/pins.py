"""Pins of the PISA oracle: checks against what the method and mathematics fix,
each independent of the oracle's own code.

Every ``check_*`` takes an oracle library handle so that the same checks can be
run against deliberately broken builds of the oracle (see
``test_oracle_mutants.py``): each plausible mistake must fail at least one pin.

Method source: "Block Sparse Attention with Log-Linear Complexity" (PISA), the
hyper.ai page; sections named in each docstring.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
from scipy.special import logsumexp

import oracle
from hierarchical_block_sparse_mean_amd import inputs as I

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _bf16_valued_f32(seed: int, stream: int, shape) -> np.ndarray:
    """N(0,1) draws rounded to bf16 but stored as float32: small-mantissa values
    so that dyadic shifts of them stay exact in float32."""
    return I.bf16_bits_to_f32(I.normal(seed, stream, int(np.prod(shape)), dtype="bf16")).reshape(shape)


def tiny_inputs(N=1024, Hq=4, Hkv=1, D=64, seed=7, B=1):
    q = I.normal(seed, 1, B * Hq * N * D, dtype="f32").reshape(B, Hq, N, D)
    k = I.normal(seed, 2, B * Hkv * N * D, dtype="f32").reshape(B, Hkv, N, D)
    v = I.normal(seed, 3, B * Hkv * N * D, dtype="f32").reshape(B, Hkv, N, D)
    return q, k, v


# --------------------------------------------------------------------------
# Hand-derived worked example (tests/golden/hand_example.json)
# --------------------------------------------------------------------------
def _golden():
    with open(os.path.join(GOLDEN, "hand_example.json")) as f:
        return json.load(f)


def check_hand_example(lib) -> None:
    """All sections of the method on an 8-token example derived by hand."""
    g = _golden()
    N, D, C = g["N"], g["D"], g["C"]
    k = np.array(g["k"], np.float32).reshape(1, 1, N, D)
    v = np.array(g["v"], np.float32).reshape(1, 1, N, D)
    q = np.tile(np.array(g["q_all"], np.float32), (1, 1, N, 1))
    ln2 = math.log(2.0)
    a = math.log(1 + math.e ** 2)

    p1 = oracle.Problem(1, N, 1, 1, D, C, 1, causal=False, scale=g["scale"])
    pyr = oracle.pyramid(p1, k, lib=lib)
    assert len(pyr) == 3
    for lvl, want in zip(pyr, g["expected"]["pyramid"]):
        np.testing.assert_allclose(lvl[0, 0], np.array(want, np.float64), rtol=0, atol=0)

    idx, score, gap, _ = oracle.select(p1, q, k, ts=[0], lib=lib)
    assert idx[0, 0, 0].tolist() == [0]
    assert abs(score[0, 0, 0, 0] - a) < 1e-12
    assert abs(gap[0, 0, 0] - (a - 1 - ln2)) < 1e-12
    o, lse = oracle.attention(p1, q, k, v, idx, ts=[0], lib=lib)
    e2 = math.e ** 2
    np.testing.assert_allclose(o[0, 0, 0], [1 / (1 + e2), e2 / (1 + e2)], rtol=0, atol=1e-12)
    assert abs(lse[0, 0, 0] - a) < 1e-12

    p2 = oracle.Problem(1, N, 1, 1, D, C, 2, causal=False, scale=g["scale"])
    idx, score, _, _ = oracle.select(p2, q, k, ts=[0], lib=lib)
    assert idx[0, 0, 0].tolist() == [0, 2]
    np.testing.assert_allclose(score[0, 0, 0], [a, math.log(math.e ** 3 + math.e ** -3)], rtol=0, atol=1e-12)

    pc = oracle.Problem(1, N, 1, 1, D, C, 1, causal=True, scale=g["scale"])
    idx, score, _, _ = oracle.select(pc, q, k, ts=[4, 1, 0], lib=lib)
    assert idx[0, 0, :, 0].tolist() == [0, 0, 0]
    np.testing.assert_allclose(score[0, 0, :, 0], [a, a, 0.0], rtol=0, atol=1e-12)
    o, _ = oracle.attention(pc, q, k, v, idx, ts=[4, 1, 0], lib=lib)
    np.testing.assert_allclose(o[0, 0, 2], [1.0, 0.0], rtol=0, atol=1e-12)

    fidx, fscore = oracle.flat_select(p1, q, k, ts=[0], lib=lib)
    assert fidx[0, 0, 0].tolist() == [0]
    assert abs(fscore[0, 0, 0, 0] - 1.0) < 1e-12


# --------------------------------------------------------------------------
# Pyramid closed forms ([PYR] mean-pooling equation)
# --------------------------------------------------------------------------
def check_pyramid_closed_form(lib) -> None:
    """Without a ragged tail (N = C 2^m) a level-l summary is the plain mean of
    its C 2^(l-1) raw keys; with N = 330, C = 64 the ragged chain follows the
    children-mean reading, written out by hand."""
    q, k, _ = tiny_inputs(N=1024, D=16)
    p = oracle.Problem(1, 1024, 4, 1, 16, 64, 4)
    pyr = oracle.pyramid(p, k, lib=lib)
    assert len(pyr) == 5 and [x.shape[2] for x in pyr] == [16, 8, 4, 2, 1]
    kk = k[0, 0].astype(np.float64)
    for l, lvl in enumerate(pyr, start=1):
        span = 64 * 2 ** (l - 1)
        want = kk.reshape(-1, span, 16).mean(axis=1)
        np.testing.assert_allclose(lvl[0, 0], want, rtol=1e-13, atol=1e-15)

    k330 = k[:, :, :330, :]
    p = oracle.Problem(1, 330, 4, 1, 16, 64, 4)
    pyr = oracle.pyramid(p, np.ascontiguousarray(k330), lib=lib)
    assert [x.shape[2] for x in pyr] == [6, 3, 2, 1]
    m = lambda a, b: kk[a:b].mean(axis=0)  # noqa: E731
    l2_2 = (m(256, 320) + m(320, 330)) / 2
    l3_0 = ((m(0, 64) + m(64, 128)) / 2 + (m(128, 192) + m(192, 256)) / 2) / 2
    l3_1 = l2_2  # single child
    root = (l3_0 + l3_1) / 2
    np.testing.assert_allclose(pyr[0][0, 0, 5], m(320, 330), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(pyr[1][0, 0, 2], l2_2, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(pyr[2][0, 0, 1], l3_1, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(pyr[3][0, 0, 0], root, rtol=1e-13, atol=1e-15)
    # the raw-key mean of the whole sequence is NOT the root under this reading
    assert np.abs(root - kk[:330].mean(axis=0)).max() > 1e-6


# --------------------------------------------------------------------------
# Independent table-driven PISA (score every block at every level, then descend)
# --------------------------------------------------------------------------
def table_descent(q, k, C, K, causal, scale):
    """q: [G][N][D] float64 (one KV group), k: [N][D] float64.
    Returns idx [N][K] (ascending, -1 padded), score [N][K], gap [N]."""
    G, N, D = q.shape
    leaves = [k[j * C:min(j * C + C, N)].mean(axis=0) for j in range(-(-N // C))]
    levels = {1: np.stack(leaves)}
    while levels[len(levels)].shape[0] > 1:
        prev = levels[len(levels)]
        levels[len(levels) + 1] = np.stack([prev[2 * j:2 * j + 2].mean(axis=0) for j in range((len(prev) + 1) // 2)])
    L = len(levels)
    t_idx = np.arange(N)
    raw = np.einsum("gtd,nd->gtn", q, k) * scale  # [G][N][N]
    if causal:
        raw = np.where(t_idx[None, None, :] <= t_idx[None, :, None], raw, -np.inf)
    tables = {}
    M1 = levels[1].shape[0]
    leaf_tab = np.empty((N, M1))
    for j in range(M1):
        with np.errstate(divide="ignore"):
            leaf_tab[:, j] = logsumexp(raw[:, :, j * C:min(j * C + C, N)], axis=2).sum(axis=0)
    tables[1] = leaf_tab
    for l in range(2, L + 1):
        child = levels[l - 1]
        cl = np.einsum("gtd,rd->gtr", q, child) * scale
        if causal:
            start = np.arange(child.shape[0]) * C * 2 ** (l - 2)
            cl = np.where(start[None, None, :] <= t_idx[None, :, None], cl, -np.inf)
        tab = np.empty((N, levels[l].shape[0]))
        for j in range(levels[l].shape[0]):
            with np.errstate(divide="ignore"):
                tab[:, j] = logsumexp(cl[:, :, 2 * j:2 * j + 2], axis=2).sum(axis=0)
        tables[l] = tab
    idx = -np.ones((N, K), np.int64)
    score = np.full((N, K), -np.inf)
    gaps = np.full(N, np.inf)
    for t in range(N):
        A = [0]
        for l in range(L, 0, -1):
            A = [j for j in A if j < levels[l].shape[0] and (not causal or j * C * 2 ** (l - 1) <= t)]
            if len(A) > K:
                order = sorted(A, key=lambda j: (-tables[l][t, j], j))
                gaps[t] = min(gaps[t], tables[l][t, order[K - 1]] - tables[l][t, order[K]])
                kept = order[:K]
            else:
                kept = list(A)
            if l > 1:
                A = [r for j in kept for r in (2 * j, 2 * j + 1) if r < levels[l - 1].shape[0]]
        kept = sorted(kept)
        idx[t, :len(kept)] = kept
        score[t, :len(kept)] = tables[1][t, kept]
    return idx, score, gaps


def check_table_descent(lib, causal: bool, K: int = 4, N: int = 1024, G: int = 4) -> None:
    """The oracle's on-the-fly descent equals an independent table-driven one
    (all sections of the method), on tiny inputs."""
    D = 32
    q, k, _ = tiny_inputs(N=N, Hq=G, Hkv=1, D=D, seed=11 + causal)
    scale = 1 / math.sqrt(D)
    p = oracle.Problem(1, N, G, 1, D, 64, K, causal=causal)
    idx, score, gap, cnt = oracle.select(p, q, k, lib=lib)
    tidx, tscore, tgap = table_descent(q[0].astype(np.float64), k[0, 0].astype(np.float64), 64, K, causal, scale)
    safe = np.minimum(gap[0, 0], tgap) > 1e-9
    assert safe.mean() > 0.95
    assert (idx[0, 0][safe] == tidx[safe]).all()
    fin = np.isfinite(tscore) & safe[:, None]
    np.testing.assert_allclose(score[0, 0][fin], tscore[fin], rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(gap[0, 0][safe], tgap[safe], rtol=1e-9, atol=1e-11)


# --------------------------------------------------------------------------
# Leaf score = exact raw-key LSE summed over the GQA group ([SEL] score eq.
# at l = 1, [KER] GQA sum)
# --------------------------------------------------------------------------
def check_leaf_scores(lib, causal: bool) -> None:
    N, G, D = 512, 4, 32
    q, k, _ = tiny_inputs(N=N, Hq=G, Hkv=1, D=D, seed=21)
    p = oracle.Problem(1, N, G, 1, D, 64, 3, causal=causal)
    ts = [0, 63, 64, 100, 300, 511]
    idx, score, _, _ = oracle.select(p, q, k, ts=ts, lib=lib)
    qq = np.array(q[0], dtype=np.longdouble)
    kk = np.array(k[0, 0], dtype=np.longdouble)
    scale = np.longdouble(1) / np.sqrt(np.longdouble(D))
    for s, t in enumerate(ts):
        for a, j in enumerate(idx[0, 0, s]):
            if j < 0:
                assert score[0, 0, s, a] == -np.inf
                continue
            hi = min(j * 64 + 64, N)
            if causal:
                hi = min(hi, t + 1)
            total = np.longdouble(0)
            for g in range(G):
                z = (kk[j * 64:hi] @ qq[g, t]) * scale
                m = z.max()
                total += m + np.log(np.exp(z - m).sum())
            assert abs(float(total) - score[0, 0, s, a]) < 1e-11 * max(1.0, abs(float(total)))


def check_leaf_score_entry(lib, causal: bool) -> None:
    """oracle_leaf_scores scores arbitrary leaf lists (any order, -1 entries,
    the ragged last leaf, leaves past the causal frontier) by the same
    long-double brute force; on the descent's own sets it gives the scores
    the descent reports."""
    N, G, D, C = 1000, 4, 32, 64
    q, k, _ = tiny_inputs(N=N, Hq=G, Hkv=1, D=D, seed=23)
    p = oracle.Problem(1, N, G, 1, D, C, 3, causal=causal)
    ts = [0, 63, 64, 130, 511, 999]
    lists = np.array([[15, 0, -1, 3, 7], [0, 1, 15, 2, -1], [1, 0, 9, 15, 4], [2, 1, 0, 3, 12],
                      [7, 8, 3, -1, 15], [15, 14, 0, 6, 2]], np.int32)[None, None]
    got = oracle.leaf_scores(p, q, k, lists, ts=ts, lib=lib)
    qq = np.array(q[0], dtype=np.longdouble)
    kk = np.array(k[0, 0], dtype=np.longdouble)
    scale = np.longdouble(1) / np.sqrt(np.longdouble(D))
    for s, t in enumerate(ts):
        for a, j in enumerate(lists[0, 0, s]):
            lo, hi = j * C, min(j * C + C, N)
            if causal:
                hi = min(hi, t + 1)
            if j < 0 or hi <= lo:
                assert got[0, 0, s, a] == -np.inf, (t, j)
                continue
            total = np.longdouble(0)
            for g in range(G):
                z = (kk[lo:hi] @ qq[g, t]) * scale
                m = z.max()
                total += m + np.log(np.exp(z - m).sum())
            assert abs(float(total) - got[0, 0, s, a]) < 1e-11 * max(1.0, abs(float(total))), (t, j)
    idx, score, _, _ = oracle.select(p, q, k, ts=ts, lib=lib)
    again = oracle.leaf_scores(p, q, k, idx, ts=ts, lib=lib)
    np.testing.assert_array_equal(again, score)


# --------------------------------------------------------------------------
# Work counters: closed forms on shapes whose candidate sets the rules of
# [SEL] fix regardless of the data (non-causal: every block valid; causal:
# keys that grow with their index, so every top-K keeps the highest valid
# blocks and the valid children can be counted by hand)
# --------------------------------------------------------------------------
def check_counters_noncausal(lib) -> None:
    """N = 1024, C = 64, K = 4, levels 16 -> 8 -> 4 -> 2 -> 1, every block
    valid: levels 5..3 hold 1, 2 and 4 candidates (kept without scoring);
    level 2 holds the 8 children of those 4 and scores them (8 blocks, 2 child
    summaries each); the 4 kept give 8 candidate leaves, scored on 64 raw keys
    each.  Per query: 8 scored blocks, 16 child dots, 8 leaf pairs, 512 leaf
    key dots, one scored level >= 2."""
    N, G, D = 1024, 4, 16
    q, k, _ = tiny_inputs(N=N, Hq=G, Hkv=1, D=D, seed=27)
    p = oracle.Problem(1, N, G, 1, D, 64, 4, causal=False)
    ts = list(range(0, N, 7))
    nt = len(ts)
    _, _, _, c = oracle.select(p, q, k, ts=ts, lib=lib)
    assert c["queries"] == nt
    assert c["scored_blocks"] == 8 * nt, c
    assert c["child_dots"] == 16 * nt, c
    assert c["leaf_pairs"] == 8 * nt, c
    assert c["leaf_key_dots"] == 512 * nt, c
    assert c["scored_levels"] == nt, c
    assert c["max_candidates"] == 8 and c["max_kept"] == 4, c
    assert c["per_level_candidates"][1:6] == [8 * nt, 8 * nt, 4 * nt, 2 * nt, nt], c["per_level_candidates"][:6]


def check_counters_causal(lib) -> None:
    """Causal, N = 1024, C = 64, K = 2, two query heads equal to e_0 and keys
    k_i = 0.375 i e_0 (logit 0.046875 i at D = 64): later blocks always score
    higher, so each scored level keeps its two highest valid blocks.  Counted
    by hand from the validity rule (a block is valid iff its first token is
    <= t) for three positions:
      t = 100: levels 5..2 hold the single valid block 0, level 1 the leaves
               {0, 1} -- nothing scored, idx {0, 1};
      t = 700: level 3 {0, 1, 2} scored (children 0..5 all valid: 6 dots),
               keeps {1, 2}; level 2 {2, 3, 4, 5} scored (children 4..10
               valid, 11 starts at 704: 7 dots), keeps {4, 5}; leaves
               {8, 9, 10} valid (64 + 64 + 61 keys), idx {9, 10};
      t = 1023: level 3 {0..3} (8 dots) keeps {2, 3}; level 2 {4..7} (8 dots)
               keeps {6, 7}; leaves {12..15} (256 keys), idx {14, 15}.
    The group sum adds per-head scores; the counters count per KV group."""
    N, D, C, K = 1024, 64, 64, 2
    q = np.zeros((1, 2, N, D), np.float32)
    q[..., 0] = 1.0
    k = np.zeros((1, 1, N, D), np.float32)
    k[0, 0, :, 0] = 0.375 * np.arange(N, dtype=np.float32)
    p = oracle.Problem(1, N, 2, 1, D, C, K, causal=True)
    expect = {
        100: dict(idx=[0, 1], scored_blocks=0, child_dots=0, leaf_pairs=0, leaf_key_dots=0, scored_levels=0,
                  levels=[2, 1, 1, 1, 1]),
        700: dict(idx=[9, 10], scored_blocks=7, child_dots=13, leaf_pairs=3, leaf_key_dots=189, scored_levels=2,
                  levels=[3, 4, 3, 2, 1]),
        1023: dict(idx=[14, 15], scored_blocks=8, child_dots=16, leaf_pairs=4, leaf_key_dots=256, scored_levels=2,
                   levels=[4, 4, 4, 2, 1]),
    }
    for t, e in expect.items():
        idx, _, _, c = oracle.select(p, q, k, ts=[t], lib=lib)
        assert idx[0, 0, 0].tolist() == e["idx"], (t, idx[0, 0, 0])
        for name in ("scored_blocks", "child_dots", "leaf_pairs", "leaf_key_dots", "scored_levels"):
            assert c[name] == e[name], (t, name, c[name], e[name])
        assert c["per_level_candidates"][1:6] == e["levels"], (t, c["per_level_candidates"][:6])


# --------------------------------------------------------------------------
# Bounds ([SEL]: candidate sets <= gK, kept <= K)
# --------------------------------------------------------------------------
def check_bounds(lib) -> None:
    for causal in (False, True):
        for K in (1, 3, 4, 5):
            q, k, _ = tiny_inputs(N=1000, D=16, seed=31)
            p = oracle.Problem(1, 1000, 4, 1, 16, 64, K, causal=causal)
            idx, _, _, cnt = oracle.select(p, q, k, lib=lib)
            assert cnt["max_candidates"] <= 2 * K
            assert cnt["max_kept"] <= K
            for row in idx[0, 0]:
                sel = row[row >= 0]
                assert len(sel) == min(K, len(set(sel.tolist())))
                assert (np.diff(sel) > 0).all()
                assert (row[len(sel):] == -1).all()


# --------------------------------------------------------------------------
# K >= M1: dense attention ([BSA] o_t equation with every block kept)
# --------------------------------------------------------------------------
def dense_attention(q, k, v, causal, scale):
    z = np.einsum("gtd,nd->gtn", q, k) * scale
    if causal:
        N = k.shape[0]
        z = np.where(np.arange(N)[None, None, :] <= np.arange(N)[None, :, None], z, -np.inf)
    m = z.max(axis=2, keepdims=True)
    e = np.exp(z - m)
    return (e @ v) / e.sum(axis=2, keepdims=True), (m[..., 0] + np.log(e.sum(axis=2)))


def check_dense_equivalence(lib, causal: bool) -> None:
    N, G, D = 1024, 4, 64
    q, k, v = tiny_inputs(N=N, Hq=G, Hkv=1, D=D, seed=41)
    p = oracle.Problem(1, N, G, 1, D, 64, 16, causal=causal)
    idx, _, _, _ = oracle.select(p, q, k, lib=lib)
    for t in (0, 5, 64, 500, 1023):
        want = list(range(0, t // 64 + 1)) if causal else list(range(16))
        assert idx[0, 0, t][: len(want)].tolist() == want
    o, lse = oracle.attention(p, q, k, v, idx, lib=lib)
    ro, rl = dense_attention(q[0].astype(np.float64), k[0, 0].astype(np.float64), v[0, 0].astype(np.float64),
                             causal, 1 / math.sqrt(D))
    np.testing.assert_allclose(o[0], ro, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[0], rl, rtol=1e-13, atol=1e-12)


# --------------------------------------------------------------------------
# K >= ceil(M1/2): every leaf is a candidate -> brute-force top-K of exact leaf
# LSE over all leaves ([SEL]: all kept while <= K, then leaf LSE, top-K)
# --------------------------------------------------------------------------
def check_bruteforce_leaf_topk(lib, causal: bool) -> None:
    N, G, D, C, K = 1024, 4, 32, 64, 8
    q, k, _ = tiny_inputs(N=N, Hq=G, Hkv=1, D=D, seed=51)
    p = oracle.Problem(1, N, G, 1, D, C, K, causal=causal)
    idx, score, _, _ = oracle.select(p, q, k, lib=lib)
    qq, kk = q[0].astype(np.float64), k[0, 0].astype(np.float64)
    z = np.einsum("gtd,nd->gtn", qq, kk) / math.sqrt(D)
    for t in range(0, N, 37):
        nleaf = t // C + 1 if causal else N // C
        u = []
        for j in range(nleaf):
            hi = min(j * C + C, t + 1) if causal else j * C + C
            u.append(sum(logsumexp(z[g, t, j * C:hi]) for g in range(G)))
        order = sorted(range(nleaf), key=lambda j: (-u[j], j))[:K]
        assert idx[0, 0, t][: len(order)].tolist() == sorted(order)
        np.testing.assert_allclose(score[0, 0, t][: len(order)], [u[j] for j in sorted(order)], rtol=1e-12)


# --------------------------------------------------------------------------
# Exact leaf top-K (quality reference): the top K over every valid leaf of the
# raw-key LSE summed over the group, against numpy/scipy brute force, with K
# small enough that the descent prunes (so it cannot stand in for it)
# --------------------------------------------------------------------------
def check_exact_topk(lib, causal: bool) -> None:
    N, G, D, C, K = 1000, 4, 32, 64, 3
    q, k, _ = tiny_inputs(N=N, Hq=G, Hkv=1, D=D, seed=53)
    p = oracle.Problem(1, N, G, 1, D, C, K, causal=causal)
    ts = np.arange(0, N, 13)
    idx, score = oracle.exact_topk(p, q, k, ts=ts, lib=lib)
    qq, kk = q[0].astype(np.float64), k[0, 0].astype(np.float64)
    z = np.einsum("gtd,nd->gtn", qq, kk) / math.sqrt(D)
    M1 = -(-N // C)
    pruned = 0
    d_idx, _, _, _ = oracle.select(p, q, k, ts=ts, lib=lib)
    for s_, t in enumerate(ts):
        nleaf = min(t // C + 1, M1) if causal else M1
        u = []
        for j in range(nleaf):
            hi = min(j * C + C, N, t + 1) if causal else min(j * C + C, N)
            u.append(sum(logsumexp(z[g, t, j * C:hi]) for g in range(G)))
        order = sorted(range(nleaf), key=lambda j: (-u[j], j))[:K]
        got = idx[0, 0, s_]
        assert got[: len(order)].tolist() == sorted(order), (t, got, sorted(order))
        assert (got[len(order):] == -1).all()
        np.testing.assert_allclose(score[0, 0, s_][: len(order)], [u[j] for j in sorted(order)], rtol=1e-12)
        pruned += int(d_idx[0, 0, s_].tolist() != got.tolist())
    assert pruned > 0  # the descent really differs somewhere: two independent paths


# --------------------------------------------------------------------------
# Attention backward: the gradients of L = sum_t dO_t . o_t over a fixed
# selection ([BSA] o_t equation; no gradient through the index-valued
# selection).  Pinned by central finite differences of the forward oracle on
# dyadic-exact perturbations, and by torch fp64 autograd of dense attention
# when every leaf is kept.
# --------------------------------------------------------------------------
def _random_selection(rng, B, Hkv, N, C, K, causal):
    M1 = -(-N // C)
    idx = np.full((B, Hkv, N, K), -1, np.int32)
    for b in range(B):
        for h in range(Hkv):
            for t in range(N):
                nvalid = min(t // C + 1, M1) if causal else M1
                pick = np.sort(rng.choice(nvalid, size=min(K, nvalid), replace=False))
                idx[b, h, t, : len(pick)] = pick
    return idx


def check_backward_finite_difference(lib, causal: bool) -> None:
    B, N, G, Hkv, D, C, K = 1, 150, 2, 2, 16, 32, 2
    Hq = G * Hkv
    q = _bf16_valued_f32(71, 1, (B, Hq, N, D))
    k = _bf16_valued_f32(71, 2, (B, Hkv, N, D))
    v = _bf16_valued_f32(71, 3, (B, Hkv, N, D))
    dO = _bf16_valued_f32(71, 4, (B, Hq, N, D))
    rng = np.random.default_rng(72)
    idx = _random_selection(rng, B, Hkv, N, C, K, causal)
    p = oracle.Problem(B, N, Hq, Hkv, D, C, K, causal=causal)
    dq, dk, dv = oracle.attention_backward(p, q, k, v, idx, dO, lib=lib)

    def loss(qq, kk, vv):
        o, _ = oracle.attention(p, qq, kk, vv, idx, lib=lib)
        return float((o * dO.astype(np.float64)).sum())

    h = 2.0 ** -9  # x +- h stays exact in float32 for bf16-valued x
    for name, arr, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for flat in rng.choice(arr.size, size=12, replace=False):
            at = np.unravel_index(flat, arr.shape)
            xp, xm = arr.copy(), arr.copy()
            xp[at] += h
            xm[at] -= h
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = xp, xm
            fd = (loss(args_p["q"], args_p["k"], args_p["v"]) - loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * h)
            assert abs(fd - grad[at]) <= 2e-4 * max(1.0, abs(grad[at])), (name, at, fd, grad[at])


def check_backward_dense(lib, causal: bool) -> None:
    import torch

    N, G, D, C = 256, 2, 32, 64
    q, k, v = tiny_inputs(N=N, Hq=G, Hkv=1, D=D, seed=73)
    dO = I.normal(73, 4, G * N * D, dtype="f32").reshape(1, G, N, D)
    M1 = N // C
    idx = np.broadcast_to(np.arange(M1, dtype=np.int32), (1, 1, N, M1)).copy()
    if causal:
        for t in range(N):
            idx[0, 0, t, t // C + 1:] = -1
    p = oracle.Problem(1, N, G, 1, D, C, M1, causal=causal)
    dq, dk, dv = oracle.attention_backward(p, q, k, v, idx, dO, lib=lib)
    tq = torch.tensor(q[0], dtype=torch.float64, requires_grad=True)
    tk = torch.tensor(k[0, 0], dtype=torch.float64, requires_grad=True)
    tv = torch.tensor(v[0, 0], dtype=torch.float64, requires_grad=True)
    z = torch.einsum("gtd,nd->gtn", tq, tk) / math.sqrt(D)
    if causal:
        mask = torch.arange(N)[None, None, :] > torch.arange(N)[None, :, None]
        z = z.masked_fill(mask, float("-inf"))
    o = torch.softmax(z, dim=-1) @ tv
    (o * torch.tensor(dO[0], dtype=torch.float64)).sum().backward()
    np.testing.assert_allclose(dq[0], tq.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk[0, 0], tk.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv[0, 0], tv.grad.numpy(), rtol=1e-10, atol=1e-12)


# --------------------------------------------------------------------------
# Shift invariance: k -> k + b shifts every LSE of a query head by q.b*scale
# ([SEL] LSE score; [BSA] softmax), so idx and o are unchanged
# --------------------------------------------------------------------------
def check_shift_invariance(lib, causal: bool) -> None:
    N, G, D = 1024, 4, 32
    q = _bf16_valued_f32(61, 1, (1, G, N, D))
    k = _bf16_valued_f32(61, 2, (1, 1, N, D))
    v = _bf16_valued_f32(61, 3, (1, 1, N, D))
    b = (np.round(I.normal(61, 9, D) * 4) / 4).astype(np.float32)  # dyadic: k + b is exact
    k2 = k + b[None, None, None, :]
    assert np.array_equal(k2.astype(np.float64) - b.astype(np.float64), k.astype(np.float64))
    p = oracle.Problem(1, N, G, 1, D, 64, 4, causal=causal)
    idx1, s1, gap1, _ = oracle.select(p, q, k, lib=lib)
    idx2, s2, gap2, _ = oracle.select(p, q, k2, lib=lib)
    safe = gap1[0, 0] > 1e-8
    assert (idx1[0, 0][safe] == idx2[0, 0][safe]).all()
    shift = (q[0].astype(np.float64) @ b.astype(np.float64)).sum(axis=0) / math.sqrt(D)  # [N]
    fin = np.isfinite(s1[0, 0]) & safe[:, None]
    np.testing.assert_allclose(s2[0, 0][fin] - s1[0, 0][fin], np.broadcast_to(shift[:, None], s1[0, 0].shape)[fin],
                               rtol=0, atol=1e-9)
    o1, _ = oracle.attention(p, q, k, v, idx1, lib=lib)
    o2, _ = oracle.attention(p, q, k2, v, idx1, lib=lib)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-11)


# --------------------------------------------------------------------------
# GQA ([KER] score-sum equation): G_Q = 1 is per-head selection; permuting the
# query heads of a group changes nothing; heads map to KV head h' // G_Q
# --------------------------------------------------------------------------
def check_gqa(lib) -> None:
    N, D = 512, 32
    q, k, _ = tiny_inputs(N=N, Hq=4, Hkv=2, D=D, seed=71)
    p = oracle.Problem(1, N, 4, 2, D, 64, 3, causal=True)
    idx, score, gap, _ = oracle.select(p, q, k, lib=lib)
    qp = q[:, [1, 0, 3, 2]]
    idx2, score2, _, _ = oracle.select(p, np.ascontiguousarray(qp), k, lib=lib)
    safe = gap > 1e-9
    assert (idx[safe] == idx2[safe]).all()
    # KV head 1 sees exactly query heads 2, 3
    p1 = oracle.Problem(1, N, 2, 1, D, 64, 3, causal=True)
    idx3, score3, _, _ = oracle.select(p1, np.ascontiguousarray(q[:, 2:4]), np.ascontiguousarray(k[:, 1:2]), lib=lib)
    assert (idx[:, 1][safe[:, 1]] == idx3[:, 0][safe[:, 1]]).all()
    # G_Q = 1: each head routed alone
    p2 = oracle.Problem(1, N, 2, 2, D, 64, 3, causal=True)
    idx4, _, gap4, _ = oracle.select(p2, np.ascontiguousarray(q[:, [0, 2]]), k, lib=lib)
    for h in range(2):
        pa = oracle.Problem(1, N, 1, 1, D, 64, 3, causal=True)
        i5, _, _, _ = oracle.select(pa, np.ascontiguousarray(q[:, [2 * h]]), np.ascontiguousarray(k[:, h:h + 1]), lib=lib)
        ok = gap4[0, h] > 1e-9
        assert (idx4[0, h][ok] == i5[0, 0][ok]).all()


# --------------------------------------------------------------------------
# Special cases: causal t < C keeps only leaf 0; N <= C is one level, dense
# attention; at t = N-1 causal equals non-causal ([SEL] validity, [BSA])
# --------------------------------------------------------------------------
def check_special_cases(lib) -> None:
    N, G, D = 1024, 4, 32
    q, k, v = tiny_inputs(N=N, Hq=G, Hkv=1, D=D, seed=81)
    p = oracle.Problem(1, N, G, 1, D, 64, 4, causal=True)
    ts = list(range(64))
    idx, _, _, _ = oracle.select(p, q, k, ts=ts, lib=lib)
    assert (idx[0, 0, :, 0] == 0).all() and (idx[0, 0, :, 1:] == -1).all()
    o, _ = oracle.attention(p, q, k, v, idx, ts=ts, lib=lib)
    ro, _ = dense_attention(q[0, :, :64].astype(np.float64), k[0, 0, :64].astype(np.float64),
                            v[0, 0, :64].astype(np.float64), True, 1 / math.sqrt(D))
    np.testing.assert_allclose(o[0], ro, rtol=0, atol=1e-12)

    for n in (1, 17, 64):
        qs, ks, vs = (np.ascontiguousarray(x[:, :, :n]) for x in (q, k, v))
        for causal in (False, True):
            pn = oracle.Problem(1, n, G, 1, D, 64, 4, causal=causal)
            assert oracle.levels(n, 64, lib=lib) == 1
            idx, _, gap, cnt = oracle.select(pn, qs, ks, lib=lib)
            assert (idx[0, 0, :, 0] == 0).all() and (idx[0, 0, :, 1:] == -1).all()
            assert np.isinf(gap).all()
            o, _ = oracle.attention(pn, qs, ks, vs, idx, lib=lib)
            ro, _ = dense_attention(qs[0].astype(np.float64), ks[0, 0].astype(np.float64),
                                    vs[0, 0].astype(np.float64), causal, 1 / math.sqrt(D))
            np.testing.assert_allclose(o[0], ro, rtol=0, atol=1e-12)

    pc = oracle.Problem(1, N, G, 1, D, 64, 4, causal=True)
    pn = oracle.Problem(1, N, G, 1, D, 64, 4, causal=False)
    a = oracle.select(pc, q, k, ts=[N - 1], lib=lib)
    b = oracle.select(pn, q, k, ts=[N - 1], lib=lib)
    assert (a[0] == b[0]).all()
    np.testing.assert_array_equal(a[1], b[1])


# --------------------------------------------------------------------------
# Needle: a leaf whose keys are 20 * unit(q) is always selected
# --------------------------------------------------------------------------
def check_needle(lib) -> None:
    N, D = 2048, 32
    q, k, _ = tiny_inputs(N=N, Hq=1, Hkv=1, D=D, seed=91)
    t = 1900
    host = 7
    u = q[0, 0, t].astype(np.float64)
    u /= np.linalg.norm(u)
    k = k.copy()
    k[0, 0, host * 64:(host + 1) * 64] = (20 * u).astype(np.float32)
    for K in (1, 2, 4):
        p = oracle.Problem(1, N, 1, 1, D, 64, K, causal=True)
        idx, _, _, _ = oracle.select(p, q, k, ts=[t], lib=lib)
        assert host in idx[0, 0, 0].tolist()


# --------------------------------------------------------------------------
# Flat selector ([BSA] flat selection): brute force over all leaf means
# --------------------------------------------------------------------------
def check_flat(lib) -> None:
    N, G, D, C, K = 1000, 4, 32, 64, 5
    q, k, _ = tiny_inputs(N=N, Hq=G, Hkv=1, D=D, seed=101)
    for causal in (False, True):
        p = oracle.Problem(1, N, G, 1, D, C, K, causal=causal)
        idx, score = oracle.flat_select(p, q, k, lib=lib)
        kk = k[0, 0].astype(np.float64)
        means = np.stack([kk[j * C:min(j * C + C, N)].mean(axis=0) for j in range(-(-N // C))])
        qs = q[0].astype(np.float64).sum(axis=0)
        for t in range(0, N, 29):
            nleaf = t // C + 1 if causal else len(means)
            u = means[:nleaf] @ qs[t] / math.sqrt(D)
            order = sorted(range(nleaf), key=lambda j: (-u[j], j))[:K]
            assert idx[0, 0, t][: len(order)].tolist() == sorted(order)
            np.testing.assert_allclose(score[0, 0, t][: len(order)], u[sorted(order)], rtol=1e-11, atol=1e-12)


# --------------------------------------------------------------------------
# Decode ([KER] decode paragraph): the new token at position n-1 of an n-token
# prefix, pyramid of the prefix, every block valid -> equals the independent
# table-driven descent over the prefix at its last position, and attention
# over its leaves
# --------------------------------------------------------------------------
def check_decode_reference(lib) -> None:
    G, D, C, K = 4, 32, 64, 3
    q, k, v = tiny_inputs(N=1024, Hq=G, Hkv=1, D=D, seed=111)
    for n in (700, 704, 705, 129, 65):
        p = oracle.Problem(1, n, G, 1, D, C, K)
        kp, vp = np.ascontiguousarray(k[:, :, :n]), np.ascontiguousarray(v[:, :, :n])
        idx, score, gap, o, lse = oracle.decode_reference(p, q[:, :, n - 1], kp, vp, lib=lib)
        tidx, tscore, tgap = table_descent(q[0, :, :n].astype(np.float64), kp[0, 0].astype(np.float64), C, K, False,
                                           1 / math.sqrt(D))
        if np.isinf(tgap[n - 1]):
            assert np.isinf(gap[0, 0])
        else:
            assert abs(gap[0, 0] - tgap[n - 1]) < 1e-9
        if tgap[n - 1] > 1e-9:
            assert idx[0, 0].tolist() == tidx[n - 1].tolist()
            fin = np.isfinite(tscore[n - 1])
            np.testing.assert_allclose(score[0, 0][fin], tscore[n - 1][fin], rtol=1e-11)
        keys = np.concatenate([np.arange(j * C, min(j * C + C, n)) for j in idx[0, 0] if j >= 0])
        z = np.einsum("gd,nd->gn", q[0, :, n - 1].astype(np.float64), kp[0, 0, keys].astype(np.float64)) / math.sqrt(D)
        w = np.exp(z - z.max(axis=1, keepdims=True))
        want = (w @ vp[0, 0, keys].astype(np.float64)) / w.sum(axis=1, keepdims=True)
        np.testing.assert_allclose(o[0], want, rtol=0, atol=1e-12)


ALL_CHECKS = [
    ("hand_example", lambda lib: check_hand_example(lib)),
    ("pyramid_closed_form", lambda lib: check_pyramid_closed_form(lib)),
    ("table_descent_noncausal", lambda lib: check_table_descent(lib, False)),
    ("table_descent_causal", lambda lib: check_table_descent(lib, True)),
    ("leaf_scores_noncausal", lambda lib: check_leaf_scores(lib, False)),
    ("leaf_scores_causal", lambda lib: check_leaf_scores(lib, True)),
    ("leaf_score_entry_noncausal", lambda lib: check_leaf_score_entry(lib, False)),
    ("leaf_score_entry_causal", lambda lib: check_leaf_score_entry(lib, True)),
    ("counters_noncausal", lambda lib: check_counters_noncausal(lib)),
    ("counters_causal", lambda lib: check_counters_causal(lib)),
    ("bounds", lambda lib: check_bounds(lib)),
    ("dense_noncausal", lambda lib: check_dense_equivalence(lib, False)),
    ("dense_causal", lambda lib: check_dense_equivalence(lib, True)),
    ("bruteforce_leaf_topk_noncausal", lambda lib: check_bruteforce_leaf_topk(lib, False)),
    ("bruteforce_leaf_topk_causal", lambda lib: check_bruteforce_leaf_topk(lib, True)),
    ("exact_topk_noncausal", lambda lib: check_exact_topk(lib, False)),
    ("exact_topk_causal", lambda lib: check_exact_topk(lib, True)),
    ("backward_fd_noncausal", lambda lib: check_backward_finite_difference(lib, False)),
    ("backward_fd_causal", lambda lib: check_backward_finite_difference(lib, True)),
    ("backward_dense_noncausal", lambda lib: check_backward_dense(lib, False)),
    ("backward_dense_causal", lambda lib: check_backward_dense(lib, True)),
    ("shift_noncausal", lambda lib: check_shift_invariance(lib, False)),
    ("shift_causal", lambda lib: check_shift_invariance(lib, True)),
    ("gqa", lambda lib: check_gqa(lib)),
    ("special_cases", lambda lib: check_special_cases(lib)),
    ("needle", lambda lib: check_needle(lib)),
    ("flat", lambda lib: check_flat(lib)),
    ("decode_reference", lambda lib: check_decode_reference(lib)),
]
