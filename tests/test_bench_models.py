"""The benchmark's work models, which every roofline figure divides by a
kernel's time, checked on the CPU against brute-force counts and against the
oracle's pinned work counters ("Block Sparse Attention with Log-Linear
Complexity", hyper.ai page: the o_t equation of "block-sparse attention" for
the attended keys; "coarse-to-fine top-K selection" for the descent the
decode byte model follows; "complexity" for the flat selector's work).

No GPU: the counting helpers take CPU tensors."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import bench
import oracle
from hierarchical_block_sparse_mean_amd import inputs as I


def random_selection(B, H, N, C, K, causal, seed):
    """idx [B][H][N][K]: per row up to K distinct valid leaves, ascending,
    -1 padded (some rows short), as a selector hands them to attention."""
    rng = np.random.default_rng(seed)
    M1 = -(-N // C)
    idx = np.full((B, H, N, K), -1, np.int32)
    for b in range(B):
        for h in range(H):
            for t in range(N):
                nvalid = min(M1, t // C + 1) if causal else M1
                want = int(rng.integers(1, min(K, nvalid) + 1))
                row = np.sort(rng.choice(nvalid, size=want, replace=False))
                idx[b, h, t, :want] = row
    return idx


@pytest.mark.parametrize("causal", [True, False])
def test_attended_keys_brute_force(causal):
    B, H, N, C, K = 2, 2, 203, 16, 5  # ragged last leaf (203 = 12 * 16 + 11)
    idx = random_selection(B, H, N, C, K, causal, seed=5 + causal)
    want = 0
    for b in range(B):
        for h in range(H):
            for t in range(N):
                for j in idx[b, h, t]:
                    if j < 0:
                        continue
                    for s in range(j * C, min(j * C + C, N)):
                        want += (not causal) or s <= t
    assert bench.attended_keys(torch.from_numpy(idx), N, C, causal) == want


def test_attention_partials_brute_force():
    B, H, N, C, K = 1, 3, 150, 8, 6
    idx = random_selection(B, H, N, C, K, True, seed=11)
    kept = pairs = 0
    for row in idx.reshape(-1, K):
        v = [int(j) for j in row if j >= 0]
        kept += len(v)
        i = 0
        while i < len(v):  # an even leaf followed by its odd sibling shares one record
            if v[i] % 2 == 0 and i + 1 < len(v) and v[i + 1] == v[i] + 1:
                pairs += 1
                i += 2
            else:
                i += 1
    t = torch.from_numpy(idx)
    assert bench.attention_partials(t, paired=False) == kept
    assert bench.attention_partials(t, paired=True) == kept - pairs


@pytest.mark.parametrize("causal", [True, False])
def test_stage1_scored_keys_brute_force(causal):
    B, H, N, C, K = 1, 2, 333, 8, 4
    M2 = -(-(-(-N // C)) // 2)
    rng = np.random.default_rng(17)
    blk2 = np.full((B, H, N, K), -1, np.int32)
    for h in range(H):
        for t in range(N):
            nvalid = min(M2, t // (2 * C) + 1) if causal else M2
            want = int(rng.integers(1, min(K, nvalid) + 1))
            blk2[0, h, t, :want] = np.sort(rng.choice(nvalid, size=want, replace=False))
    keys = npairs = 0
    for h in range(H):
        for t in range(N):
            for j2 in blk2[0, h, t]:
                if j2 < 0:
                    continue
                npairs += 1
                for s in range(2 * j2 * C, min(2 * j2 * C + 2 * C, N)):
                    keys += (not causal) or s <= t
    assert bench.stage1_scored_keys(torch.from_numpy(blk2), N, C, causal) == (keys, npairs)


@pytest.mark.parametrize("causal", [True, False])
def test_flat_work_brute_force(causal):
    N, C, D, B, Hkv = 1000, 64, 32, 2, 3
    M1 = -(-N // C)
    valid = sum((min(M1, t // C + 1) if causal else M1) for t in range(N))
    assert bench.flat_work(N, C, D, B, Hkv, causal) == 2.0 * D * valid * B * Hkv


# (n, C, K): n = C * 2^m has full sibling pairs at every level; the others
# have a ragged last block on some levels
DECODE_CASES = [(4096, 64, 16), (2048, 32, 8), (1024, 64, 16), (1000, 16, 4), (777, 8, 3), (5000, 32, 6)]


@pytest.mark.parametrize("n,C,K", DECODE_CASES)
def test_decode_bytes_model_matches_oracle_counters(n, C, K):
    """Summary rows and leaf keys of the decode byte model against the
    oracle's work counters for the query at t = n - 1 (every block valid):
    equal where every level has full sibling pairs, otherwise at most one
    extra row per level and one extra leaf."""
    D, G = 16, 2
    q = I.normal(41, 1, G * D, dtype="f32").reshape(1, G, 1, D)
    k = I.normal(41, 2, n * D, dtype="f32").reshape(1, 1, n, D)
    p = oracle.Problem(1, n, G, 1, D, C, K, causal=True)
    _, _, _, c = oracle.select(p, q, k, ts=[n - 1], q_sampled=True)
    m = bench.decode_bytes_model(n, C, K, D, G, esz=2)
    model_leaf = m["leaf_keys"] // (D * 2)
    full = n % C == 0 and ((n // C) & (n // C - 1)) == 0
    if full:
        assert m["summary_rows"] == c["child_dots"], (m, c)
    else:
        assert 0 <= m["summary_rows"] - c["child_dots"] <= m["levels"], (m, c)
    if c["leaf_key_dots"] == 0:  # at most K candidate leaves: kept unscored, their keys read once
        assert model_leaf == min(-(-n // C), K) * C or not full, (m, c)
        assert model_leaf <= K * C
    elif full:
        assert model_leaf == c["leaf_key_dots"], (m, c)
    else:
        assert 0 <= model_leaf - c["leaf_key_dots"] <= 2 * C, (m, c)


def test_decode_bytes_model_hand_count():
    """n = 131072, C = 64, K = 16 (2048 leaves, 12 levels): levels 12..8 keep
    all their 1..16 candidates; levels 7..2 each hold 32 candidates and score
    their 64 children; the 32 candidate leaves' 2048 raw keys are scored and
    the 16 kept leaves' 1024 values read."""
    m = bench.decode_bytes_model(131072, 64, 16, 128, 4, esz=2)
    assert m["levels"] == 12
    assert m["summary_rows"] == 6 * 64
    assert m["summaries"] == 384 * (128 * 2 + 4)
    assert m["leaf_keys"] == 2048 * 128 * 2
    assert m["values"] == 1024 * 128 * 2
