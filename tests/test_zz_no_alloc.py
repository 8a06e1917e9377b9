"""pisa_select_noalloc (selection with the library's own per-GPU scratch, no
workspace argument) against pisa_select with a caller workspace, through
the C ABI: the same kernels run, so the indices must be identical and the
scores bit-identical.  Two calls in a row on one GPU, the second with a
smaller problem (the scratch keeps the first call's contents, which must not
matter), then the first problem again."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from gpu_util import log, to_dev
from hierarchical_block_sparse_mean_amd import inputs as I
from hierarchical_block_sparse_mean_amd import pisa

pytestmark = pytest.mark.gpu

BIG = I.workload("prefill_32k")  # needs about 68 MB of the 128 MiB scratch
SMALL = I.Workload("noalloc_small", 1, 4133, 8, 2, 64, 48, 8, "f32", False, seed=31)


def _run(w: I.Workload):
    data = I.generate(w, with_v=False)
    p = pisa.Problem(w.B, w.N, w.Hq, w.Hkv, w.D, w.C, w.K, causal=w.causal, dtype=w.dtype)
    need = pisa.select_workspace_bytes(p)
    assert 0 < need <= pisa.NOALLOC_SCRATCH_BYTES, need
    q, k = to_dev(data["q"]), to_dev(data["k"])
    pyr = pisa.build_pyramid(p, k)
    ref_idx, ref_score = pisa.select(p, q, k, pyr)
    idx = torch.full_like(ref_idx, -7)
    score = torch.full_like(ref_score, 7.0)
    pisa.select_noalloc(p, q, k, pyr, idx, score)
    torch.cuda.synchronize()
    a, b = ref_idx.cpu().numpy(), idx.cpu().numpy()
    assert np.array_equal(a, b), f"{w.name}: {int((a != b).any(-1).sum())} rows differ"
    sa, sb = ref_score.cpu().numpy(), score.cpu().numpy()
    assert np.array_equal(sa.view(np.uint32), sb.view(np.uint32)), f"{w.name}: scores not bit-identical"
    log(f"[noalloc {w.name}] scratch need {need / 2**20:.1f} MiB: identical to pisa_select "
        f"({int((b >= 0).sum())} kept leaves)")


def test_noalloc_matches_select_twice_smaller_second():
    _run(BIG)
    _run(SMALL)
    _run(BIG)
