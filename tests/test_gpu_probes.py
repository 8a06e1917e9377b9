"""The measurement probes the benchmark takes its HBM ceilings from (not part
of the method): pisa_probe_stream's copy reproduces its source exactly, and
its read mode folds every 16-byte piece into the checksum of the thread that
owns it (thread i reads pieces i, i + T, i + 2T, ... for T threads), checked
against the same fold done with numpy."""
import numpy as np
import pytest
import torch

from hierarchical_block_sparse_mean_amd import pisa

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n16,wgs", [(1 << 16, 4), (12345, 3), ((1 << 20) + 7, 64)])
def test_probe_stream(n16, wgs):
    print(f"[probe_stream] pieces={n16} workgroups={wgs}", flush=True)
    g = torch.Generator().manual_seed(n16)
    host = torch.randint(-(1 << 31), (1 << 31) - 1, (n16 * 4,), generator=g, dtype=torch.int64).to(torch.int32)
    src = host.cuda()
    dst = torch.zeros_like(src)
    pisa.probe_stream(src, dst, n16 * 16, 1, wgs, None)
    torch.cuda.synchronize()
    assert torch.equal(dst.cpu(), host)

    threads = wgs * 256
    sink = torch.full((threads,), -1, dtype=torch.int32, device="cuda")
    pisa.probe_stream(src, None, n16 * 16, 0, wgs, sink)
    torch.cuda.synchronize()
    words = host.numpy().view(np.uint32).reshape(n16, 4)
    piece = words[:, 0] ^ words[:, 1] ^ words[:, 2] ^ words[:, 3]
    pad = (-n16) % threads
    folded = np.bitwise_xor.reduce(np.concatenate([piece, np.zeros(pad, np.uint32)]).reshape(-1, threads), axis=0)
    assert np.array_equal(sink.cpu().numpy().view(np.uint32), folded)
