"""The matrix-core rate probe (halo_mfma_rate_probe, the measurement aid bench.py sets the
products against): every instruction kind launches and completes, and the operation count it
reports is that of its grid, 256 workgroups of 8 waves, each wave issuing `iters` (rounded up
to even) groups of 8 MFMAs (16 of the 16 x 16 x 128 kind)."""
import pytest
import torch

import hadamard_rotated_precision_halo_amd as H

pytestmark = pytest.mark.gpu

# operations (2 x multiply-adds) of one group of MFMAs per wave, per kind
GROUP_OPS = {0: 8 * 2 * 32 * 32 * 32, 1: 8 * 2 * 32 * 32 * 64, 2: 16 * 2 * 16 * 16 * 128}


@pytest.mark.parametrize("kind", [0, 1, 2])
@pytest.mark.parametrize("iters", [2, 3, 64])
def test_probe_runs_and_counts(kind, iters):
    print(f"probe kind {kind}, iters {iters}", flush=True)
    st = torch.cuda.current_stream()
    ops = H.mfma_rate_probe(kind, iters, st)
    torch.cuda.synchronize()
    groups = (iters + 1) // 2 * 2
    assert ops == 256 * 8 * groups * GROUP_OPS[kind]
