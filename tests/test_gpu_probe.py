"""The matrix-core rate probe (a measurement aid of the benchmark) runs and counts its products."""

import pytest

pytestmark = pytest.mark.gpu


def test_mfma_peak_probe_counts_its_products_and_runs():
    import torch

    import prefix_tree_packed_dfs_amd as lib
    print("case mfma peak probe: 64 blocks x 100 iterations", flush=True)
    sink = torch.zeros(256, dtype=torch.float32, device="cuda")
    flops = lib.tree_mfma_peak(64, 100, sink)
    torch.cuda.synchronize()
    assert flops == 64 * 4 * 100 * 4 * 32 * 32 * 16 * 2
    assert not sink.any()  # the guarded store never fires for the probe's operands
    with pytest.raises(lib.TreeAttnError):
        lib.tree_mfma_peak(0, 100, sink)
