"""The memory-path calibration entry point (pma_gather_ceiling): wavefront w
folds with XOR the 1 KB rows rows[w * per .. w * per + per - 1] of the table,
lane l holding bytes 16 l .. 16 l + 15 of each row, and row indices outside
the table read its last row. Checked bit for bit against the same fold on
the host."""
import numpy as np
import pytest
import torch

import graph_sparse_head_amd as pma

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n,per", [(103, 5), (64, 64), (1, 1), (1000, 8), (999, 7)])
def test_gather_ceiling_folds_the_rows(n, per):
    print(f"[calibrate] n={n} per={per}", flush=True)
    rng = np.random.default_rng(n + per)
    n_tab = 37
    table = rng.integers(0, 2**32, size=(n_tab, 256), dtype=np.uint64).astype(np.uint32)
    rows = rng.integers(-3, n_tab + 5, size=n).astype(np.int32)   # some past either end
    waves = -(-n // per)
    t_dev = torch.from_numpy(table.view(np.int32)).cuda()
    r_dev = torch.from_numpy(rows).cuda()
    sink = torch.full((waves * 256,), -1, dtype=torch.int32, device="cuda")
    pma.pma_gather_ceiling(t_dev, r_dev, per, sink)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32).reshape(waves, 256)
    clamped = np.where((rows < 0) | (rows >= n_tab), n_tab - 1, rows)
    for w in range(waves):
        want = np.bitwise_xor.reduce(table[clamped[w * per:(w + 1) * per]], axis=0)
        assert np.array_equal(got[w], want), w


def test_gather_ceiling_binding_rejects():
    t = torch.zeros(256, dtype=torch.int32, device="cuda")
    r = torch.zeros(4, dtype=torch.int32, device="cuda")
    with pytest.raises(pma.PmaError) as e:
        pma.pma_gather_ceiling(t, r.to(torch.int64), 2, torch.zeros(512, dtype=torch.int32, device="cuda"))
    assert e.value.name == "PMA_E_DTYPE"
    with pytest.raises(pma.PmaError) as e:
        pma.pma_gather_ceiling(t, r, 2, torch.zeros(256, dtype=torch.int32, device="cuda"))
    assert e.value.name == "PMA_E_SIZE"                     # 2 wavefronts need 2 KiB
    with pytest.raises(pma.PmaError) as e:
        pma.pma_gather_ceiling(t[:100], r, 2, torch.zeros(512, dtype=torch.int32, device="cuda"))
    assert e.value.name == "PMA_E_ARG"                      # 400 bytes: not whole KiB
