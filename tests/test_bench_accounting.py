"""The bench's algorithmic work counts against brute force (host only).

The roofline figures divide these counts by measured time, so a miscount would
misstate every TFLOP/s figure: visible (query, key) pairs of a causal prefill
with a window, and with a block-sparse mask (a query block always sees its own
block)."""
import importlib.util
import os

import numpy as np
import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_spec = importlib.util.spec_from_file_location("bench_module", os.path.join(ROOT, "bench.py"))
bench = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(bench)


@pytest.mark.parametrize("L,W", [(1, 0), (7, 0), (7, 3), (300, 0), (300, 128), (300, 299),
                                 (300, 300), (300, 1000), (4096, 1024)])
def test_visible_pairs_counts_the_causal_band(L, W):
    i, j = np.arange(L)[:, None], np.arange(L)[None, :]
    band = (j <= i) & ((j > i - W) if W > 0 else True)
    assert bench.visible_pairs(L, W) == int(band.sum())


@pytest.mark.parametrize("L,density,seed", [(128, 0.5, 1), (700, 0.3, 2), (1030, 0.0, 3),
                                            (1030, 1.0, 4), (4096, 0.25, 5)])
def test_masked_pairs_counts_the_expanded_mask(L, density, seed):
    nb = -(-L // 128)
    m = synth.block_mask(seed, (2, 3, nb, nb), density)
    i, j = np.arange(L)[:, None], np.arange(L)[None, :]
    qb, kb = i // 128, j // 128
    total = 0
    for b in range(2):
        for h in range(3):
            vis = (j <= i) & ((qb == kb) | (m[b, h][qb, kb] != 0))
            total += int(vis.sum())
    assert bench.masked_pairs(m, L) == total


def test_elementwise_relative_error_skips_near_zero_references():
    import bench
    ref = np.array([[1.0, -0.5, 1e-9, 0.25]])
    o = ref * np.array([[1.002, 0.997, 50.0, 1.001]])  # the 1e-9 element is far off
    # the near-zero element is below 1% of the row's largest and is left out
    assert abs(bench.elementwise_rel_err(o, ref) - 0.003) < 1e-12
