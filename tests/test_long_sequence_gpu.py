"""Long sequences through the prefill and its backward: L = 65536 (16 times the
training workload's length, 512 key tiles per head, 32 MB per head and tensor).

- Causal prefill, every key visible to the last rows: sampled rows across the range
  (the last ones see all 65536 keys) and their lse against the oracle row by row.
- With a 256-key window: the whole output and all four gradients against the oracle
  (the window keeps the oracle's work to seconds)."""
import numpy as np
import pytest

import oracle
import parameterized_local_linear_amd as plx
import synth
from gpu_util import assert_parity, from_gpu, to_gpu

pytestmark = pytest.mark.gpu

B, HQ, HKV, L, D = 1, 2, 1, 65536, 128
S128 = 1.0 / np.sqrt(128.0)


def _inputs(seed):
    q, r = (synth.normal(seed, tid, (B, HQ, L, D), S128, synth.BF16) for tid in (synth.TID_Q, synth.TID_R))
    k, v = (synth.normal(seed, tid, (B, HKV, L, D), S128, synth.BF16) for tid in (synth.TID_K, synth.TID_V))
    do = synth.normal(seed, synth.TID_DO, (B, HQ, L, D), 1.0, synth.BF16)
    return q, r, k, v, do


def test_long_causal_prefill_sampled_rows():
    q, r, k, v, _ = _inputs(970)
    t = [to_gpu(x, synth.BF16) for x in (q, r, k, v)]
    o, lse, _ = plx.prefill(*t, return_stats=True)
    o, lse = from_gpu(o), lse.cpu().numpy().astype(np.float64)
    g = np.random.default_rng(970)
    rows = np.concatenate([
        np.array([[0, 0, 0], [0, 1, 1], [0, 0, L - 1], [0, 1, L - 1], [0, 0, L - 2], [0, 1, 32767]]),
        np.stack([np.zeros(10, dtype=np.int64), g.integers(0, HQ, 10), g.integers(0, L, 10)], axis=1)])
    ref, ref_lse, _ = oracle.prefill(q, r, k, v, rows=rows, stats=True)
    assert_parity(o[rows[:, 0], rows[:, 1], rows[:, 2]], ref, synth.BF16, "L=65536 sampled rows")
    got_lse = lse[rows[:, 0], rows[:, 1], rows[:, 2]]
    assert np.abs(got_lse - ref_lse).max() <= 1e-4 * max(1.0, np.abs(ref_lse).max())


def test_long_windowed_prefill_and_backward():
    W = 256
    q, r, k, v, do = _inputs(971)
    t = [to_gpu(x, synth.BF16) for x in (q, r, k, v, do)]
    o, lse, sbar = plx.prefill(*t[:4], return_stats=True, window=W)
    assert_parity(from_gpu(o), oracle.prefill(q, r, k, v, window=W), synth.BF16, "L=65536 window")
    grads = plx.prefill_backward(*t[:4], o, t[4], lse, sbar, window=W)
    ref = oracle.prefill_backward(q, r, k, v, do, window=W)
    for name, a, b in zip(("dq", "dr", "dk", "dv"), grads, ref):
        a = from_gpu(a)
        err = np.abs(a - b).max() / np.abs(b).max()
        assert err <= 1e-2, f"L=65536 window backward {name}: max-norm error {err:.3e}"
