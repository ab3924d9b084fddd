"""Parity at the size limits the kernels' 32-bit offsets set.

- Decode: one split may span at most 2^31 bytes of K (its keys plus the keys the
  streaming loop reads ahead). With 64 KV heads a token is 16 KB, so a cache of
  140,000 keys cannot run as one split: the plan must raise a forced single split to
  two, each spanning about 1.1 GB, and the output must still match the oracle; the
  default plan is checked on the same cache.
- Prefill: the longest sequence the prefill takes is 2^22 tokens (a head's [L, D]
  tensor addressed with 32-bit offsets). A windowed prefill at that length is checked
  on sampled rows across the whole range, the last ones 1 GB into each tensor, with
  their lse; one token more is refused before anything runs.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import parameterized_local_linear_amd as plx
import synth
from gpu_util import assert_parity, from_gpu, to_gpu

pytestmark = pytest.mark.gpu

MAX_PREFILL_LEN = 1 << 22  # the limit stated for parallax_prefill


def test_decode_split_raised_past_32bit_span():
    B, Hq, Hkv, D, L = 1, 64, 64, 128, 140_000
    assert plx.decode_num_splits(B, Hq, Hkv, D, L, plx.PLX_BF16, 1) >= 2
    s = 1.0 / math.sqrt(D)
    q, r = (synth.normal(990, tid, (B, Hq, D), s, synth.BF16) for tid in (0, 1))
    k, v = (synth.normal(990, tid, (B, L, Hkv, D), s, synth.BF16) for tid in (2, 3))
    t = [to_gpu(x, synth.BF16) for x in (q, r, k, v)]
    ref = oracle.decode(q, r, k, v)
    for splits in (1, 0):
        o = from_gpu(plx.decode(*t, num_splits=splits))
        assert_parity(o, ref, synth.BF16, f"decode over 140000 keys x 64 KV heads, splits={splits}")


def test_prefill_at_the_longest_sequence():
    B, H, D, W, L = 1, 1, 128, 256, MAX_PREFILL_LEN
    s = 1.0 / math.sqrt(D)
    q, r = (synth.normal(991, tid, (B, H, L, D), s, synth.BF16) for tid in (synth.TID_Q, synth.TID_R))
    k, v = (synth.normal(991, tid, (B, H, L, D), s, synth.BF16) for tid in (synth.TID_K, synth.TID_V))
    t = [to_gpu(x, synth.BF16) for x in (q, r, k, v)]
    o, lse, _ = plx.prefill(*t, return_stats=True, window=W)
    o, lse = from_gpu(o), lse.cpu().numpy().astype(np.float64)
    g = np.random.default_rng(991)
    pos = np.concatenate([[0, 1, W - 1, W, L // 2, L - W, L - 2, L - 1], g.integers(0, L, 8)])
    rows = np.stack([np.zeros_like(pos), np.zeros_like(pos), pos], axis=1)
    ref, ref_lse, _ = oracle.prefill(q, r, k, v, rows=rows, stats=True, window=W)
    assert_parity(o[0, 0, pos], ref, synth.BF16, "prefill at L = 2^22, window 256")
    assert np.abs(lse[0, 0, pos] - ref_lse).max() <= 1e-4 * max(1.0, np.abs(ref_lse).max())
    del t, o, lse
    torch.cuda.empty_cache()

    big = [torch.empty((B, H, L + 1, D), dtype=torch.bfloat16, device="cuda") for _ in range(4)]
    with pytest.raises(plx.ParallaxError):
        plx.prefill(*big, window=W)
