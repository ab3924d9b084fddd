"""GPU parity of parallax_prefill (causal) against the double oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
import parameterized_local_linear_amd as plx
import synth
from gpu_util import assert_parity, from_gpu, to_gpu

pytestmark = pytest.mark.gpu

S128 = 1.0 / math.sqrt(128.0)


def inputs(B, Hq, Hkv, L, D, dtype, scale, seed):
    q = synth.normal(seed, synth.TID_Q, (B, Hq, L, D), scale, dtype)
    r = synth.normal(seed, synth.TID_R, (B, Hq, L, D), scale, dtype)
    k = synth.normal(seed, synth.TID_K, (B, Hkv, L, D), scale, dtype)
    v = synth.normal(seed, synth.TID_V, (B, Hkv, L, D), scale, dtype)
    return q, r, k, v


@pytest.mark.parametrize("dtype,D", [(synth.BF16, 128), (synth.F32, 64), (synth.BF16, 64),
                                     (synth.F32, 128)])
@pytest.mark.parametrize("L", [1, 7, 64, 65, 200])
def test_prefill_small(dtype, D, L):
    B, Hq, Hkv = 2, 4, 2
    q, r, k, v = inputs(B, Hq, Hkv, L, D, dtype, 1.0, 40 + L)
    t = [to_gpu(x, dtype) for x in (q, r, k, v)]
    o, lse, sbar = plx.prefill(*t, return_stats=True)
    ref, ref_lse, ref_sbar = oracle.prefill(q, r, k, v, stats=True)
    assert_parity(from_gpu(o), ref, dtype, f"prefill L={L}")
    lse = lse.cpu().numpy().astype(np.float64)
    sbar = sbar.cpu().numpy().astype(np.float64)
    assert np.abs(lse - ref_lse).max() <= 1e-4 * max(1.0, np.abs(ref_lse).max())
    tol = 1e-4 if dtype == synth.F32 else 1e-2
    assert np.abs(sbar - ref_sbar).max() <= tol * max(1.0, np.abs(ref_sbar).max())


@pytest.mark.parametrize("scale", [S128, 1.0])
def test_prefill_gqa_bf16(scale):
    B, Hq, Hkv, L, D = 1, 8, 2, 300, 128
    q, r, k, v = inputs(B, Hq, Hkv, L, D, synth.BF16, scale, 77)
    t = [to_gpu(x, synth.BF16) for x in (q, r, k, v)]
    assert_parity(from_gpu(plx.prefill(*t)), oracle.prefill(q, r, k, v), synth.BF16, "gqa")


def test_prefill_row_matches_decode_on_prefix():
    B, Hq, Hkv, L, D = 1, 4, 2, 130, 128
    q, r, k, v = inputs(B, Hq, Hkv, L, D, synth.BF16, S128, 78)
    t = [to_gpu(x, synth.BF16) for x in (q, r, k, v)]
    o = from_gpu(plx.prefill(*t))
    for i in (0, 64, 129):
        kd = t[2][:, :, : i + 1].transpose(1, 2).contiguous()
        vd = t[3][:, :, : i + 1].transpose(1, 2).contiguous()
        od = from_gpu(plx.decode(t[0][:, :, i].contiguous(), t[1][:, :, i].contiguous(), kd, vd))
        assert np.abs(od - o[:, :, i]).max() <= 1e-2 * np.abs(o[:, :, i]).max()


@pytest.mark.parametrize("Hq,Hkv", [(4, 2), (2, 2), (8, 2), (6, 2), (3, 1)])
@pytest.mark.parametrize("L", [1, 31, 64, 100, 257])
def test_prefill_mfma_shapes(Hq, Hkv, L):
    """bf16, head_dim 128: the MFMA kernel across q-tile, KV-tile and diagonal
    boundaries, for group sizes 1, even (two query heads per work item) and odd
    (one)."""
    B, D = 2, 128
    q, r, k, v = inputs(B, Hq, Hkv, L, D, synth.BF16, 1.0, 300 + L + Hq)
    t = [to_gpu(x, synth.BF16) for x in (q, r, k, v)]
    o, lse, sbar = plx.prefill(*t, return_stats=True)
    ref, ref_lse, ref_sbar = oracle.prefill(q, r, k, v, stats=True)
    assert_parity(from_gpu(o), ref, synth.BF16, f"Hq={Hq} Hkv={Hkv} L={L}")
    lse = lse.cpu().numpy().astype(np.float64)
    assert np.abs(lse - ref_lse).max() <= 1e-3 * max(1.0, np.abs(ref_lse).max())
    sbar = sbar.cpu().numpy().astype(np.float64)
    assert np.abs(sbar - ref_sbar).max() <= 1e-2 * max(1.0, np.abs(ref_sbar).max())


def test_prefill_workload_sampled_rows():
    """B=8, L=4096, Hq=16, Hkv=8, D=128, bf16, N(0,1)/sqrt(128): sampled rows
    across the causal range (every row's oracle cost is its prefix)."""
    spec = synth.prefill_spec(5)
    B, Hq, Hkv, L, D = spec.B, spec.Hq, spec.Hkv, spec.L, spec.D
    q, r, k, v = inputs(B, Hq, Hkv, L, D, spec.dtype, spec.scale, spec.seed)
    t = [to_gpu(x, spec.dtype) for x in (q, r, k, v)]
    o = plx.prefill(*t)
    g = np.random.default_rng(5)
    rows = np.stack([g.integers(0, B, 96), g.integers(0, Hq, 96), g.integers(0, L, 96)], axis=1)
    rows = np.concatenate([rows, [[0, 0, 0], [B - 1, Hq - 1, L - 1], [3, 7, 63], [3, 7, 64],
                                  [5, 2, 127], [5, 2, 128]]])
    ref = oracle.prefill(q, r, k, v, rows=rows)
    got = from_gpu(o[rows[:, 0], rows[:, 1], rows[:, 2]])
    assert_parity(got, ref, spec.dtype, "prefill workload rows")


def test_prefill_workload_full_output():
    """B=8, L=4096, Hq=16, Hkv=8, D=128, bf16, N(0,1)/sqrt(128): every output row of
    every (sequence, query head), with lse and sbar, against the oracle."""
    spec = synth.prefill_spec(5)
    B, Hq, Hkv, L, D = spec.B, spec.Hq, spec.Hkv, spec.L, spec.D
    q, r, k, v = inputs(B, Hq, Hkv, L, D, spec.dtype, spec.scale, spec.seed)
    t = [to_gpu(x, spec.dtype) for x in (q, r, k, v)]
    o, lse, sbar = plx.prefill(*t, return_stats=True)
    o, lse, sbar = from_gpu(o), lse.cpu().numpy(), sbar.cpu().numpy()
    ref, ref_lse, ref_sbar = oracle.prefill(q, r, k, v, stats=True)
    assert_parity(o, ref, spec.dtype, "causal prefill workload")
    assert np.abs(lse - ref_lse).max() <= 1e-4 * max(1.0, np.abs(ref_lse).max())
    assert np.abs(sbar - ref_sbar).max() <= 1e-2 * max(1.0, np.abs(ref_sbar).max())


@pytest.mark.parametrize("L", [65, 300])
def test_prefill_shifted_keys_and_probe_scale(L):
    """Keys shifted by a constant vector (a large common part in every r.k and
    q.k) with a probe scale other than 1: the pivot must centre the probe scores
    and the scale must reach B, S and the pivot alike (bf16, the MFMA path)."""
    B, Hq, Hkv, D = 1, 4, 2, 128
    q, r, k, v = inputs(B, Hq, Hkv, L, D, synth.BF16, 1.0, 500 + L)
    c = 3.0 * synth.key_shift(500 + L, D)
    ks = np.array([synth.bf16_from_double(x) for x in (synth.bf16_bits_to_f32(k) + c).ravel()],
                  dtype=np.uint16).reshape(k.shape)
    t = [to_gpu(x, synth.BF16) for x in (q, r, ks, v)]
    o, lse, sbar = plx.prefill(*t, 0.05, 0.6, return_stats=True)
    ref, ref_lse, ref_sbar = oracle.prefill(q, r, ks, v, qk_scale=0.05, rk_scale=0.6, stats=True)
    assert_parity(from_gpu(o), ref, synth.BF16, f"shifted keys L={L}")
    lse = lse.cpu().numpy().astype(np.float64)
    assert np.abs(lse - ref_lse).max() <= 1e-3 * max(1.0, np.abs(ref_lse).max())
    sbar = sbar.cpu().numpy().astype(np.float64)
    assert np.abs(sbar - ref_sbar).max() <= 1e-2 * max(1.0, np.abs(ref_sbar).max())
