"""GPU parity of the sliding window (prefill, decode, backward) against the oracle.

Query i of a prefill sees keys i - W + 1 .. i; a decode query the last W keys
of its sequence. Same bars as the unwindowed tests: max-norm 1e-2 for bf16
inputs, 1e-5 (outputs) / 1e-4 (gradients) for fp32.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import parameterized_local_linear_amd as plx
import synth
from gpu_util import assert_parity, decode_inputs, from_gpu, to_gpu

pytestmark = pytest.mark.gpu

S128 = 1.0 / math.sqrt(128.0)
GTOL = {synth.F32: 1e-4, synth.BF16: 1e-2}


def prefill_inputs(B, Hq, Hkv, L, D, dtype, scale, seed, with_do=False):
    q = synth.normal(seed, synth.TID_Q, (B, Hq, L, D), scale, dtype)
    r = synth.normal(seed, synth.TID_R, (B, Hq, L, D), scale, dtype)
    k = synth.normal(seed, synth.TID_K, (B, Hkv, L, D), scale, dtype)
    v = synth.normal(seed, synth.TID_V, (B, Hkv, L, D), scale, dtype)
    if with_do:
        return q, r, k, v, synth.normal(seed, synth.TID_DO, (B, Hq, L, D), 1.0, dtype)
    return q, r, k, v


@pytest.mark.parametrize("dtype,D", [(synth.BF16, 128), (synth.F32, 64)])
@pytest.mark.parametrize("L,W", [(7, 1), (7, 3), (130, 1), (130, 64), (257, 100), (257, 128),
                                 (600, 129), (600, 300), (600, 599)])
def test_prefill_window(dtype, D, L, W):
    host = prefill_inputs(2, 4, 2, L, D, dtype, S128 if D == 128 else 1.0, 300 + L + W)
    t = [to_gpu(x, dtype) for x in host]
    o, lse, sbar = plx.prefill(*t, return_stats=True, window=W)
    ref, ref_lse, ref_sbar = oracle.prefill(*host, stats=True, window=W)
    assert_parity(from_gpu(o), ref, dtype, f"prefill L={L} W={W}")
    lse = lse.cpu().numpy().astype(np.float64)
    assert np.abs(lse - ref_lse).max() <= 1e-4 * max(1.0, np.abs(ref_lse).max())
    tol = 1e-4 if dtype == synth.F32 else 1e-2
    sbar = sbar.cpu().numpy().astype(np.float64)
    assert np.abs(sbar - ref_sbar).max() <= tol * max(1.0, np.abs(ref_sbar).max())


def test_prefill_window_unscaled_inputs_and_gqa():
    # large logits: rows whose first sub-tiles hold none of their keys must stay finite
    host = prefill_inputs(1, 8, 2, 513, 128, synth.BF16, 1.0, 320)
    t = [to_gpu(x, synth.BF16) for x in host]
    for W in (17, 200):
        assert_parity(from_gpu(plx.prefill(*t, window=W)), oracle.prefill(*host, window=W),
                      synth.BF16, f"W={W}")


@pytest.mark.parametrize("dtype,D,Hq,Hkv", [(synth.BF16, 128, 16, 8), (synth.F32, 64, 4, 4),
                                            (synth.BF16, 128, 6, 2)])
@pytest.mark.parametrize("W,splits", [(1, 0), (50, 0), (50, 3), (1000, 0), (1000, 1),
                                      (5000, 0)])
def test_decode_window_dense(dtype, D, Hq, Hkv, W, splits):
    q, r, k, v = decode_inputs(2, Hq, Hkv, D, [2000, 2000], dtype, S128, 330 + W)
    t = [to_gpu(x, dtype) for x in (q, r, k, v)]
    o = from_gpu(plx.decode(*t, window=W, num_splits=splits))
    assert_parity(o, oracle.decode(q, r, k, v, window=W), dtype, f"decode W={W}")
    o0 = from_gpu(plx.softmax_decode(t[0], t[2], t[3], window=W, num_splits=splits))
    assert_parity(o0, oracle.decode(q, None, k, v, window=W), dtype, f"softmax W={W}")


@pytest.mark.parametrize("splits", [0, 2])
def test_decode_window_packed_varlen(splits):
    lens = np.array([0, 1, 37, 300, 1024, 77])
    W = 64
    q, r, k, v = decode_inputs(len(lens), 16, 8, 128, lens, synth.BF16, S128, 340, packed=True)
    cu = np.concatenate([[0], np.cumsum(lens)])
    t = [to_gpu(x, synth.BF16) for x in (q, r, k, v)]
    cu_t = torch.from_numpy(cu.astype(np.int32)).cuda()
    o = from_gpu(plx.decode(*t, cu_seqlens_k=cu_t, kv_len=int(lens.max()), window=W,
                            num_splits=splits))
    ref = oracle.decode(q, r, k, v, seq_start=cu[:-1], seq_len=lens, window=W)
    assert np.all(o[0] == 0)
    assert_parity(o[1:], ref[1:], synth.BF16, "packed window")


@pytest.mark.parametrize("dtype,D", [(synth.BF16, 128), (synth.F32, 64)])
@pytest.mark.parametrize("L,W", [(130, 1), (130, 33), (300, 128), (300, 200), (257, 64)])
def test_backward_window(dtype, D, L, W):
    host = prefill_inputs(2, 4, 2, L, D, dtype, S128 if D == 128 else 1.0, 350 + L + W, True)
    t = [to_gpu(x, dtype) for x in host]
    vbar = torch.empty_like(t[0]) if L != 257 else None  # both backward variants
    o, lse, sbar = plx.prefill(*t[:4], return_stats=True, window=W, vbar_out=vbar)
    got = [from_gpu(g) for g in plx.prefill_backward(*t[:4], o, t[4], lse, sbar, window=W,
                                                      vbar=vbar)]
    ref = oracle.prefill_backward(*host, window=W)
    largest = max(np.abs(b).max() for b in ref)
    for name, a, b in zip(("dq", "dr", "dk", "dv"), got, ref):
        bmax = np.abs(b).max()
        err = np.abs(a - b).max() / (bmax if bmax > 0 else largest)
        assert err <= GTOL[dtype], f"L={L} W={W} {name}: {err:.3e}"


def test_window_full_size_prefill_rows_and_backward_unit():
    """B=8, Hq=16, Hkv=8, L=4096, D=128 bf16 with a 1024-key window: sampled forward rows
    and the complete gradients of one (sequence, KV head) unit."""
    spec = synth.prefill_spec(5)
    B, Hq, Hkv, L, D, W = spec.B, spec.Hq, spec.Hkv, spec.L, spec.D, 1024
    host = prefill_inputs(B, Hq, Hkv, L, D, synth.BF16, spec.scale, spec.seed, True)
    t = [to_gpu(x, synth.BF16) for x in host]
    o, lse, sbar = plx.prefill(*t[:4], return_stats=True, window=W)
    rows = np.array([[0, 0, 0], [0, 1, 1023], [3, 7, 1024], [7, 15, 4095], [5, 9, 2500]])
    ref = oracle.prefill(*host[:4], rows=rows, window=W)
    got = from_gpu(o[rows[:, 0], rows[:, 1], rows[:, 2]])
    assert np.abs(got - ref).max(axis=1).max() <= 1e-2 * np.abs(ref).max()
    grads = plx.prefill_backward(*t[:4], o, t[4], lse, sbar, window=W)
    b, hk = 6, 3
    gref = oracle.prefill_backward(*host, units=[[b, hk]], window=W)
    sel = [grads[0][b, 2 * hk:2 * hk + 2], grads[1][b, 2 * hk:2 * hk + 2], grads[2][b, hk],
           grads[3][b, hk]]
    for name, a, r in zip(("dq", "dr", "dk", "dv"), sel, gref):
        a = from_gpu(a)
        err = np.abs(a - r[0]).max() / np.abs(r[0]).max()
        assert err <= 1e-2, f"{name}: {err:.3e}"
