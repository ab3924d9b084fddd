"""Seeded random-shape sweep against the oracle.

Each case draws its shape, dtype, head group, layout (dense or packed, with empty
sequences), window, split count, scales and (last, so that the other draws do not
depend on it) an optional block-sparse mask from a fixed numpy generator, so the
cases are the same on every run. Decode cases run both entry points (Parallax and
the softmax baseline); prefill cases check o, lse, sbar and the four gradients.
Every group size takes the matrix-core kernels for bf16 at D = 128 (odd groups
with one query head per work item), the generic kernels otherwise. Bars as in
the other parity tests, for scaled and unscaled inputs alike: max-norm 1e-2 (bf16)
/ 1e-5 (fp32) for outputs, 1e-2 / 1e-4 for gradients.

Unscaled N(0,1) inputs at D = 128 give probe scores about sqrt(D) times those of
the scaled workloads, so they test the two numerical safeguards:
- the forward's probe pivot follows the running weighted mean of s (re-based
  exactly when it drifts), so the bf16 operand P o (s - pivot) and the factor
  (sbar - pivot) that multiplies the rounding of P stay small;
- the backward corrects delta = g.o and ubar from the sums of its own fp32 dz and
  ds (sweeping again where the correction is above bf16 rounding), so that dz,
  a difference of terms up to |1 + s - sbar| times larger than itself, does not
  carry the rounding of the forward's bf16 outputs.
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

GTOL = {synth.F32: 1e-4, synth.BF16: 1e-2}


def _draw_common(g):
    dtype = synth.BF16 if g.random() < 0.7 else synth.F32
    D = 128 if (dtype == synth.BF16 and g.random() < 0.75) else int(g.choice([64, 128]))
    G = int(g.choice([1, 2, 3, 4, 8]))
    Hkv = int(g.choice([1, 2, 3, 4]))
    scale = float(g.choice([1.0, 1.0 / math.sqrt(D)]))
    qk = float(g.choice([1.0 / math.sqrt(D), 0.3]))
    rk = float(g.choice([1.0, 0.5]))
    return dtype, D, G, Hkv, scale, qk, rk


@pytest.mark.parametrize("case", range(24))
def test_random_decode(case):
    g = np.random.default_rng(7100 + case)
    dtype, D, G, Hkv, scale, qk, rk = _draw_common(g)
    Hq = G * Hkv
    B = int(g.integers(1, 6))
    packed = bool(g.random() < 0.5)
    if packed:
        lens = g.integers(0, 2500, size=B)
        lens[int(g.integers(0, B))] = int(g.integers(1, 2500))  # at least one non-empty
    else:
        lens = np.full(B, int(g.integers(1, 2500)))
    W = int(g.choice([0, 0, 1, 17, 300, 5000]))
    splits = int(g.choice([0, 0, 1, 2, 7]))
    seed = 7200 + case
    q, r, k, v = (synth.normal(seed, tid, shp, scale, dtype) for tid, shp in (
        (synth.TID_Q, (B, Hq, D)), (synth.TID_R, (B, Hq, D)),
        (synth.TID_K, (int(lens.sum()), Hkv, D) if packed else (B, int(lens[0]), Hkv, D)),
        (synth.TID_V, (int(lens.sum()), Hkv, D) if packed else (B, int(lens[0]), Hkv, D))))
    t = [to_gpu(x, dtype) for x in (q, r, k, v)]
    kv_len = int(lens.max())
    mask = None
    if g.random() < 0.4:
        mask = (g.random((B, Hkv, -(-kv_len // 128))) < g.uniform(0.1, 0.7)).astype(np.uint8)
    what = (f"case {case}: B={B} Hq={Hq} Hkv={Hkv} D={D} lens={lens.tolist()} W={W} "
            f"splits={splits} mask={mask is not None}")
    mask_t = None if mask is None else torch.from_numpy(mask).cuda()
    if packed:
        cu = np.concatenate([[0], np.cumsum(lens)])
        cu_t = torch.from_numpy(cu.astype(np.int32)).cuda()
        kw = dict(cu_seqlens_k=cu_t, kv_len=kv_len, num_splits=splits, window=W,
                  block_mask=mask_t)
        okw = dict(seq_start=cu[:-1], seq_len=lens, window=W, block_mask=mask)
    else:
        kw = dict(num_splits=splits, window=W, block_mask=mask_t)
        okw = dict(window=W, block_mask=mask)
    live = lens > 0
    o = from_gpu(plx.decode(*t, qk, rk, **kw))
    ref = oracle.decode(q, r, k, v, qk_scale=qk, rk_scale=rk, **okw)
    assert np.all(o[~live] == 0), what
    assert_parity(o[live], ref[live], dtype, what)
    o0 = from_gpu(plx.softmax_decode(t[0], t[2], t[3], qk, **kw))
    ref0 = oracle.decode(q, None, k, v, qk_scale=qk, **okw)
    assert np.all(o0[~live] == 0), what
    assert_parity(o0[live], ref0[live], dtype, "softmax " + what)


def _check_grads(got, ref, dtype, what):
    tol = GTOL[dtype]
    largest = max(np.abs(b).max() for b in ref)
    for name, a, b in zip(("dq", "dr", "dk", "dv"), got, ref):
        bmax = np.abs(b).max()
        err = np.abs(a - b).max() / (bmax if bmax > 0 else largest)
        assert err <= tol, f"{what} {name}: {err:.3e}"


@pytest.mark.parametrize("case", range(16))
def test_random_prefill_and_backward(case):
    g = np.random.default_rng(7300 + case)
    dtype, D, G, Hkv, scale, qk, rk = _draw_common(g)
    G = min(G, 4)
    Hq = G * Hkv
    packed = bool(g.random() < 0.4)
    W = int(g.choice([0, 0, 1, 33, 200]))
    seed = 7400 + case
    what = f"case {case}: Hq={Hq} Hkv={Hkv} D={D} W={W}"

    def draw_mask(B, L):
        if g.random() >= 0.4:
            return None, None
        nb = -(-L // 128)
        m = (g.random((B, Hkv, nb, nb)) < g.uniform(0.1, 0.7)).astype(np.uint8)
        return m, torch.from_numpy(m).cuda()

    if packed:
        lens = g.integers(0, 400, size=int(g.integers(1, 5)))
        lens[0] = max(int(lens[0]), 1)
        T = int(lens.sum())
        cu = np.concatenate([[0], np.cumsum(lens)])
        q, r, k, v = (synth.normal(seed, tid, (T, H, D), scale, dtype) for tid, H in (
            (synth.TID_Q, Hq), (synth.TID_R, Hq), (synth.TID_K, Hkv), (synth.TID_V, Hkv)))
        do = synth.normal(seed, synth.TID_DO, (T, Hq, D), 1.0, dtype)
        t = [to_gpu(x, dtype) for x in (q, r, k, v, do)]
        cu_t = torch.from_numpy(cu.astype(np.int32)).cuda()
        m, mt = draw_mask(len(lens), int(lens.max()))
        what += f" lens={lens.tolist()} mask={m is not None}"
        o, lse, sbar = plx.prefill_varlen(*t[:4], cu_t, None, qk, rk, return_stats=True, window=W,
                                          block_mask=mt)
        ref, ref_lse, ref_sbar = oracle.prefill_varlen(q, r, k, v, cu, qk_scale=qk, rk_scale=rk,
                                                       window=W, stats=True, block_mask=m)
        grads = plx.prefill_varlen_backward(*t[:4], o, t[4], lse, sbar, cu_t, None, qk, rk,
                                            window=W, block_mask=mt)
        ref_g = oracle.prefill_varlen_backward(q, r, k, v, do, cu, qk_scale=qk, rk_scale=rk,
                                               window=W, block_mask=m)
    else:
        B = int(g.integers(1, 4))
        L = int(g.integers(1, 400))
        q, r, k, v = (synth.normal(seed, tid, (B, H, L, D), scale, dtype) for tid, H in (
            (synth.TID_Q, Hq), (synth.TID_R, Hq), (synth.TID_K, Hkv), (synth.TID_V, Hkv)))
        do = synth.normal(seed, synth.TID_DO, (B, Hq, L, D), 1.0, dtype)
        t = [to_gpu(x, dtype) for x in (q, r, k, v, do)]
        m, mt = draw_mask(B, L)
        what += f" B={B} L={L} mask={m is not None}"
        o, lse, sbar = plx.prefill(*t[:4], qk, rk, return_stats=True, window=W, block_mask=mt)
        ref, ref_lse, ref_sbar = oracle.prefill(q, r, k, v, qk_scale=qk, rk_scale=rk, window=W,
                                                stats=True, block_mask=m)
        grads = plx.prefill_backward(*t[:4], o, t[4], lse, sbar, qk, rk, window=W, block_mask=mt)
        ref_g = oracle.prefill_backward(q, r, k, v, do, qk_scale=qk, rk_scale=rk, window=W,
                                        block_mask=m)
    assert_parity(from_gpu(o), ref, dtype, what)
    lse = lse.cpu().numpy().astype(np.float64)
    assert np.abs(lse - ref_lse).max() <= 1e-4 * max(1.0, np.abs(ref_lse).max()), what
    stol = 1e-4 if dtype == synth.F32 else 1e-2
    sbar = sbar.cpu().numpy().astype(np.float64)
    assert np.abs(sbar - ref_sbar).max() <= stol * max(1.0, np.abs(ref_sbar).max()), what
    _check_grads([from_gpu(x) for x in grads], ref_g, dtype, what)


@pytest.mark.parametrize("splits", [0, 1, 2, 7])
def test_unscaled_group8_masked_decode(splits):
    """The decode the fixed first-key pivot served worst (it measured 1.03e-2
    under every split plan): unscaled bf16 inputs, eight query heads per KV head,
    qk_scale 0.3, rk_scale 0.5, a packed batch of four, and a block mask keeping
    about a fifth of the blocks. With the drifting pivot it is held to half the
    bf16 bar."""
    g = np.random.default_rng(7102)
    dtype, D, G, Hkv, scale, qk, rk = _draw_common(g)
    assert (dtype, D, G, Hkv, scale, qk, rk) == (synth.BF16, 128, 8, 1, 1.0, 0.3, 0.5)
    Hq, B = G * Hkv, int(g.integers(1, 6))
    assert bool(g.random() < 0.5)  # packed
    lens = g.integers(0, 2500, size=B)
    lens[int(g.integers(0, B))] = int(g.integers(1, 2500))
    g.choice([0, 0, 1, 17, 300, 5000]), g.choice([0, 0, 1, 2, 7])  # window 0, split draw
    kv_len = int(lens.max())
    assert g.random() < 0.4
    mask = (g.random((B, Hkv, -(-kv_len // 128))) < g.uniform(0.1, 0.7)).astype(np.uint8)
    seed = 7202
    T = int(lens.sum())
    q, r, k, v = (synth.normal(seed, tid, shp, scale, dtype) for tid, shp in (
        (synth.TID_Q, (B, Hq, D)), (synth.TID_R, (B, Hq, D)),
        (synth.TID_K, (T, Hkv, D)), (synth.TID_V, (T, Hkv, D))))
    cu = np.concatenate([[0], np.cumsum(lens)])
    t = [to_gpu(x, dtype) for x in (q, r, k, v)]
    o = from_gpu(plx.decode(*t, qk, rk, cu_seqlens_k=torch.from_numpy(cu.astype(np.int32)).cuda(),
                            kv_len=kv_len, num_splits=splits, block_mask=torch.from_numpy(mask).cuda()))
    ref = oracle.decode(q, r, k, v, qk_scale=qk, rk_scale=rk, seq_start=cu[:-1], seq_len=lens,
                        block_mask=mask)
    live = lens > 0
    assert_parity(o[live], ref[live], dtype, f"lens={lens.tolist()} splits={splits}", tol=5e-3)
