"""GPU parity of block-sparse masks (decode, prefill, varlen, backward) against the oracle.

Masks cover blocks of 128 positions, one per (sequence, KV head); a query always
sees its own block. The oracle takes the same mask bytes (``block=128``). Same
bars as the unmasked tests: max-norm 1e-2 (bf16) / 1e-5 (fp32) for outputs,
1e-2 / 1e-4 for gradients. An all-ones mask must reproduce the unmasked call bit
for bit (the mask only decides which tiles are streamed).
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
BS = 128


def nblocks(n):
    return -(-n // BS)


def mask_gpu(m):
    return torch.from_numpy(np.ascontiguousarray(m, dtype=np.uint8)).cuda()


# ---------------------------------------------------------------- decode
@pytest.mark.parametrize("dtype,D,Hq,Hkv", [(synth.BF16, 128, 16, 8), (synth.BF16, 128, 8, 1),
                                            (synth.BF16, 128, 6, 2), (synth.F32, 64, 4, 2)])
@pytest.mark.parametrize("L,density,splits,W", [(1000, 0.4, 0, 0), (4100, 0.25, 0, 0),
                                               (4100, 0.0, 3, 0), (4100, 0.5, 1, 0),
                                               (3000, 0.5, 0, 1500), (300, 0.5, 2, 200)])
def test_decode_block_mask_dense(dtype, D, Hq, Hkv, L, density, splits, W):
    B = 3
    seed = 800 + L + int(density * 10) + splits + W
    host = decode_inputs(B, Hq, Hkv, D, [L] * B, dtype, S128 if D == 128 else 1.0, seed)
    t = [to_gpu(x, dtype) for x in host]
    m = synth.block_mask(seed, (B, Hkv, nblocks(L)), density)
    what = f"decode L={L} density={density} splits={splits} W={W} G={Hq // Hkv}"
    o = from_gpu(plx.decode(*t, num_splits=splits, window=W, block_mask=mask_gpu(m)))
    ref = oracle.decode(*host, window=W, block_mask=m)
    assert_parity(o, ref, dtype, what)
    o0 = from_gpu(plx.softmax_decode(t[0], t[2], t[3], num_splits=splits, window=W,
                                     block_mask=mask_gpu(m)))
    ref0 = oracle.decode(host[0], None, host[2], host[3], window=W, block_mask=m)
    assert_parity(o0, ref0, dtype, "softmax " + what)


@pytest.mark.parametrize("splits", [0, 2])
def test_decode_block_mask_packed(splits):
    dtype, D, Hq, Hkv = synth.BF16, 128, 16, 8
    lens = np.array([0, 1, 129, 2000, 4096, 700, 5000])
    B = len(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    host = decode_inputs(B, Hq, Hkv, D, lens, dtype, S128, 810 + splits, packed=True)
    t = [to_gpu(x, dtype) for x in host]
    kv_len = int(lens.max())
    m = synth.block_mask(811, (B, Hkv, nblocks(kv_len)), 0.35)
    cu_t = torch.from_numpy(cu).cuda()
    o = from_gpu(plx.decode(*t, cu_seqlens_k=cu_t, kv_len=kv_len, num_splits=splits,
                            block_mask=mask_gpu(m)))
    ref = oracle.decode(*host, seq_start=cu[:-1], seq_len=lens, block_mask=m)
    live = lens > 0
    assert np.all(o[~live] == 0)
    assert_parity(o[live], ref[live], dtype, f"packed decode splits={splits}")


def test_decode_all_ones_mask_is_bitwise_the_unmasked_call():
    B, Hq, Hkv, D, L = 2, 16, 8, 128, 5000
    host = decode_inputs(B, Hq, Hkv, D, [L] * B, synth.BF16, S128, 820)
    t = [to_gpu(x, synth.BF16) for x in host]
    ones = torch.ones((B, Hkv, nblocks(L)), dtype=torch.uint8, device="cuda")
    for splits in (0, 1, 5):
        a = plx.decode(*t, num_splits=splits)
        b = plx.decode(*t, num_splits=splits, block_mask=ones)
        assert torch.equal(a, b), splits


def test_decode_partial_and_merge_with_mask():
    B, Hq, Hkv, D, L = 2, 8, 4, 128, 3000
    host = decode_inputs(B, Hq, Hkv, D, [L] * B, synth.BF16, S128, 830)
    t = [to_gpu(x, synth.BF16) for x in host]
    m = synth.block_mask(830, (B, Hkv, nblocks(L)), 0.3)
    recs, n = plx.decode_partial(*t, num_splits=6, block_mask=mask_gpu(m))
    o = from_gpu(plx.decode_merge(recs))
    assert_parity(o, oracle.decode(*host, block_mask=m), synth.BF16, "partial + merge")


# ---------------------------------------------------------------- prefill
def prefill_inputs(B, Hq, Hkv, L, D, dtype, scale, seed):
    q = synth.normal(seed, synth.TID_Q, (B, Hq, L, D), scale, dtype)
    r = synth.normal(seed, synth.TID_R, (B, Hq, L, D), scale, dtype)
    k = synth.normal(seed, synth.TID_K, (B, Hkv, L, D), scale, dtype)
    v = synth.normal(seed, synth.TID_V, (B, Hkv, L, D), scale, dtype)
    do = synth.normal(seed, synth.TID_DO, (B, Hq, L, D), 1.0, dtype)
    return q, r, k, v, do


def check_stats(lse, sbar, ref_lse, ref_sbar, dtype):
    lse = lse.cpu().numpy().astype(np.float64)
    assert np.abs(lse - ref_lse).max() <= 1e-4 * max(1.0, np.abs(ref_lse).max())
    tol = 1e-4 if dtype == synth.F32 else 1e-2
    sbar = sbar.cpu().numpy().astype(np.float64)
    assert np.abs(sbar - ref_sbar).max() <= tol * max(1.0, np.abs(ref_sbar).max())


def check_grads(got, ref, dtype, what):
    # a gradient that is exactly zero (every row sees one key: dr = 0) is measured
    # against the largest of the four
    largest = max(np.abs(b).max() for b in ref)
    for name, a, b in zip(("dq", "dr", "dk", "dv"), got, ref):
        bmax = np.abs(b).max()
        err = np.abs(from_gpu(a) - b).max() / (bmax if bmax > 0 else largest)
        assert err <= GTOL[dtype], f"{what} {name}: {err:.3e}"


@pytest.mark.parametrize("dtype,D,Hq,Hkv", [(synth.BF16, 128, 4, 2), (synth.BF16, 128, 3, 3),
                                            (synth.BF16, 128, 8, 2), (synth.F32, 64, 4, 2)])
@pytest.mark.parametrize("L,density,W", [(700, 0.4, 0), (700, 0.0, 0), (1030, 0.6, 0),
                                         (700, 0.5, 300)])
def test_prefill_and_backward_block_mask(dtype, D, Hq, Hkv, L, density, W):
    B = 2
    seed = 840 + L + int(10 * density) + W + Hq
    q, r, k, v, do = prefill_inputs(B, Hq, Hkv, L, D, dtype, S128 if D == 128 else 1.0, seed)
    m = synth.block_mask(seed, (B, Hkv, nblocks(L), nblocks(L)), density)
    mg = mask_gpu(m)
    t = [to_gpu(x, dtype) for x in (q, r, k, v, do)]
    what = f"L={L} density={density} W={W} G={Hq // Hkv} D={D}"
    o, lse, sbar = plx.prefill(*t[:4], return_stats=True, window=W, block_mask=mg)
    ref, ref_lse, ref_sbar = oracle.prefill(q, r, k, v, stats=True, window=W, block_mask=m)
    assert_parity(from_gpu(o), ref, dtype, "prefill " + what)
    check_stats(lse, sbar, ref_lse, ref_sbar, dtype)
    ref_g = oracle.prefill_backward(q, r, k, v, do, window=W, block_mask=m)
    for vbar in (False, True):
        vb = None
        if vbar:
            vb = torch.empty_like(t[0])
            plx.prefill(*t[:4], window=W, block_mask=mg, vbar_out=vb)
        g = plx.prefill_backward(*t[:4], o, t[4], lse, sbar, window=W, vbar=vb, block_mask=mg)
        check_grads(g, ref_g, dtype, f"backward vbar={vbar} " + what)


def test_prefill_all_ones_mask_is_bitwise_the_unmasked_call():
    q, r, k, v, do = prefill_inputs(1, 4, 2, 900, 128, synth.BF16, S128, 850)
    t = [to_gpu(x, synth.BF16) for x in (q, r, k, v, do)]
    ones = torch.ones((1, 2, nblocks(900), nblocks(900)), dtype=torch.uint8, device="cuda")
    a = plx.prefill(*t[:4], return_stats=True)
    b = plx.prefill(*t[:4], return_stats=True, block_mask=ones)
    assert all(torch.equal(x, y) for x, y in zip(a, b))
    ga = plx.prefill_backward(*t[:4], a[0], t[4], a[1], a[2])
    gb = plx.prefill_backward(*t[:4], a[0], t[4], a[1], a[2], block_mask=ones)
    assert all(torch.equal(x, y) for x, y in zip(ga, gb))


def test_parallax_func_autograd_with_mask():
    q, r, k, v, do = prefill_inputs(1, 4, 2, 520, 128, synth.BF16, S128, 860)
    m = synth.block_mask(860, (1, 2, nblocks(520), nblocks(520)), 0.5)
    t = [to_gpu(x, synth.BF16).requires_grad_(True) for x in (q, r, k, v)]
    o = plx.parallax_func(*t, block_mask=mask_gpu(m))
    o.backward(to_gpu(do, synth.BF16))
    assert_parity(from_gpu(o.detach()), oracle.prefill(q, r, k, v, block_mask=m), synth.BF16)
    check_grads([x.grad for x in t], oracle.prefill_backward(q, r, k, v, do, block_mask=m),
                synth.BF16, "autograd")


@pytest.mark.parametrize("dtype,D", [(synth.BF16, 128), (synth.F32, 64)])
def test_varlen_prefill_and_backward_block_mask(dtype, D):
    lens = np.array([300, 0, 1, 650, 129])
    cu = np.concatenate([[0], np.cumsum(lens)])
    T, Hq, Hkv = int(cu[-1]), 4, 2
    seed = 870 + D
    scale = S128 if D == 128 else 1.0
    q, r = (synth.normal(seed, tid, (T, Hq, D), scale, dtype) for tid in (synth.TID_Q, synth.TID_R))
    k, v = (synth.normal(seed, tid, (T, Hkv, D), scale, dtype) for tid in (synth.TID_K, synth.TID_V))
    do = synth.normal(seed, synth.TID_DO, (T, Hq, D), 1.0, dtype)
    nb = nblocks(int(lens.max()))
    m = synth.block_mask(seed, (len(lens), Hkv, nb, nb), 0.4)
    mg = mask_gpu(m)
    t = [to_gpu(x, dtype) for x in (q, r, k, v, do)]
    cu_t = torch.from_numpy(cu.astype(np.int32)).cuda()
    o, lse, sbar = plx.prefill_varlen(*t[:4], cu_t, None, return_stats=True, block_mask=mg)
    ref, ref_lse, ref_sbar = oracle.prefill_varlen(q, r, k, v, cu, stats=True, block_mask=m)
    assert_parity(from_gpu(o), ref, dtype, "varlen prefill")
    check_stats(lse, sbar, ref_lse, ref_sbar, dtype)
    g = plx.prefill_varlen_backward(*t[:4], o, t[4], lse, sbar, cu_t, None, block_mask=mg)
    check_grads(g, oracle.prefill_varlen_backward(q, r, k, v, do, cu, block_mask=m), dtype,
                "varlen backward")


def test_long_prefill_sparse_mask_sampled_rows():
    """B=1, L=4096 with a sparse mask at the full workload's head shape: sampled rows
    of every query head against the oracle, computed row by row."""
    B, Hq, Hkv, L, D = 1, 16, 8, 4096, 128
    q, r, k, v, _ = prefill_inputs(B, Hq, Hkv, L, D, synth.BF16, S128, 880)
    m = synth.block_mask(880, (B, Hkv, 32, 32), 0.2)
    t = [to_gpu(x, synth.BF16) for x in (q, r, k, v)]
    o = from_gpu(plx.prefill(*t, block_mask=mask_gpu(m)))
    g = np.random.default_rng(880)
    rows = np.stack([np.zeros(64, dtype=np.int64), g.integers(0, Hq, 64),
                     g.integers(0, L, 64)], axis=1)
    ref = oracle.prefill(q, r, k, v, rows=rows, block_mask=m)
    got = o[rows[:, 0], rows[:, 1], rows[:, 2]]
    assert_parity(got, ref, synth.BF16, "sampled rows")


@pytest.mark.parametrize("splits", [0, 1])
def test_decode_block_mask_longer_than_one_staging(splits):
    """600,000 keys: more than the 4096 blocks a workgroup stages, so each split walks
    the visible blocks of its own key range (a forced single split becomes two)."""
    B, Hq, Hkv, D, L = 1, 2, 1, 128, 600_000
    host = decode_inputs(B, Hq, Hkv, D, [L], synth.BF16, S128, 890 + splits)
    t = [to_gpu(x, synth.BF16) for x in host]
    m = synth.block_mask(890, (B, Hkv, nblocks(L)), 0.3)
    o = from_gpu(plx.decode(*t, num_splits=splits, block_mask=mask_gpu(m)))
    assert_parity(o, oracle.decode(*host, block_mask=m), synth.BF16, f"L={L} splits={splits}")


@pytest.mark.parametrize("L,W", [(128, 0), (129, 0), (300, 1), (300, 129), (400, 64)])
def test_prefill_block_mask_small_and_windowed(L, W):
    q, r, k, v, do = prefill_inputs(1, 4, 2, L, 128, synth.BF16, S128, 900 + L + W)
    m = synth.block_mask(900 + W, (1, 2, nblocks(L), nblocks(L)), 0.3)
    t = [to_gpu(x, synth.BF16) for x in (q, r, k, v, do)]
    o, lse, sbar = plx.prefill(*t[:4], return_stats=True, window=W, block_mask=mask_gpu(m))
    ref, ref_lse, ref_sbar = oracle.prefill(q, r, k, v, stats=True, window=W, block_mask=m)
    assert_parity(from_gpu(o), ref, synth.BF16, f"L={L} W={W}")
    check_stats(lse, sbar, ref_lse, ref_sbar, synth.BF16)
    g = plx.prefill_backward(*t[:4], o, t[4], lse, sbar, window=W, block_mask=mask_gpu(m))
    check_grads(g, oracle.prefill_backward(q, r, k, v, do, window=W, block_mask=m), synth.BF16,
                f"backward L={L} W={W}")
