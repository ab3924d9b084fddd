"""parallax_decode_noalloc (the decode entry point that allocates nothing: its split
records live in the library's own device array) against parallax_decode with a caller
workspace, both called through the C ABI on the same inputs: the outputs must agree bit
for bit (same kernels and plan), on two calls in a row, the second with a smaller input
and a different plan, and the shared array must not carry anything between them."""
import ctypes
import math

import numpy as np
import pytest
import torch

import oracle
import parameterized_local_linear_amd as plx
import synth
from gpu_util import assert_parity, from_gpu, to_gpu

pytestmark = pytest.mark.gpu


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _both(q, r, k, v, cu, B, Hq, Hkv, D, kv_len, splits):
    """o from parallax_decode (torch workspace) and from parallax_decode_noalloc."""
    L = plx.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    qk = 1.0 / math.sqrt(D)
    need = plx.decode_workspace_bytes(B, Hq, Hkv, D, kv_len, plx.PLX_BF16, splits)
    assert 0 < need <= plx.NOALLOC_SCRATCH_BYTES
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    o_ref = torch.empty((B, Hq, D), dtype=torch.bfloat16, device="cuda")
    o_new = torch.full((B, Hq, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    st = L.parallax_decode(_ptr(q), _ptr(r), _ptr(k), _ptr(v), _ptr(o_ref), _ptr(cu), B, Hq, Hkv,
                           D, kv_len, 0, None, qk, 1.0, plx.PLX_BF16, splits, _ptr(ws), need, stream)
    assert st == 0, st
    st = L.parallax_decode_noalloc(_ptr(q), _ptr(r), _ptr(k), _ptr(v), _ptr(o_new), _ptr(cu), B,
                                   Hq, Hkv, D, kv_len, 0, None, qk, 1.0, plx.PLX_BF16, splits,
                                   stream)
    assert st == 0, st
    torch.cuda.synchronize()
    return o_ref, o_new


def test_noalloc_decode_matches_workspace_decode_on_two_calls():
    Hq, Hkv, D = 16, 8, 128
    # call 1: a packed batch of 32 mixed lengths (the stream-K plan; its records fill
    # ~2.6 MB of the library's array)
    g = np.random.default_rng(900)
    lens = g.integers(100, 3001, size=32)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(lens.sum())
    s = 1.0 / math.sqrt(D)
    q, r = (synth.normal(901, tid, (32, Hq, D), s, synth.BF16) for tid in (0, 1))
    k, v = (synth.normal(901, tid, (T, Hkv, D), s, synth.BF16) for tid in (2, 3))
    t = [to_gpu(x, synth.BF16) for x in (q, r, k, v)]
    cu_t = torch.from_numpy(cu).cuda()
    o_ref, o_new = _both(*t, cu_t, 32, Hq, Hkv, D, int(lens.max()), 0)
    assert torch.equal(o_new, o_ref)
    ref = oracle.decode(q, r, k, v, seq_start=cu[:-1].astype(np.int64), seq_len=lens)
    assert_parity(from_gpu(o_new), ref, synth.BF16, "noalloc, packed batch")

    # call 2: a smaller dense batch with seven splits (fewer records, other layout)
    B, L = 2, 3000
    q2, r2 = (synth.normal(902, tid, (B, Hq, D), s, synth.BF16) for tid in (0, 1))
    k2, v2 = (synth.normal(902, tid, (B, L, Hkv, D), s, synth.BF16) for tid in (2, 3))
    t2 = [to_gpu(x, synth.BF16) for x in (q2, r2, k2, v2)]
    o_ref2, o_new2 = _both(*t2, None, B, Hq, Hkv, D, L, 7)
    assert torch.equal(o_new2, o_ref2)
    assert_parity(from_gpu(o_new2), oracle.decode(q2, r2, k2, v2), synth.BF16, "noalloc, dense")


def test_noalloc_decode_python_binding_and_fused_plan():
    # one short sequence runs as a single fused split (no records at all)
    Hq, Hkv, D, L = 4, 2, 128, 300
    s = 1.0 / math.sqrt(D)
    q, r = (synth.normal(903, tid, (1, Hq, D), s, synth.BF16) for tid in (0, 1))
    k, v = (synth.normal(903, tid, (1, L, Hkv, D), s, synth.BF16) for tid in (2, 3))
    t = [to_gpu(x, synth.BF16) for x in (q, r, k, v)]
    assert torch.equal(plx.decode_noalloc(*t), plx.decode(*t))
    assert torch.equal(plx.decode_noalloc(*t, num_splits=2), plx.decode(*t, num_splits=2))


def test_noalloc_decode_generic_kernel_window_and_block_mask():
    # fp32 at D = 64 runs the generic kernel; a window moves every split's range
    B, Hq, Hkv, D, L = 2, 4, 2, 64, 700
    q, r = (synth.normal(904, tid, (B, Hq, D), 1.0, synth.F32) for tid in (0, 1))
    k, v = (synth.normal(904, tid, (B, L, Hkv, D), 1.0, synth.F32) for tid in (2, 3))
    t = [to_gpu(x, synth.F32) for x in (q, r, k, v)]
    for splits in (3, 0):
        a = plx.decode_noalloc(*t, num_splits=splits, window=100)
        assert torch.equal(a, plx.decode(*t, num_splits=splits, window=100))
    assert_parity(from_gpu(a), oracle.decode(q, r, k, v, window=100), synth.F32, "noalloc, fp32 window")

    # bf16 with a seeded block mask over 128-key blocks, then a smaller unmasked call
    B, Hq, Hkv, D, L = 2, 16, 8, 128, 1500
    s = 1.0 / math.sqrt(D)
    q, r = (synth.normal(905, tid, (B, Hq, D), s, synth.BF16) for tid in (0, 1))
    k, v = (synth.normal(905, tid, (B, L, Hkv, D), s, synth.BF16) for tid in (2, 3))
    t = [to_gpu(x, synth.BF16) for x in (q, r, k, v)]
    nb = -(-L // plx.MASK_BLOCK)
    mask = (np.random.default_rng(905).random((B, Hkv, nb)) < 0.5).astype(np.uint8)
    mask_t = torch.from_numpy(mask).cuda()
    a = plx.decode_noalloc(*t, num_splits=4, block_mask=mask_t)
    assert torch.equal(a, plx.decode(*t, num_splits=4, block_mask=mask_t))
    assert_parity(from_gpu(a), oracle.decode(q, r, k, v, block_mask=mask), synth.BF16,
                  "noalloc, block mask")
    t_small = [(x[:1] if x.dim() == 3 else x[:1, :700]).contiguous() for x in t]
    assert torch.equal(plx.decode_noalloc(*t_small, num_splits=2), plx.decode(*t_small, num_splits=2))


def test_noalloc_refuses_by_the_plan_it_runs():
    """The array must hold the records of the plan the call runs, not the bound over both
    plans that parallax_decode_workspace_bytes gives: a dense batch whose own split records
    fit runs, though a packed cache of the same sizes would take the stream-K plan, whose
    records (Hq (4 CUs / Hkv + B - 1) of them) do not fit and are refused before anything
    runs."""
    B, Hq, Hkv, D, L = 64, 16, 2, 128, 600
    assert plx.decode_workspace_bytes(B, Hq, Hkv, D, L, plx.PLX_BF16) > plx.NOALLOC_SCRATCH_BYTES
    s = 1.0 / math.sqrt(D)
    q, r = (synth.normal(906, tid, (B, Hq, D), s, synth.BF16) for tid in (0, 1))
    k, v = (synth.normal(906, tid, (B, L, Hkv, D), s, synth.BF16) for tid in (2, 3))
    t = [to_gpu(x, synth.BF16) for x in (q, r, k, v)]
    splits = plx.decode_num_splits(B, Hq, Hkv, D, L, plx.PLX_BF16)
    assert B * Hq * splits * (2 * D + 4) * 4 <= plx.NOALLOC_SCRATCH_BYTES
    a = plx.decode_noalloc(*t)
    assert torch.equal(a, plx.decode(*t))
    assert_parity(from_gpu(a), oracle.decode(q, r, k, v), synth.BF16, "noalloc, dense G=8")
    cu = torch.arange(0, (B + 1) * L, L, dtype=torch.int32, device="cuda")
    kp, vp = (x.reshape(B * L, Hkv, D) for x in t[2:])
    with pytest.raises(plx.ParallaxError) as e:
        plx.decode_noalloc(t[0], t[1], kp, vp, cu_seqlens_k=cu, kv_len=L)
    assert e.value.status == 3
