"""GPU parity of the packed-sequence (varlen) prefill and its backward against
the oracle (each sequence an independent causal prefill)."""
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
GTOL = {synth.F32: 1e-4, synth.BF16: 1e-2}


def packed_inputs(lens, Hq, Hkv, D, dtype, scale, seed):
    T = int(np.sum(lens))
    q = synth.normal(seed, synth.TID_Q, (T, Hq, D), scale, dtype)
    r = synth.normal(seed, synth.TID_R, (T, Hq, D), scale, dtype)
    k = synth.normal(seed, synth.TID_K, (T, Hkv, D), scale, dtype)
    v = synth.normal(seed, synth.TID_V, (T, Hkv, D), scale, dtype)
    do = synth.normal(seed, synth.TID_DO, (T, Hq, D), 1.0, dtype)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return (q, r, k, v, do), cu


def check_grads(got, ref, dtype, what):
    largest = max(np.abs(b).max() for b in ref)
    for name, a, b in zip(("dq", "dr", "dk", "dv"), got, ref):
        bmax = np.abs(b).max()
        err = np.abs(a - b).max() / (bmax if bmax > 0 else largest)
        assert err <= GTOL[dtype], f"{what} {name}: {err:.3e}"


@pytest.mark.parametrize("dtype,D", [(synth.BF16, 128), (synth.F32, 64), (synth.BF16, 64)])
@pytest.mark.parametrize("W", [0, 50])
def test_varlen_forward_and_backward(dtype, D, W):
    lens = [63, 0, 1, 200, 64, 513, 65]
    host, cu = packed_inputs(lens, 4, 2, D, dtype, S128 if D == 128 else 1.0, 400 + D + W)
    t = [to_gpu(x, dtype) for x in host]
    cu_t = torch.from_numpy(cu.astype(np.int32)).cuda()
    o, lse, sbar = plx.prefill_varlen(*t[:4], cu_t, return_stats=True, window=W)
    ref, ref_lse, ref_sbar = oracle.prefill_varlen(*host[:4], cu, stats=True, window=W)
    assert_parity(from_gpu(o), ref, dtype, f"varlen W={W}")
    assert np.abs(lse.cpu().numpy() - ref_lse).max() <= 1e-4 * np.abs(ref_lse).max()
    tol = 1e-4 if dtype == synth.F32 else 1e-2
    assert np.abs(sbar.cpu().numpy() - ref_sbar).max() <= tol * max(1.0, np.abs(ref_sbar).max())
    got = plx.prefill_varlen_backward(*t[:4], o, t[4], lse, sbar, cu_t, window=W)
    ref_g = oracle.prefill_varlen_backward(*host, cu, window=W)
    check_grads([from_gpu(g) for g in got], ref_g, dtype, f"varlen W={W}")
    # and with the forward's softmax readout in place of the first sweep
    vbar = torch.empty_like(t[0])
    plx.prefill_varlen(*t[:4], cu_t, window=W, vbar_out=vbar)
    got = plx.prefill_varlen_backward(*t[:4], o, t[4], lse, sbar, cu_t, window=W, vbar=vbar)
    check_grads([from_gpu(g) for g in got], ref_g, dtype, f"varlen vbar W={W}")


@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (8, 2), (3, 1)])
def test_varlen_groups(Hq, Hkv):
    lens = [130, 7, 300]
    host, cu = packed_inputs(lens, Hq, Hkv, 128, synth.BF16, S128, 420 + Hq)
    t = [to_gpu(x, synth.BF16) for x in host]
    cu_t = torch.from_numpy(cu.astype(np.int32)).cuda()
    o, lse, sbar = plx.prefill_varlen(*t[:4], cu_t, return_stats=True)
    assert_parity(from_gpu(o), oracle.prefill_varlen(*host[:4], cu), synth.BF16, "groups")
    got = plx.prefill_varlen_backward(*t[:4], o, t[4], lse, sbar, cu_t)
    check_grads([from_gpu(g) for g in got], oracle.prefill_varlen_backward(*host, cu),
                synth.BF16, f"Hq={Hq} Hkv={Hkv}")


def test_varlen_matches_dense_batch_and_autograd_entry_point():
    # equal lengths: the packed call equals the dense call on the same values
    B, Hq, Hkv, L, D = 3, 4, 2, 150, 128
    host, cu = packed_inputs([L] * B, Hq, Hkv, D, synth.BF16, S128, 430)
    t = [to_gpu(x, synth.BF16) for x in host]
    cu_t = torch.from_numpy(cu.astype(np.int32)).cuda()
    dense = [x.view(B, L, x.shape[1], D).transpose(1, 2).contiguous() for x in t]
    o_d = plx.prefill(*dense[:4])
    o_p = plx.prefill_varlen(*t[:4], cu_t, L)
    assert torch.equal(o_p.view(B, L, Hq, D).transpose(1, 2), o_d)
    leaves = [x.clone().requires_grad_(True) for x in t[:4]]
    out = plx.parallax_varlen_func(*leaves, cu_t)
    out.backward(t[4])
    vbar = torch.empty_like(t[0])
    o, lse, sbar = plx.prefill_varlen(*t[:4], cu_t, return_stats=True, vbar_out=vbar)
    ref = plx.prefill_varlen_backward(*t[:4], o, t[4], lse, sbar, cu_t, vbar=vbar)
    for leaf, g in zip(leaves, ref):
        assert torch.equal(leaf.grad, g)


def test_varlen_training_sized_batch_sampled():
    """16 sequences of U[256, 4096] tokens (Hq16 Hkv8 D128 bf16): full forward output and
    the gradients of three sequences against the oracle."""
    spec = synth.prefill_varlen_spec()
    host, cu = packed_inputs(spec.lengths, spec.Hq, spec.Hkv, spec.D, spec.dtype, spec.scale,
                             spec.seed)
    t = [to_gpu(x, synth.BF16) for x in host]
    cu_t = torch.from_numpy(cu.astype(np.int32)).cuda()
    o, lse, sbar = plx.prefill_varlen(*t[:4], cu_t, return_stats=True)
    got = plx.prefill_varlen_backward(*t[:4], o, t[4], lse, sbar, cu_t)
    for b in (0, 7, 15):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        sub = [np.ascontiguousarray(x[s0:s1]) for x in host]
        scu = np.array([0, s1 - s0])
        ref_o = oracle.prefill_varlen(*sub[:4], scu)
        assert_parity(from_gpu(o[s0:s1]), ref_o, synth.BF16, f"seq {b}")
        check_grads([from_gpu(g[s0:s1]) for g in got], oracle.prefill_varlen_backward(*sub, scu),
                    synth.BF16, f"seq {b}")
