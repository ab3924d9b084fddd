"""GPU parity of parallax_prefill_backward (dq, dr, dk, dv) against the
double oracle's gradients.

The backward takes the GPU forward's own o, lse and sbar (as in training);
the oracle recomputes everything in double from q, r, k, v and d_o. The bar
is the pages' ("Helion" section of the PyPI README: output and all four
gradients within 1e-2 max-norm relative error of an fp32 reference) for bf16
inputs, taken as max |g - g_ref| <= 1e-2 max |g_ref| per gradient; fp32
inputs get 1e-4 (fp32 sums over up to a few hundred keys, each gradient a
difference of terms of the size of the result).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import parameterized_local_linear_amd as plx
import synth
from gpu_util import from_gpu, to_gpu

pytestmark = pytest.mark.gpu

S128 = 1.0 / math.sqrt(128.0)
GTOL = {synth.F32: 1e-4, synth.BF16: 1e-2}


def inputs(B, Hq, Hkv, L, D, dtype, scale, seed):
    q = synth.normal(seed, synth.TID_Q, (B, Hq, L, D), scale, dtype)
    r = synth.normal(seed, synth.TID_R, (B, Hq, L, D), scale, dtype)
    k = synth.normal(seed, synth.TID_K, (B, Hkv, L, D), scale, dtype)
    v = synth.normal(seed, synth.TID_V, (B, Hkv, L, D), scale, dtype)
    do = synth.normal(seed, synth.TID_DO, (B, Hq, L, D), 1.0, dtype)
    return q, r, k, v, do


def gpu_backward(host, dtype, qk_scale=None, rk_scale=1.0, keep_on_gpu=False, use_vbar=False):
    q, r, k, v, do = (to_gpu(x, dtype) for x in host)
    vbar = torch.empty_like(q) if use_vbar else None
    o, lse, sbar = plx.prefill(q, r, k, v, qk_scale, rk_scale, return_stats=True, vbar_out=vbar)
    grads = plx.prefill_backward(q, r, k, v, o, do, lse, sbar, qk_scale, rk_scale, vbar=vbar)
    return grads if keep_on_gpu else [from_gpu(g) for g in grads]


def check(got, ref, dtype, what):
    # A gradient that is exactly zero (dq, dr and dk when every row sees a
    # single key) is measured against the largest of the four gradients
    # instead of its own zero maximum.
    largest = max(np.abs(b).max() for b in ref)
    for name, a, b in zip(("dq", "dr", "dk", "dv"), got, ref):
        assert a.shape == b.shape, (name, a.shape, b.shape)
        assert np.all(np.isfinite(a)), f"{what} {name}: non-finite"
        bmax = np.abs(b).max()
        err = np.abs(a - b).max() / (bmax if bmax > 0 else largest)
        assert err <= GTOL[dtype], f"{what} {name}: max-norm error {err:.3e} > {GTOL[dtype]:.0e}"


@pytest.mark.parametrize("dtype,D", [(synth.BF16, 128), (synth.F32, 64), (synth.BF16, 64),
                                     (synth.F32, 128)])
@pytest.mark.parametrize("L", [1, 7, 64, 130, 257])
def test_backward_small(dtype, D, L):
    B, Hq, Hkv = 2, 4, 2
    host = inputs(B, Hq, Hkv, L, D, dtype, 1.0 if D == 64 else S128, 140 + L)
    got = gpu_backward(host, dtype)
    ref = oracle.prefill_backward(*host)
    check(got, ref, dtype, f"L={L} D={D}")


@pytest.mark.parametrize("dtype,D", [(synth.BF16, 128), (synth.F32, 64), (synth.BF16, 64)])
@pytest.mark.parametrize("L", [1, 130, 257])
def test_backward_with_stored_vbar(dtype, D, L):
    # the forward's softmax readout replaces the backward's first sweep over the keys
    host = inputs(2, 4, 2, L, D, dtype, S128 if D == 128 else 1.0, 240 + L)
    q, r, k, v, do = (to_gpu(x, dtype) for x in host)
    vbar = torch.empty_like(q)
    plx.prefill(q, r, k, v, vbar_out=vbar)
    # vbar is the softmax readout: the oracle at r = 0
    tol = 1e-5 if dtype == synth.F32 else 1e-2
    ref_vbar = oracle.prefill(*host[:1], None, *host[2:4])
    assert np.abs(from_gpu(vbar) - ref_vbar).max() <= tol * np.abs(ref_vbar).max()
    check(gpu_backward(host, dtype, use_vbar=True), oracle.prefill_backward(*host), dtype,
          f"vbar L={L} D={D}")


@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (3, 1), (8, 2), (4, 1)])
def test_backward_groups_bf16(Hq, Hkv):
    # G = 1 and even G run on the matrix-core kernels, G = 3 on the generic ones
    host = inputs(1, Hq, Hkv, 200, 128, synth.BF16, S128, 150 + Hq)
    check(gpu_backward(host, synth.BF16), oracle.prefill_backward(*host), synth.BF16,
          f"Hq={Hq} Hkv={Hkv}")


@pytest.mark.parametrize("scale", [S128, 1.0])
def test_backward_scales_and_tile_multiples(scale):
    # L a multiple of every tile (128 keys, 64 rows) and a ragged one, large logits
    for L in (256, 383):
        host = inputs(1, 4, 2, L, 128, synth.BF16, scale, 160 + L)
        check(gpu_backward(host, synth.BF16, qk_scale=0.11, rk_scale=0.7),
              oracle.prefill_backward(*host, qk_scale=0.11, rk_scale=0.7), synth.BF16,
              f"L={L} scale={scale}")


def test_backward_r_zero_is_softmax_attention_gradient():
    host = list(inputs(1, 4, 2, 190, 128, synth.BF16, S128, 170))
    host[1] = np.zeros_like(host[1])
    got = gpu_backward(host, synth.BF16)
    ref = oracle.prefill_backward(*host)
    check(got, ref, synth.BF16, "r=0")
    # and against torch's own autograd of causal softmax attention (fp32 on GPU)
    q, _, k, v, do = (to_gpu(x, synth.BF16).float().requires_grad_(True) for x in host)
    o = torch.nn.functional.scaled_dot_product_attention(
        q, k.repeat_interleave(2, 1), v.repeat_interleave(2, 1), is_causal=True)
    o.backward(do.detach())
    for name, a, t in (("dq", got[0], q), ("dv", got[3], v)):
        b = t.grad.double().cpu().numpy()
        assert np.abs(a - b).max() <= 1e-2 * np.abs(b).max(), name


def test_backward_deterministic_and_autograd_entry_point():
    host = inputs(2, 4, 2, 150, 128, synth.BF16, S128, 180)
    q, r, k, v, do = (to_gpu(x, synth.BF16) for x in host)
    vbar = torch.empty_like(q)
    o, lse, sbar = plx.prefill(q, r, k, v, return_stats=True, vbar_out=vbar)
    g1 = plx.prefill_backward(q, r, k, v, o, do, lse, sbar, vbar=vbar)
    g2 = plx.prefill_backward(q, r, k, v, o, do, lse, sbar, vbar=vbar)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)
    leaves = [t.clone().requires_grad_(True) for t in (q, r, k, v)]
    out = plx.parallax_func(*leaves)
    assert torch.equal(out, o)
    out.backward(do)
    for leaf, g in zip(leaves, g1):
        assert torch.equal(leaf.grad, g)


def test_backward_pages_training_example_loss():
    # the pages' training call: o.float().pow(2).mean().backward()
    host = inputs(1, 2, 2, 96, 128, synth.BF16, 1.0, 190)
    leaves = [to_gpu(x, synth.BF16).requires_grad_(True) for x in host[:4]]
    o = plx.parallax_func(*leaves)
    o.float().pow(2).mean().backward()
    do = (2.0 * o.detach().float() / o.numel()).to(torch.bfloat16)
    do_bits = do.cpu().view(torch.int16).numpy().view(np.uint16).copy()
    ref = oracle.prefill_backward(*host[:4], do_bits)
    check([from_gpu(t.grad) for t in leaves], ref, synth.BF16, "pages' loss")


def test_backward_full_size_units():
    """B=8, Hq=16, Hkv=8, L=4096, D=128 bf16 (the causal-prefill workload): complete
    dq, dr, dk, dv of two (sequence, KV head) units against the oracle."""
    spec = synth.prefill_spec(5)
    B, Hq, Hkv, L, D = spec.B, spec.Hq, spec.Hkv, spec.L, spec.D
    host = inputs(B, Hq, Hkv, L, D, synth.BF16, spec.scale, spec.seed)
    got = gpu_backward(host, synth.BF16, keep_on_gpu=True, use_vbar=True)
    G = Hq // Hkv
    units = np.array([[0, 0], [B - 1, Hkv - 1]])
    ref = oracle.prefill_backward(*host, units=units)
    for n, (b, hk) in enumerate(units):
        sel = [from_gpu(got[0][b, hk * G:(hk + 1) * G]), from_gpu(got[1][b, hk * G:(hk + 1) * G]),
               from_gpu(got[2][b, hk]), from_gpu(got[3][b, hk])]
        check(sel, [ref[0][n], ref[1][n], ref[2][n], ref[3][n]], synth.BF16, f"unit {b},{hk}")


@pytest.mark.parametrize("G,Hkv", [(3, 2), (5, 1)])
@pytest.mark.parametrize("scale", [S128, 1.0])
def test_odd_group_sizes_on_matrix_cores(G, Hkv, scale):
    """Odd query-head groups (one query head per work item on the matrix-core
    forward and backward): output, statistics and the four gradients."""
    B, L, D = 2, 300, 128
    Hq = G * Hkv
    host = inputs(B, Hq, Hkv, L, D, synth.BF16, scale, 600 + G)
    q, r, k, v, do = (to_gpu(x, synth.BF16) for x in host)
    o, lse, sbar = plx.prefill(q, r, k, v, return_stats=True)
    ref, ref_lse, ref_sbar = oracle.prefill(*host[:4], stats=True)
    err = np.abs(from_gpu(o) - ref).max() / np.abs(ref).max()
    assert err <= 1e-2, f"G={G} o: {err:.3e}"
    assert np.abs(lse.cpu().numpy() - ref_lse).max() <= 1e-4 * max(1.0, np.abs(ref_lse).max())
    grads = plx.prefill_backward(q, r, k, v, o, do, lse, sbar)
    check([from_gpu(x) for x in grads], oracle.prefill_backward(*host), synth.BF16, f"G={G}")


@pytest.mark.parametrize("use_vbar", [False, True])
@pytest.mark.parametrize("L", [2, 3, 9, 40, 200])
def test_unscaled_short_rows_delta_correction(L, use_vbar):
    """Unscaled N(0,1) inputs with a sharp softmax (qk_scale 0.3): rows with a
    few keys whose probe scores lie far apart, where dz is a small difference
    of terms |1 + s - sbar| times larger. delta and ubar taken from the
    forward's bf16 outputs are corrected by the row pass's own fp32 sums."""
    B, Hq, Hkv, D = 2, 4, 2, 128
    host = inputs(B, Hq, Hkv, L, D, synth.BF16, 1.0, 700 + L)
    got = gpu_backward(host, synth.BF16, qk_scale=0.3, use_vbar=use_vbar)
    ref = oracle.prefill_backward(*host, qk_scale=0.3)
    check(got, ref, synth.BF16, f"L={L} vbar={use_vbar}")
