"""Pins for the oracle's prefill gradients (dq, dr, dk, dv).

The pages train through parallax_func with autograd (PyPI README of
parallax-kernel, "Training (Triton)") and hold the four gradients to the
same tolerance as the output ("Helion" section). They print no gradient
formula, so the gradient is pinned to what fixes it independently of the
oracle's reverse pass:
  - central finite differences of the (separately pinned) forward oracle,
  - torch's float64 autograd through scaled_dot_product_attention at r = 0
    (softmax attention, encorp.ai article: W_R = 0 gives it back exactly),
  - exact identities of the forward: invariance under a common key shift,
    linearity in v (and the softmax-plus-centred weights summing to one),
    and the derivative along the probe scale, whose value is o minus the
    softmax readout.
A wrong sign in any adjoint, a dropped sbar path, an off-by-one causal
range or a wrong GQA head fails at least one of them.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def _inputs(seed, B, Hq, Hkv, L, D, scale=1.0):
    g = np.random.default_rng(seed)
    q, r, do = (g.standard_normal((B, Hq, L, D)) * scale for _ in range(3))
    k, v = (g.standard_normal((B, Hkv, L, D)) * scale for _ in range(2))
    return q, r, k, v, do


@pytest.mark.parametrize("Hq,Hkv,L,D,tau,rho,with_r", [
    (2, 1, 6, 4, None, 1.0, True),
    (2, 2, 5, 3, 0.7, 1.3, True),
    (3, 1, 4, 4, None, 1.0, False),
])
def test_finite_differences_of_forward(Hq, Hkv, L, D, tau, rho, with_r):
    q, r, k, v, do = _inputs(11, 1, Hq, Hkv, L, D)
    if not with_r:
        r = None
    dq, dr, dk, dv = oracle.prefill_backward(q, r, k, v, do, qk_scale=tau, rk_scale=rho)
    args = dict(q=q, r=r if with_r else np.zeros_like(q), k=k, v=v)

    def loss(a):
        return float((oracle.prefill(a["q"], a["r"], a["k"], a["v"], qk_scale=tau,
                                     rk_scale=rho) * do).sum())

    h = 1e-6
    for name, grad in (("q", dq), ("r", dr), ("k", dk), ("v", dv)):
        x = args[name]
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            a = dict(args)
            xp = x.copy(); xp[idx] += h
            xm = x.copy(); xm[idx] -= h
            a[name] = xp
            lp = loss(a)
            a[name] = xm
            fd[idx] = (lp - loss(a)) / (2 * h)
        np.testing.assert_allclose(grad, fd, rtol=0, atol=2e-8 * max(1.0, np.abs(fd).max()),
                                   err_msg=name)


@pytest.mark.parametrize("B,Hq,Hkv,L,D", [(2, 4, 2, 19, 8), (1, 2, 2, 33, 16)])
def test_r_zero_matches_torch_autograd_of_softmax_attention(B, Hq, Hkv, L, D):
    q, _, k, v, do = _inputs(3, B, Hq, Hkv, L, D)
    tau = 1.0 / math.sqrt(D)
    dq, dr, dk, dv = oracle.prefill_backward(q, np.zeros_like(q), k, v, do)
    tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=tau,
                                                         enable_gqa=True)
    o.backward(torch.from_numpy(do))
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=0, atol=1e-12)
    # at r = 0, dr_i = rho * sum_j w_ij (g_i.v_j - g_i.vbar_i) k_j: the
    # w-weighted covariance of (g.v, k), taken here with numpy's cov
    G = q.shape[1] // k.shape[1]
    for b in range(B):
        for h in range(Hq):
            for i in (0, L // 2, L - 1):
                z = tau * k[b, h // G, : i + 1] @ q[b, h, i]
                w = np.exp(z - z.max()); w /= w.sum()
                u = v[b, h // G, : i + 1] @ do[b, h, i]
                if i == 0:
                    ref = np.zeros(D)
                else:
                    c = np.cov(np.vstack([u, k[b, h // G, : i + 1].T]), aweights=w, bias=True)
                    ref = c[0, 1:]
                np.testing.assert_allclose(dr[b, h, i], ref, rtol=0, atol=1e-12)


def test_key_shift_invariance_sum_of_dk_is_zero():
    # adding one vector to every key shifts each row's logits and probe scores
    # by a per-row constant: w and s - sbar are unchanged, so is o
    q, r, k, v, do = _inputs(5, 2, 4, 2, 23, 8)
    _, _, dk, _ = oracle.prefill_backward(q, r, k, v, do, rk_scale=0.8)
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-11)
    assert np.abs(dk).max() > 0.1


def test_values_linear_and_constant_shift():
    # o is linear in v (sum_j v_j.dv_j = sum_i g_i.o_i), and the weights
    # w_j (1 + s_j - sbar) of each row sum to one (sum_j dv_j = sum_i g_i)
    q, r, k, v, do = _inputs(6, 1, 4, 2, 29, 8)
    o = oracle.prefill(q, r, k, v)
    _, _, _, dv = oracle.prefill_backward(q, r, k, v, do)
    lhs = (v * dv).sum(axis=(2, 3))
    rhs = (o * do).reshape(1, 2, 2, 29, 8).sum(axis=(2, 3, 4))
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-11)
    np.testing.assert_allclose(dv.sum(axis=2), do.reshape(1, 2, 2, 29, 8).sum(axis=(2, 3)),
                               rtol=0, atol=1e-11)


def test_probe_scale_derivative():
    # o((1 + e) r) = vbar + (1 + e)(o - vbar): per row, r_i.dr_i = g_i.(o_i - vbar_i)
    # with vbar the softmax readout (the forward at r = 0)
    q, r, k, v, do = _inputs(7, 2, 2, 1, 17, 8)
    o = oracle.prefill(q, r, k, v)
    vbar = oracle.prefill(q, None, k, v)
    _, dr, _, _ = oracle.prefill_backward(q, r, k, v, do)
    np.testing.assert_allclose((r * dr).sum(-1), (do * (o - vbar)).sum(-1), rtol=0, atol=1e-11)


def test_query_scale_derivative():
    # o((1 + e) q) sharpens the softmax: dw_j/de = w_j (z_j - zbar); per row
    # q_i.dq_i = g_i.[sum_j w_j (z_j - zbar)(1 + s_j - sbar) v_j - Cov_w(z, s) vbar]
    q, r, k, v, do = _inputs(8, 1, 2, 1, 13, 8)
    D = 8
    tau = 1.0 / math.sqrt(D)
    dq, _, _, _ = oracle.prefill_backward(q, r, k, v, do)
    for h in range(2):
        for i in range(13):
            kk, vv = k[0, 0, : i + 1], v[0, 0, : i + 1]
            z = tau * kk @ q[0, h, i]
            s = kk @ r[0, h, i]
            w = np.exp(z - z.max()); w /= w.sum()
            zb, sb = w @ z, w @ s
            vbar = w @ vv
            do_de = (w * (z - zb) * (1 + s - sb)) @ vv - (w @ ((z - zb) * (s - sb))) * vbar
            assert abs(q[0, h, i] @ dq[0, h, i] - do[0, h, i] @ do_de) < 1e-11


def test_units_subset_matches_full_and_bf16_widening():
    q, r, k, v, do = _inputs(9, 2, 4, 2, 21, 8)
    full = oracle.prefill_backward(q, r, k, v, do)
    sub = oracle.prefill_backward(q, r, k, v, do, units=[[1, 0], [0, 1]])
    for (b, hk), n in (((1, 0), 0), ((0, 1), 1)):
        np.testing.assert_array_equal(sub[0][n], full[0][b, 2 * hk: 2 * hk + 2])
        np.testing.assert_array_equal(sub[1][n], full[1][b, 2 * hk: 2 * hk + 2])
        np.testing.assert_array_equal(sub[2][n], full[2][b, hk])
        np.testing.assert_array_equal(sub[3][n], full[3][b, hk])
    # bf16 inputs are widened exactly: same as the float64 of the same values
    tb = [torch.from_numpy(x).to(torch.bfloat16) for x in (q, r, k, v, do)]
    bits = [t.view(torch.int16).numpy().view(np.uint16).copy() for t in tb]
    wide = [t.to(torch.float64).numpy().copy() for t in tb]
    gb = oracle.prefill_backward(*bits)
    gw = oracle.prefill_backward(*wide)
    for a, b_ in zip(gb, gw):
        np.testing.assert_array_equal(a, b_)
