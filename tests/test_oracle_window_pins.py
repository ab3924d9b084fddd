"""Pins for the oracle's sliding window (prefill, decode and the gradients).

The pages name sliding windows as structurally compatible with Parallax
(PyPI README of parallax-kernel, overview) without defining one; the reading
taken is the usual one: with window W > 0 query i sees keys i - W + 1 .. i,
and a decode query the last W cached keys. These checks tie it to torch's
float64 SDPA with an explicit band mask (r = 0), to slicing the inputs in
numpy, to the one-key closed form, and to finite differences.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def band_mask(L, W):
    i = np.arange(L)[:, None]
    j = np.arange(L)[None, :]
    return torch.from_numpy((j <= i) & (j > i - W))


def _rand(seed, *shapes):
    g = np.random.default_rng(seed)
    return [g.standard_normal(s) for s in shapes]


@pytest.mark.parametrize("W", [1, 2, 5, 16])
def test_prefill_window_r_zero_is_banded_softmax_attention(W):
    B, Hq, Hkv, L, D = 2, 4, 2, 23, 8
    q, k, v = _rand(1, (B, Hq, L, D), (B, Hkv, L, D), (B, Hkv, L, D))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        attn_mask=band_mask(L, W), enable_gqa=True).numpy()
    np.testing.assert_allclose(oracle.prefill(q, None, k, v, window=W), ref, rtol=0, atol=1e-13)


def test_window_at_least_the_length_is_no_window():
    q, r, k, v = _rand(2, (1, 2, 19, 8), (1, 2, 19, 8), (1, 1, 19, 8), (1, 1, 19, 8))
    full = oracle.prefill(q, r, k, v, stats=True)
    for W in (19, 50):
        for a, b in zip(oracle.prefill(q, r, k, v, stats=True, window=W), full):
            np.testing.assert_array_equal(a, b)


def test_window_one_returns_each_rows_own_value():
    q, r, k, v = _rand(3, (2, 2, 11, 8), (2, 2, 11, 8), (2, 2, 11, 8), (2, 2, 11, 8))
    o, lse, sbar = oracle.prefill(q, r, k, v, stats=True, window=1, qk_scale=0.3, rk_scale=0.7)
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, 0.3 * (q * k).sum(-1), rtol=0, atol=1e-13)
    np.testing.assert_allclose(sbar, 0.7 * (r * k).sum(-1), rtol=0, atol=1e-13)


@pytest.mark.parametrize("W", [3, 10])
def test_prefill_window_row_equals_oracle_on_the_sliced_keys(W):
    B, Hq, Hkv, L, D = 1, 2, 1, 17, 8
    q, r, k, v = _rand(4, (B, Hq, L, D), (B, Hq, L, D), (B, Hkv, L, D), (B, Hkv, L, D))
    o = oracle.prefill(q, r, k, v, window=W)
    for i in (0, W - 1, W, L - 1):
        lo = max(0, i - W + 1)
        ks = np.ascontiguousarray(k[:, :, lo:i + 1].transpose(0, 2, 1, 3))
        vs = np.ascontiguousarray(v[:, :, lo:i + 1].transpose(0, 2, 1, 3))
        ref = oracle.decode(np.ascontiguousarray(q[:, :, i]), np.ascontiguousarray(r[:, :, i]),
                            ks, vs)
        np.testing.assert_allclose(o[:, :, i], ref, rtol=0, atol=1e-14)


def test_decode_window_keeps_the_last_keys_of_each_sequence():
    Hq, Hkv, D, W = 4, 2, 8, 6
    lens = np.array([3, 6, 7, 20, 0])
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
    q, r, k, v = _rand(5, (5, Hq, D), (5, Hq, D), (lens.sum(), Hkv, D), (lens.sum(), Hkv, D))
    o = oracle.decode(q, r, k, v, seq_start=starts, seq_len=lens, window=W)
    for b, (s0, n) in enumerate(zip(starts, lens)):
        lo = s0 + max(0, n - W)
        ref = oracle.decode(q[b:b + 1], r[b:b + 1], k[lo:s0 + n], v[lo:s0 + n],
                            seq_start=np.array([0]), seq_len=np.array([s0 + n - lo]))
        np.testing.assert_allclose(o[b], ref[0], rtol=0, atol=1e-14)


def test_window_gradients_by_finite_differences():
    Hq, Hkv, L, D, W = 2, 1, 6, 3, 3
    q, r, k, v, do = _rand(6, (1, Hq, L, D), (1, Hq, L, D), (1, Hkv, L, D), (1, Hkv, L, D),
                           (1, Hq, L, D))
    grads = dict(zip("qrkv", oracle.prefill_backward(q, r, k, v, do, window=W)))
    args = dict(q=q, r=r, k=k, v=v)
    h = 1e-6
    for name in "qrkv":
        x = args[name]
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            a = dict(args)
            xp = x.copy(); xp[idx] += h
            xm = x.copy(); xm[idx] -= h
            a[name] = xp
            lp = (oracle.prefill(a["q"], a["r"], a["k"], a["v"], window=W) * do).sum()
            a[name] = xm
            lm = (oracle.prefill(a["q"], a["r"], a["k"], a["v"], window=W) * do).sum()
            fd[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(grads[name], fd, rtol=0, atol=2e-8 * max(1, np.abs(fd).max()),
                                   err_msg=name)


def test_window_gradients_r_zero_match_torch_autograd():
    B, Hq, Hkv, L, D, W = 1, 4, 2, 21, 8, 5
    q, k, v, do = _rand(7, (B, Hq, L, D), (B, Hkv, L, D), (B, Hkv, L, D), (B, Hq, L, D))
    dq, _, dk, dv = oracle.prefill_backward(q, np.zeros_like(q), k, v, do, window=W)
    tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v))
    torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=band_mask(L, W), scale=1 / math.sqrt(D),
        enable_gqa=True).backward(torch.from_numpy(do))
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=0, atol=1e-12)
