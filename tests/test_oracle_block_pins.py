"""Pins of the oracle's block-sparse masks (CPU).

The pages call block sparsity structurally compatible with Parallax and define
none; the reading the oracle takes is: blocks of `block` positions from the
start of each sequence, one byte mask per (sequence, KV head), a query always
seeing its own block (prefill: the diagonal block; decode: the block holding
the last key), on top of causality and the window. These tests tie that to
computations outside the oracle:
- r = 0: torch's float64 scaled_dot_product_attention with the element mask the
  block mask expands to (GQA, with and without a window);
- r != 0: each row against numpy's weighted covariance over the row's visible
  keys, gathered by index;
- gradients: central finite differences of the masked forward, and torch's
  float64 autograd of the masked SDPA at r = 0;
- an all-ones mask returns exactly the unmasked result, and packed sequences
  take their own slice of the mask.
"""
import math

import numpy as np
import pytest
import torch
from scipy.special import softmax

import oracle


def element_mask(bm, L, block, window=0):
    """[B, Hkv, L, L] bool: key j visible to query i."""
    i, j = np.arange(L)[:, None], np.arange(L)[None, :]
    vis = j <= i
    if window:
        vis &= j > i - window
    qb, kb = i // block, j // block
    return vis[None, None] & ((qb == kb)[None, None] | bm[:, :, qb, kb])


def sdpa(q, k, v, mask, scale):
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        attn_mask=torch.from_numpy(mask), scale=scale, enable_gqa=True).numpy()


@pytest.mark.parametrize("seed,window", [(0, 0), (1, 0), (2, 7), (3, 1)])
def test_prefill_r0_matches_sdpa_with_the_expanded_mask(seed, window):
    g = np.random.default_rng(seed)
    B, Hq, Hkv, L, D, bs = 2, 4, 2, 37, 8, 5
    nb = -(-L // bs)
    q = g.standard_normal((B, Hq, L, D))
    k, v = g.standard_normal((B, Hkv, L, D)), g.standard_normal((B, Hkv, L, D))
    bm = g.random((B, Hkv, nb, nb)) < 0.4
    em = np.repeat(element_mask(bm, L, bs, window), Hq // Hkv, axis=1)
    ref = sdpa(q, k, v, em, 0.3)
    got = oracle.prefill(q, None, k, v, qk_scale=0.3, window=window, block_mask=bm, block=bs)
    assert np.abs(got - ref).max() < 1e-12


def test_decode_r0_matches_sdpa_dense_and_packed():
    g = np.random.default_rng(5)
    B, Hq, Hkv, D, bs = 3, 6, 3, 8, 4
    lens = np.array([17, 1, 30])
    nkb = -(-lens.max() // bs)
    q = g.standard_normal((B, Hq, D))
    T = int(lens.sum())
    k, v = g.standard_normal((T, Hkv, D)), g.standard_normal((T, Hkv, D))
    bm = g.random((B, Hkv, nkb)) < 0.5
    start = np.concatenate([[0], np.cumsum(lens)[:-1]])
    got = oracle.decode(q, None, k, v, seq_start=start, seq_len=lens, qk_scale=0.7,
                        block_mask=bm, block=bs)
    for b in range(B):
        n = lens[b]
        jj = np.arange(n)
        kb = k[start[b]:start[b] + n].transpose(1, 0, 2)[None]
        vb = v[start[b]:start[b] + n].transpose(1, 0, 2)[None]
        em = np.stack([(jj // bs == (n - 1) // bs) | bm[b, h // 2][jj // bs]
                       for h in range(Hq)])[None, :, None]
        ref = sdpa(np.ascontiguousarray(q[b:b + 1, :, None]), np.ascontiguousarray(kb),
                   np.ascontiguousarray(vb), em, 0.7)[0, :, 0]
        assert np.abs(got[b] - ref).max() < 1e-12
    # the same cache laid out dense gives the same rows (sequence 2 is the longest)
    kd = k[start[2]:][None].copy()
    vd = v[start[2]:][None].copy()
    dense = oracle.decode(q[2:3].copy(), None, kd, vd, qk_scale=0.7, block_mask=bm[2:3], block=bs)
    assert np.array_equal(dense[0], got[2])


@pytest.mark.parametrize("seed", [11, 12])
def test_correction_matches_weighted_covariance_on_visible_keys(seed):
    g = np.random.default_rng(seed)
    Hkv, L, D, bs, rho = 1, 29, 6, 4, 1.3
    nb = -(-L // bs)
    q, r = g.standard_normal((1, 1, L, D)), g.standard_normal((1, 1, L, D))
    k, v = g.standard_normal((1, Hkv, L, D)), g.standard_normal((1, Hkv, L, D))
    bm = g.random((1, Hkv, nb, nb)) < 0.5
    o = oracle.prefill(q, r, k, v, qk_scale=0.4, rk_scale=rho, block_mask=bm, block=bs)
    vis = element_mask(bm, L, bs)[0, 0]
    for i in range(L):
        J = np.nonzero(vis[i])[0]
        Kj, Vj = k[0, 0, J], v[0, 0, J]
        w = softmax(0.4 * Kj @ q[0, 0, i])
        s = rho * Kj @ r[0, 0, i]
        cov = np.array([np.cov(s, Vj[:, d], aweights=w, bias=True)[0, 1] for d in range(D)]) \
            if len(J) > 1 else np.zeros(D)
        assert np.abs(o[0, 0, i] - (w @ Vj + cov)).max() < 1e-12


def test_all_ones_mask_is_exactly_no_mask():
    g = np.random.default_rng(3)
    q, r = g.standard_normal((1, 2, 33, 8)), g.standard_normal((1, 2, 33, 8))
    k, v = g.standard_normal((1, 1, 33, 8)), g.standard_normal((1, 1, 33, 8))
    ones = np.ones((1, 1, 9, 9), dtype=bool)
    for w in (0, 6):
        a = oracle.prefill(q, r, k, v, window=w, stats=True)
        b = oracle.prefill(q, r, k, v, window=w, stats=True, block_mask=ones, block=4)
        assert all(np.array_equal(x, y) for x, y in zip(a, b))
    qd, rd = g.standard_normal((2, 2, 8)), g.standard_normal((2, 2, 8))
    kd, vd = g.standard_normal((2, 21, 1, 8)), g.standard_normal((2, 21, 1, 8))
    assert np.array_equal(oracle.decode(qd, rd, kd, vd),
                          oracle.decode(qd, rd, kd, vd, block_mask=np.ones((2, 1, 3)), block=8))


def test_hidden_blocks_do_not_influence_a_row():
    """Changing keys and values in blocks a row cannot see leaves that row alone."""
    g = np.random.default_rng(8)
    L, D, bs = 24, 5, 4
    q, r = g.standard_normal((1, 1, L, D)), g.standard_normal((1, 1, L, D))
    k, v = g.standard_normal((1, 1, L, D)), g.standard_normal((1, 1, L, D))
    bm = np.zeros((1, 1, 6, 6), dtype=bool)
    bm[0, 0, 5, 1] = True  # the last block also sees block 1
    o = oracle.prefill(q, r, k, v, block_mask=bm, block=bs)
    k2, v2 = k.copy(), v.copy()
    k2[0, 0, 8:12] += 3.0  # block 2: seen only by its own rows
    v2[0, 0, 8:12] -= 2.0
    o2 = oracle.prefill(q, r, k2, v2, block_mask=bm, block=bs)
    changed = np.abs(o2 - o).max(axis=-1)[0, 0] > 0
    assert np.array_equal(np.nonzero(changed)[0], np.arange(8, 12))


def test_varlen_takes_each_sequence_slice_of_the_mask():
    g = np.random.default_rng(9)
    lens = np.array([13, 0, 22])
    cu = np.concatenate([[0], np.cumsum(lens)])
    T, Hq, Hkv, D, bs = int(cu[-1]), 2, 1, 6, 4
    q, r = g.standard_normal((T, Hq, D)), g.standard_normal((T, Hq, D))
    k, v = g.standard_normal((T, Hkv, D)), g.standard_normal((T, Hkv, D))
    nb = -(-lens.max() // bs)
    bm = g.random((3, Hkv, nb, nb)) < 0.5
    o = oracle.prefill_varlen(q, r, k, v, cu, block_mask=bm, block=bs)
    s0, n = cu[2], lens[2]
    dense = oracle.prefill(*(np.ascontiguousarray(x[s0:s0 + n].transpose(1, 0, 2)[None])
                             for x in (q, r, k, v)), block_mask=bm[2:3], block=bs)
    assert np.array_equal(o[s0:s0 + n], dense[0].transpose(1, 0, 2))


def test_masked_gradients_match_finite_differences():
    g = np.random.default_rng(21)
    Hq, Hkv, L, D, bs = 2, 1, 7, 3, 2
    nb = -(-L // bs)
    q, r, do = (g.standard_normal((1, Hq, L, D)) for _ in range(3))
    k, v = (g.standard_normal((1, Hkv, L, D)) for _ in range(2))
    bm = g.random((1, Hkv, nb, nb)) < 0.5
    kw = dict(rk_scale=0.8, block_mask=bm, block=bs, window=5)
    grads = dict(zip("qrkv", oracle.prefill_backward(q, r, k, v, do, **kw)))
    args = dict(q=q, r=r, k=k, v=v)
    h = 1e-6
    for name in "qrkv":
        x = args[name]
        for idx in np.ndindex(x.shape):
            a = dict(args)
            xp = x.copy(); xp[idx] += h
            xm = x.copy(); xm[idx] -= h
            a[name] = xp
            lp = (oracle.prefill(a["q"], a["r"], a["k"], a["v"], **kw) * do).sum()
            a[name] = xm
            lm = (oracle.prefill(a["q"], a["r"], a["k"], a["v"], **kw) * do).sum()
            assert abs((lp - lm) / (2 * h) - grads[name][idx]) < 1e-6, (name, idx)


def test_masked_gradients_at_r0_match_sdpa_autograd():
    g = np.random.default_rng(22)
    B, Hq, Hkv, L, D, bs = 2, 4, 2, 19, 4, 3
    nb = -(-L // bs)
    q, do = g.standard_normal((B, Hq, L, D)), g.standard_normal((B, Hq, L, D))
    k, v = g.standard_normal((B, Hkv, L, D)), g.standard_normal((B, Hkv, L, D))
    bm = g.random((B, Hkv, nb, nb)) < 0.5
    em = np.repeat(element_mask(bm, L, bs), Hq // Hkv, axis=1)
    tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v))
    torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=torch.from_numpy(em), scale=1 / math.sqrt(D),
        enable_gqa=True).backward(torch.from_numpy(do))
    dq, _, dk, dv = oracle.prefill_backward(q, np.zeros_like(q), k, v, do, block_mask=bm,
                                            block=bs)
    for a, b in ((dq, tq), (dk, tk), (dv, tv)):
        assert np.abs(a - b.grad.numpy()).max() < 1e-12
