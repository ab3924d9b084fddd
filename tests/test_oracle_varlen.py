"""The oracle's packed-sequence (varlen) prefill: each sequence of a packed
batch is the dense causal prefill of its own tokens, and nothing crosses a
sequence boundary (the pages name parallax_varlen_func and define no more)."""
import numpy as np
import torch

import oracle


def test_equal_lengths_equal_the_dense_batch():
    g = np.random.default_rng(0)
    B, Hq, Hkv, L, D = 3, 4, 2, 9, 8
    q, r, do = (g.standard_normal((B, Hq, L, D)) for _ in range(3))
    k, v = (g.standard_normal((B, Hkv, L, D)) for _ in range(2))
    pack = lambda x: np.ascontiguousarray(x.transpose(0, 2, 1, 3).reshape(B * L, x.shape[1], D))
    cu = np.arange(B + 1) * L
    o, lse, sbar = oracle.prefill(q, r, k, v, stats=True, window=4)
    po, plse, psbar = oracle.prefill_varlen(pack(q), pack(r), pack(k), pack(v), cu, stats=True,
                                            window=4)
    np.testing.assert_array_equal(po, pack(o))
    np.testing.assert_array_equal(plse, lse.transpose(0, 2, 1).reshape(B * L, Hq))
    np.testing.assert_array_equal(psbar, sbar.transpose(0, 2, 1).reshape(B * L, Hq))
    dense = oracle.prefill_backward(q, r, k, v, do, window=4)
    packed = oracle.prefill_varlen_backward(pack(q), pack(r), pack(k), pack(v), pack(do), cu,
                                            window=4)
    for a, b in zip(packed, dense):
        np.testing.assert_array_equal(a, pack(b))


def test_sequences_do_not_see_each_other_r_zero_is_sdpa():
    g = np.random.default_rng(1)
    lens = [4, 0, 7, 1, 12]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T, Hq, Hkv, D = cu[-1], 2, 1, 8
    q, k, v = g.standard_normal((T, Hq, D)), g.standard_normal((T, Hkv, D)), \
        g.standard_normal((T, Hkv, D))
    o = oracle.prefill_varlen(q, None, k, v, cu)
    # block-diagonal causal mask over the packed tokens
    seq = np.repeat(np.arange(len(lens)), lens)
    i, j = np.arange(T)[:, None], np.arange(T)[None, :]
    mask = torch.from_numpy((j <= i) & (seq[:, None] == seq[None, :]))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q.transpose(1, 0, 2).copy())[None],
        torch.from_numpy(k.transpose(1, 0, 2).copy())[None],
        torch.from_numpy(v.transpose(1, 0, 2).copy())[None], attn_mask=mask,
        enable_gqa=True)[0].numpy().transpose(1, 0, 2)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-13)
