"""The pins must catch plausible mistakes in the oracle.

Each case compiles a copy of oracle/oracle.c with one deliberate mistake (on
the CPU, in a temporary directory), routes the oracle through it, and checks
that at least one independent check rejects it. The checks are the ones the
pins use: torch's float64 SDPA (r = 0, GQA, causal), numpy's weighted
covariance, and the local-linear least-squares intercept.
"""
import math
import os
import subprocess
import tempfile

import numpy as np
import pytest
import torch
from scipy.special import softmax

import oracle

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                   "oracle.c")

MUTANTS = {
    "dropped correction": ("o[d] += wj * vd + cj * vd;", "o[d] += wj * vd;"),
    "wrong sign": ("o[d] += wj * vd + cj * vd;", "o[d] += wj * vd - cj * vd;"),
    "not centred": ("double cj = z[j] * (s[j] - sb);", "double cj = z[j] * s[j];"),
    "gqa index": ("int64_t hk = h / g;\n                size_t qo = ((size_t)b",
                  "int64_t hk = h % Hkv;\n                size_t qo = ((size_t)b"),
    "prefill gqa index": ("int64_t hk = h / g;\n                size_t qo = (((size_t)b",
                          "int64_t hk = h % Hkv;\n                size_t qo = (((size_t)b"),
    "causal off by one": ("for (int64_t p = first; p <= i; ++p)", "for (int64_t p = first; p < i; ++p)"),
    "logit scale dropped": ("z[j] = tau * zq;", "z[j] = zq;"),
    "keys and values swapped": (
        "double kd = elem(k, dtype, kb + d);\n            zq += elem(q, dtype, q_off + d) * kd;"
        "\n            if (r)\n                sr += elem(r, dtype, r_off",
        "double kd = elem(v, dtype, kb + d);\n            zq += elem(q, dtype, q_off + d) * kd;"
        "\n            if (r)\n                sr += elem(r, dtype, r_off"),
    "sample covariance": ("z[j] /= l;", "z[j] /= (l - z[j] / l * 0.5);"),
    "prefill window off by one": (
        "int64_t first = (window > 0 && i + 1 > window) ? i + 1 - window : 0, n = 0;",
        "int64_t first = (window > 0 && i + 1 > window) ? i - window : 0, n = 0;"),
    "decode window keeps the first keys": ("first = len - window;", "first = 0;"),
    "block mask diagonal not forced": ("if (!mrow || p / block == i / block || mrow[",
                                       "if (!mrow || mrow["),
    "block mask transposed": ("mrow[(size_t)(i / block) * nb + p / block]",
                              "mrow[(size_t)(p / block) * nb + i / block]"),
    "decode mask drops the last-block rule": ("if (block_mask && p / block != (len - 1) / block)",
                                              "if (block_mask)"),
    "decode mask ignored": ("(size_t)(p / block)] != 0;", "(size_t)(p / block)] != 2;"),
}

# mistakes in the reverse pass (the forward code is untouched)
BACKWARD_MUTANTS = {
    "bwd sbar adjoint dropped": ("a_sb -= w[j] * t;", "a_sb -= 0.0 * t;"),
    "bwd softmax jacobian sign": ("aw[j] = w[j] * (aw[j] - waw);", "aw[j] = w[j] * (aw[j] + waw);"),
    "bwd causal off by one": ("qo, kvo, keys, n, D, dtype", "qo, kvo, keys, n - 1, D, dtype"),
    "bwd probe adjoint uses q": ("cs * elem(r, dtype, q_off + d)", "cs * elem(q, dtype, q_off + d)"),
    "bwd dv without correction": ("double cv = w[j] * (1.0 + s[j] - sb);", "double cv = w[j];"),
    "bwd dq misses tau": ("double cz = tau * aw[j], cs", "double cz = aw[j], cs"),
}


def build_mutant(name, tmp):
    old, new = {**MUTANTS, **BACKWARD_MUTANTS}[name]
    src = open(SRC).read()
    assert src.count(old) == 1, name
    path = os.path.join(tmp, "oracle_mutant.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    so = os.path.join(tmp, "liboracle_mutant.so")
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", path, "-o", so,
                    "-lm"], check=True)
    return so


def independent_checks_pass():
    """True if every independent check accepts the current oracle."""
    g = np.random.default_rng(123)
    ok = True
    # r = 0 against SDPA, GQA 4:2 (decode)
    B, Hq, Hkv, L, D = 2, 4, 2, 23, 8
    q, k, v = g.standard_normal((B, Hq, D)), g.standard_normal((B, L, Hkv, D)), \
        g.standard_normal((B, L, Hkv, D))
    tau = 1 / math.sqrt(D)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[:, :, None], torch.from_numpy(np.ascontiguousarray(
            k.transpose(0, 2, 1, 3))), torch.from_numpy(np.ascontiguousarray(
                v.transpose(0, 2, 1, 3))), scale=tau, enable_gqa=True)[:, :, 0].numpy()
    ok &= np.abs(oracle.decode(q, None, k, v, qk_scale=tau) - ref).max() < 1e-12
    # causal prefill r = 0 against SDPA with GQA
    Q, K, V = g.standard_normal((1, 4, 19, D)), g.standard_normal((1, 2, 19, D)), \
        g.standard_normal((1, 2, 19, D))
    refp = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Q), torch.from_numpy(K), torch.from_numpy(V), is_causal=True,
        enable_gqa=True).numpy()
    ok &= np.abs(oracle.prefill(Q, np.zeros_like(Q), K, V) - refp).max() < 1e-12
    # sliding window (prefill and decode) against SDPA with a band mask
    i, j = np.arange(19)[:, None], np.arange(19)[None, :]
    band = torch.from_numpy((j <= i) & (j > i - 4))
    refw = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Q), torch.from_numpy(K), torch.from_numpy(V), attn_mask=band,
        enable_gqa=True).numpy()
    ok &= np.abs(oracle.prefill(Q, None, K, V, window=4) - refw).max() < 1e-12
    kd = np.ascontiguousarray(K.transpose(0, 2, 1, 3))
    vd = np.ascontiguousarray(V.transpose(0, 2, 1, 3))
    ok &= np.abs(oracle.decode(np.ascontiguousarray(Q[:, :, 18]), None, kd, vd, window=4)
                 - refw[:, :, 18]).max() < 1e-12
    # block-sparse masks (blocks of 4 positions) against SDPA with the element mask
    bm = g.random((1, 2, 5, 5)) < 0.5
    bm[0, 0, 2, 2] = bm[0, 1, 4, 4] = False  # diagonal entries must not matter
    qb, kb = i // 4, j // 4
    em = np.stack([(j <= i) & ((qb == kb) | bm[0, h // 2][qb, kb]) for h in range(4)])[None]
    refb = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Q), torch.from_numpy(K), torch.from_numpy(V),
        attn_mask=torch.from_numpy(em), enable_gqa=True).numpy()
    ok &= np.abs(oracle.prefill(Q, None, K, V, block_mask=bm, block=4) - refb).max() < 1e-12
    dm = g.random((2, 2, 6)) < 0.5
    dm[0, 0, 5] = dm[1, 1, 5] = False  # the block holding the last key is always visible
    dm[1, 0, :5] = False
    jj = np.arange(23)
    em_d = np.stack([np.stack([(jj // 4 == 5) | dm[b, h // 2][jj // 4] for h in range(4)])
                     for b in range(2)])[:, :, None]
    refd = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[:, :, None], torch.from_numpy(np.ascontiguousarray(
            k.transpose(0, 2, 1, 3))), torch.from_numpy(np.ascontiguousarray(
                v.transpose(0, 2, 1, 3))), attn_mask=torch.from_numpy(em_d), scale=tau,
        enable_gqa=True)[:, :, 0].numpy()
    ok &= np.abs(oracle.decode(q, None, k, v, qk_scale=tau, block_mask=dm, block=4) - refd).max() \
        < 1e-12
    # correction = weighted covariance
    L, D = 30, 5
    q1, r1 = g.standard_normal((1, 1, D)), g.standard_normal((1, 1, D))
    k1, v1 = g.standard_normal((1, L, 1, D)), g.standard_normal((1, L, 1, D))
    w = softmax((k1[0, :, 0] @ q1[0, 0]) / math.sqrt(D))
    s = k1[0, :, 0] @ r1[0, 0]
    cov = np.array([np.cov(s, v1[0, :, 0, d], aweights=w, bias=True)[0, 1] for d in range(D)])
    o = oracle.decode(q1, r1, k1, v1)[0, 0]
    ok &= np.abs(o - (w @ v1[0, :, 0] + cov)).max() < 1e-12
    # local-linear intercept
    L, D = 50, 3
    q2, k2 = g.standard_normal((1, 1, D)), g.standard_normal((1, L, 1, D))
    v2 = g.standard_normal((1, L, 1, D)) + k2 @ g.standard_normal((D, D))
    K2, V2 = k2[0, :, 0], v2[0, :, 0]
    w2 = softmax(0.5 * (K2 @ q2[0, 0]))
    rv = np.linalg.solve(np.cov(K2.T, aweights=w2, bias=True), q2[0, 0] - w2 @ K2)
    X = np.concatenate([np.ones((L, 1)), K2 - q2[0, 0]], axis=1)
    coef, *_ = np.linalg.lstsq(np.sqrt(w2)[:, None] * X, np.sqrt(w2)[:, None] * V2, rcond=None)
    ok &= np.abs(oracle.decode(q2, rv[None, None], k2, v2, qk_scale=0.5)[0, 0] - coef[0]).max() \
        < 1e-10
    return bool(ok)


def test_unmutated_oracle_passes_the_checks():
    assert independent_checks_pass()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    with tempfile.TemporaryDirectory() as tmp:
        so = build_mutant(name, tmp)
        with oracle.using_library(so):
            assert not independent_checks_pass(), f"mutant '{name}' passed every check"


def backward_checks_pass():
    """True if the oracle's gradients pass finite differences of its forward
    (tiny GQA case) and torch's float64 autograd of causal SDPA at r = 0."""
    g = np.random.default_rng(321)
    Hq, Hkv, L, D = 2, 1, 5, 3
    q, r, do = (g.standard_normal((1, Hq, L, D)) for _ in range(3))
    k, v = (g.standard_normal((1, Hkv, L, D)) for _ in range(2))
    grads = dict(zip("qrkv", oracle.prefill_backward(q, r, k, v, do, rk_scale=1.2)))
    args = dict(q=q, r=r, k=k, v=v)
    h = 1e-6
    for name in "qrkv":
        x = args[name]
        for idx in np.ndindex(x.shape):
            a = dict(args)
            xp = x.copy(); xp[idx] += h
            xm = x.copy(); xm[idx] -= h
            a[name] = xp
            lp = (oracle.prefill(a["q"], a["r"], a["k"], a["v"], rk_scale=1.2) * do).sum()
            a[name] = xm
            lm = (oracle.prefill(a["q"], a["r"], a["k"], a["v"], rk_scale=1.2) * do).sum()
            if abs((lp - lm) / (2 * h) - grads[name][idx]) > 1e-6:
                return False
    tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v))
    torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True,
                                                     enable_gqa=True).backward(
        torch.from_numpy(do))
    dq, _, dk, dv = oracle.prefill_backward(q, np.zeros_like(q), k, v, do)
    return bool(np.abs(dq - tq.grad.numpy()).max() < 1e-12
                and np.abs(dk - tk.grad.numpy()).max() < 1e-12
                and np.abs(dv - tv.grad.numpy()).max() < 1e-12)


def test_unmutated_oracle_passes_the_backward_checks():
    assert backward_checks_pass()


@pytest.mark.parametrize("name", sorted(BACKWARD_MUTANTS))
def test_backward_mutant_is_caught(name):
    with tempfile.TemporaryDirectory() as tmp:
        so = build_mutant(name, tmp)
        with oracle.using_library(so):
            assert not backward_checks_pass(), f"mutant '{name}' passed every check"
