"""Pins for the CPU oracle: checks against what the pages and the mathematics fix.

None of these compares the oracle with a retyped copy of its own formula
(the mpmath check at the end only bounds round-off). Each is chosen so that
a plausible slip -- a dropped correction term, a wrong sign, a wrong GQA
index, an off-by-one causal mask, a transposed operand, 1/(n-1) instead of
1/n -- fails at least one of them.

Passages: "Parallax: Parameterized Local Linear Attention for Language
Modeling" (neuraltrendhub summary, "What the paper found", and the original
abstract) -- a learned query-like projector probes the KV covariance and the
solver of Local Linear Attention is removed; the cere-bro blog's diagram --
softmax is the local-constant estimate, LLA the local-linear one; the
encorp.ai article (section on the conjugate-gradient solver and the FAQ) --
W_R = 0 gives softmax attention exactly; the PyPI README quickstart -- shapes,
causal training call, decode qk_scale = 1/sqrt(D).
"""
import json
import math
import os

import mpmath
import numpy as np
import pytest
import torch
from scipy.special import softmax

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rng(seed):
    return np.random.default_rng(seed)


def rand(g, *shape):
    return g.standard_normal(shape)


def sdpa_decode(q, k, v, tau):
    """torch SDPA in float64: q [B,Hq,D], k/v [B,L,Hkv,D] -> [B,Hq,D]."""
    qt = torch.from_numpy(q)[:, :, None, :]
    kt = torch.from_numpy(np.ascontiguousarray(k.transpose(0, 2, 1, 3)))
    vt = torch.from_numpy(np.ascontiguousarray(v.transpose(0, 2, 1, 3)))
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=tau, enable_gqa=True)
    return o[:, :, 0, :].numpy()


# ---------------------------------------------------------------- P1
@pytest.mark.parametrize("B,Hq,Hkv,D,L", [(2, 4, 4, 8, 37), (3, 8, 2, 16, 50), (1, 2, 1, 64, 256)])
def test_r_zero_is_softmax_attention_decode(B, Hq, Hkv, D, L):
    """W_R = 0 reduces exactly to softmax attention (encorp.ai FAQ and solver section)."""
    g = rng(1)
    q, k, v = rand(g, B, Hq, D), rand(g, B, L, Hkv, D), rand(g, B, L, Hkv, D)
    tau = 1.0 / math.sqrt(D)
    ref = sdpa_decode(q, k, v, tau)
    o0 = oracle.decode(q, np.zeros_like(q), k, v, qk_scale=tau)
    on = oracle.decode(q, None, k, v, qk_scale=tau)
    np.testing.assert_allclose(o0, ref, rtol=0, atol=1e-13)
    np.testing.assert_array_equal(o0, on)


@pytest.mark.parametrize("B,Hq,Hkv,L,D", [(2, 4, 2, 33, 8), (1, 6, 3, 70, 16)])
def test_r_zero_is_causal_softmax_attention_prefill(B, Hq, Hkv, L, D):
    g = rng(2)
    q, k, v = rand(g, B, Hq, L, D), rand(g, B, Hkv, L, D), rand(g, B, Hkv, L, D)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), is_causal=True,
        enable_gqa=True).numpy()  # default scale 1/sqrt(D)
    o = oracle.prefill(q, np.zeros_like(q), k, v)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-13)


# ---------------------------------------------------------------- P2, P3
def test_correction_is_weighted_covariance():
    """o(r) - o(0) is the w-weighted covariance of the probe scores and the values
    ("probes the KV covariance"), taken with numpy's cov (aweights, 1/sum w)."""
    g = rng(3)
    L, D = 40, 6
    q, r = rand(g, 1, 1, D), rand(g, 1, 1, D)
    k, v = rand(g, 1, L, 1, D), rand(g, 1, L, 1, D)
    tau = 0.7
    w = softmax(tau * (k[0, :, 0] @ q[0, 0]))
    s = k[0, :, 0] @ r[0, 0]
    corr = np.array([np.cov(s, v[0, :, 0, d], aweights=w, bias=True)[0, 1] for d in range(D)])
    o = oracle.decode(q, r, k, v, qk_scale=tau)[0, 0]
    o0 = oracle.decode(q, None, k, v, qk_scale=tau)[0, 0]
    np.testing.assert_allclose(o - o0, corr, rtol=0, atol=1e-13)
    np.testing.assert_allclose(o0, w @ v[0, :, 0], rtol=0, atol=1e-13)


def test_correction_is_cross_covariance_times_probe():
    """Same correction by the matrix route: Sigma_vk r with Sigma_vk the D x D
    weighted cross-covariance of values and keys."""
    g = rng(4)
    L, D = 29, 5
    q, r = rand(g, 1, 1, D), rand(g, 1, 1, D)
    k, v = rand(g, 1, L, 1, D), rand(g, 1, L, 1, D)
    K, V = k[0, :, 0], v[0, :, 0]
    w = softmax((K @ q[0, 0]) / math.sqrt(D))
    C = np.cov(np.concatenate([V, K], axis=1).T, aweights=w, bias=True)
    sigma_vk = C[:D, D:]
    o = oracle.decode(q, r, k, v)[0, 0]
    np.testing.assert_allclose(o, w @ V + sigma_vk @ r[0, 0], rtol=0, atol=1e-13)


# ---------------------------------------------------------------- P4
@pytest.mark.parametrize("seed", [5, 6])
def test_plus_sign_from_local_linear_intercept(seed):
    """Local Linear Attention (cere-bro diagram: slope + intercept; the solve that
    Parallax removes). With the probe set to the solver's output
    r = Sigma_kk^{-1} (q - kbar), the oracle must return the intercept of the
    w-weighted least-squares fit of v on [1, k - q] -- computed here by
    numpy.linalg.lstsq. This fixes the sign and the centring."""
    g = rng(seed)
    L, D, Dv = 60, 4, 3
    q = rand(g, 1, 1, D)
    k = rand(g, 1, L, 1, D)
    v = np.zeros((1, L, 1, D))
    v[0, :, 0, :Dv] = rand(g, L, Dv) + k[0, :, 0, :Dv] @ rand(g, Dv, Dv) * 0.5
    v[0, :, 0, Dv:] = rand(g, L, D - Dv)
    K, V = k[0, :, 0], v[0, :, 0]
    tau = 0.5
    w = softmax(tau * (K @ q[0, 0]))
    kbar = w @ K
    sigma_kk = np.cov(K.T, aweights=w, bias=True)
    rvec = np.linalg.solve(sigma_kk, q[0, 0] - kbar)
    X = np.concatenate([np.ones((L, 1)), K - q[0, 0]], axis=1)
    sw = np.sqrt(w)[:, None]
    coef, *_ = np.linalg.lstsq(sw * X, sw * V, rcond=None)
    intercept = coef[0]
    o = oracle.decode(q, rvec[None, None, :], k, v, qk_scale=tau)[0, 0]
    np.testing.assert_allclose(o, intercept, rtol=0, atol=1e-11)
    # the opposite sign would be far away
    assert np.abs(2 * (w @ V) - o - intercept).max() > 1e-3


# ---------------------------------------------------------------- P5, P6
def test_key_shift_invariance():
    g = rng(7)
    B, Hq, Hkv, L, D = 2, 4, 2, 45, 8
    q, r = rand(g, B, Hq, D), rand(g, B, Hq, D)
    k, v = rand(g, B, L, Hkv, D), rand(g, B, L, Hkv, D)
    c = rand(g, D) * 3.0
    o = oracle.decode(q, r, k, v)
    os_ = oracle.decode(q, r, k + c, v)
    np.testing.assert_allclose(os_, o, rtol=0, atol=1e-12)


def test_value_constant_shift_and_scale():
    g = rng(8)
    B, Hq, Hkv, L, D = 1, 2, 2, 31, 6
    q, r = rand(g, B, Hq, D), rand(g, B, Hq, D)
    k, v = rand(g, B, L, Hkv, D), rand(g, B, L, Hkv, D)
    c = rand(g, D)
    const_v = np.broadcast_to(c, v.shape).copy()
    np.testing.assert_allclose(oracle.decode(q, r, k, const_v), np.broadcast_to(c, q.shape),
                               rtol=0, atol=1e-13)
    o = oracle.decode(q, r, k, v)
    np.testing.assert_allclose(oracle.decode(q, r, k, v + c), o + c, rtol=0, atol=1e-12)
    np.testing.assert_allclose(oracle.decode(q, r, k, 2.5 * v), 2.5 * o, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- P7
def test_single_key_returns_its_value():
    g = rng(9)
    q, r = rand(g, 1, 2, 8), rand(g, 1, 2, 8)
    k, v = rand(g, 1, 1, 2, 8), rand(g, 1, 1, 2, 8)
    np.testing.assert_array_equal(oracle.decode(q, r, k, v), v[:, 0])
    Q, R = rand(g, 1, 2, 5, 8), rand(g, 1, 2, 5, 8)
    K, V = rand(g, 1, 2, 5, 8), rand(g, 1, 2, 5, 8)
    o = oracle.prefill(Q, R, K, V)
    np.testing.assert_array_equal(o[:, :, 0], V[:, :, 0])


def test_two_keys_closed_form():
    """o = w1 v1 + w2 v2 + w1 w2 (s1 - s2)(v1 - v2) for two visible keys."""
    g = rng(10)
    D = 7
    q, r = rand(g, 1, 1, D), rand(g, 1, 1, D)
    k, v = rand(g, 1, 2, 1, D), rand(g, 1, 2, 1, D)
    tau = 0.3
    z = tau * (k[0, :, 0] @ q[0, 0])
    w1 = 1.0 / (1.0 + math.exp(z[1] - z[0]))
    w2 = 1.0 - w1
    s1, s2 = k[0, 0, 0] @ r[0, 0], k[0, 1, 0] @ r[0, 0]
    v1, v2 = v[0, 0, 0], v[0, 1, 0]
    ref = w1 * v1 + w2 * v2 + w1 * w2 * (s1 - s2) * (v1 - v2)
    np.testing.assert_allclose(oracle.decode(q, r, k, v, qk_scale=tau)[0, 0], ref, rtol=0,
                               atol=1e-14)


def test_golden_hand_worked_examples():
    """Small examples worked by hand (tests/golden/hand_worked.json)."""
    with open(os.path.join(GOLDEN, "hand_worked.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        q = np.array(c["q"], dtype=np.float64)[None, None]
        r = np.array(c["r"], dtype=np.float64)[None, None]
        k = np.array(c["k"], dtype=np.float64)[None, :, None]
        v = np.array(c["v"], dtype=np.float64)[None, :, None]
        o = oracle.decode(q, r, k, v, qk_scale=c["qk_scale"], rk_scale=c.get("rk_scale", 1.0))
        np.testing.assert_allclose(o[0, 0], np.array(c["o"]), rtol=0, atol=1e-14,
                                   err_msg=c["name"])


# ---------------------------------------------------------------- P8
def test_zero_query_gives_uniform_weights_and_population_covariance():
    g = rng(11)
    L, D = 23, 4
    q = np.zeros((1, 1, D))
    r = rand(g, 1, 1, D)
    k, v = rand(g, 1, L, 1, D), rand(g, 1, L, 1, D)
    s = k[0, :, 0] @ r[0, 0]
    ref = v[0, :, 0].mean(axis=0) + np.array(
        [np.cov(s, v[0, :, 0, d], bias=True)[0, 1] for d in range(D)])
    np.testing.assert_allclose(oracle.decode(q, r, k, v)[0, 0], ref, rtol=0, atol=1e-13)


# ---------------------------------------------------------------- P9
def test_linear_in_probe_and_rk_scale():
    g = rng(12)
    B, Hq, Hkv, L, D = 1, 2, 1, 19, 8
    q, r1, r2 = rand(g, B, Hq, D), rand(g, B, Hq, D), rand(g, B, Hq, D)
    k, v = rand(g, B, L, Hkv, D), rand(g, B, L, Hkv, D)
    o0 = oracle.decode(q, None, k, v)
    d1 = oracle.decode(q, r1, k, v) - o0
    d2 = oracle.decode(q, r2, k, v) - o0
    d12 = oracle.decode(q, r1 + r2, k, v) - o0
    np.testing.assert_allclose(d12, d1 + d2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(oracle.decode(q, r1, k, v, rk_scale=0.25),
                               oracle.decode(q, 0.25 * r1, k, v), rtol=0, atol=1e-13)


# ---------------------------------------------------------------- P10
def test_gqa_equals_mha_with_repeated_kv_heads():
    g = rng(13)
    B, Hq, Hkv, L, D = 2, 8, 2, 21, 4
    q, r = rand(g, B, Hq, D), rand(g, B, Hq, D)
    k, v = rand(g, B, L, Hkv, D), rand(g, B, L, Hkv, D)
    rep = Hq // Hkv
    k_mha = np.repeat(k, rep, axis=2)   # head h reads KV head h // rep
    v_mha = np.repeat(v, rep, axis=2)
    np.testing.assert_array_equal(oracle.decode(q, r, k, v), oracle.decode(q, r, k_mha, v_mha))
    # and r = 0 agrees with torch's own GQA mapping
    np.testing.assert_allclose(oracle.decode(q, None, k, v, qk_scale=0.5),
                               sdpa_decode(q, k, v, 0.5), rtol=0, atol=1e-13)


# ---------------------------------------------------------------- P11
def test_prefill_row_equals_decode_on_prefix():
    g = rng(14)
    B, Hq, Hkv, L, D = 1, 4, 2, 17, 8
    Q, R = rand(g, B, Hq, L, D), rand(g, B, Hq, L, D)
    K, V = rand(g, B, Hkv, L, D), rand(g, B, Hkv, L, D)
    o = oracle.prefill(Q, R, K, V)
    for i in (0, 1, 7, L - 1):
        kd = np.ascontiguousarray(K[:, :, : i + 1].transpose(0, 2, 1, 3))
        vd = np.ascontiguousarray(V[:, :, : i + 1].transpose(0, 2, 1, 3))
        od = oracle.decode(np.ascontiguousarray(Q[:, :, i]), np.ascontiguousarray(R[:, :, i]),
                           kd, vd)
        np.testing.assert_allclose(o[:, :, i], od, rtol=0, atol=1e-13)


def test_prefill_stats():
    g = rng(15)
    B, Hq, Hkv, L, D = 1, 2, 1, 9, 4
    Q, R = rand(g, B, Hq, L, D), rand(g, B, Hq, L, D)
    K, V = rand(g, B, Hkv, L, D), rand(g, B, Hkv, L, D)
    o, lse, sbar = oracle.prefill(Q, R, K, V, stats=True)
    tau = 0.5
    for h in range(Hq):
        for i in range(L):
            z = tau * (K[0, 0, : i + 1] @ Q[0, h, i])
            s = K[0, 0, : i + 1] @ R[0, h, i]
            assert abs(lse[0, h, i] - np.log(np.exp(z).sum())) < 1e-13
            assert abs(sbar[0, h, i] - softmax(z) @ s) < 1e-13


def test_prefill_stats_through_other_paths():
    """lse and sbar pinned without their own formula:
    - d lse / d q = qk_scale * kbar, where kbar = sum_j w_j k_j is the oracle's
      softmax readout (r = 0) with the keys as values (central differences);
    - sbar = rk_scale * r . kbar (the same readout), and also
      sbar = rk_scale * d/dt lse(q + (t / qk_scale) r) at t = 0 (the probe score
      is the slope of the log-partition along r: central differences);
    - shifting every key by c adds qk_scale * q . c to lse (logits all move by it);
    - one visible key: lse = its logit; two: numpy's logaddexp of the two."""
    g = rng(25)
    B, Hq, Hkv, L, D = 1, 2, 1, 9, 4
    Q, R = rand(g, B, Hq, L, D), rand(g, B, Hq, L, D)
    K, V = rand(g, B, Hkv, L, D), rand(g, B, Hkv, L, D)
    tau, rho = 0.7, 1.3
    _, lse, sbar = oracle.prefill(Q, R, K, V, qk_scale=tau, rk_scale=rho, stats=True)
    kbar = oracle.prefill(Q, None, K, K, qk_scale=tau)  # sum_j w_j k_j per row
    np.testing.assert_allclose(sbar, rho * np.einsum("bhld,bhld->bhl", R, kbar), rtol=0,
                               atol=1e-12)
    eps = 1e-5
    for d in range(D):
        e = np.zeros(D)
        e[d] = eps
        _, lp, _ = oracle.prefill(Q + e, R, K, V, qk_scale=tau, stats=True)
        _, lm, _ = oracle.prefill(Q - e, R, K, V, qk_scale=tau, stats=True)
        np.testing.assert_allclose((lp - lm) / (2 * eps), tau * kbar[..., d], rtol=0, atol=1e-8)
    t = 1e-5
    _, lp, _ = oracle.prefill(Q + (t / tau) * R, R, K, V, qk_scale=tau, stats=True)
    _, lm, _ = oracle.prefill(Q - (t / tau) * R, R, K, V, qk_scale=tau, stats=True)
    np.testing.assert_allclose(rho * (lp - lm) / (2 * t), sbar, rtol=0, atol=1e-8)
    c = rand(g, D)
    _, ls, _ = oracle.prefill(Q, R, K + c, V, qk_scale=tau, stats=True)
    np.testing.assert_allclose(ls, lse + tau * (Q @ c), rtol=0, atol=1e-12)
    z0 = tau * (Q[0, :, 0] @ K[0, 0, 0])
    np.testing.assert_allclose(lse[0, :, 0], z0, rtol=0, atol=1e-14)
    z1 = tau * (Q[0, :, 1] @ K[0, 0, 1])
    zz = tau * (Q[0, :, 1] @ K[0, 0, 0])
    np.testing.assert_allclose(lse[0, :, 1], np.logaddexp(zz, z1), rtol=0, atol=1e-14)


# ---------------------------------------------------------------- varlen
def test_packed_varlen_equals_per_sequence_and_empty_sequence_is_zero():
    g = rng(16)
    Hq, Hkv, D = 4, 2, 8
    lens = np.array([5, 0, 1, 12], dtype=np.int64)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
    T = int(lens.sum())
    q, r = rand(g, len(lens), Hq, D), rand(g, len(lens), Hq, D)
    k, v = rand(g, T, Hkv, D), rand(g, T, Hkv, D)
    o = oracle.decode(q, r, k, v, seq_start=starts, seq_len=lens)
    for b, (s0, n) in enumerate(zip(starts, lens)):
        if n == 0:
            np.testing.assert_array_equal(o[b], 0.0)
            continue
        ob = oracle.decode(q[b:b + 1], r[b:b + 1], k[None, s0:s0 + n], v[None, s0:s0 + n])
        np.testing.assert_allclose(o[b], ob[0], rtol=0, atol=1e-14)
        np.testing.assert_allclose(
            oracle.decode(q[b:b + 1], None, k[None, s0:s0 + n], v[None, s0:s0 + n])[0],
            sdpa_decode(q[b:b + 1], k[None, s0:s0 + n], v[None, s0:s0 + n], 1 / math.sqrt(D))[0],
            rtol=0, atol=1e-13)


def test_rows_subset_matches_full():
    g = rng(17)
    q, r = rand(g, 2, 4, 8), rand(g, 2, 4, 8)
    k, v = rand(g, 2, 13, 2, 8), rand(g, 2, 13, 2, 8)
    full = oracle.decode(q, r, k, v)
    rows = np.array([[1, 3], [0, 0], [1, 1]])
    sub = oracle.decode(q, r, k, v, rows=rows)
    np.testing.assert_array_equal(sub, full[rows[:, 0], rows[:, 1]])
    Q, R = rand(g, 2, 2, 9, 4), rand(g, 2, 2, 9, 4)
    K, V = rand(g, 2, 1, 9, 4), rand(g, 2, 1, 9, 4)
    full = oracle.prefill(Q, R, K, V)
    rows = np.array([[1, 1, 8], [0, 0, 0], [1, 0, 4]])
    np.testing.assert_array_equal(oracle.prefill(Q, R, K, V, rows=rows),
                                  full[rows[:, 0], rows[:, 1], rows[:, 2]])


def test_bf16_and_f32_inputs_are_widened_exactly():
    import synth
    g = rng(18)
    x = (rand(g, 1, 2, 16) * 0.3).astype(np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)       # truncation: exact bf16 values
    xb = synth.bf16_bits_to_f32(bits)
    kb = (rand(g, 1, 9, 2, 16).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    vb = (rand(g, 1, 9, 2, 16).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    o_bits = oracle.decode(bits, bits, kb, vb)
    o_f32 = oracle.decode(xb, xb, synth.bf16_bits_to_f32(kb), synth.bf16_bits_to_f32(vb))
    o_f64 = oracle.decode(xb.astype(np.float64), xb.astype(np.float64),
                          synth.bf16_bits_to_f32(kb).astype(np.float64),
                          synth.bf16_bits_to_f32(vb).astype(np.float64))
    np.testing.assert_array_equal(o_bits, o_f32)
    np.testing.assert_array_equal(o_bits, o_f64)


# ---------------------------------------------------------------- split-state algebra
def test_split_state_merge_algebra_matches_oracle():
    """The streaming state the GPU kernels carry -- running max m, l = sum e,
    S = sum e (s - pi), A = sum e v, B = sum e (s - pi) v, with a fixed pivot
    pi -- merged over an arbitrary partition of the keys and finalised as
    o = (A + B - (S / l) A) / l, equals the oracle (exact algebra)."""
    g = rng(19)
    L, D = 77, 6
    q, r = rand(g, 1, 1, D), rand(g, 1, 1, D) * 3
    k, v = rand(g, 1, L, 1, D) + 5.0, rand(g, 1, L, 1, D)
    K, V = k[0, :, 0], v[0, :, 0]
    z = (K @ q[0, 0]) / math.sqrt(D)
    s = K @ r[0, 0]
    pi = s[0]
    cuts = [0, 5, 6, 40, 41, 77]
    parts = []
    for a, b in zip(cuts[:-1], cuts[1:]):
        m = z[a:b].max()
        e = np.exp(z[a:b] - m)
        sp = s[a:b] - pi
        parts.append((m, e.sum(), e @ sp, e @ V[a:b], (e * sp) @ V[a:b]))
    M = max(p[0] for p in parts)
    al = [math.exp(p[0] - M) for p in parts]
    l = sum(a * p[1] for a, p in zip(al, parts))
    S = sum(a * p[2] for a, p in zip(al, parts))
    A = sum(a * p[3] for a, p in zip(al, parts))
    Bm = sum(a * p[4] for a, p in zip(al, parts))
    o = (A + Bm - (S / l) * A) / l
    np.testing.assert_allclose(o, oracle.decode(q, r, k, v)[0, 0], rtol=0, atol=1e-12)


# ---------------------------------------------------------------- P13 (round-off only)
def test_mpmath_fifty_digits_tiny():
    mpmath.mp.dps = 50
    g = rng(20)
    for L, D in [(1, 3), (3, 2), (8, 4)]:
        q, r = rand(g, 1, 1, D), rand(g, 1, 1, D)
        k, v = rand(g, 1, L, 1, D), rand(g, 1, L, 1, D)
        tau = mpmath.mpf(1) / mpmath.sqrt(D)
        K = [[mpmath.mpf(float(x)) for x in row] for row in k[0, :, 0]]
        Vv = [[mpmath.mpf(float(x)) for x in row] for row in v[0, :, 0]]
        qq = [mpmath.mpf(float(x)) for x in q[0, 0]]
        rr = [mpmath.mpf(float(x)) for x in r[0, 0]]
        z = [tau * mpmath.fsum(a * b for a, b in zip(qq, kr)) for kr in K]
        s = [mpmath.fsum(a * b for a, b in zip(rr, kr)) for kr in K]
        e = [mpmath.exp(x) for x in z]
        tot = mpmath.fsum(e)
        w = [x / tot for x in e]
        sb = mpmath.fsum(a * b for a, b in zip(w, s))
        ref = [mpmath.fsum(w[j] * (1 + s[j] - sb) * Vv[j][d] for j in range(L)) for d in range(D)]
        o = oracle.decode(q, r, k, v)[0, 0]
        np.testing.assert_allclose(o, np.array([float(x) for x in ref]), rtol=0, atol=2e-15)
