"""Shared helpers for the GPU parity tests: seeded inputs (from ``synth``) moved to
the GPU, and the max-norm parity bar.

The bar: max |o - o_ref| <= tol * max |o_ref| with tol = 1e-5 for fp32 inputs
and 1e-2 for bf16 inputs, o_ref from the double-precision oracle on exactly
the values handed to the GPU.
"""
from __future__ import annotations

import numpy as np
import torch

import synth

TOL = {synth.F32: 1e-5, synth.BF16: 1e-2}


def to_gpu(a: np.ndarray, dtype: int) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype == synth.BF16:
        t = t.view(torch.bfloat16)
    return t.cuda()


def from_gpu(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def max_norm_err(o: np.ndarray, ref: np.ndarray) -> float:
    return float(np.abs(o - ref).max() / np.abs(ref).max())


def assert_parity(o: np.ndarray, ref: np.ndarray, dtype: int, what: str = "", tol=None):
    assert o.shape == ref.shape, (o.shape, ref.shape)
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    tol = TOL[dtype] if tol is None else tol
    err = max_norm_err(o, ref)
    assert err <= tol, f"{what}: max-norm error {err:.3e} > {tol:.0e}"
    return err


def decode_inputs(B, Hq, Hkv, D, lens, dtype, scale, seed, packed=False):
    """q, r [B,Hq,D]; K, V dense [B,L,Hkv,D] (lens all equal) or packed [T,Hkv,D]."""
    lens = np.asarray(lens, dtype=np.int64)
    q = synth.normal(seed, synth.TID_Q, (B, Hq, D), scale, dtype)
    r = synth.normal(seed, synth.TID_R, (B, Hq, D), scale, dtype)
    if packed:
        T = int(lens.sum())
        k = synth.normal(seed, synth.TID_K, (T, Hkv, D), scale, dtype)
        v = synth.normal(seed, synth.TID_V, (T, Hkv, D), scale, dtype)
    else:
        L = int(lens[0])
        assert np.all(lens == L)
        k = synth.normal(seed, synth.TID_K, (B, L, Hkv, D), scale, dtype)
        v = synth.normal(seed, synth.TID_V, (B, L, Hkv, D), scale, dtype)
    return q, r, k, v


def upload_decode_cache(spec: synth.DecodeSpec, tid: int, total_tokens: int,
                        chunk_tokens: int = 1 << 16) -> torch.Tensor:
    """Generate a K or V cache of ``total_tokens`` rows chunk by chunk into the GPU."""
    row = spec.Hkv * spec.D
    out = torch.empty((total_tokens, spec.Hkv, spec.D), dtype=torch.bfloat16
                      if spec.dtype == synth.BF16 else torch.float32, device="cuda")
    host = torch.empty((chunk_tokens, spec.Hkv, spec.D), dtype=out.dtype, pin_memory=True)
    hview = host.view(torch.int16).numpy().view(np.uint16) if spec.dtype == synth.BF16 \
        else host.numpy()
    t0 = 0
    while t0 < total_tokens:
        n = min(chunk_tokens, total_tokens - t0)
        buf = hview[:n]
        synth.normal(spec.seed, tid, (n, spec.Hkv, spec.D), spec.scale, spec.dtype,
                     first=t0 * row, out=buf)
        out[t0:t0 + n].copy_(host[:n])
        t0 += n
    torch.cuda.synchronize()
    return out
