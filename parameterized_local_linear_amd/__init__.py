"""Python binding of the MI355X Parallax attention library.

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libparallax_hip.so`` (built in-tree by
``python -m parameterized_local_linear_amd.build``). PyTorch provides device
memory and the current stream; there is no CPU or PyTorch fallback, and a
missing library raises.

Entry points mirror the C ABI (include/parallax.h):
  decode(q, r, k, v, ...)          Parallax decode, q/r [B, Hq, D] or [B, 1, Hq, D]
  decode_noalloc(q, r, k, v, ...)  the same with the library's own device workspace
  softmax_decode(q, k, v, ...)     the same kernels with the probe path compiled out
  prefill(q, r, k, v, ...)         causal Parallax prefill on [B, H, L, D]
  prefill_backward(...)            its gradients dq, dr, dk, dv
  prefill_varlen(...), prefill_varlen_backward(...)
                                   the same on packed [T, H, D] sequences
The pages' names: ``parallax_decode`` aliases decode, and ``parallax_func``
is the prefill as a differentiable torch function (forward and backward on
these kernels).
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libparallax_hip.so")

PLX_F32, PLX_BF16 = 0, 1
NOALLOC_SCRATCH_BYTES = 8 << 20  # PLX_NOALLOC_SCRATCH_BYTES
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported configuration",
          3: "workspace missing or too small", 4: "HIP runtime error"}

_lib = None


class ParallaxError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {STATUS.get(status, status)} (status {status})")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m parameterized_local_linear_amd.build` (there is no fallback)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        L.parallax_abi_version.argtypes = []
        L.parallax_abi_version.restype = i32
        L.parallax_status_string.argtypes = [i32]
        L.parallax_status_string.restype = ctypes.c_char_p
        L.parallax_decode_workspace_bytes.argtypes = [i32] * 8
        L.parallax_decode_workspace_bytes.restype = sz
        L.parallax_decode_num_splits.argtypes = [i32] * 8
        L.parallax_decode_num_splits.restype = i32
        L.parallax_decode.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp,
                                      f32, f32, i32, i32, vp, sz, vp]
        L.parallax_decode.restype = i32
        L.parallax_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                              vp, f32, f32, i32, i32, vp]
        L.parallax_decode_noalloc.restype = i32
        L.softmax_decode.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp, f32,
                                     i32, i32, vp, sz, vp]
        L.softmax_decode.restype = i32
        L.parallax_prefill.argtypes = [vp] * 8 + [i32] * 6 + [vp, f32, f32, i32, vp]
        L.parallax_prefill.restype = i32
        L.parallax_decode_record_bytes.argtypes = [i32, i32, i32, i32]
        L.parallax_decode_record_bytes.restype = sz
        L.parallax_decode_partial.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp,
                                              f32, f32, i32, i32, vp, sz, vp]
        L.parallax_decode_partial.restype = i32
        L.parallax_decode_merge.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, vp]
        L.parallax_decode_merge.restype = i32
        L.parallax_prefill_backward_workspace_bytes.argtypes = [i32, i32, i32]
        L.parallax_prefill_backward_workspace_bytes.restype = sz
        L.parallax_prefill_backward.argtypes = [vp] * 13 + [i32] * 6 + [vp, f32, f32, i32, vp, sz,
                                                                         vp]
        L.parallax_prefill_backward.restype = i32
        L.parallax_prefill_varlen.argtypes = [vp] * 9 + [i32] * 7 + [vp, f32, f32, i32, vp, sz, vp]
        L.parallax_prefill_varlen_workspace_bytes.argtypes = [i32, i32, i32]
        L.parallax_prefill_varlen_workspace_bytes.restype = sz
        L.parallax_prefill_varlen.restype = i32
        L.parallax_prefill_varlen_backward.argtypes = [vp] * 14 + [i32] * 7 + [vp, f32, f32, i32,
                                                                              vp, sz, vp]
        L.parallax_prefill_varlen_backward.restype = i32
        _lib = L
    return _lib


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return PLX_F32
    if t.dtype == torch.bfloat16:
        return PLX_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(t: torch.Tensor, name: str, dtype, device):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype or t.device != device:
        raise ValueError(f"{name} must be {dtype} on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


MASK_BLOCK = 128  # positions per block of a block-sparse mask


def _check_mask(m, shape, device):
    """A block mask: None, or a contiguous bool / uint8 GPU tensor of `shape`."""
    if m is None:
        return None
    if not m.is_cuda or m.device != device or m.dtype not in (torch.bool, torch.uint8):
        raise ValueError(f"block_mask must be a bool or uint8 tensor on {device}")
    if not m.is_contiguous() or tuple(m.shape) != tuple(shape):
        raise ValueError(f"block_mask must be contiguous {tuple(shape)}")
    return m


def decode_workspace_bytes(B, Hq, Hkv, D, kv_len, dtype_code, num_splits=0, window=0) -> int:
    return int(lib().parallax_decode_workspace_bytes(B, Hq, Hkv, D, kv_len, window, dtype_code,
                                                     num_splits))


def decode_num_splits(B, Hq, Hkv, D, kv_len, dtype_code, num_splits=0, window=0) -> int:
    return int(lib().parallax_decode_num_splits(B, Hq, Hkv, D, kv_len, window, dtype_code,
                                                num_splits))


def _decode_impl(q, r, k, v, qk_scale, rk_scale, cu_seqlens_k, kv_len, num_splits, out,
                 workspace, parallax, window, block_mask=None, noalloc=False):
    L_ = lib()
    squeeze = q.dim() == 4
    if squeeze:                       # the pages' (B, 1, H, D)
        if q.shape[1] != 1:
            raise ValueError("decode takes one query token per sequence")
        q = q[:, 0]
        if r is not None:
            r = r[:, 0]
    B, Hq, D = q.shape
    dev, dt = q.device, q.dtype
    _check(q, "q", dt, dev)
    if parallax:
        _check(r, "r", dt, dev)
        if r.shape != q.shape:
            raise ValueError("r must have q's shape")
    _check(k, "k", dt, dev)
    _check(v, "v", dt, dev)
    if k.shape != v.shape:
        raise ValueError("k and v must have the same shape")
    if cu_seqlens_k is None:
        if k.dim() != 4 or k.shape[0] != B or k.shape[3] != D:
            raise ValueError("dense k/v must be [B, kv_len, Hkv, D]")
        kv_len = k.shape[1]
        Hkv = k.shape[2]
    else:
        _check(cu_seqlens_k, "cu_seqlens_k", torch.int32, dev)
        if cu_seqlens_k.shape != (B + 1,):
            raise ValueError("cu_seqlens_k must be int32 [B + 1]")
        if k.dim() != 3 or k.shape[2] != D:
            raise ValueError("packed k/v must be [total_tokens, Hkv, D]")
        if kv_len is None:
            raise ValueError("packed decode needs kv_len (the maximum sequence length)")
        Hkv = k.shape[1]
    code = _dtype_code(q)
    _check_mask(block_mask, (B, Hkv, -(-int(kv_len) // MASK_BLOCK)), dev)
    if qk_scale is None:
        qk_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=dt, device=dev)
    else:
        _check(out, "out", dt, dev)
        if out.shape != (B, Hq, D):
            raise ValueError("out must be [B, Hq, D]")
    stream = _stream_handle(dev)
    if noalloc:
        st = L_.parallax_decode_noalloc(_ptr(q), _ptr(r), _ptr(k), _ptr(v), _ptr(out),
                                        _ptr(cu_seqlens_k), B, Hq, Hkv, D, int(kv_len), int(window),
                                        _ptr(block_mask), float(qk_scale), float(rk_scale), code,
                                        int(num_splits), stream)
        if st != 0:
            raise ParallaxError(st, "parallax_decode_noalloc")
        return out[:, None] if squeeze else out
    need = decode_workspace_bytes(B, Hq, Hkv, D, int(kv_len), code, num_splits, window)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if parallax:
        st = L_.parallax_decode(_ptr(q), _ptr(r), _ptr(k), _ptr(v), _ptr(out), _ptr(cu_seqlens_k),
                                B, Hq, Hkv, D, int(kv_len), int(window), _ptr(block_mask),
                                float(qk_scale), float(rk_scale), code, int(num_splits),
                                _ptr(workspace), ws_bytes, stream)
        what = "parallax_decode"
    else:
        st = L_.softmax_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(cu_seqlens_k), B, Hq, Hkv,
                               D, int(kv_len), int(window), _ptr(block_mask), float(qk_scale),
                               code, int(num_splits), _ptr(workspace), ws_bytes, stream)
        what = "softmax_decode"
    if st != 0:
        raise ParallaxError(st, what)
    return out[:, None] if squeeze else out


def decode(q, r, k, v, qk_scale=None, rk_scale=1.0, *, cu_seqlens_k=None, kv_len=None,
           num_splits=0, out=None, workspace=None, window=0, block_mask=None):
    """Parallax decode. q, r: [B, Hq, D] (or [B, 1, Hq, D]); k, v: [B, kv_len, Hkv, D],
    or packed [T, Hkv, D] with int32 ``cu_seqlens_k`` [B + 1] and ``kv_len`` = max length.
    ``window`` > 0: each sequence's last ``window`` keys only. ``block_mask``: optional
    bool/uint8 [B, Hkv, ceil(kv_len / 128)] over 128-key blocks (the block holding a
    sequence's last key is always visible)."""
    return _decode_impl(q, r, k, v, qk_scale, rk_scale, cu_seqlens_k, kv_len, num_splits, out,
                        workspace, True, window, block_mask)


def decode_noalloc(q, r, k, v, qk_scale=None, rk_scale=1.0, *, cu_seqlens_k=None, kv_len=None,
                   num_splits=0, out=None, window=0, block_mask=None):
    """decode() through parallax_decode_noalloc: the split records live in the
    library's own device array (NOALLOC_SCRATCH_BYTES per device), so the call
    needs no workspace. Calls on one device must not overlap in time."""
    return _decode_impl(q, r, k, v, qk_scale, rk_scale, cu_seqlens_k, kv_len, num_splits, out,
                        None, True, window, block_mask, noalloc=True)


def softmax_decode(q, k, v, qk_scale=None, *, cu_seqlens_k=None, kv_len=None, num_splits=0,
                   out=None, workspace=None, window=0, block_mask=None):
    """Softmax-attention decode on the same kernels (the Parallax correction compiled out)."""
    return _decode_impl(q, None, k, v, qk_scale, 1.0, cu_seqlens_k, kv_len, num_splits, out,
                        workspace, False, window, block_mask)


def decode_partial(q, r, k, v, qk_scale=None, rk_scale=1.0, *, cu_seqlens_k=None, kv_len=None,
                   num_splits=0, records=None, window=0, block_mask=None):
    """Streaming half of decode: returns (records, n) with records a float32
    [B, Hq, n, 2D + 4] tensor (A, B, m, l, S, pi per split). r=None: softmax records."""
    L_ = lib()
    B, Hq, D = q.shape
    dev, dt = q.device, q.dtype
    _check(q, "q", dt, dev)
    if r is not None:
        _check(r, "r", dt, dev)
    _check(k, "k", dt, dev)
    _check(v, "v", dt, dev)
    if cu_seqlens_k is None:
        kv_len, Hkv = k.shape[1], k.shape[2]
    else:
        _check(cu_seqlens_k, "cu_seqlens_k", torch.int32, dev)
        Hkv = k.shape[1]
    code = _dtype_code(q)
    _check_mask(block_mask, (B, Hkv, -(-int(kv_len) // MASK_BLOCK)), dev)
    if qk_scale is None:
        qk_scale = 1.0 / math.sqrt(D)
    n = decode_num_splits(B, Hq, Hkv, D, int(kv_len), code, num_splits, window)
    if n == 0:
        raise ParallaxError(1, "parallax_decode_partial")
    if records is None:
        records = torch.empty((B, Hq, n, 2 * D + 4), dtype=torch.float32, device=dev)
    st = L_.parallax_decode_partial(_ptr(q), _ptr(r), _ptr(k), _ptr(v), _ptr(cu_seqlens_k), B, Hq,
                                    Hkv, D, int(kv_len), int(window), _ptr(block_mask),
                                    float(qk_scale), float(rk_scale), code,
                                    int(num_splits), _ptr(records),
                                    records.numel() * records.element_size(), _stream_handle(dev))
    if st != 0:
        raise ParallaxError(st, "parallax_decode_partial")
    return records, n


def decode_merge(records, dtype=torch.bfloat16, with_probe=True, out=None):
    """Merge records [B, Hq, n, 2D + 4] (float32) into o [B, Hq, D]."""
    L_ = lib()
    B, Hq, n, F = records.shape
    D = (F - 4) // 2
    _check(records, "records", torch.float32, records.device)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=dtype, device=records.device)
    st = L_.parallax_decode_merge(_ptr(records), _ptr(out), B, Hq, D, n, _dtype_code(out),
                                  1 if with_probe else 0, _stream_handle(records.device))
    if st != 0:
        raise ParallaxError(st, "parallax_decode_merge")
    return out


def prefill(q, r, k, v, qk_scale=None, rk_scale=1.0, *, out=None, return_stats=False, window=0,
            vbar_out=None, block_mask=None):
    """Causal Parallax prefill. q, r: [B, Hq, L, D]; k, v: [B, Hkv, L, D] -> o [B, Hq, L, D]
    (plus fp32 lse and sbar [B, Hq, L] with return_stats=True). ``window`` > 0: query i
    sees keys i - window + 1 .. i. ``vbar_out``: optional tensor shaped like o that
    receives the softmax readout (a backward statistic). ``block_mask``: optional
    bool/uint8 [B, Hkv, nb, nb], nb = ceil(L / 128): [qb, kb] lets query block qb see
    key block kb (the diagonal block is always visible)."""
    L_ = lib()
    B, Hq, L, D = q.shape
    dev, dt = q.device, q.dtype
    for t, name in ((q, "q"), (r, "r"), (k, "k"), (v, "v")):
        _check(t, name, dt, dev)
    if r.shape != q.shape:
        raise ValueError("r must have q's shape")
    if k.shape != v.shape or k.dim() != 4 or k.shape[0] != B or k.shape[2] != L or k.shape[3] != D:
        raise ValueError("k, v must be [B, Hkv, L, D]")
    Hkv = k.shape[1]
    code = _dtype_code(q)
    nb = -(-L // MASK_BLOCK)
    _check_mask(block_mask, (B, Hkv, nb, nb), dev)
    if qk_scale is None:
        qk_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check(out, "out", dt, dev)
        if out.shape != q.shape:
            raise ValueError("out must have q's shape")
    lse = sbar = None
    if return_stats:
        lse = torch.empty((B, Hq, L), dtype=torch.float32, device=dev)
        sbar = torch.empty((B, Hq, L), dtype=torch.float32, device=dev)
    if vbar_out is not None:
        _check(vbar_out, "vbar_out", dt, dev)
        if vbar_out.shape != q.shape:
            raise ValueError("vbar_out must have q's shape")
    st = L_.parallax_prefill(_ptr(q), _ptr(r), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(sbar),
                             _ptr(vbar_out), B, Hq, Hkv, L, D, int(window), _ptr(block_mask),
                             float(qk_scale), float(rk_scale), code, _stream_handle(dev))
    if st != 0:
        raise ParallaxError(st, "parallax_prefill")
    return (out, lse, sbar) if return_stats else out


def prefill_backward(q, r, k, v, o, d_o, lse, sbar, qk_scale=None, rk_scale=1.0, *,
                     workspace=None, out=None, window=0, vbar=None, block_mask=None):
    """Gradients of the causal prefill: (dq, dr, dk, dv) for the upstream
    gradient ``d_o``, from the forward's o, lse and sbar (prefill with
    return_stats=True on the same inputs and scales). ``out``: optional
    preallocated (dq, dr, dk, dv)."""
    L_ = lib()
    B, Hq, L, D = q.shape
    dev, dt = q.device, q.dtype
    for t, name in ((q, "q"), (r, "r"), (k, "k"), (v, "v"), (o, "o"), (d_o, "d_o")):
        _check(t, name, dt, dev)
    for t, name in ((lse, "lse"), (sbar, "sbar")):
        _check(t, name, torch.float32, dev)
        if t.shape != (B, Hq, L):
            raise ValueError(f"{name} must be float32 [B, Hq, L]")
    if r.shape != q.shape or o.shape != q.shape or d_o.shape != q.shape:
        raise ValueError("r, o and d_o must have q's shape")
    if k.shape != v.shape or k.dim() != 4 or k.shape[0] != B or k.shape[2] != L or k.shape[3] != D:
        raise ValueError("k, v must be [B, Hkv, L, D]")
    Hkv = k.shape[1]
    nb = -(-L // MASK_BLOCK)
    _check_mask(block_mask, (B, Hkv, nb, nb), dev)
    if qk_scale is None:
        qk_scale = 1.0 / math.sqrt(D)
    need = int(L_.parallax_prefill_backward_workspace_bytes(B, Hq, L))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    if out is None:
        out = (torch.empty_like(q), torch.empty_like(r), torch.empty_like(k), torch.empty_like(v))
    dq, dr, dk, dv = out
    for t, ref, name in ((dq, q, "dq"), (dr, q, "dr"), (dk, k, "dk"), (dv, k, "dv")):
        _check(t, name, dt, dev)
        if t.shape != ref.shape:
            raise ValueError(f"{name} must have shape {tuple(ref.shape)}")
    if vbar is not None:
        _check(vbar, "vbar", dt, dev)
        if vbar.shape != q.shape:
            raise ValueError("vbar must have q's shape")
    st = L_.parallax_prefill_backward(
        _ptr(q), _ptr(r), _ptr(k), _ptr(v), _ptr(o), _ptr(d_o), _ptr(lse), _ptr(sbar), _ptr(vbar),
        _ptr(dq),
        _ptr(dr), _ptr(dk), _ptr(dv), B, Hq, Hkv, L, D, int(window), _ptr(block_mask),
        float(qk_scale), float(rk_scale),
        _dtype_code(q), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream_handle(dev))
    if st != 0:
        raise ParallaxError(st, "parallax_prefill_backward")
    return dq, dr, dk, dv


class _ParallaxFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, r, k, v, qk_scale, rk_scale, window, save_vbar, block_mask):
        vbar = torch.empty_like(q) if save_vbar else None
        o, lse, sbar = prefill(q, r, k, v, qk_scale, rk_scale, return_stats=True, window=window,
                               vbar_out=vbar, block_mask=block_mask)
        ctx.save_for_backward(q, r, k, v, o, lse, sbar, vbar, block_mask)
        ctx.scales = (qk_scale, rk_scale)
        ctx.window = window
        return o

    @staticmethod
    def backward(ctx, d_o):
        q, r, k, v, o, lse, sbar, vbar, block_mask = ctx.saved_tensors
        grads = prefill_backward(q, r, k, v, o, d_o.contiguous(), lse, sbar, *ctx.scales,
                                 window=ctx.window, vbar=vbar, block_mask=block_mask)
        return (*grads, None, None, None, None, None)


def parallax_func(q, r, k, v, qk_scale=None, rk_scale=1.0, *, window=0, save_vbar=True,
                  block_mask=None):
    """Causal Parallax attention on [B, H, L, D] tensors, differentiable in
    q, r, k and v (the pages' training entry point); ``window`` and ``block_mask``
    as in prefill. ``save_vbar`` keeps the softmax readout for the backward (one
    more o-sized activation, one sweep over the keys fewer in the backward)."""
    if torch.is_grad_enabled() and any(t.requires_grad for t in (q, r, k, v)):
        return _ParallaxFunction.apply(q, r, k, v, qk_scale, rk_scale, window, save_vbar,
                                       block_mask)
    return prefill(q, r, k, v, qk_scale, rk_scale, window=window, block_mask=block_mask)


def _varlen_shapes(q, k, cu_seqlens, max_len):
    if q.dim() != 3 or k.dim() != 3 or q.shape[0] != k.shape[0] or q.shape[2] != k.shape[2]:
        raise ValueError("varlen q must be [T, Hq, D] and k [T, Hkv, D]")
    _check(cu_seqlens, "cu_seqlens", torch.int32, q.device)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be int32 [B + 1]")
    if max_len is None:  # one host read of the lengths when the caller does not know it
        max_len = int((cu_seqlens[1:] - cu_seqlens[:-1]).max().item())
    return cu_seqlens.numel() - 1, q.shape[1], k.shape[1], q.shape[2], max(int(max_len), 1)


def prefill_varlen(q, r, k, v, cu_seqlens, max_len=None, qk_scale=None, rk_scale=1.0, *,
                   out=None, return_stats=False, window=0, workspace=None, vbar_out=None,
                   block_mask=None):
    """Causal prefill of packed sequences: q, r [T, Hq, D]; k, v [T, Hkv, D]; int32
    ``cu_seqlens`` [B + 1]. Returns o [T, Hq, D] (plus fp32 lse, sbar [T, Hq]).
    ``block_mask``: optional [B, Hkv, nb, nb], nb = ceil(max_len / 128), over
    sequence-local blocks."""
    L_ = lib()
    dev, dt = q.device, q.dtype
    for t, name in ((q, "q"), (r, "r"), (k, "k"), (v, "v")):
        _check(t, name, dt, dev)
    if r.shape != q.shape or v.shape != k.shape:
        raise ValueError("r must have q's shape and v k's")
    B, Hq, Hkv, D, max_len = _varlen_shapes(q, k, cu_seqlens, max_len)
    T = q.shape[0]
    nb = -(-max_len // MASK_BLOCK)
    _check_mask(block_mask, (B, Hkv, nb, nb), dev)
    if qk_scale is None:
        qk_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    lse = sbar = None
    if return_stats:
        lse = torch.empty((T, Hq), dtype=torch.float32, device=dev)
        sbar = torch.empty((T, Hq), dtype=torch.float32, device=dev)
    if workspace is None:
        need = int(L_.parallax_prefill_varlen_workspace_bytes(Hq, T, 0))
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if vbar_out is not None:
        _check(vbar_out, "vbar_out", dt, dev)
        if vbar_out.shape != q.shape:
            raise ValueError("vbar_out must have q's shape")
    st = L_.parallax_prefill_varlen(_ptr(q), _ptr(r), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                    _ptr(sbar), _ptr(vbar_out), _ptr(cu_seqlens), B, Hq, Hkv, max_len, T, D,
                                    int(window), _ptr(block_mask), float(qk_scale),
                                    float(rk_scale), _dtype_code(q),
                                    _ptr(workspace), workspace.numel() * workspace.element_size(),
                                    _stream_handle(dev))
    if st != 0:
        raise ParallaxError(st, "parallax_prefill_varlen")
    return (out, lse, sbar) if return_stats else out


def prefill_varlen_backward(q, r, k, v, o, d_o, lse, sbar, cu_seqlens, max_len=None,
                            qk_scale=None, rk_scale=1.0, *, window=0, workspace=None, out=None,
                            vbar=None, block_mask=None):
    """Gradients (dq, dr, dk, dv) of prefill_varlen from its o, lse and sbar."""
    L_ = lib()
    dev, dt = q.device, q.dtype
    for t, name in ((q, "q"), (r, "r"), (k, "k"), (v, "v"), (o, "o"), (d_o, "d_o")):
        _check(t, name, dt, dev)
    B, Hq, Hkv, D, max_len = _varlen_shapes(q, k, cu_seqlens, max_len)
    T = q.shape[0]
    for t, name in ((lse, "lse"), (sbar, "sbar")):
        _check(t, name, torch.float32, dev)
        if t.shape != (T, Hq):
            raise ValueError(f"{name} must be float32 [T, Hq]")
    nb = -(-max_len // MASK_BLOCK)
    _check_mask(block_mask, (B, Hkv, nb, nb), dev)
    if qk_scale is None:
        qk_scale = 1.0 / math.sqrt(D)
    need = int(L_.parallax_prefill_varlen_workspace_bytes(Hq, T, 1))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    if out is None:
        out = (torch.empty_like(q), torch.empty_like(r), torch.empty_like(k), torch.empty_like(v))
    dq, dr, dk, dv = out
    if vbar is not None:
        _check(vbar, "vbar", dt, dev)
        if vbar.shape != q.shape:
            raise ValueError("vbar must have q's shape")
    st = L_.parallax_prefill_varlen_backward(
        _ptr(q), _ptr(r), _ptr(k), _ptr(v), _ptr(o), _ptr(d_o), _ptr(lse), _ptr(sbar), _ptr(vbar),
        _ptr(cu_seqlens), _ptr(dq), _ptr(dr), _ptr(dk), _ptr(dv), B, Hq, Hkv, max_len, T, D,
        int(window), _ptr(block_mask), float(qk_scale), float(rk_scale), _dtype_code(q),
        _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream_handle(dev))
    if st != 0:
        raise ParallaxError(st, "parallax_prefill_varlen_backward")
    return dq, dr, dk, dv


class _ParallaxVarlenFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, r, k, v, cu_seqlens, max_len, qk_scale, rk_scale, window, save_vbar,
                block_mask):
        vbar = torch.empty_like(q) if save_vbar else None
        o, lse, sbar = prefill_varlen(q, r, k, v, cu_seqlens, max_len, qk_scale, rk_scale,
                                      return_stats=True, window=window, vbar_out=vbar,
                                      block_mask=block_mask)
        ctx.save_for_backward(q, r, k, v, o, lse, sbar, cu_seqlens, vbar, block_mask)
        ctx.args = (max_len, qk_scale, rk_scale, window)
        return o

    @staticmethod
    def backward(ctx, d_o):
        q, r, k, v, o, lse, sbar, cu, vbar, block_mask = ctx.saved_tensors
        max_len, qk_scale, rk_scale, window = ctx.args
        grads = prefill_varlen_backward(q, r, k, v, o, d_o.contiguous(), lse, sbar, cu, max_len,
                                        qk_scale, rk_scale, window=window, vbar=vbar,
                                        block_mask=block_mask)
        return (*grads, None, None, None, None, None, None, None)


def parallax_varlen_func(q, r, k, v, cu_seqlens, max_len=None, qk_scale=None, rk_scale=1.0, *,
                         window=0, save_vbar=True, block_mask=None):
    """Differentiable causal Parallax attention on packed sequences (the pages'
    parallax_varlen_func): q, r [T, Hq, D]; k, v [T, Hkv, D]; int32 cu_seqlens [B + 1]."""
    if max_len is None:
        max_len = int((cu_seqlens[1:] - cu_seqlens[:-1]).max().item())
    if torch.is_grad_enabled() and any(t.requires_grad for t in (q, r, k, v)):
        return _ParallaxVarlenFunction.apply(q, r, k, v, cu_seqlens, max_len, qk_scale, rk_scale,
                                             window, save_vbar, block_mask)
    return prefill_varlen(q, r, k, v, cu_seqlens, max_len, qk_scale, rk_scale, window=window,
                          block_mask=block_mask)


parallax_decode = decode

__all__ = ["decode", "softmax_decode", "prefill", "prefill_backward", "prefill_varlen",
           "prefill_varlen_backward", "parallax_varlen_func", "decode_partial",
           "decode_merge", "parallax_decode", "parallax_func", "decode_workspace_bytes",
           "decode_num_splits", "lib", "ParallaxError", "LIB_PATH"]
