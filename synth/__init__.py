"""Seeded synthetic inputs for the Parallax attention tests and benchmark.

This package draws numbers and nothing else: no attention arithmetic lives
here. Both the CPU oracle side and the GPU side of the tests take their inputs
from it, so the two see bit-identical values. The generator is counter based
(SplitMix64 words -> Box-Muller normals, see ``synth.c``), so any slice of a
tensor can be regenerated on its own: a sampled check at a large size only
regenerates the sequences it looks at.

Arrays come back as numpy: ``float32`` for fp32 and ``uint16`` bit patterns
for bf16 (numpy has no bfloat16; ``torch.from_numpy(a).view(torch.bfloat16)``
reinterprets them without a copy).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# PLX_SANITIZED_HOST_LIBS=1 selects the AddressSanitizer + UBSan build
# (libsynth_san.so, from build(sanitize=True)); the process must then preload
# gcc's libasan and libubsan.
_SANITIZED = os.environ.get("PLX_SANITIZED_HOST_LIBS") == "1"
_LIB_PATH = os.path.join(_HERE, "libsynth_san.so" if _SANITIZED else "libsynth.so")
_lib = None

F32 = 0
BF16 = 1
BASE_SEED = 20261203
# tensor ids inside one seed: one independent stream each
TID_Q, TID_R, TID_K, TID_V, TID_SHIFT, TID_LENGTHS = 0, 1, 2, 3, 4, 5
TID_DO = 6  # upstream gradient dLoss/do of the training backward
TID_MASK = 7  # block-sparse masks


def build(sanitize: bool = False) -> str:
    """Compile ``libsynth.so`` next to this file (gcc, OpenMP).
    sanitize=True builds libsynth_san.so with AddressSanitizer and UBSan
    instead (host test tier)."""
    out = os.path.join(_HERE, "libsynth_san.so" if sanitize else "libsynth.so")
    opt = (["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
            "-fno-sanitize-recover=undefined"] if sanitize else ["-O2"])
    cmd = ["gcc", *opt, "-fopenmp", "-fPIC", "-shared", "-std=c11",
           os.path.join(_HERE, "synth.c"), "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(_LIB_PATH)
        lib.synth_normal.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                     ctypes.c_uint64, ctypes.c_double, ctypes.c_int,
                                     ctypes.c_void_p]
        lib.synth_normal.restype = None
        lib.synth_uniform_int.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                          ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
        lib.synth_uniform_int.restype = None
        lib.synth_word.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64]
        lib.synth_word.restype = ctypes.c_uint64
        lib.synth_bf16_from_double.argtypes = [ctypes.c_double]
        lib.synth_bf16_from_double.restype = ctypes.c_uint16
        _lib = lib
    return _lib


def word(seed: int, tid: int, p: int) -> int:
    """SplitMix64 output ``p`` of the stream (seed, tid)."""
    return int(_load().synth_word(seed, tid, p))


def bf16_from_double(x: float) -> int:
    return int(_load().synth_bf16_from_double(float(x)))


def normal(seed: int, tid: int, shape, scale: float = 1.0, dtype: int = F32,
           first: int = 0, out: np.ndarray | None = None) -> np.ndarray:
    """Elements ``first ..`` of stream (seed, tid) as N(0,1)*scale, rounded once."""
    count = int(np.prod(shape)) if len(tuple(shape)) else 1
    npdt = np.float32 if dtype == F32 else np.uint16
    if out is None:
        out = np.empty(shape, dtype=npdt)
    assert out.dtype == npdt and out.size == count and out.flags.c_contiguous
    _load().synth_normal(seed, tid, first, count, float(scale), dtype,
                         out.ctypes.data_as(ctypes.c_void_p))
    return out


def uniform_int(seed: int, tid: int, count: int, lo: int, hi: int) -> np.ndarray:
    out = np.empty(count, dtype=np.int64)
    _load().synth_uniform_int(seed, tid, count, lo, hi, out.ctypes.data_as(ctypes.c_void_p))
    return out


def block_mask(seed: int, shape, density: float) -> np.ndarray:
    """A uint8 block mask of the given shape: each entry 1 with probability
    ``density`` (independent draws of stream (seed, TID_MASK), in units of 1/1e6)."""
    count = int(np.prod(shape))
    u = uniform_int(seed, TID_MASK, count, 0, 999999)
    return (u < int(round(density * 1e6))).astype(np.uint8).reshape(shape)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32 exactly."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def to_f64(a: np.ndarray, dtype: int) -> np.ndarray:
    return (a if dtype == F32 else bf16_bits_to_f32(a)).astype(np.float64)


# --------------------------------------------------------------------------
# Workload recipes. Shapes and distributions of the five measured workloads;
# index 1..5 in the order they are listed in the benchmark description.
# --------------------------------------------------------------------------
@dataclass
class DecodeSpec:
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    L: int                     # dense length, or max length when varlen
    dtype: int
    scale: float               # std of q, r, K, V
    seed: int
    varlen: tuple | None = None  # (lo, hi) inclusive length range
    lengths: np.ndarray | None = field(default=None, repr=False)

    def seq_lengths(self) -> np.ndarray:
        if self.lengths is not None:
            return self.lengths
        if self.varlen is None:
            return np.full(self.B, self.L, dtype=np.int64)
        lo, hi = self.varlen
        return uniform_int(self.seed, TID_LENGTHS, self.B, lo, hi)


@dataclass
class PrefillSpec:
    name: str
    B: int
    Hq: int
    Hkv: int
    L: int
    D: int
    dtype: int
    scale: float
    seed: int


def decode_spec(idx: int) -> DecodeSpec:
    s = 1.0 / np.sqrt(128.0)
    if idx == 1:
        return DecodeSpec("tiny-decode-fp32 B1 Hq2 Hkv2 D64 L256", 1, 2, 2, 64, 256, F32, 1.0,
                          BASE_SEED + 1)
    if idx == 2:
        return DecodeSpec("long-decode-bf16 B1 Hq16 Hkv8 D128 L32768", 1, 16, 8, 128, 32768, BF16,
                          s, BASE_SEED + 2)
    if idx == 3:
        spec = DecodeSpec("varlen-decode-bf16 B64 Hq16 Hkv8 D128 L~U[1024,8192]", 64, 16, 8, 128,
                          8192, BF16, s, BASE_SEED + 3, varlen=(1024, 8192))
        spec.L = int(spec.seq_lengths().max())
        return spec
    if idx == 4:
        return DecodeSpec("large-batch-decode-bf16 B2048 Hq16 Hkv8 D128 L2048", 2048, 16, 8, 128,
                          2048, BF16, s, BASE_SEED + 4)
    raise ValueError(idx)


def pages_decode_grid() -> list:
    """The decode shapes of the pages' benchmark tables (PyPI README of
    parallax-kernel, small- and large-batch decode tables): multi-head
    (Hq = Hkv = 8), D = 128, bf16, B in {1, 32}, L in {512, 1024, 4096, 16384}."""
    s = 1.0 / np.sqrt(128.0)
    out = []
    for i, (B, L) in enumerate((B, L) for B in (1, 32) for L in (512, 1024, 4096, 16384)):
        out.append(DecodeSpec(f"pages-grid-decode-bf16 B{B} H8 D128 L{L}", B, 8, 8, 128, L, BF16,
                              s, BASE_SEED + 100 + i))
    return out


def prefill_spec(idx: int = 5) -> PrefillSpec:
    assert idx == 5
    return PrefillSpec("causal-prefill-bf16 B8 L4096 Hq16 Hkv8 D128", 8, 16, 8, 4096, 128, BF16,
                       1.0 / np.sqrt(128.0), BASE_SEED + 5)


@dataclass
class VarlenPrefillSpec:
    name: str
    lengths: np.ndarray
    Hq: int
    Hkv: int
    D: int
    dtype: int
    scale: float
    seed: int


def prefill_varlen_spec() -> VarlenPrefillSpec:
    """Packed training batch: 16 sequences of U{256 .. 4096} tokens, Hq16 Hkv8 D128 bf16
    (the causal-prefill workload's heads with a length mix instead of one length)."""
    seed = BASE_SEED + 40
    lens = uniform_int(seed, TID_LENGTHS, 16, 256, 4096)
    return VarlenPrefillSpec("varlen-prefill-bf16 16 seqs L~U[256,4096] Hq16 Hkv8 D128", lens, 16,
                             8, 128, BF16, 1.0 / np.sqrt(128.0), seed)


def decode_qr(spec: DecodeSpec, r_zero: bool = False):
    """q, r as [B, Hq, D] arrays of the spec's dtype."""
    shp = (spec.B, spec.Hq, spec.D)
    q = normal(spec.seed, TID_Q, shp, spec.scale, spec.dtype)
    r = normal(spec.seed, TID_R, shp, spec.scale, spec.dtype)
    if r_zero:
        r[...] = 0
    return q, r


def decode_kv_rows(spec: DecodeSpec, tid: int, first_token: int, n_tokens: int,
                   out: np.ndarray | None = None) -> np.ndarray:
    """Tokens first_token .. +n_tokens of the K (tid 2) or V (tid 3) cache.

    The cache is one stream over the flattened [tokens, Hkv, D] array, dense
    [B, L, Hkv, D] or packed [sum L_b, Hkv, D] alike, so a sequence's rows can
    be regenerated without the rest.
    """
    row = spec.Hkv * spec.D
    return normal(spec.seed, tid, (n_tokens, spec.Hkv, spec.D), spec.scale, spec.dtype,
                  first=first_token * row, out=out)


def key_shift(seed: int, D: int) -> np.ndarray:
    """The constant key shift c ~ N(0,1)^D (float64, unrounded)."""
    x = normal(seed, TID_SHIFT, (D,), 1.0, F32)
    return x.astype(np.float64)
