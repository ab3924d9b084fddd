"""The C ABI library: it loads, exports every declared symbol, and rejects bad
arguments on the host before any launch (so these run without a GPU)."""
import ctypes
import os
import re

import pytest

import parameterized_local_linear_amd as plx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation first


def declared_functions():
    names = []
    inc = os.path.join(ROOT, "include")
    for fn in os.listdir(inc):
        if fn.endswith(".h"):
            text = open(os.path.join(inc, fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"^[A-Za-z_][\w\s\*]*?\b(\w+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "defined")))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert {"parallax_decode", "softmax_decode", "parallax_prefill",
            "parallax_decode_workspace_bytes", "parallax_abi_version"} <= set(names)
    lib = ctypes.CDLL(plx.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings():
    L = plx.lib()
    assert L.parallax_abi_version() == 5
    for s in range(5):
        assert L.parallax_status_string(s).decode() == plx.STATUS[s]
    assert L.parallax_status_string(99) == b"unknown status"


def _decode(**kw):
    a = dict(q=FAKE, r=FAKE, k=FAKE, v=FAKE, o=FAKE, cu=None, B=1, Hq=4, Hkv=2, D=128, L=64,
             W=0, mask=None, qk=0.1, rk=1.0, dt=1, ns=0, ws=None, wsb=0, stream=None)
    a.update(kw)
    return plx.lib().parallax_decode(a["q"], a["r"], a["k"], a["v"], a["o"], a["cu"], a["B"],
                                     a["Hq"], a["Hkv"], a["D"], a["L"], a["W"], a["mask"], a["qk"],
                                     a["rk"], a["dt"], a["ns"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), 1), (dict(Hq=0), 1), (dict(L=0), 1), (dict(Hq=6, Hkv=4), 1),
    (dict(q=None), 1), (dict(r=None), 1), (dict(k=None), 1), (dict(o=None), 1),
    (dict(D=96), 2), (dict(D=256), 2), (dict(dt=2), 2), (dict(ns=-1), 1),
    (dict(qk=float("nan")), 1), (dict(rk=float("inf")), 1), (dict(qk=0.0), 1),
    (dict(qk=-0.1), 1), (dict(W=-1), 1),
    (dict(ns=4, L=4096), 3), (dict(ns=4, L=4096, ws=FAKE, wsb=16), 3),
])
def test_decode_rejects_on_host(kw, status):
    # every case must fail validation: FAKE pointers may never reach a launch
    assert status != 0
    assert _decode(**kw) == status


def test_softmax_decode_and_prefill_reject_on_host():
    L = plx.lib()
    assert L.softmax_decode(FAKE, FAKE, FAKE, FAKE, None, 1, 4, 3, 128, 10, 0, None, 0.1, 1, 0, None, 0,
                            None) == 1
    assert L.softmax_decode(FAKE, FAKE, FAKE, FAKE, None, 1, 4, 2, 80, 10, 0, None, 0.1, 1, 0, None, 0,
                            None) == 2
    assert L.softmax_decode(FAKE, FAKE, FAKE, FAKE, None, 1, 4, 2, 128, 10, -3, None, 0.1, 1, 0, None, 0,
                            None) == 1
    args = [FAKE] * 5 + [None, None, None]
    assert L.parallax_prefill(*args, 1, 4, 2, 0, 128, 0, None, 0.1, 1.0, 1, None) == 1
    assert L.parallax_prefill(*args, 1, 4, 3, 16, 128, 0, None, 0.1, 1.0, 1, None) == 1
    assert L.parallax_prefill(*args, 1, 4, 2, 16, 72, 0, None, 0.1, 1.0, 1, None) == 2
    assert L.parallax_prefill(*args, 1, 4, 2, 16, 128, 0, None, 0.1, 1.0, 5, None) == 2
    assert L.parallax_prefill(*args, 1, 4, 2, 16, 128, -1, None, 0.1, 1.0, 1, None) == 1
    assert L.parallax_prefill(*args, 1, 4, 2, 16, 128, 0, None, -0.1, 1.0, 1, None) == 1
    assert L.parallax_prefill(None, *args[1:], 1, 4, 2, 16, 128, 0, None, 0.1, 1.0, 1, None) == 1


def test_workspace_plan():
    ws = plx.decode_workspace_bytes
    ns = plx.decode_num_splits
    assert ws(1, 16, 8, 128, 32768, 1, 1) == 0
    assert ns(1, 16, 8, 128, 32768, 1, 1) == 1
    # forced split counts: records of 2D + 4 floats per (b, hq, split)
    assert ns(1, 16, 8, 128, 32768, 1, 64) == 64
    assert ws(1, 16, 8, 128, 32768, 1, 64) == 16 * 64 * (2 * 128 + 4) * 4
    # at least 32 keys per split on the generic path (fp32), 128 on the MFMA path (bf16, D=128)
    assert ns(2, 4, 2, 128, 100, 0, 1000) == 4
    assert ns(2, 4, 2, 128, 100, 1, 1000) == 1
    assert ns(2, 4, 2, 128, 1000, 1, 1000) == 8
    # monotone in the length for a fixed request
    prev = 0
    for L in (1, 33, 64, 500, 4096, 70000):
        cur = ws(4, 8, 2, 64, L, 0, 16)
        assert cur >= prev
        prev = cur
    assert ws(0, 16, 8, 128, 64, 1, 0) == 0 and ns(1, 16, 5, 128, 64, 1, 0) == 0
    # the automatic plan keeps at least one 32-key tile per wave (4 waves per split on the
    # MFMA path, 1 on the generic one) and targets one workgroup per CU
    s = ns(1, 16, 8, 128, 32768, 1, 0)
    assert 1 < s <= 32768 // 128
    s = ns(1, 16, 8, 64, 32768, 1, 0)
    assert 1 < s <= 32768 // 32
    assert ns(1, 8, 8, 128, 1024, 1, 0) == 8       # short sequence: split down to 128 keys
    # up to 512 visible keys the matrix-core path runs one fused split (no merge launch)
    assert ns(1, 8, 8, 128, 512, 1, 0) == 1 and ns(1, 8, 8, 128, 513, 1, 0) > 1
    assert ns(1, 8, 8, 128, 32768, 1, 0, 512) == 1  # a window of 512 keys
    assert ns(2048, 16, 8, 128, 2048, 1, 0) == 1   # large batch: one split


def test_workspace_covers_stream_k_plan():
    """The decode workspace size also covers a packed cache's stream-K plan: four ranges per
    CU in all (4 CUs / Hkv per KV head; with no device the CU count falls back to 256), and
    one record per sequence piece, (ranges + B - 1) per query head. Windows, forced split
    counts and the generic path do not take that plan."""
    ws = plx.decode_workspace_bytes
    rec = (2 * 128 + 4) * 4
    for B, Hq, Hkv in ((64, 16, 8), (3, 2, 1), (5, 6, 3), (1, 8, 8)):
        parts = 4 * 256 // Hkv
        assert ws(B, Hq, Hkv, 128, 8192, 1, 0) >= Hq * (parts + B - 1) * rec
        # the split plan's records where stream-K does not apply (none for one fused split)
        s = plx.decode_num_splits(B, Hq, Hkv, 128, 8192, 1, 0, 1000)
        assert ws(B, Hq, Hkv, 128, 8192, 1, 0, 1000) == (B * Hq * s * rec if s > 1 else 0)
        assert ws(B, Hq, Hkv, 128, 8192, 1, 7) == B * Hq * 7 * rec
    # workload 3's plan: 16 x (128 + 63) records
    assert ws(64, 16, 8, 128, 8192, 1, 0) == 16 * (128 + 63) * rec


def _backward(**kw):
    a = dict(q=FAKE, r=FAKE, k=FAKE, v=FAKE, o=FAKE, do=FAKE, lse=FAKE, sbar=FAKE, vbar=None, dq=FAKE,
             dr=FAKE, dk=FAKE, dv=FAKE, B=1, Hq=4, Hkv=2, L=64, D=128, W=0, mask=None, qk=0.1,
             rk=1.0, dt=1, ws=None, wsb=0, stream=None)
    a.update(kw)
    return plx.lib().parallax_prefill_backward(
        a["q"], a["r"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["sbar"], a["vbar"], a["dq"],
        a["dr"],
        a["dk"], a["dv"], a["B"], a["Hq"], a["Hkv"], a["L"], a["D"], a["W"], a["mask"], a["qk"],
        a["rk"], a["dt"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), 1), (dict(L=0), 1), (dict(Hq=6, Hkv=4), 1), (dict(q=None), 1),
    (dict(do=None), 1), (dict(lse=None), 1), (dict(sbar=None), 1), (dict(dk=None), 1),
    (dict(D=96), 2), (dict(dt=3), 2), (dict(L=(1 << 22) + 1), 2), (dict(rk=float("nan")), 1),
    (dict(W=-2), 1), (dict(qk=0.0), 1),
    (dict(), 3), (dict(ws=FAKE, wsb=4 * 64 * 16 - 1), 3),
])
def test_prefill_backward_rejects_on_host(kw, status):
    # every case must fail validation: FAKE pointers may never reach a launch
    assert status != 0
    assert _backward(**kw) == status


def test_prefill_backward_workspace_size():
    f = plx.lib().parallax_prefill_backward_workspace_bytes
    assert f(2, 16, 4096) == 2 * 16 * 4096 * 16
    assert f(0, 16, 4096) == 0 and f(1, 1, 0) == 0


def test_varlen_prefill_rejects_on_host():
    L = plx.lib()
    p8 = [FAKE] * 5 + [None, None, None]
    # cu_seqlens missing, negative total, too long a packed head, empty batch is a no-op
    ws = (FAKE, 256)
    assert L.parallax_prefill_varlen(*p8, None, 2, 4, 2, 64, 100, 128, 0, None, 0.1, 1.0, 1, *ws,
                                     None) == 1
    assert L.parallax_prefill_varlen(*p8, FAKE, 2, 4, 2, 64, -1, 128, 0, None, 0.1, 1.0, 1, *ws,
                                     None) == 1
    assert L.parallax_prefill_varlen(*p8, FAKE, 2, 64, 8, 1 << 21, 100, 128, 0, None, 0.1, 1.0, 1, *ws,
                                     None) == 2
    assert L.parallax_prefill_varlen(*p8, FAKE, 2, 4, 2, 64, 100, 128, 0, None, 0.1, 1.0, 1, FAKE, 255,
                                     None) == 3
    assert L.parallax_prefill_varlen(*p8, FAKE, 2, 4, 2, 64, 0, 128, 0, None, 0.1, 1.0, 1, *ws,
                                     None) == 0
    assert L.parallax_prefill_varlen_workspace_bytes(4, 100, 0) == 256
    assert L.parallax_prefill_varlen_workspace_bytes(4, 100, 1) == 256 + 4 * 100 * 16
    b13 = [FAKE] * 8 + [None] + [FAKE] + [FAKE] * 4
    assert L.parallax_prefill_varlen_backward(*b13, 2, 4, 2, 64, 100, 128, 0, None, 0.1, 1.0, 1, None,
                                              0, None) == 3
    assert L.parallax_prefill_varlen_backward(*b13, 2, 4, 2, 64, 100, 128, 0, None, 0.1, 1.0, 1, FAKE,
                                              256 + 4 * 100 * 16 - 1, None) == 3


@pytest.mark.parametrize("Hkv,D,code", [(64, 128, plx.PLX_BF16), (8, 128, plx.PLX_F32),
                                        (128, 64, plx.PLX_F32), (1, 64, plx.PLX_BF16)])
def test_split_plan_keeps_read_ahead_inside_32bit_offsets(Hkv, D, code):
    """Kernels address a split's keys with 32-bit byte offsets, and the streaming loop
    reads up to two 128-key strides and a 32-key tile past the split's end: every plan,
    even a forced single split over a huge cache, must keep that inside 2^31 bytes."""
    tok = Hkv * D * (2 if code == plx.PLX_BF16 else 4)
    for kv_len in (1 << 20, (1 << 21) + 77, 1 << 24):
        for forced in (0, 1, 3):
            s = plx.decode_num_splits(1, Hkv, Hkv, D, kv_len, code, forced)
            per = -(-kv_len // s)
            chunk = -(-per // 128) * 128
            assert (chunk + 2 * 128 + 32) * tok + 1024 < 2 ** 31, (kv_len, forced, s)
            # a workgroup stages the block-sparse visibility of at most 4096 blocks
            assert chunk <= (4096 - 2) * 128, (kv_len, forced, s)


def test_noalloc_decode_refuses_plans_beyond_its_array_on_host():
    # 64 sequences x 64 query heads x 64 forced splits of records: 272 MB > 8 MiB
    L = plx.lib()
    need = L.parallax_decode_workspace_bytes(64, 64, 8, 128, 32768, 0, 1, 64)
    assert need > plx.NOALLOC_SCRATCH_BYTES
    st = L.parallax_decode_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, None, 64, 64, 8, 128, 32768, 0,
                                   None, 0.1, 1.0, 1, 64, None)
    assert st == 3
    # invalid sizes are reported as by parallax_decode, also before any device call
    assert L.parallax_decode_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, 4, 2, 128, 64, 0,
                                     None, 0.1, 1.0, 1, 0, None) == 1
