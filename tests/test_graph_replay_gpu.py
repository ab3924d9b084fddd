"""HIP graph capture and replay of the prefill, its backward and their packed-sequence
forms. Each call is captured once into a graph with caller-held outputs and workspace,
then replayed several times with the outputs cleared before each replay and eager calls
on the same workspace in between: every replay must reproduce the eager result bit for
bit. The packed forms draw work items from per-XCD queues whose counters a small kernel
clears at the start of every call, so a replay that left them dirty would skip items.
"""
import math

import numpy as np
import pytest
import torch

import parameterized_local_linear_amd as plx
import synth
from gpu_util import to_gpu

pytestmark = pytest.mark.gpu

S128 = 1.0 / math.sqrt(128.0)
REPLAYS = 4


def _replay_check(fn, outs, what):
    """fn() writes into the tensors `outs`; capture it, replay, compare with eager."""
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        fn()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        fn()
    for rep in range(REPLAYS):
        for o in outs:
            o.zero_()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, eager)):
            assert torch.equal(o, e), f"{what}: replay {rep}, output {i}"
        # eager work on the same workspace and outputs between replays
        with torch.cuda.stream(stream):
            fn()
        torch.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, eager)):
            assert torch.equal(o, e), f"{what}: eager call after replay {rep}, output {i}"


@pytest.mark.parametrize("dtype,D", [(synth.BF16, 128), (synth.F32, 64)])
def test_prefill_and_backward_graph_replays(dtype, D):
    B, Hq, Hkv, L = 2, 8, 4, 333
    s = 1.0 / math.sqrt(D)
    q, r = (to_gpu(synth.normal(930, tid, (B, Hq, L, D), s, dtype), dtype) for tid in (synth.TID_Q, synth.TID_R))
    k, v = (to_gpu(synth.normal(930, tid, (B, Hkv, L, D), s, dtype), dtype) for tid in (synth.TID_K, synth.TID_V))
    do = to_gpu(synth.normal(930, synth.TID_DO, (B, Hq, L, D), 1.0, dtype), dtype)
    o = torch.empty_like(q)
    vbar = torch.empty_like(q)
    o_, lse, sbar = plx.prefill(q, r, k, v, return_stats=True, vbar_out=vbar)
    o.copy_(o_)

    def fwd():
        plx.prefill(q, r, k, v, out=o, window=100)

    _replay_check(fwd, [o], f"prefill window 100 D={D}")

    o.copy_(o_)
    ws = torch.empty(int(plx.lib().parallax_prefill_backward_workspace_bytes(B, Hq, L)),
                     dtype=torch.uint8, device="cuda")
    grads = [torch.empty_like(x) for x in (q, r, k, v)]

    def bwd():
        plx.prefill_backward(q, r, k, v, o, do, lse, sbar, workspace=ws, out=grads, vbar=vbar)

    _replay_check(bwd, grads, f"prefill backward D={D}")


def test_packed_prefill_and_backward_graph_replays():
    lens = np.array([700, 1, 0, 129, 2300, 64])
    Hq, Hkv, D = 8, 4, 128
    T = int(lens.sum())
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)).cuda()
    q, r = (to_gpu(synth.normal(931, tid, (T, Hq, D), S128, synth.BF16), synth.BF16) for tid in (synth.TID_Q, synth.TID_R))
    k, v = (to_gpu(synth.normal(931, tid, (T, Hkv, D), S128, synth.BF16), synth.BF16) for tid in (synth.TID_K, synth.TID_V))
    do = to_gpu(synth.normal(931, synth.TID_DO, (T, Hq, D), 1.0, synth.BF16), synth.BF16)
    max_len = int(lens.max())
    ws_f = torch.empty(int(plx.lib().parallax_prefill_varlen_workspace_bytes(Hq, T, 0)),
                       dtype=torch.uint8, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((T, Hq), dtype=torch.float32, device="cuda")
    sbar = torch.empty_like(lse)
    o_, lse_, sbar_ = plx.prefill_varlen(q, r, k, v, cu, max_len, return_stats=True, workspace=ws_f)

    def fwd():
        plx.prefill_varlen(q, r, k, v, cu, max_len, out=o, workspace=ws_f)

    _replay_check(fwd, [o], "packed prefill")

    o.copy_(o_)
    ws_b = torch.empty(int(plx.lib().parallax_prefill_varlen_workspace_bytes(Hq, T, 1)),
                       dtype=torch.uint8, device="cuda")
    grads = [torch.empty_like(x) for x in (q, r, k, v)]

    def bwd():
        plx.prefill_varlen_backward(q, r, k, v, o, do, lse_, sbar_, cu, max_len, workspace=ws_b,
                                    out=grads)

    _replay_check(bwd, grads, "packed prefill backward")
