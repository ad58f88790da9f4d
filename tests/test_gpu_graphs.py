"""The entry points under HIP graph capture, on side streams and without allocation.

Every entry point enqueues its kernels on the caller's stream and allocates
nothing, so a caller can capture a call (with preallocated outputs and workspace)
into a graph and replay it.  Each replay, with eager work and synchronisations
between replays, must reproduce the eager result bit for bit."""
import numpy as np
import pytest
import torch

import flashattention_forward_fwd_amd as fa
from flashattention_forward_fwd_amd.inputs import random_dout, random_qkv
from tests.parity import say

pytestmark = pytest.mark.gpu


def _replays_match(run, outputs, eager, n=3):
    """Capture run() on a side stream, replay n times and compare outputs with eager."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()                                   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        run()
    torch.cuda.synchronize()
    for i in range(n):
        for t in outputs:
            t.fill_(float("nan"))               # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, e in zip(outputs, eager):
            assert torch.equal(t, e), "replay %d differs" % i
    say("  %d replays match" % n)


def test_forward_in_graph():
    say("case graph forward bf16 causal (1, 4, 700, 700, 128)")
    q, k, v = (t.cuda() for t in random_qkv(1, 4, 700, 700, 128, "bf16", seed=71))
    eager = fa.forward(q, k, v, causal=True)
    o = torch.empty_like(q)
    lse = torch.empty(1, 4, 700, device="cuda")
    _replays_match(lambda: fa.forward(q, k, v, causal=True, out=o, lse=lse), (o, lse), eager)


def test_splitkv_in_graph():
    say("case graph split-KV bf16 (2, 2, 100, 3000, 64), 4 splits")
    q, k, v = (t.cuda() for t in random_qkv(2, 2, 100, 3000, 64, "bf16", seed=72))
    eager = fa.forward(q, k, v, num_splits=4)
    need = fa.fa2_splitkv_workspace_bytes(2, 2, 100, 3000, 64, 0, 4)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty(2, 2, 100, device="cuda")
    _replays_match(lambda: fa.forward(q, k, v, num_splits=4, workspace=ws, out=o, lse=lse), (o, lse), eager)


def test_backward_in_graph():
    say("case graph backward bf16 causal (1, 2, 500, 500, 128)")
    q, k, v = (t.cuda() for t in random_qkv(1, 2, 500, 500, 128, "bf16", seed=73))
    do = random_dout(1, 2, 500, 128, "bf16", seed=73).cuda()
    o, lse = fa.forward(q, k, v, causal=True)
    eager = fa.backward(q, k, v, o, lse, do, causal=True)
    ws = torch.empty(fa.fa2_bwd_workspace_bytes(1, 2, 500), dtype=torch.uint8, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    _replays_match(lambda: fa.backward(q, k, v, o, lse, do, causal=True, dq=dq, dk=dk, dv=dv, workspace=ws),
                   (dq, dk, dv), eager)


def test_dropout_in_graph():
    say("case graph dropout forward bf16 (1, 2, 300, 300, 64) p=0.2")
    q, k, v = (t.cuda() for t in random_qkv(1, 2, 300, 300, 64, "bf16", seed=74))
    eager = fa.forward(q, k, v, dropout=(0.2, 5, 6))
    o = torch.empty_like(q)
    lse = torch.empty(1, 2, 300, device="cuda")
    _replays_match(lambda: fa.forward(q, k, v, dropout=(0.2, 5, 6), out=o, lse=lse), (o, lse), eager)


def test_non_default_stream():
    """Work enqueued on a side stream (the current stream inside the context)
    gives the default-stream result once that stream is synchronised."""
    say("case side stream forward + backward bf16 (2, 2, 400, 400, 64)")
    q, k, v = (t.cuda() for t in random_qkv(2, 2, 400, 400, 64, "bf16", seed=75))
    do = random_dout(2, 2, 400, 64, "bf16", seed=75).cuda()
    o1, l1 = fa.forward(q, k, v, causal=True)
    g1 = fa.backward(q, k, v, o1, l1, do, causal=True)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        o2, l2 = fa.forward(q, k, v, causal=True)
        g2 = fa.backward(q, k, v, o2, l2, do, causal=True)
    side.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert all(torch.equal(a, b) for a, b in zip(g1, g2))
    assert np.isfinite(o2.float().cpu().numpy()).all()


def test_preallocated_calls_allocate_nothing():
    """With outputs and workspace passed in, forward (one-pass and split-KV) and
    backward allocate no device memory (the library allocates none itself)."""
    say("case no allocation with caller buffers: forward, split-KV, backward (1, 2, 640, 640, 64)")
    q, k, v = (t.cuda() for t in random_qkv(1, 2, 640, 640, 64, "bf16", seed=76))
    do = random_dout(1, 2, 640, 64, "bf16", seed=76).cuda()
    o, lse = torch.empty_like(q), torch.empty(1, 2, 640, device="cuda")
    ws = torch.empty(fa.fa2_splitkv_workspace_bytes(1, 2, 640, 640, 64, 1, 3), dtype=torch.uint8, device="cuda")
    bws = torch.empty(fa.fa2_bwd_workspace_bytes(1, 2, 640), dtype=torch.uint8, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    fa.forward(q, k, v, causal=True, out=o, lse=lse)          # warm-up (library load)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    fa.forward(q, k, v, causal=True, out=o, lse=lse)
    fa.forward(q, k, v, causal=True, num_splits=3, workspace=ws, out=o, lse=lse)
    fa.backward(q, k, v, o, lse, do, causal=True, dq=dq, dk=dk, dv=dv, workspace=bws)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before


def test_two_streams_concurrently():
    """Calls in flight on two streams at once (different inputs, shared library
    state) give the results each gives alone."""
    say("case two streams: forward + backward on (1, 4, 900, 900, 128) and (2, 2, 333, 777, 64)")
    shapes = [((1, 4, 900, 900, 128), True, 77), ((2, 2, 333, 777, 64), False, 78)]
    ins, alone = [], []
    for (B, H, Lq, Lk, d), causal, seed in shapes:
        q, k, v = (t.cuda() for t in random_qkv(B, H, Lq, Lk, d, "bf16", seed=seed))
        do = random_dout(B, H, Lq, d, "bf16", seed=seed).cuda()
        o, lse = fa.forward(q, k, v, causal=causal)
        alone.append((o, lse) + tuple(fa.backward(q, k, v, o, lse, do, causal=causal)))
        ins.append((q, k, v, do, causal))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    got = [None, None]
    for _ in range(3):
        for i, (s, (q, k, v, do, causal)) in enumerate(zip(streams, ins)):
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                o, lse = fa.forward(q, k, v, causal=causal)
                got[i] = (o, lse) + tuple(fa.backward(q, k, v, o, lse, do, causal=causal))
        torch.cuda.synchronize()
        for a, b in zip(got, alone):
            assert all(torch.equal(x, y) for x, y in zip(a, b))
