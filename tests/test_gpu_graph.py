"""Graph capture: the library's entry points only launch kernels on the
caller's stream (no allocation, memset, copy or synchronisation inside), so a
call can be recorded into a HIP graph and replayed.

Each case records its calls once, then replays the graph three times with
eager work and a synchronisation between replays (every output poisoned with
NaN first), and checks every replay bit for bit against the same calls run
eagerly: the whole-share forward on the ping-pong kernel, on the four-wave
kernel with its key split and merge kernel, and on the fp32 kernel; the
per-block ring (state init, one update per block, finalize, and a
log-sum-exp merge); the backward; decode with a workspace and the
allocation-free decode. The eager results of the forward cases are also held
to the oracle on sampled rows, so the comparison is between right answers.
A last case enqueues independent calls on two streams at once and checks
that each result is the one the call gives alone.
"""
import numpy as np
import pytest
import torch

import cakv_synth as syn
import context_attention_kv_amd as cakv
from gpu_util import Inputs, compare, gather_rows, oracle_rows, say, to_dev

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _bits(t: torch.Tensor) -> torch.Tensor:
    if t.dtype == torch.float32:
        return t.view(torch.int32)
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16)
    return t


def _replays_match(call, outs, what):
    """Run call() eagerly, record it into a graph, replay the graph REPLAYS
    times; every replay's outputs must equal the eager ones bit for bit."""
    call()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for i in range(REPLAYS):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for j, (o, r) in enumerate(zip(outs, ref)):
            n = int((_bits(o) != _bits(r)).sum())
            assert n == 0, f"{what}: replay {i}, output {j}: {n} elements differ from eager"
        say(f"  {what}: replay {i} bit-identical to the eager call")
    del g
    return ref


@pytest.mark.parametrize("case", [
    # (B, Hq, Hkv, T, N, D, dtype, causal, rank, kernel)
    (1, 8, 2, 2048, 4, 128, "bf16", True, 3, "ping-pong"),
    (1, 8, 8, 4096, 4, 128, "bf16", True, 3, "four-wave, key split + merge"),
    (1, 2, 1, 1024, 4, 64, "f32", True, 2, "fp32"),
])
def test_forward_graph(case):
    B, Hq, Hkv, T, N, D, dtype, causal, r, kernel = case
    w = syn.Workload("graph", B=B, Hq=Hq, Hkv=Hkv, T=T, N=N, D=D, dtype=dtype, causal=causal,
                     ranks=(r,), seed=91)
    inp = Inputs(w)
    say(f"forward graph: {kernel} {case[:-1]}")
    out = torch.empty((B, w.C, Hq, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq, w.C), dtype=torch.float32, device="cuda")
    nb = cakv.cakv_forward_workspace_size(cakv.CAKV_BF16 if dtype == "bf16" else cakv.CAKV_F32,
                                          B, Hq, Hkv, w.C, D)
    if kernel.startswith("four-wave"):
        assert nb > 0, "this shape is meant to take the key-split path"
    ws = torch.empty(nb // 4 + 4, dtype=torch.float32, device="cuda") if nb else None

    def call():
        cakv.cakv_local_shard_forward(inp.qd[r], inp.kb, inp.vb, r, causal, out, lse,
                                      workspace=ws)

    ref_out, ref_lse = _replays_match(call, [out, lse], f"forward {kernel}")
    rows = syn.sample_rows(w, per_head=16, seed=4)
    ro, rl = oracle_rows(inp, r, rows)
    go, gl = gather_rows(ref_out, ref_lse, rows)
    compare(go, gl, ro, rl, dtype, f"forward {kernel} vs oracle", rows)


def test_per_block_ring_graph():
    """init, one update per block in ring order, finalize, then a merge of the
    result with itself (lse + ln 2, same out), all in one graph."""
    w = syn.Workload("graph-ring", B=1, Hq=4, Hkv=2, T=1024, N=4, D=128, dtype="bf16",
                     causal=True, ranks=(2,), seed=92)
    inp = Inputs(w)
    r, C = 2, w.C
    m = torch.empty((1, w.Hq, C), device="cuda")
    l = torch.empty((1, w.Hq, C), device="cuda")
    o = torch.empty((1, C, w.Hq, w.D), device="cuda")
    out = torch.empty((1, C, w.Hq, w.D), device="cuda")
    lse = torch.empty((1, w.Hq, C), device="cuda")
    mo = torch.empty((1, C, w.Hq, w.D), device="cuda")
    ml = torch.empty((1, w.Hq, C), device="cuda")
    blocks, _ = cakv.cakv_schedule(r, w.N, C, True)
    kb = [t.contiguous() for t in inp.kb]
    vb = [t.contiguous() for t in inp.vb]

    def call():
        cakv.cakv_state_init(m, l, o)
        for j in blocks:
            cakv.cakv_block_update(inp.qd[r], kb[j], vb[j], r * C, j * C, True, m, l, o)
        cakv.cakv_finalize(m, l, o, out, lse)
        cakv.cakv_lse_merge(out, lse, out, lse, mo, ml)

    say("per-block ring graph: init, updates, finalize, merge")
    ref = _replays_match(call, [m, l, o, out, lse, mo, ml], "per-block ring")
    # a result merged with itself keeps its out and gains ln 2 in lse
    assert torch.allclose(ref[5], ref[3], atol=1e-6, rtol=1e-6)
    fin = torch.isfinite(ref[4])
    assert torch.allclose(ref[6][fin], ref[4][fin] + float(np.log(2.0)), atol=1e-5, rtol=0)
    rows = syn.sample_rows(w, per_head=16, seed=6)
    ro, rl = oracle_rows(inp, r, rows)
    go, gl = gather_rows(ref[3], ref[4], rows)
    compare(go, gl, ro, rl, "bf16", "per-block ring vs oracle", rows)


def test_backward_graph():
    B, Hq, Hkv, T, D = 1, 4, 2, 600, 128
    w = syn.Workload("graph-bwd", B=B, Hq=Hq, Hkv=Hkv, T=T, N=1, D=D, dtype="bf16",
                     causal=True, ranks=(0,), seed=93)
    q, k, v = syn.make_q_full(w), syn.make_kv_full(w, "k"), syn.make_kv_full(w, "v")
    dout = np.empty((B, T, Hq, D), np.uint16)
    syn.fill(dout, seed=93, tensor=7)
    qd, kd, vd, dod = to_dev(q), to_dev(k), to_dev(v), to_dev(dout)
    spans = [(0, 250), (250, 350)]
    kb = [kd[:, a:a + n].contiguous() for a, n in spans]
    vb = [vd[:, a:a + n].contiguous() for a, n in spans]
    offs = [a for a, _ in spans]
    out = torch.empty((B, T, Hq, D), device="cuda")
    lse = torch.empty((B, Hq, T), device="cuda")
    cakv.cakv_forward_blocks(qd, kb, vb, offs, 0, True, out, lse)
    torch.cuda.synchronize()
    dq = torch.empty((B, T, Hq, D), device="cuda")
    dk = [torch.empty(t.shape, device="cuda") for t in kb]
    dv = [torch.empty(t.shape, device="cuda") for t in kb]
    ws = torch.empty(cakv.cakv_backward_workspace_size(B, Hq, T) // 4 + 4, device="cuda")

    def call():
        cakv.cakv_backward_blocks(qd, kb, vb, offs, 0, True, out, lse, dod, dq, dk, dv,
                                  workspace=ws)

    say("backward graph")
    _replays_match(call, [dq] + dk + dv, "backward")


@pytest.mark.parametrize("noalloc", [False, True])
def test_decode_graph(noalloc):
    w = syn.scaled(syn.DECODE_WORKLOADS[1], Tn=3)
    q, k, v = syn.make_decode(w)
    bounds = w.portions()
    kd, vd = to_dev(k), to_dev(v)
    kp = [kd[:, a:a + n].contiguous() for a, n in bounds]
    vp = [vd[:, a:a + n].contiguous() for a, n in bounds]
    offs = [a for a, _ in bounds]
    qd = to_dev(q)
    B, Tn, Hq, D = qd.shape
    out = torch.empty((B, Tn, Hq, D), device="cuda")
    lse = torch.empty((B, Hq, Tn), device="cuda")
    nb = cakv.cakv_decode_workspace_size(B, Hq, w.Hkv, Tn, D, [t.shape[1] for t in kp])
    ws = torch.empty(max(nb, 16) // 4 + 4, device="cuda")

    def call():
        if noalloc:
            cakv.cakv_decode_noalloc(qd, kp, vp, offs, w.hist, True, out, lse)
        else:
            cakv.cakv_decode(qd, kp, vp, offs, w.hist, True, out, lse, workspace=ws)

    what = "allocation-free decode" if noalloc else "decode"
    say(f"{what} graph: B={B} Hq={Hq} Hkv={w.Hkv} hist={w.hist} Tn={Tn}")
    _replays_match(call, [out, lse], what)


def test_calls_on_two_streams_at_once():
    """Two whole-share forwards (each with its own workspace: the key-split
    path) and a decode, enqueued on two streams of default priority so that
    they can run at the same time: each result equals the same call run
    alone, bit for bit (the library keeps no state between calls other than
    the allocation-free decode's scratch, which this test does not use)."""
    w = syn.Workload("two-streams", B=1, Hq=8, Hkv=8, T=4096, N=4, D=128, dtype="bf16",
                     causal=True, ranks=(2, 3), seed=94)
    inp = Inputs(w)
    nb = cakv.cakv_forward_workspace_size(cakv.CAKV_BF16, 1, w.Hq, w.Hkv, w.C, w.D)
    assert nb > 0

    def fwd_bufs():
        return (torch.empty((1, w.C, w.Hq, w.D), device="cuda"),
                torch.empty((1, w.Hq, w.C), device="cuda"),
                torch.empty(nb // 4 + 4, device="cuda"))

    dw = syn.scaled(syn.DECODE_WORKLOADS[1], Tn=2)
    q, k, v = syn.make_decode(dw)
    bounds = dw.portions()
    kd, vd = to_dev(k), to_dev(v)
    kp = [kd[:, a:a + n].contiguous() for a, n in bounds]
    vp = [vd[:, a:a + n].contiguous() for a, n in bounds]
    offs = [a for a, _ in bounds]
    qd = to_dev(q)
    B, Tn, Hq, D = qd.shape

    def dec_bufs():
        need = cakv.cakv_decode_workspace_size(B, Hq, dw.Hkv, Tn, D, [t.shape[1] for t in kp])
        return (torch.empty((B, Tn, Hq, D), device="cuda"), torch.empty((B, Hq, Tn), device="cuda"),
                torch.empty(max(need, 16) // 4 + 4, device="cuda"))

    def fwd(r, bufs, stream=None):
        out, lse, ws = bufs
        cakv.cakv_local_shard_forward(inp.qd[r], inp.kb, inp.vb, r, True, out, lse, workspace=ws,
                                      stream=stream)

    def dec(bufs, stream=None):
        out, lse, ws = bufs
        cakv.cakv_decode(qd, kp, vp, offs, dw.hist, True, out, lse, workspace=ws, stream=stream)

    # alone, one after another
    a2, a3, ad = fwd_bufs(), fwd_bufs(), dec_bufs()
    fwd(2, a2)
    fwd(3, a3)
    dec(ad)
    torch.cuda.synchronize()
    # together: rank 2 and decode on one stream, rank 3 on the other
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    b2, b3, bd = fwd_bufs(), fwd_bufs(), dec_bufs()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        fwd(2, b2, stream=s1.cuda_stream)
        fwd(3, b3, stream=s2.cuda_stream)
        dec(bd, stream=s1.cuda_stream)
    torch.cuda.synchronize()
    say("two streams: forward ranks 2 and 3 and a decode, three rounds")
    for what, x, y in (("rank 2", a2, b2), ("rank 3", a3, b3), ("decode", ad, bd)):
        for j in range(2):
            assert torch.equal(_bits(x[j]), _bits(y[j])), f"{what}: output {j} differs on two streams"
