"""Ordering check: results do not depend on which workgroup takes which unit
of work.

Every kernel maps its workgroup id to a unit (a query tile, a key tile, a
key-range part, a decode split) and no workgroup waits for another: each
output element is written by one wave, summed in a fixed order. So the same
call with the logical workgroup ids permuted (cakv_diag_set_workgroup_order:
1 scrambled, 2 reversed) must give bit-identical out, lse, tile counts and
gradients. A dependence on launch order or residency (a race between
workgroups, a read of another workgroup's output) would show up here as a
difference. The forward results of the default order are also checked
against the oracle on sampled rows, so the comparison is between right
answers.
"""
import numpy as np
import pytest
import torch

import cakv_synth as syn
import context_attention_kv_amd as cakv
from gpu_util import Inputs, compare, gather_rows, oracle_rows, say, to_dev

pytestmark = pytest.mark.gpu

ORDERS = (0, 1, 2)


@pytest.fixture(autouse=True)
def _default_order_after():
    yield
    cakv.cakv_diag_set_workgroup_order(0)


def _bits(t: torch.Tensor) -> np.ndarray:
    """Raw bits of a device tensor (so NaN patterns and -0.0 count too)."""
    a = t.detach().contiguous().cpu()
    if a.dtype in (torch.float32, torch.int32):
        return a.view(torch.int32).numpy()
    if a.dtype == torch.bfloat16:
        return a.view(torch.int16).numpy()
    return a.numpy()


def _same_for_all_orders(run, what):
    """run() -> list of device tensors; equal bits under every order."""
    ref = None
    for order in ORDERS:
        cakv.cakv_diag_set_workgroup_order(order)
        got = [_bits(t) for t in run()]
        torch.cuda.synchronize()
        if ref is None:
            ref = got
            continue
        for i, (a, b) in enumerate(zip(ref, got)):
            n = int((a != b).sum())
            assert n == 0, f"{what}: output {i} differs in {n} elements under order {order}"
        say(f"  {what}: order {order} bit-identical to order 0")
    cakv.cakv_diag_set_workgroup_order(0)


@pytest.mark.parametrize("case", [
    # (B, Hq, Hkv, T, N, D, dtype, causal, rank, workspace)
    (1, 8, 2, 4096, 4, 128, "bf16", True, 3, "auto"),    # ping-pong kernel, grouped heads
    (1, 8, 8, 8192, 4, 128, "bf16", True, 3, "auto"),    # four-wave kernel, key split in parts
    (2, 3, 3, 999, 3, 64, "bf16", False, 0, None),       # four-wave, d = 64, ragged tail
    (1, 2, 1, 1024, 4, 64, "f32", True, 3, None),        # fp32 kernel
])
def test_forward_independent_of_workgroup_order(case):
    B, Hq, Hkv, T, N, D, dtype, causal, r, ws = case
    w = syn.Workload("order", B=B, Hq=Hq, Hkv=Hkv, T=T, N=N, D=D, dtype=dtype, causal=causal,
                     ranks=(r,), seed=77)
    inp = Inputs(w)
    say(f"forward order case {case}")

    def run():
        out = torch.empty((B, w.C, Hq, D), dtype=torch.float32, device="cuda")
        lse = torch.empty((B, Hq, w.C), dtype=torch.float32, device="cuda")
        tc = torch.zeros(3, dtype=torch.int64, device="cuda")
        cakv.cakv_local_shard_forward(inp.qd[r], inp.kb, inp.vb, r, causal, out, lse,
                                      tile_counters=tc, workspace=ws)
        torch.cuda.synchronize()
        return [out, lse, tc]

    _same_for_all_orders(run, f"forward {case}")
    out, lse, _ = run()
    rows = syn.sample_rows(w, per_head=16, seed=5)
    ref_o, ref_l = oracle_rows(inp, r, rows)
    got_o, got_l = gather_rows(out, lse, rows)
    compare(got_o, got_l, ref_o, ref_l, dtype, f"forward {case} vs oracle", rows)


def test_forward_blocks_independent_of_workgroup_order():
    """Blocks of unequal length, a gap, an empty block and a future block."""
    w = syn.Workload("order-blocks", B=1, Hq=4, Hkv=2, T=2048, N=1, D=128, dtype="bf16",
                     causal=True, ranks=(0,), seed=78)
    q = syn.make_q_full(w)
    k = syn.make_kv_full(w, "k")
    v = syn.make_kv_full(w, "v")
    qd, kd, vd = to_dev(np.ascontiguousarray(q[:, 1000:1500])), to_dev(k), to_dev(v)
    spans = [(1300, 400), (0, 700), (900, 0), (800, 300), (1800, 200)]
    kb = [kd[:, o:o + n].contiguous() for o, n in spans]
    vb = [vd[:, o:o + n].contiguous() for o, n in spans]
    offs = [o for o, _ in spans]

    def run():
        out = torch.empty((1, 500, 4, 128), dtype=torch.float32, device="cuda")
        lse = torch.empty((1, 4, 500), dtype=torch.float32, device="cuda")
        tc = torch.zeros(3, dtype=torch.int64, device="cuda")
        cakv.cakv_forward_blocks(qd, kb, vb, offs, 1000, True, out, lse, tile_counters=tc)
        torch.cuda.synchronize()
        return [out, lse, tc]

    _same_for_all_orders(run, "forward_blocks")


def test_backward_independent_of_workgroup_order():
    B, Hq, Hkv, T, D = 1, 4, 2, 700, 128
    w = syn.Workload("order-bwd", B=B, Hq=Hq, Hkv=Hkv, T=T, N=1, D=D, dtype="bf16",
                     causal=True, ranks=(0,), seed=79)
    q, k, v = syn.make_q_full(w), syn.make_kv_full(w, "k"), syn.make_kv_full(w, "v")
    dout = np.empty((B, T, Hq, D), np.uint16)
    syn.fill(dout, seed=79, tensor=7)
    qd, kd, vd, dod = to_dev(q), to_dev(k), to_dev(v), to_dev(dout)
    spans = [(0, 300), (300, 400)]
    kb = [kd[:, o:o + n].contiguous() for o, n in spans]
    vb = [vd[:, o:o + n].contiguous() for o, n in spans]
    offs = [o for o, _ in spans]
    out = torch.empty((B, T, Hq, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device="cuda")
    cakv.cakv_forward_blocks(qd, kb, vb, offs, 0, True, out, lse)
    torch.cuda.synchronize()

    def run():
        dq = torch.empty((B, T, Hq, D), dtype=torch.float32, device="cuda")
        dk = [torch.empty(t.shape, dtype=torch.float32, device="cuda") for t in kb]
        dv = [torch.empty(t.shape, dtype=torch.float32, device="cuda") for t in kb]
        cakv.cakv_backward_blocks(qd, kb, vb, offs, 0, True, out, lse, dod, dq, dk, dv)
        torch.cuda.synchronize()
        return [dq] + dk + dv

    _same_for_all_orders(run, "backward")


def test_decode_independent_of_workgroup_order():
    w = syn.scaled(syn.DECODE_WORKLOADS[1], Tn=4)
    q, k, v = syn.make_decode(w)
    bounds = w.portions()
    kd, vd = to_dev(k), to_dev(v)
    kp = [kd[:, o:o + n].contiguous() for o, n in bounds]
    vp = [vd[:, o:o + n].contiguous() for o, n in bounds]
    offs = [o for o, _ in bounds]
    qd = to_dev(q)
    B, Tn, Hq, D = qd.shape

    def run():
        out = torch.empty((B, Tn, Hq, D), dtype=torch.float32, device="cuda")
        lse = torch.empty((B, Hq, Tn), dtype=torch.float32, device="cuda")
        cakv.cakv_decode(qd, kp, vp, offs, w.hist, True, out, lse)
        torch.cuda.synchronize()
        return [out, lse]

    _same_for_all_orders(run, "decode")
