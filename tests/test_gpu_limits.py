"""The ABI's limits and the method's degenerate shapes on the GPU.

* The most blocks one call takes (CAKV_MAX_CHUNKS = 64): the ring of web page
  "Sequence parallelism -- splitting the token dimension across GPUs",
  section "A better mental model: move blocks past the queries", with 64
  ranks, for the first, a middle and the last rank (the causal rule of
  section "Causal attention gives us another optimization" skips every block
  in a rank's future); 64 blocks of any length, order and offset through
  cakv_forward_blocks; 64 blocks through the backward; decode against 64
  history portions (section "Training and inference stress this dimension
  differently").
* One-token chunks: each rank owns a single query, and the last rank sees
  64 blocks of one key each, every tile ragged.

Every output row is compared with the fp64 oracle; tile counts with its
brute-force classification (O3), bit for bit.
"""
import numpy as np
import pytest
import torch

import cakv_synth as syn
import context_attention_kv_amd as cakv
import oracle
from gpu_util import all_rows, compare, expected_tiles, gather_rows, say, to_dev

pytestmark = pytest.mark.gpu

NMAX = cakv.CAKV_MAX_CHUNKS


@pytest.mark.parametrize("C,Hq,Hkv,D,dtype", [
    (24, 4, 2, 128, "bf16"),   # ping-pong kernel, ragged 24-key blocks
    (1, 4, 4, 64, "bf16"),     # one-token chunks, four-wave kernel
    (7, 2, 1, 64, "f32"),      # fp32 kernel
])
def test_ring_with_the_most_blocks(C, Hq, Hkv, D, dtype):
    w = syn.Workload("max-ring", B=1, Hq=Hq, Hkv=Hkv, T=NMAX * C, N=NMAX, D=D, dtype=dtype,
                     causal=True, ranks=(0, 21, NMAX - 1), seed=61)
    q_full = syn.make_q_full(w)
    k = syn.make_kv_full(w, "k")
    v = syn.make_kv_full(w, "v")
    kd, vd = to_dev(k), to_dev(v)
    kb = [kd[:, j * C:(j + 1) * C] for j in range(NMAX)]
    vb = [vd[:, j * C:(j + 1) * C] for j in range(NMAX)]
    for r in w.ranks:
        say(f"ring of {NMAX} blocks: C={C} Hq={Hq} Hkv={Hkv} D={D} {dtype} rank {r}")
        q = np.ascontiguousarray(q_full[:, r * C:(r + 1) * C])
        out = torch.empty((1, C, Hq, D), dtype=torch.float32, device="cuda")
        lse = torch.empty((1, Hq, C), dtype=torch.float32, device="cuda")
        tc = torch.zeros(3, dtype=torch.int64, device="cuda")
        cakv.cakv_local_shard_forward(to_dev(q), kb, vb, r, True, out, lse, tile_counters=tc)
        torch.cuda.synchronize()
        rows = all_rows(1, Hq, C)
        ro, rl = oracle.attention(q, k, v, q_off=r * C, causal=True, rows=rows)
        go, gl = gather_rows(out, lse, rows)
        compare(go, gl, ro, rl, dtype, f"ring N={NMAX} C={C} rank {r}", rows)
        assert tc.cpu().tolist() == list(expected_tiles(w, r))


def test_forward_blocks_with_the_most_blocks():
    """64 blocks of random lengths (some empty) at random offsets, some in the
    queries' future, some overlapping, in shuffled order."""
    rng = np.random.default_rng(62)
    T, Tq, q_off = 1500, 300, 900
    w = syn.Workload("max-blocks", B=1, Hq=4, Hkv=2, T=T, N=1, D=128, dtype="bf16",
                     causal=True, ranks=(0,), seed=62)
    q = np.ascontiguousarray(syn.make_q_full(w)[:, q_off:q_off + Tq])
    k = syn.make_kv_full(w, "k")
    v = syn.make_kv_full(w, "v")
    blocks = []
    for _ in range(NMAX):
        n = int(rng.integers(0, 60))
        o = int(rng.integers(0, T - n + 1))
        blocks.append((o, n))
    kd, vd = to_dev(k), to_dev(v)
    kb = [kd[:, o:o + n].contiguous() for o, n in blocks]
    vb = [vd[:, o:o + n].contiguous() for o, n in blocks]
    out = torch.empty((1, Tq, 4, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((1, 4, Tq), dtype=torch.float32, device="cuda")
    tc = torch.zeros(3, dtype=torch.int64, device="cuda")
    cakv.cakv_forward_blocks(to_dev(q), kb, vb, [o for o, _ in blocks], q_off, True, out, lse,
                             tile_counters=tc)
    torch.cuda.synchronize()
    rows = all_rows(1, 4, Tq)
    acc_o = acc_l = None
    for o, n in blocks:
        if n == 0:
            continue
        po, pl = oracle.attention(q, k[:, o:o + n], v[:, o:o + n], q_off=q_off, k_off=o,
                                  causal=True, rows=rows)
        acc_o, acc_l = (po, pl) if acc_o is None else oracle.lse_merge(acc_o, acc_l, po, pl)
    go, gl = gather_rows(out, lse, rows)
    compare(go, gl, acc_o, acc_l, "bf16", f"forward_blocks with {NMAX} blocks", rows)
    starts = np.array([o for o, _ in blocks])
    lens = np.array([n for _, n in blocks])
    _, _, tiles = oracle.classify(Tq, q_off, starts, lens, causal=True, B=1, Hq=4,
                                  tile_q=cakv.CAKV_TILE_Q, tile_k=cakv.CAKV_TILE_K)
    assert tc.cpu().tolist() == list(tiles)


def test_backward_with_the_most_blocks():
    """Gradients through 64 contiguous blocks of 11 keys (the sequence's
    first 704 keys), queries at 600..699, against O4."""
    B, Hq, Hkv, D, T = 1, 4, 2, 128, 704
    w = syn.Workload("max-bwd", B=B, Hq=Hq, Hkv=Hkv, T=T, N=1, D=D, dtype="bf16",
                     causal=True, ranks=(0,), seed=63)
    q_full, k, v = syn.make_q_full(w), syn.make_kv_full(w, "k"), syn.make_kv_full(w, "v")
    q_off, Tq = 600, 100
    q = np.ascontiguousarray(q_full[:, q_off:q_off + Tq])
    dout = np.empty((B, Tq, Hq, D), np.uint16)
    syn.fill(dout, seed=63, tensor=7)
    L = T // NMAX
    spans = [(j * L, L) for j in range(NMAX)]
    qd, kd, vd, dod = to_dev(q), to_dev(k), to_dev(v), to_dev(dout)
    kb = [kd[:, o:o + n].contiguous() for o, n in spans]
    vb = [vd[:, o:o + n].contiguous() for o, n in spans]
    offs = [o for o, _ in spans]
    out = torch.empty((B, Tq, Hq, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq, Tq), dtype=torch.float32, device="cuda")
    cakv.cakv_forward_blocks(qd, kb, vb, offs, q_off, True, out, lse)
    dq = torch.empty((B, Tq, Hq, D), dtype=torch.float32, device="cuda")
    dk = [torch.empty(t.shape, dtype=torch.float32, device="cuda") for t in kb]
    dv = [torch.empty(t.shape, dtype=torch.float32, device="cuda") for t in kb]
    cakv.cakv_backward_blocks(qd, kb, vb, offs, q_off, True, out, lse, dod, dq, dk, dv)
    torch.cuda.synchronize()
    rdq, rdk, rdv = oracle.attention_backward(q, k, v, dout, q_off=q_off, causal=True)
    got_dk = torch.cat(dk, 1).cpu().numpy()
    got_dv = torch.cat(dv, 1).cpu().numpy()
    for name, got, ref in (("dq", dq.cpu().numpy(), rdq), ("dk", got_dk, rdk), ("dv", got_dv, rdv)):
        d = np.abs(got.astype(np.float64) - ref)
        rms = max(float(np.sqrt((ref ** 2).mean())), 1e-3)
        say(f"  {name}: max {d.max():.3e} mean {d.mean():.3e} rms_ref {rms:.3e}")
        assert not np.isnan(got).any(), name
        assert d.max() <= 1e-1 * rms and d.mean() <= 4e-3 * rms, name


def test_decode_with_the_most_portions():
    """Four new tokens against a 1,000-token history in 64 portions of uneven
    length (one empty), shuffled."""
    rng = np.random.default_rng(64)
    w = syn.scaled(syn.DECODE_WORKLOADS[1], Tn=4)
    q, k, v = syn.make_decode(w)
    cuts = np.sort(rng.choice(np.arange(1, w.hist), size=NMAX - 2, replace=False))
    edges = [0] + cuts.tolist() + [w.hist]
    bounds = [(edges[j], edges[j + 1] - edges[j]) for j in range(len(edges) - 1)]
    bounds.append((w.hist, 0))
    bounds = [bounds[j] for j in rng.permutation(len(bounds))]
    assert len(bounds) == NMAX
    kd, vd = to_dev(k), to_dev(v)
    # the new tokens' own keys follow the history in the last portion
    kp = [kd[:, o:o + n].contiguous() for o, n in bounds]
    vp = [vd[:, o:o + n].contiguous() for o, n in bounds]
    last = max(range(NMAX), key=lambda j: bounds[j][0] + bounds[j][1])
    o, n = bounds[last]
    kp[last] = kd[:, o:o + n + w.Tn].contiguous()
    vp[last] = vd[:, o:o + n + w.Tn].contiguous()
    bounds[last] = (o, n + w.Tn)
    qd = to_dev(q)
    B, Tn, Hq, D = qd.shape
    out = torch.empty((B, Tn, Hq, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq, Tn), dtype=torch.float32, device="cuda")
    cakv.cakv_decode(qd, kp, vp, [o for o, _ in bounds], w.hist, True, out, lse)
    torch.cuda.synchronize()
    rows = all_rows(B, Hq, Tn)
    ro, rl = oracle.attention(q, k, v, q_off=w.hist, k_off=0, causal=True, rows=rows)
    go, gl = gather_rows(out, lse, rows)
    compare(go, gl, ro, rl, "bf16", f"decode with {NMAX} portions", rows)
