"""GPU parity of decode over a KV history held in portions (web page
"Sequence parallelism -- splitting the token dimension across GPUs", section
"Training and inference stress this dimension differently": the new query
is evaluated against the portions and the partial results are combined).

Every case compares cakv_decode (through the C ABI) with the fp64 oracle on
the same seeded inputs, to the bf16 tolerances of gpu_util.TOL. The oracle
side is either one attention over the whole contiguous history or, where the
portions are shuffled, gapped or empty, one attention per portion combined
with the oracle's log-sum-exp merge.
"""
import numpy as np
import pytest
import torch

import cakv_synth as syn
import context_attention_kv_amd as cakv
import oracle
from gpu_util import all_rows, compare, gather_rows, say, to_dev

pytestmark = pytest.mark.gpu


def _portions_dev(k, v, bounds):
    kd, vd = to_dev(k), to_dev(v)
    kp = [kd[:, o:o + l].contiguous() for o, l in bounds]
    vp = [vd[:, o:o + l].contiguous() for o, l in bounds]
    return kp, vp


def _run(qd, kp, vp, offs, q_off, causal, out_dtype=torch.float32):
    B, Tn, Hq, D = qd.shape
    out = torch.empty((B, Tn, Hq, D), dtype=out_dtype, device="cuda")
    lse = torch.empty((B, Hq, Tn), dtype=torch.float32, device="cuda")
    cakv.cakv_decode(qd, kp, vp, offs, q_off, causal, out, lse)
    torch.cuda.synchronize()
    return out, lse


def _oracle_by_portions(q, k, v, bounds, q_off, causal, rows):
    """One fp64 attention per portion, combined with the oracle merge."""
    acc_o, acc_l = None, None
    for o, l in bounds:
        if l == 0:
            continue
        po, pl = oracle.attention(q, k[:, o:o + l], v[:, o:o + l], q_off=q_off, k_off=o,
                                  causal=causal, rows=rows)
        if acc_o is None:
            acc_o, acc_l = po, pl
        else:
            acc_o, acc_l = oracle.lse_merge(acc_o, acc_l, po, pl)
    return acc_o, acc_l


@pytest.mark.parametrize("Tn", [1, 4, 16])
def test_decode_small_all_rows(Tn):
    w = syn.scaled(syn.DECODE_WORKLOADS[1], Tn=Tn)
    q, k, v = syn.make_decode(w)
    bounds = w.portions()
    kp, vp = _portions_dev(k, v, bounds)
    say(f"decode {w.name} Tn={Tn} portions={bounds}")
    out, lse = _run(to_dev(q), kp, vp, [o for o, _ in bounds], w.hist, True)
    rows = all_rows(w.B, w.Hq, w.Tn)
    ro, rl = oracle.attention(q, k, v, q_off=w.hist, k_off=0, causal=True, rows=rows)
    go, gl = gather_rows(out, lse, rows)
    compare(go, gl, ro, rl, "bf16", f"decode Tn={Tn}", rows)


def test_decode_d64_bidirectional_bf16_out():
    w = syn.scaled(syn.DECODE_WORKLOADS[1], D=64, Hq=12, Hkv=3, hist=777, N=3, Tn=3,
                   causal=False, seed=2011)
    q, k, v = syn.make_decode(w)
    bounds = w.portions()
    kp, vp = _portions_dev(k, v, bounds)
    out, lse = _run(to_dev(q), kp, vp, [o for o, _ in bounds], w.hist, False,
                    out_dtype=torch.bfloat16)
    rows = all_rows(w.B, w.Hq, w.Tn)
    ro, rl = oracle.attention(q, k, v, q_off=w.hist, k_off=0, causal=False, rows=rows)
    go, gl = gather_rows(out, lse, rows)
    compare(go, gl, ro, rl, "bf16", "decode d=64 bidirectional, bf16 out", rows,
            out_bf16=True)


def test_decode_shuffled_gapped_empty_portions():
    """Portions in any order, not adjacent (a gap of history left out), one
    empty and one shorter than a tile."""
    w = syn.scaled(syn.DECODE_WORKLOADS[1], hist=1500, Tn=2, seed=2012)
    q, k, v = syn.make_decode(w)
    bounds = [(900, 602), (0, 300), (300, 0), (310, 37), (347, 500)]   # 847..899 left out
    order = [3, 0, 4, 2, 1]
    bounds = [bounds[i] for i in order]
    kp, vp = _portions_dev(k, v, bounds)
    out, lse = _run(to_dev(q), kp, vp, [o for o, _ in bounds], w.hist, True)
    rows = all_rows(w.B, w.Hq, w.Tn)
    ro, rl = _oracle_by_portions(q, k, v, bounds, w.hist, True, rows)
    go, gl = gather_rows(out, lse, rows)
    compare(go, gl, ro, rl, "bf16", "decode shuffled / gapped / empty portions", rows)


def test_decode_per_portion_partials_then_merge():
    """Each portion alone gives its normalised partial (o_j, lse_j); the LSE
    merge kernel combines them into the same result as one call over all."""
    w = syn.DECODE_WORKLOADS[1]
    q, k, v = syn.make_decode(w)
    bounds = w.portions()
    kp, vp = _portions_dev(k, v, bounds)
    qd = to_dev(q)
    acc_o = acc_l = None
    for j, (o, _) in enumerate(bounds):
        po, pl = _run(qd, [kp[j]], [vp[j]], [o], w.hist, True)
        if acc_o is None:
            acc_o, acc_l = po, pl
        else:
            cakv.cakv_lse_merge(acc_o, acc_l, po, pl, acc_o, acc_l)
    torch.cuda.synchronize()
    rows = all_rows(w.B, w.Hq, w.Tn)
    ro, rl = oracle.attention(q, k, v, q_off=w.hist, k_off=0, causal=True, rows=rows)
    go, gl = gather_rows(acc_o, acc_l, rows)
    compare(go, gl, ro, rl, "bf16", "per-portion partials + merge", rows)
    full_o, full_l = _run(qd, kp, vp, [o for o, _ in bounds], w.hist, True)
    fo, fl = gather_rows(full_o, full_l, rows)
    assert np.abs(fo - go).max() <= 1e-3 and np.abs(fl - gl).max() <= 1e-4


def test_decode_rows_without_keys_and_noops():
    """All keys after the queries (causal): out = 0, lse = -inf. B = 0 and
    Tn = 0 launch nothing."""
    w = syn.scaled(syn.DECODE_WORKLOADS[1], hist=256, Tn=2, seed=2013)
    q, k, v = syn.make_decode(w)
    kp, vp = _portions_dev(k, v, [(0, 256)])
    out, lse = _run(to_dev(q), kp, vp, [10_000], 0, True)   # keys at 10000.. > queries 0, 1
    assert float(out.abs().max()) == 0.0
    assert torch.isinf(lse).all() and (lse < 0).all()
    z = torch.empty((0, 2, w.Hq, w.D), dtype=torch.bfloat16, device="cuda")
    cakv.cakv_decode(z, [kp[0][:0]], [vp[0][:0]], [0], 0, True,
                     torch.empty((0, 2, w.Hq, w.D), device="cuda"))
    torch.cuda.synchronize()


def test_decode_million_token_history_all_rows():
    """The benchmarked decode workload at full size: one new token per batch
    against a 1,048,576-token history in 8 portions (its own key in the last),
    every query row against the oracle."""
    w = syn.DECODE_WORKLOADS[2]
    q, k, v = syn.make_decode(w)
    bounds = w.portions()
    kp, vp = _portions_dev(k, v, bounds)
    say(f"decode {w.name}")
    out, lse = _run(to_dev(q), kp, vp, [o for o, _ in bounds], w.hist, True)
    rows = all_rows(w.B, w.Hq, w.Tn)
    ro, rl = oracle.attention(q, k, v, q_off=w.hist, k_off=0, causal=True, rows=rows)
    go, gl = gather_rows(out, lse, rows)
    compare(go, gl, ro, rl, "bf16", "decode million-token history", rows)


def _decode_sweep_case(i):
    """Seeded random decode shape: batch, head grouping, d, history length,
    1-16 new tokens, and the whole sequence's keys cut into 1-6 portions at
    random points, some dropped (gaps), now and then an empty one, in random
    order; every third case bidirectional."""
    rng = np.random.default_rng(7000 + i)
    B = int(rng.integers(1, 3))
    Hq, Hkv = [(1, 1), (4, 1), (4, 2), (8, 2), (6, 3), (32, 8)][int(rng.integers(0, 6))]
    D = int(rng.choice([64, 128]))
    hist = int(rng.integers(1, 5000))
    Tn = int(rng.integers(1, 17))
    causal = i % 3 != 2
    total = hist + Tn
    nb = int(rng.integers(1, 7))
    cuts = (np.sort(rng.choice(np.arange(1, total), size=min(nb - 1, total - 1), replace=False))
            if nb > 1 else [])
    edges = [0, *[int(c) for c in cuts], total]
    bounds = [(edges[j], edges[j + 1] - edges[j]) for j in range(len(edges) - 1)]
    bounds = [bd for bd in bounds if rng.random() < 0.8] or [bounds[-1]]
    if rng.random() < 0.3:
        bounds.append((int(rng.integers(0, total)), 0))
    order = rng.permutation(len(bounds))
    return B, Hq, Hkv, D, hist, Tn, causal, [bounds[j] for j in order]


@pytest.mark.parametrize("i", range(8))
def test_decode_random_shapes_sweep(i):
    """Eight seeded random decode shapes through cakv_decode, every row
    against the oracle's per-portion attention merged by log-sum-exp."""
    B, Hq, Hkv, D, hist, Tn, causal, bounds = _decode_sweep_case(i)
    say(f"decode sweep {i}: B={B} Hq={Hq} Hkv={Hkv} D={D} hist={hist} Tn={Tn} "
        f"causal={causal} portions={bounds}")
    w = syn.DecodeWorkload("decode-sweep", B=B, Hq=Hq, Hkv=Hkv, hist=hist, N=1, Tn=Tn, D=D,
                           causal=causal, seed=7000 + i)
    q, k, v = syn.make_decode(w)
    kp, vp = _portions_dev(k, v, bounds)
    out, lse = _run(to_dev(q), kp, vp, [o for o, _ in bounds], hist, causal)
    rows = all_rows(B, Hq, Tn)
    ro, rl = _oracle_by_portions(q, k, v, bounds, hist, causal, rows)
    go, gl = gather_rows(out, lse, rows)
    compare(go, gl, ro, rl, "bf16", f"decode sweep {i}", rows)


@pytest.mark.parametrize("case", [
    # (B, Hq, Hkv, D, hist, Tn, causal, portions)
    (2, 16, 8, 64, 3000, 5, True, [(1800, 700), (0, 900), (2500, 505), (900, 0), (900, 900)]),
    (1, 8, 4, 128, 2500, 20, False, [(0, 1000), (1000, 1), (1001, 1519)]),
    (3, 4, 4, 64, 900, 1, True, [(0, 901)]),
])
def test_decode_four_heads_per_workgroup(case):
    """Shapes whose kv-head count is a multiple of four, which the split
    kernel serves with four heads' waves per workgroup: d = 64 and 128, two
    32-row blocks (Tn = 20 at G = 2), a tiny history with fewer tiles than
    the plan's splits, portions shuffled and one empty, every row against
    the oracle's per-portion attention merged by log-sum-exp."""
    B, Hq, Hkv, D, hist, Tn, causal, bounds = case
    say(f"decode, four heads per workgroup: B={B} Hq={Hq} Hkv={Hkv} D={D} hist={hist} "
        f"Tn={Tn} causal={causal} portions={bounds}")
    w = syn.DecodeWorkload("decode-hpw4", B=B, Hq=Hq, Hkv=Hkv, hist=hist, N=1, Tn=Tn, D=D,
                           causal=causal, seed=7100 + B * 10 + Hkv)
    q, k, v = syn.make_decode(w)
    kp, vp = _portions_dev(k, v, bounds)
    out, lse = _run(to_dev(q), kp, vp, [o for o, _ in bounds], hist, causal)
    rows = all_rows(B, Hq, Tn)
    ro, rl = _oracle_by_portions(q, k, v, bounds, hist, causal, rows)
    go, gl = gather_rows(out, lse, rows)
    compare(go, gl, ro, rl, "bf16", f"decode four heads per workgroup {case[:7]}", rows)
