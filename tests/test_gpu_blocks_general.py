"""GPU parity of cakv_forward_blocks: queries at any global offset against
key/value blocks of unequal lengths at arbitrary offsets, in any order, with
gaps, empty blocks, blocks straddling the query range and blocks wholly in
the queries' future (web page "Sequence parallelism -- splitting the token
dimension across GPUs": sections "Causal attention gives us another
optimization" for the per-position rule, "Training and inference stress this
dimension differently" for a KV history appended turn by turn).

Expected values come from the fp64 oracle: one attention over the contiguous
sequence where the blocks cover every visible key, else one attention per
block combined with the oracle's log-sum-exp merge. Tile counters must equal
the oracle's brute-force tile classification exactly.
"""
import numpy as np
import pytest
import torch

import cakv_synth as syn
import context_attention_kv_amd as cakv
import oracle
from gpu_util import all_rows, compare, gather_rows, say, to_dev

pytestmark = pytest.mark.gpu


def _seq(B, Hq, Hkv, T, D, dtype, seed):
    w = syn.Workload("general-blocks", B=B, Hq=Hq, Hkv=Hkv, T=T, N=1, D=D, dtype=dtype,
                     causal=True, ranks=(0,), seed=seed)
    return syn.make_q_full(w), syn.make_kv_full(w, "k"), syn.make_kv_full(w, "v")


def _run(q, k, v, blocks, q_off, causal, counters=False):
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    kb = [kd[:, o:o + l].contiguous() for o, l in blocks]
    vb = [vd[:, o:o + l].contiguous() for o, l in blocks]
    B, Tq, Hq, D = q.shape
    out = torch.empty((B, Tq, Hq, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq, Tq), dtype=torch.float32, device="cuda")
    tc = torch.zeros(3, dtype=torch.int64, device="cuda") if counters else None
    cakv.cakv_forward_blocks(qd, kb, vb, [o for o, _ in blocks], q_off, causal, out, lse,
                             tile_counters=tc)
    torch.cuda.synchronize()
    return out, lse, tc


def _oracle_merged(q, k, v, blocks, q_off, causal, rows):
    acc_o = acc_l = None
    for o, l in blocks:
        if l == 0:
            continue
        po, pl = oracle.attention(q, k[:, o:o + l], v[:, o:o + l], q_off=q_off, k_off=o,
                                  causal=causal, rows=rows)
        if acc_o is None:
            acc_o, acc_l = po, pl
        else:
            acc_o, acc_l = oracle.lse_merge(acc_o, acc_l, po, pl)
    return acc_o, acc_l


@pytest.mark.parametrize("Hq,Hkv,D", [(8, 2, 128), (4, 4, 128), (4, 4, 64)])
def test_unequal_straddling_and_future_blocks_causal(Hq, Hkv, D):
    # grouped heads at d=128 run the ping-pong kernel, the others the four-wave one
    q, k, v = _seq(2, Hq, Hkv, 2100, D, "bf16", 3001)
    q_off, Tq = 1000, 300
    qs = np.ascontiguousarray(q[:, q_off:q_off + Tq])
    # straddles the query range / before it / wholly after it / straddles its
    # end / a short block; keys 1481..1999 are missing but no query sees them
    blocks = [(581, 700), (0, 517), (2000, 100), (1281, 200), (517, 64)]
    out, lse, tc = _run(qs, k, v, blocks, q_off, True, counters=True)
    rows = all_rows(2, Hq, Tq)
    ro, rl = oracle.attention(qs, k, v, q_off=q_off, k_off=0, causal=True, rows=rows)
    go, gl = gather_rows(out, lse, rows)
    compare(go, gl, ro, rl, "bf16", "unequal / straddling / future blocks", rows)
    starts = np.array([o for o, _ in blocks])
    lens = np.array([l for _, l in blocks])
    _, _, tiles = oracle.classify(Tq, q_off, starts, lens, causal=True, B=2, Hq=Hq,
                                  tile_q=cakv.CAKV_TILE_Q, tile_k=cakv.CAKV_TILE_K)
    got = tc.cpu().numpy()
    say(f"  tiles: gpu {got.tolist()} oracle {list(tiles)}")
    assert got.tolist() == list(tiles), "tile counts (full, masked, skipped) differ"


def test_kv_appended_across_turns():
    """A new turn's queries against the previous turns' blocks plus the
    current turn's own block (diagonal)."""
    q, k, v = _seq(1, 4, 4, 1600, 128, "bf16", 3002)
    q_off, Tq = 1500, 100
    qs = np.ascontiguousarray(q[:, q_off:q_off + Tq])
    blocks = [(1500, 100), (1000, 500), (0, 1000)]
    out, lse, _ = _run(qs, k, v, blocks, q_off, True)
    rows = all_rows(1, 4, Tq)
    ro, rl = oracle.attention(qs, k, v, q_off=q_off, k_off=0, causal=True, rows=rows)
    go, gl = gather_rows(out, lse, rows)
    compare(go, gl, ro, rl, "bf16", "KV appended across turns", rows)


def test_bidirectional_gaps_and_empty_block():
    q, k, v = _seq(1, 12, 3, 1400, 64, "bf16", 3003)
    q_off, Tq = 200, 257
    qs = np.ascontiguousarray(q[:, q_off:q_off + Tq])
    blocks = [(700, 333), (0, 300), (1100, 0), (1200, 50)]
    out, lse, _ = _run(qs, k, v, blocks, q_off, False)
    rows = all_rows(1, 12, Tq)
    ro, rl = _oracle_merged(qs, k, v, blocks, q_off, False, rows)
    go, gl = gather_rows(out, lse, rows)
    compare(go, gl, ro, rl, "bf16", "bidirectional, gaps, empty block", rows)


def test_fp32_unequal_blocks_causal():
    q, k, v = _seq(1, 2, 1, 900, 64, "f32", 3004)
    q_off, Tq = 500, 150
    qs = np.ascontiguousarray(q[:, q_off:q_off + Tq])
    blocks = [(300, 260), (0, 300), (560, 90), (650, 250)]
    out, lse, _ = _run(qs, k, v, blocks, q_off, True)
    rows = all_rows(1, 2, Tq)
    ro, rl = oracle.attention(qs, k, v, q_off=q_off, k_off=0, causal=True, rows=rows)
    go, gl = gather_rows(out, lse, rows)
    compare(go, gl, ro, rl, "f32", "fp32 unequal blocks", rows)


def _sweep_case(i):
    """Seeded random shape: batch, head grouping, d, query offset and count,
    and 1-5 blocks cut from [0, T) at random points, some dropped (gaps), an
    empty one added now and then, in random order; every third case
    bidirectional; in every fourth the block at position 0 is dropped, so
    that early causal rows may see no key."""
    rng = np.random.default_rng(5000 + i)
    B = int(rng.integers(1, 3))
    Hq, Hkv = [(1, 1), (2, 1), (4, 1), (4, 2), (4, 4), (8, 2), (6, 3)][int(rng.integers(0, 7))]
    D = int(rng.choice([64, 128]))
    T = int(rng.integers(64, 2500))
    Tq = int(rng.integers(1, min(700, T) + 1))
    q_off = int(rng.integers(0, T - Tq + 1))
    causal = i % 3 != 2
    nb = int(rng.integers(1, 6))
    cuts = np.sort(rng.choice(np.arange(1, T), size=nb - 1, replace=False)) if nb > 1 else []
    edges = [0, *[int(c) for c in cuts], T]
    blocks = [(edges[j], edges[j + 1] - edges[j]) for j in range(nb)]
    keep = [bl for bl in blocks if rng.random() < 0.8] or [blocks[-1]]
    if i % 4 == 3 and len(keep) > 1:
        keep = [bl for bl in keep if bl[0] != 0]
    if rng.random() < 0.3:
        keep.append((int(rng.integers(0, T)), 0))
    order = rng.permutation(len(keep))
    return B, Hq, Hkv, D, T, Tq, q_off, causal, [keep[j] for j in order]


@pytest.mark.parametrize("i", range(16))
def test_random_shapes_sweep(i):
    """Sixteen seeded random shapes through cakv_forward_blocks (both bf16
    kernels: grouped heads at d = 128 take the ping-pong kernel, the rest the
    four-wave one), every row against the oracle's per-block attention
    merged by log-sum-exp, and the tile counters against the brute-force
    classification."""
    B, Hq, Hkv, D, T, Tq, q_off, causal, blocks = _sweep_case(i)
    say(f"sweep {i}: B={B} Hq={Hq} Hkv={Hkv} D={D} T={T} Tq={Tq} q_off={q_off} "
        f"causal={causal} blocks={blocks}")
    q, k, v = _seq(B, Hq, Hkv, T, D, "bf16", 5000 + i)
    qs = np.ascontiguousarray(q[:, q_off:q_off + Tq])
    out, lse, tc = _run(qs, k, v, blocks, q_off, causal, counters=True)
    rows = all_rows(B, Hq, Tq)
    ro, rl = _oracle_merged(qs, k, v, blocks, q_off, causal, rows)
    go, gl = gather_rows(out, lse, rows)
    compare(go, gl, ro, rl, "bf16", f"sweep {i}", rows)
    starts = np.array([o for o, _ in blocks])
    lens = np.array([l for _, l in blocks])
    _, _, tiles = oracle.classify(Tq, q_off, starts, lens, causal=causal, B=B, Hq=Hq,
                                  tile_q=cakv.CAKV_TILE_Q, tile_k=cakv.CAKV_TILE_K)
    got = tc.cpu().numpy()
    say(f"  tiles: gpu {got.tolist()} oracle {list(tiles)}")
    assert got.tolist() == list(tiles), "tile counts (full, masked, skipped) differ"


@pytest.mark.parametrize("i", range(100, 106))
def test_random_shapes_sweep_fp32(i):
    """Six more seeded random shapes with fp32 inputs (the fp32 kernel),
    every row against the oracle to the fp32 tolerances."""
    B, Hq, Hkv, D, T, Tq, q_off, causal, blocks = _sweep_case(i)
    say(f"fp32 sweep {i}: B={B} Hq={Hq} Hkv={Hkv} D={D} T={T} Tq={Tq} q_off={q_off} "
        f"causal={causal} blocks={blocks}")
    q, k, v = _seq(B, Hq, Hkv, T, D, "f32", 5000 + i)
    qs = np.ascontiguousarray(q[:, q_off:q_off + Tq])
    out, lse, _ = _run(qs, k, v, blocks, q_off, causal)
    rows = all_rows(B, Hq, Tq)
    ro, rl = _oracle_merged(qs, k, v, blocks, q_off, causal, rows)
    go, gl = gather_rows(out, lse, rows)
    compare(go, gl, ro, rl, "f32", f"fp32 sweep {i}", rows)
