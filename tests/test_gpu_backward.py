"""GPU parity of cakv_backward_blocks against the fp64 gradient oracle (O4).

The GPU side runs the forward (cakv_forward_blocks: out fp32, lse) and then
the backward on the same seeded bf16 inputs and a seeded bf16 upstream
gradient dout; the oracle differentiates the plain definition in fp64 on the
same stored values.

Tolerance, per gradient tensor, relative to the reference's scale
(rms = root-mean-square of the reference tensor): max |d| <= 1e-1 * rms' and
mean |d| <= 4e-3 * rms', rms' = max(rms, 1e-3). The kernels round p and ds to
bf16 (relative error up to 2^-9 ~ 2e-3, rms ~1.1e-3) before the products that
sum them over keys or rows, so a gradient entry's error is ~1e-3 of the rms of
its terms (measured: mean |d| ~1.3e-3 rms); the largest of ~10^5 entries
lands about 20 times higher (up to 2.3e-2 rms on rows that see many keys).
A row that sees only two keys carries a gradient several times the tensor's
rms, and there the rounding of ds alone gives 6.0e-2 rms (an fp64 model of
dq with only ds rounded to bf16 reproduces the kernel's largest error on
test_backward_rows_without_keys to four digits), hence the max bound.
"""
import numpy as np
import pytest
import torch

import cakv_synth as syn
import context_attention_kv_amd as cakv
import oracle
from gpu_util import say, to_dev

pytestmark = pytest.mark.gpu


def _seq(B, Hq, Hkv, T, D, seed):
    w = syn.Workload("backward", B=B, Hq=Hq, Hkv=Hkv, T=T, N=1, D=D, dtype="bf16",
                     causal=True, ranks=(0,), seed=seed)
    q = syn.make_q_full(w)
    k = syn.make_kv_full(w, "k")
    v = syn.make_kv_full(w, "v")
    dout = np.empty((B, T, Hq, D), np.uint16)
    syn.fill(dout, seed=seed, tensor=7)
    return q, k, v, dout


def _check(name, got, ref, floor=1e-3):
    d = np.abs(got.astype(np.float64) - ref)
    rms = max(float(np.sqrt((ref ** 2).mean())), floor)
    st = dict(max=float(d.max()), mean=float(d.mean()), rms_ref=rms)
    say(f"  {name}: {st}")
    assert not np.isnan(got).any(), name
    assert st["max"] <= 1e-1 * rms, (name, st)
    assert st["mean"] <= 4e-3 * rms, (name, st)


def _run(q, k, v, dout, blocks, q_off, causal):
    qd, kd, vd, dod = to_dev(q), to_dev(k), to_dev(v), to_dev(dout)
    kb = [kd[:, o:o + l].contiguous() for o, l in blocks]
    vb = [vd[:, o:o + l].contiguous() for o, l in blocks]
    offs = [o for o, _ in blocks]
    B, Tq, Hq, D = q.shape
    out = torch.empty((B, Tq, Hq, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq, Tq), dtype=torch.float32, device="cuda")
    cakv.cakv_forward_blocks(qd, kb, vb, offs, q_off, causal, out, lse)
    dq = torch.full((B, Tq, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    dk = [torch.full(t.shape, float("nan"), dtype=torch.float32, device="cuda") for t in kb]
    dv = [torch.full(t.shape, float("nan"), dtype=torch.float32, device="cuda") for t in kb]
    cakv.cakv_backward_blocks(qd, kb, vb, offs, q_off, causal, out, lse, dod, dq, dk, dv)
    torch.cuda.synchronize()
    return dq.cpu().numpy(), [t.cpu().numpy() for t in dk], [t.cpu().numpy() for t in dv]


def test_backward_causal_diagonal_and_future_block():
    q, k, v, dout = _seq(2, 8, 2, 700, 128, 4001)
    q_off, Tq = 300, 300
    qs = np.ascontiguousarray(q[:, q_off:q_off + Tq])
    ds = np.ascontiguousarray(dout[:, q_off:q_off + Tq])
    blocks = [(300, 300), (0, 300), (600, 100)]   # diagonal, full, wholly in the future
    say(f"backward causal blocks={blocks}")
    dq, dk, dv = _run(qs, k, v, ds, blocks, q_off, True)
    rq, rk, rv = oracle.attention_backward(qs, k, v, ds, q_off=q_off, k_off=0, causal=True)
    _check("dq", dq, rq)
    for (o, l), gk, gv in zip(blocks, dk, dv):
        _check(f"dk[{o}:{o + l}]", gk, rk[:, o:o + l])
        _check(f"dv[{o}:{o + l}]", gv, rv[:, o:o + l])
    assert not dk[2].any() and not dv[2].any()


def test_backward_bidirectional_unequal_blocks_d64_gqa():
    q, k, v, dout = _seq(1, 12, 3, 900, 64, 4002)
    q_off, Tq = 100, 257
    qs = np.ascontiguousarray(q[:, q_off:q_off + Tq])
    ds = np.ascontiguousarray(dout[:, q_off:q_off + Tq])
    blocks = [(500, 400), (0, 130), (130, 370)]
    dq, dk, dv = _run(qs, k, v, ds, blocks, q_off, False)
    rq, rk, rv = oracle.attention_backward(qs, k, v, ds, q_off=q_off, k_off=0, causal=False)
    _check("dq", dq, rq)
    for (o, l), gk, gv in zip(blocks, dk, dv):
        _check(f"dk[{o}:{o + l}]", gk, rk[:, o:o + l])
        _check(f"dv[{o}:{o + l}]", gv, rv[:, o:o + l])


def test_backward_many_tiles_causal_gqa():
    """A larger causal share: 1,100 query rows (34 row tiles and a ragged 12)
    at positions 1100..2199 against a diagonal block and two unequal full
    blocks (ragged against the 64-key and 128-key tiles), 16 query heads on
    4 key/value heads, so that many workgroups of both gradient kernels are
    resident together and every tile boundary case occurs."""
    q, k, v, dout = _seq(1, 16, 4, 2200, 128, 4003)
    q_off, Tq = 1100, 1100
    qs = np.ascontiguousarray(q[:, q_off:q_off + Tq])
    ds = np.ascontiguousarray(dout[:, q_off:q_off + Tq])
    blocks = [(1100, 1100), (0, 700), (700, 400)]
    say(f"backward many tiles: blocks={blocks}")
    dq, dk, dv = _run(qs, k, v, ds, blocks, q_off, True)
    rq, rk, rv = oracle.attention_backward(qs, k, v, ds, q_off=q_off, k_off=0, causal=True)
    _check("dq", dq, rq)
    for (o, l), gk, gv in zip(blocks, dk, dv):
        _check(f"dk[{o}:{o + l}]", gk, rk[:, o:o + l])
        _check(f"dv[{o}:{o + l}]", gv, rv[:, o:o + l])


def test_backward_rows_without_keys():
    """Causal rows 0..99 precede every key (blocks start at position 100):
    their lse is -inf, their out 0, and they give no gradient anywhere; the
    rest of the rows see a diagonal block, and a block lies wholly after all
    of them."""
    q, k, v, dout = _seq(1, 8, 2, 500, 128, 4004)
    Tq = 300
    qs = np.ascontiguousarray(q[:, :Tq])
    ds = np.ascontiguousarray(dout[:, :Tq])
    blocks = [(100, 300), (400, 100)]
    dq, dk, dv = _run(qs, k, v, ds, blocks, 0, True)
    # the oracle sees exactly the blocks' keys: positions 100..499
    ks = np.ascontiguousarray(k[:, 100:])
    vs = np.ascontiguousarray(v[:, 100:])
    rq, rk, rv = oracle.attention_backward(qs, ks, vs, ds, q_off=0, k_off=100, causal=True)
    assert not dq[:, :100].any(), "rows without keys must get no gradient"
    _check("dq", dq, rq)
    for (o, l), gk, gv in zip(blocks, dk, dv):
        _check(f"dk[{o}:{o + l}]", gk, rk[:, o - 100:o - 100 + l])
        _check(f"dv[{o}:{o + l}]", gv, rv[:, o - 100:o - 100 + l])
    assert not dk[1].any() and not dv[1].any()


@pytest.mark.parametrize("D", [128, 64])
def test_backward_one_head_per_kv_head(D):
    """Hq = Hkv (no grouping): every dq workgroup covers four row blocks of one
    head and every dk/dv query tile is one head's; causal, a diagonal block
    that starts inside the query range, a full block, ragged lengths."""
    q, k, v, dout = _seq(2, 3, 3, 650, D, 4005 + D)
    q_off, Tq = 250, 400
    qs = np.ascontiguousarray(q[:, q_off:q_off + Tq])
    ds = np.ascontiguousarray(dout[:, q_off:q_off + Tq])
    blocks = [(250, 400), (0, 250)]
    dq, dk, dv = _run(qs, k, v, ds, blocks, q_off, True)
    rq, rk, rv = oracle.attention_backward(qs, k, v, ds, q_off=q_off, k_off=0, causal=True)
    _check("dq", dq, rq)
    for (o, l), gk, gv in zip(blocks, dk, dv):
        _check(f"dk[{o}:{o + l}]", gk, rk[:, o:o + l])
        _check(f"dv[{o}:{o + l}]", gv, rv[:, o:o + l])


def test_backward_full_share_sampled():
    """The backward at full size, in the launch configuration bench.py times
    (the 131,072-token causal sequence, N = 8, rank 7's share of 16,384 rows,
    32 query heads on 8 key/value heads, d = 128; workspace from
    cakv_backward_workspace_size), checked where the oracle can compute
    outputs one by one and by identities that hold at any size.

    Sampled outputs (same bound as above): dq of the row runs [0, 4),
    [8190, 8194) and [C-4, C) (each run's gradient needs only its own rows,
    so the oracle takes those rows against every key); dk and dv of the last
    four keys, positions 131,068..131,071, which only the last four query
    rows see, so the oracle's run [C-4, C) gives their whole gradient.

    Identities over every key (the outputs start as NaN, so every element
    must be written): (i) each row's p sums to 1 over its keys, so
    sum_j dv_j = sum over rows and grouped heads of dout, per kv head and
    component. The kernels' bf16 p (rounding rms 2.3e-3 relative, summed
    over ~1.2e5 keys with sum p^2 ~ e / Tk) and the fp32 lse leave about
    1.2e-5 of sqrt(sum dout^2); bound 2e-4, while one key tile of 256
    dropped or doubled moves the sum by ~2e-3. (ii) sum_j ds_ij = 0 for
    every row (the delta term cancels the mean of dP under p), so
    sum_j dk_j = 0; bf16 ds leaves ~3e-3 of the component's norm over keys
    sqrt(sum_j dk_j^2); bound 5e-2, while leaving out delta gives ~1."""
    w = syn.scaled(syn.WORKLOADS[5], name="backward-T131072-N8-Hq32-Hkv8-d128-bf16-causal",
                   T=131072)
    r, C, G = w.ranks[-1], w.C, w.Hq // w.Hkv
    say(f"backward full share: {w.name} rank {r} C={C}")
    k = syn.make_kv_full(w, "k")
    v = syn.make_kv_full(w, "v")
    q = syn.make_q_local(w, r)
    dout = np.empty((w.B, C, w.Hq, w.D), np.uint16)
    syn.fill(dout, seed=w.seed, tensor=7)
    kd, vd, qd, dod = to_dev(k), to_dev(v), to_dev(q), to_dev(dout)
    order = [(r - s) % w.N for s in range(w.N)]
    kb = [kd[:, j * C:(j + 1) * C] for j in order]
    vb = [vd[:, j * C:(j + 1) * C] for j in order]
    offs = [j * C for j in order]
    out = torch.empty((w.B, C, w.Hq, w.D), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.B, w.Hq, C), dtype=torch.float32, device="cuda")
    cakv.cakv_forward_blocks(qd, kb, vb, offs, r * C, w.causal, out, lse)
    dq = torch.full_like(out, float("nan"))
    dk = [torch.full(t.shape, float("nan"), dtype=torch.float32, device="cuda") for t in kb]
    dv = [torch.full(t.shape, float("nan"), dtype=torch.float32, device="cuda") for t in kb]
    ws = torch.empty(cakv.cakv_backward_workspace_size(w.B, w.Hq, C) // 4, dtype=torch.float32,
                     device="cuda")
    cakv.cakv_backward_blocks(qd, kb, vb, offs, r * C, w.causal, out, lse, dod, dq, dk, dv,
                              workspace=ws)
    torch.cuda.synchronize()
    say("  gpu done")
    dq = dq.cpu().numpy()
    for t in dk + dv:
        assert not torch.isnan(t).any().item()
    assert not np.isnan(dq).any()

    # sampled rows and the last keys against the oracle
    for i0 in (0, 8190, C - 4):
        qs = np.ascontiguousarray(q[:, i0:i0 + 4])
        ds = np.ascontiguousarray(dout[:, i0:i0 + 4])
        rq, rk, rv = oracle.attention_backward(qs, k, v, ds, q_off=r * C + i0, k_off=0,
                                               causal=True)
        _check(f"dq[{i0}:{i0 + 4}]", dq[:, i0:i0 + 4], rq)
        if i0 == C - 4:
            last = r * C + C - 4   # block order[0] == r holds positions r*C .. r*C + C - 1
            # these gradients are ~3e-5 (p ~ 1 / Tk), so no floor on the scale
            _check("dk[last 4 keys]", dk[0][:, C - 4:].cpu().numpy(), rk[:, last:last + 4], 0.0)
            _check("dv[last 4 keys]", dv[0][:, C - 4:].cpu().numpy(), rv[:, last:last + 4], 0.0)
        del rq, rk, rv

    # identities over every key
    sum_dk = sum(t.double().sum(dim=1) for t in dk).cpu().numpy()          # [B, Hkv, D]
    norm_dk = np.sqrt(sum((t.double() ** 2).sum(dim=1) for t in dk).cpu().numpy())
    sum_dv = sum(t.double().sum(dim=1) for t in dv).cpu().numpy()
    do = dout.astype(np.uint32) << 16
    do = do.view(np.float32).astype(np.float64).reshape(w.B, C, w.Hkv, G, w.D)
    ref_dv = do.sum(axis=(1, 3))
    scale_dv = np.sqrt((do ** 2).sum(axis=(1, 3)))
    e_dv = float((np.abs(sum_dv - ref_dv) / scale_dv).max())
    e_dk = float((np.abs(sum_dk) / norm_dk).max())
    say(f"  sum_j dv_j vs sum dout: {e_dv:.3e} of sqrt(sum dout^2); "
        f"|sum_j dk_j|: {e_dk:.3e} of the norm over keys")
    assert e_dv <= 2e-4, e_dv
    assert e_dk <= 5e-2, e_dk


def _bwd_sweep_case(i):
    """Seeded random shape for the backward: batch, head grouping, d, query
    offset and count. Causal cases cut the keys [k0, T) into 1-4 blocks at
    random points (k0 inside the first half of the query range in every
    fourth case, so that early rows see no key); bidirectional cases may
    drop blocks (gaps); now and then an empty block; random order."""
    rng = np.random.default_rng(6000 + i)
    B = int(rng.integers(1, 3))
    Hq, Hkv = [(1, 1), (2, 1), (4, 1), (4, 2), (4, 4), (8, 2), (6, 3)][int(rng.integers(0, 7))]
    D = int(rng.choice([64, 128]))
    T = int(rng.integers(64, 1500))
    Tq = int(rng.integers(1, min(500, T) + 1))
    q_off = int(rng.integers(0, T - Tq + 1))
    causal = i % 2 == 0
    k0 = int(rng.integers(0, q_off + Tq // 2 + 1)) if causal and i % 4 == 0 else 0
    nb = int(rng.integers(1, 5))
    cuts = (np.sort(rng.choice(np.arange(k0 + 1, T), size=min(nb - 1, T - k0 - 1), replace=False))
            if nb > 1 else [])
    edges = [k0, *[int(c) for c in cuts], T]
    blocks = [(edges[j], edges[j + 1] - edges[j]) for j in range(len(edges) - 1)]
    if not causal:
        blocks = [bl for bl in blocks if rng.random() < 0.8] or [blocks[-1]]
    if rng.random() < 0.3:
        blocks.append((int(rng.integers(k0, T)), 0))
    order = rng.permutation(len(blocks))
    return B, Hq, Hkv, D, T, Tq, q_off, causal, k0, [blocks[j] for j in order]


@pytest.mark.parametrize("i", range(8))
def test_backward_random_shapes_sweep(i):
    """Eight seeded random shapes through cakv_backward_blocks against O4.
    The oracle takes one key sequence: causal cases give it the contiguous
    keys [k0, T) at their positions; bidirectional ones, where positions do
    not matter, the blocks' keys concatenated. Each block's dk, dv are
    compared with the matching rows of the oracle's."""
    B, Hq, Hkv, D, T, Tq, q_off, causal, k0, blocks = _bwd_sweep_case(i)
    say(f"backward sweep {i}: B={B} Hq={Hq} Hkv={Hkv} D={D} T={T} Tq={Tq} q_off={q_off} "
        f"causal={causal} blocks={blocks}")
    q, k, v, _ = _seq(B, Hq, Hkv, T, D, 6000 + i)
    qs = np.ascontiguousarray(q[:, q_off:q_off + Tq])
    dout = np.empty((B, Tq, Hq, D), np.uint16)
    syn.fill(dout, seed=6000 + i, tensor=7)
    dq, dk, dv = _run(qs, k, v, dout, blocks, q_off, causal)
    if causal:
        at = {bl: bl[0] - k0 for bl in blocks}
        ks, vs, k_off = np.ascontiguousarray(k[:, k0:]), np.ascontiguousarray(v[:, k0:]), k0
    else:
        nz = sorted(bl for bl in blocks if bl[1] > 0)
        at, pos = {}, 0
        for bl in nz:
            at[bl] = pos
            pos += bl[1]
        ks = np.ascontiguousarray(np.concatenate([k[:, o:o + l] for o, l in nz], axis=1))
        vs = np.ascontiguousarray(np.concatenate([v[:, o:o + l] for o, l in nz], axis=1))
        k_off = 0
    rq, rk, rv = oracle.attention_backward(qs, ks, vs, dout, q_off=q_off, k_off=k_off,
                                           causal=causal)
    _check("dq", dq, rq)
    for (o, l), gk, gv in zip(blocks, dk, dv):
        if l == 0:
            continue
        s = at[(o, l)]
        _check(f"dk[{o}:{o + l}]", gk, rk[:, s:s + l])
        _check(f"dv[{o}:{o + l}]", gv, rv[:, s:s + l])
