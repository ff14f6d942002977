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


def _check(name, got, ref):
    d = np.abs(got.astype(np.float64) - ref)
    rms = max(float(np.sqrt((ref ** 2).mean())), 1e-3)
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
