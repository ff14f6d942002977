"""Helpers shared by the GPU tests: device upload of seeded host inputs, the
ring call through the C ABI, and comparison against the fp64 oracle.

Tolerances (tests/tolerances.py): absolute bounds on out and lse, and a
scale-aware per-row bound max_c |d out| / rms(out_ref row) that still bites
where |out| is ~1e-3 (a million keys of U(-1,1) values).
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import cakv_synth as syn
import context_attention_kv_amd as cakv
import oracle
from tolerances import TOL, check_rel, row_rel_errors


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray) -> torch.Tensor:
    """Host array (float32, or uint16 holding bf16 bits) -> device tensor."""
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def blocks_from_full(full: torch.Tensor, n: int):
    """Cut a device [B, T, H, D] into n contiguous [B, T/n, H, D] blocks
    (views when B == 1)."""
    C = full.shape[1] // n
    if full.shape[0] == 1:
        return [full[:, j * C:(j + 1) * C] for j in range(n)]
    return [full[:, j * C:(j + 1) * C].contiguous() for j in range(n)]


class Inputs:
    """Seeded inputs of a workload: host copies for the oracle, device copies
    (local query shards and the N key/value blocks) for the GPU."""

    def __init__(self, w: syn.Workload, ranks=None, host_q_full=False):
        self.w = w
        self.ranks = tuple(w.ranks if ranks is None else ranks)
        self.k = syn.make_kv_full(w, "k")
        self.v = syn.make_kv_full(w, "v")
        self.q = {r: syn.make_q_local(w, r) for r in self.ranks}
        kd, vd = to_dev(self.k), to_dev(self.v)
        self.kb = blocks_from_full(kd, w.N)
        self.vb = blocks_from_full(vd, w.N)
        if w.B != 1:
            del kd, vd
        else:
            self._keep = (kd, vd)
        self.qd = {r: to_dev(self.q[r]) for r in self.ranks}


def run_forward(inp: Inputs, rank: int, out_dtype=torch.float32, counters=False,
                workspace="auto"):
    """The whole-shard call; workspace="auto" lets small shares take the
    key-split path, None keeps the single-pass path."""
    w = inp.w
    out = torch.empty((w.B, w.C, w.Hq, w.D), dtype=out_dtype, device="cuda")
    lse = torch.empty((w.B, w.Hq, w.C), dtype=torch.float32, device="cuda")
    tc = torch.zeros(3, dtype=torch.int64, device="cuda") if counters else None
    cakv.cakv_local_shard_forward(inp.qd[rank], inp.kb, inp.vb, rank, w.causal, out, lse,
                                  tile_counters=tc, workspace=workspace)
    torch.cuda.synchronize()
    return out, lse, tc


def oracle_rows(inp: Inputs, rank: int, rows=None, threads=None):
    w = inp.w
    return oracle.attention(inp.q[rank], inp.k, inp.v, q_off=rank * w.C, causal=w.causal,
                            rows=rows, threads=threads)


def gather_rows(out: torch.Tensor, lse: torch.Tensor, rows: np.ndarray):
    """GPU results at oracle row order (b, h, i)."""
    o = out.float().cpu().numpy().astype(np.float64)
    l = lse.cpu().numpy().astype(np.float64)
    b, h, i = rows[:, 0], rows[:, 1], rows[:, 2]
    return o[b, i, h, :], l[b, h, i]


def all_rows(B, H, T):
    b, h, i = np.meshgrid(np.arange(B), np.arange(H), np.arange(T), indexing="ij")
    return np.stack([b.ravel(), h.ravel(), i.ravel()], axis=1).astype(np.int64)


def compare(got_o, got_l, ref_o, ref_l, dtype: str, what: str, rows=None, out_bf16=False):
    """Assert the tolerances (absolute and per-row relative); returns the
    error statistics. `rows` (b, h, i) only labels the worst rows in the log;
    out_bf16 marks a bf16 output copy (its own rounding widens the relative
    bound)."""
    tol = TOL[dtype]
    rel_kind = "f32" if dtype == "f32" else ("bf16-out" if out_bf16 else "bf16")
    rel_ok, rel_max, rel_mean = check_rel(got_o, ref_o, rel_kind)
    d = np.abs(got_o - ref_o)
    fin = np.isfinite(ref_l)
    assert np.array_equal(fin, np.isfinite(got_l)), f"{what}: lse finiteness differs"
    dl = np.abs(got_l[fin] - ref_l[fin]) if fin.any() else np.zeros(1)
    stats = dict(max_out=float(d.max()) if d.size else 0.0,
                 mean_out=float(d.mean()) if d.size else 0.0,
                 max_lse=float(dl.max()) if dl.size else 0.0, rows=int(len(ref_l)),
                 max_rel=rel_max, mean_rel=rel_mean)
    say(f"  {what}: {stats}")
    rr = row_rel_errors(got_o, ref_o) if d.size else np.zeros(0)
    worst = np.argsort(-d.max(axis=1))[:4] if d.size else []
    for r in worst:
        lab = tuple(rows[r]) if rows is not None else r
        say(f"    row {lab}: max|d out|={d[r].max():.3e} rel={rr[r]:.3e} |d lse|="
            f"{abs(got_l[r] - ref_l[r]):.3e} lse={ref_l[r]:.4f}")
    assert not np.isnan(got_o).any(), f"{what}: NaN in output"
    assert stats["max_out"] <= tol["max_out"], f"{what}: max |d out| {stats['max_out']}"
    assert stats["mean_out"] <= tol["mean_out"], f"{what}: mean |d out| {stats['mean_out']}"
    assert stats["max_lse"] <= tol["lse"], f"{what}: max |d lse| {stats['max_lse']}"
    assert rel_ok, f"{what}: per-row relative error max {rel_max:.3e} mean {rel_mean:.3e}"
    return stats


def expected_tiles(w: syn.Workload, rank: int):
    """Brute-force FULL / masked tile counts of one rank (oracle O3)."""
    C = w.C
    starts = np.arange(w.N) * C
    lens = np.full(w.N, C)
    _, _, tiles = oracle.classify(C, rank * C, starts, lens, causal=w.causal, B=w.B, Hq=w.Hq,
                                  tile_q=cakv.CAKV_TILE_Q, tile_k=cakv.CAKV_TILE_K)
    return tiles
