#!/usr/bin/env python3
"""Benchmark: one rank's local-shard ring attention on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config 1..5] [--gpus 1]

A step is one pass of the whole hot path over resident inputs: the ring
schedule, every non-skipped key/value block folded into the running softmax
state in ring order, and the finalisation into out/lse -- one call of
cakv_local_shard_forward (config 2: one call per rank, all four ranks). The
default workload is the million-token causal context (T = 1,048,576 in 8
chunks, rank 7, 32 query heads over 8 key/value heads, d_k = 128, bf16).

Printed: ONE JSON line. value = useful TFLOP/s (4 d_k FLOPs per allowed
(query, key) pair, masked work not counted) over the timed steps; roofline =
the forward kernel's useful FLOPs per launch over its HIP-event-timed launch
duration against the bf16 dense matrix peak (256 CUs x 2.4 GHz x 4096
FLOP/clk = 2516.6 TFLOP/s), plus roofline.sustained_mfma: the rate the
matrix cores hold on this chip with back-to-back bf16 products from registers
(random and zero operands; the clock settles lower for random ones) and
frac_of_sustained = achieved / the random-operand rate; cpu_baseline = the fp64 CPU oracle timed on a
bounded row sample on this host's cores (its rows double as a parity spot
check, reported under "parity"); kernels = the bandwidth-bound finalize and
log-sum-exp merge kernels timed at this workload's row count against 8 TB/s.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 256 * 2.4e9 * 4096 / 1e12      # 2516.58
PEAK_F32_VALU_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
CEILING_ITERS = 200000   # ~0.35-0.5 s per cakv_diag_mfma_burn launch
METRIC = "local-shard attention TFLOP/s (useful causal FLOPs), % of bf16 MFMA peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fwd_bf16_traffic.json")
KERNEL_SRC = os.path.join(ROOT, "context_attention_kv_amd", "csrc", "fwd_bf16.hip")
DECODE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.json")
DECODE_SRC = os.path.join(ROOT, "context_attention_kv_amd", "csrc", "decode_bf16.hip")
BWD_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "backward_traffic.json")
BWD_SRC = os.path.join(ROOT, "context_attention_kv_amd", "csrc", "bwd_bf16.hip")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def allowed_pairs(w, rank: int) -> int:
    """Allowed (query, key) pairs per (batch, query head) of one rank: every
    earlier chunk in full plus the lower triangle (diagonal included) of its
    own chunk when causal; all N*C*C pairs when bidirectional."""
    C = w.C
    if not w.causal:
        return w.N * C * C
    return rank * C * C + C * (C + 1) // 2


def useful_flops(w, ranks) -> int:
    return sum(4 * w.D * allowed_pairs(w, r) * w.B * w.Hq for r in ranks)


def kernel_hash(path: str = KERNEL_SRC) -> str:
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def traffic_for(workload_name: str):
    """HBM bytes per launch of the forward kernel from the committed counter
    profile, if it was taken on this workload and on the current kernel source."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_sha") != kernel_hash() or rec.get("workload") != workload_name:
        return None
    return rec.get("bytes_per_launch")


def decode_traffic(workload_name: str):
    """HBM bytes per decode call (split + merge kernels) from the committed
    counter profile, if taken on this workload and the current kernel source."""
    try:
        rec = json.load(open(DECODE_TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_sha") != kernel_hash(DECODE_SRC) or rec.get("workload") != workload_name:
        return None
    return rec.get("bytes_per_call")


def backward_traffic(workload_name: str):
    """HBM bytes per backward call (delta, dq and dk/dv kernels) from the
    committed counter profile, if taken on this workload and the current
    kernel source."""
    try:
        rec = json.load(open(BWD_TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_sha") != kernel_hash(BWD_SRC) or rec.get("workload") != workload_name:
        return None
    return rec.get("bytes_per_call")


def calibrate_copy(nbytes: int):
    """One device copy of nbytes (read nbytes, write nbytes): the reference
    the FETCH_SIZE / WRITE_SIZE counters of the forward kernel are scaled by."""
    import torch
    torch.cuda.set_device(0)
    n = nbytes // 4
    src = torch.empty(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n * 4}), flush=True)


class ClockSampler:
    """Samples the GPU's graphics clock (amdsmi GPU metrics) from a host thread
    while the timed steps run, so the line can say at what clock the chip ran
    (the matrix cores' rate follows it, and it varies from chip to chip under
    the board's power limit). Reports nothing where amdsmi is not usable."""

    def __init__(self, period_s: float = 0.05):
        self.period = period_s
        self.samples = []
        self._stop = None
        self._thread = None
        self._read = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            handle = amdsmi.amdsmi_get_processor_handles()[0]

            def read():
                m = amdsmi.amdsmi_get_gpu_metrics_info(handle)
                for key in ("current_gfxclk", "average_gfxclk_frequency"):
                    v = m.get(key)
                    if isinstance(v, (int, float)) and 0 < v < 10000:
                        return float(v)
                vals = [x for x in (m.get("current_gfxclks") or [])
                        if isinstance(x, (int, float)) and 0 < x < 10000]
                if vals:
                    return float(sum(vals)) / len(vals)
                c = amdsmi.amdsmi_get_clock_info(handle, amdsmi.AmdSmiClkType.GFX)
                return float(c.get("clk", c.get("cur_clk")))

            read()
            self._read = read
        except Exception as e:   # noqa: BLE001 -- optional telemetry
            log(f"clock sampling unavailable: {type(e).__name__}: {e}")

    def __enter__(self):
        if self._read is None:
            return self
        import threading
        self._stop = threading.Event()

        def run():
            while not self._stop.is_set():
                try:
                    self.samples.append(self._read())
                except Exception:   # noqa: BLE001
                    pass
                self._stop.wait(self.period)

        self._thread = threading.Thread(target=run, daemon=True)
        self._thread.start()
        return self

    def __exit__(self, *exc):
        if self._thread is not None:
            self._stop.set()
            self._thread.join()
        return False

    def summary(self):
        if not self.samples:
            return None
        xs = sorted(self.samples)
        return {"median_MHz": xs[len(xs) // 2], "min_MHz": xs[0], "max_MHz": xs[-1],
                "samples": len(xs), "source": "amdsmi GPU metrics, sampled every 50 ms "
                                              "during the timed steps"}


def launch_stats(ms):
    """median / min / max / mean of the per-launch HIP-event times (ms)."""
    xs = sorted(ms)
    n = len(xs)
    med = xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])
    return {"median": round(med, 4), "min": round(xs[0], 4), "max": round(xs[-1], 4),
            "mean": round(sum(xs) / n, 4), "n": n}


def forward_kernel_name(w) -> str:
    """The forward kernel the library launches for this workload: fp32 inputs
    go to the fp32 kernel; bf16 at d = 64, and one query head per kv head on
    fewer than 2,048 32-row tasks, to the four-wave kernel; every other bf16
    shape to the ping-pong kernel."""
    if w.dtype != "bf16":
        return "fwd_f32_kernel"
    tasks = w.B * w.Hq * ((w.C + 31) // 32)
    if w.D == 64 or (w.Hq == w.Hkv and tasks < 2048):
        return "fwd_bf16_4w_kernel"
    return "fwd_bf16_kernel"


def bench_per_block(args):
    """One rank's share through the per-block ring-step calls, as a ring over
    several GPUs would drive them: cakv_state_init, then cakv_block_update for
    each block in ring order r, r-1, ... (the running m, l, o in HBM between
    calls; fully masked blocks launch nothing), then cakv_finalize. Same
    useful FLOPs as the fused driver."""
    import numpy as np
    import torch

    import cakv_synth as syn
    import context_attention_kv_amd as cakv

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(3)
    torch.cuda.set_device(0)
    w = syn.WORKLOADS[args.config]
    r = w.ranks[-1]
    C = w.C
    log(f"generating {w.name} (per-block calls)")

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(a).cuda()

    kd, vd = dev(syn.make_kv_full(w, "k")), dev(syn.make_kv_full(w, "v"))
    qd = dev(syn.make_q_local(w, r))
    blocks, _ = cakv.cakv_schedule(r, w.N, C, w.causal)
    kb = {j: kd[:, j * C:(j + 1) * C].contiguous() for j in blocks}
    vb = {j: vd[:, j * C:(j + 1) * C].contiguous() for j in blocks}
    del kd, vd
    m = torch.empty((w.B, w.Hq, C), dtype=torch.float32, device="cuda")
    l = torch.empty_like(m)
    o = torch.empty((w.B, C, w.Hq, w.D), dtype=torch.float32, device="cuda")
    out = torch.empty_like(o)
    lse = torch.empty_like(m)
    stream = torch.cuda.current_stream()

    def call():
        cakv.cakv_state_init(m, l, o)
        for j in blocks:
            cakv.cakv_block_update(qd, kb[j], vb[j], r * C, j * C, w.causal, m, l, o)
        cakv.cakv_finalize(m, l, o, out, lse)

    for _ in range(max(args.warmup, 1)):
        call()
    torch.cuda.synchronize()
    steps = max(args.steps, 1)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    ms = sum(a.elapsed_time(b) for a, b in ev) / steps
    flops = useful_flops(w, [r])
    tf = flops / (ms * 1e-3) / 1e12
    is_bf16 = w.dtype == "bf16"
    peak = PEAK_BF16_TFLOPS if is_bf16 else PEAK_F32_VALU_TFLOPS
    rec = {
        "metric": "per-block ring steps (state in HBM between calls): useful TFLOP/s",
        "value": round(tf, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": max(args.warmup, 1),
        "ms_per_step": round(wall_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded SplitMix64/Box-Muller inputs of the workload's shape)",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "T": w.T, "N": w.N,
                   "chunk": C, "d_k": w.D, "causal": w.causal, "ranks": [r],
                   "calls": f"state_init + {len(blocks)} x block_update + finalize"},
        "roofline": {"bound": "mfma" if is_bf16 else "alu",
                     "kernel": forward_kernel_name(w),
                     "achieved": round(tf, 2), "peak": round(peak, 1), "unit": "TFLOP/s",
                     "frac": round(tf / peak, 4), "traffic": None,
                     "avg_call_ms": round(ms, 4), "flops_per_call": flops},
    }
    print(json.dumps(rec), flush=True)


def bench_backward(args):
    """Gradients of one rank's share (dq, dk, dv from out, lse and a seeded
    upstream gradient): useful FLOPs = 2.5 x the forward's (five products of
    2 d_k FLOPs per allowed pair: the score recomputation, dP, dV, dQ, dK)."""
    import numpy as np
    import torch

    import cakv_synth as syn
    import context_attention_kv_amd as cakv

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(3)
    torch.cuda.set_device(0)
    w = syn.scaled(syn.WORKLOADS[5], name="backward-T131072-N8-Hq32-Hkv8-d128-bf16-causal",
                   T=131072)
    r = w.ranks[-1]
    C = w.C
    log(f"generating {w.name}")

    def dev(a):
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)

    kd, vd = dev(syn.make_kv_full(w, "k")), dev(syn.make_kv_full(w, "v"))
    qd = dev(syn.make_q_local(w, r))
    dout = np.empty((w.B, C, w.Hq, w.D), np.uint16)
    syn.fill(dout, seed=w.seed, tensor=7)
    dod = dev(dout)
    order = [(r - k) % w.N for k in range(w.N)]
    kb = [kd[:, j * C:(j + 1) * C] for j in order]
    vb = [vd[:, j * C:(j + 1) * C] for j in order]
    offs = [j * C for j in order]
    out = torch.empty((w.B, C, w.Hq, w.D), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.B, w.Hq, C), dtype=torch.float32, device="cuda")
    cakv.cakv_forward_blocks(qd, kb, vb, offs, r * C, w.causal, out, lse)
    dq = torch.empty_like(out)
    dk = [torch.empty(t.shape, dtype=torch.float32, device="cuda") for t in kb]
    dv = [torch.empty(t.shape, dtype=torch.float32, device="cuda") for t in kb]
    ws = torch.empty(cakv.cakv_backward_workspace_size(w.B, w.Hq, C) // 4, dtype=torch.float32,
                     device="cuda")
    stream = torch.cuda.current_stream()

    def call():
        cakv.cakv_backward_blocks(qd, kb, vb, offs, r * C, w.causal, out, lse, dod, dq, dk, dv,
                                  workspace=ws)

    for _ in range(max(args.warmup, 1)):
        call()
    torch.cuda.synchronize()
    steps = max(args.steps, 1)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    clock = ClockSampler()
    with clock:
        t0 = time.perf_counter()
        for a, b in ev:
            a.record(stream)
            call()
            b.record(stream)
        torch.cuda.synchronize()
        wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    ms = sum(a.elapsed_time(b) for a, b in ev) / steps
    flops = 2.5 * useful_flops(w, [r])
    tf = flops / (ms * 1e-3) / 1e12
    rec = {
        "metric": "backward of one rank's share: useful TFLOP/s (2.5x the forward's FLOPs)",
        "value": round(tf, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": max(args.warmup, 1),
        "ms_per_step": round(wall_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded SplitMix64/Box-Muller inputs of the workload's shape)",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "T": w.T, "N": w.N,
                   "chunk": C, "d_k": w.D, "causal": w.causal, "ranks": [r]},
        "roofline": {"bound": "mfma", "kernel": "bwd_dq_kernel + bwd_dkdv_kernel (+ bwd_delta)",
                     "achieved": round(tf, 2), "peak": round(PEAK_BF16_TFLOPS, 1),
                     "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                     "traffic": backward_traffic(w.name),
                     "avg_call_ms": round(ms, 4), "flops_per_call": flops,
                     "gfx_clock": clock.summary()},
    }
    print(json.dumps(rec), flush=True)


def bench_decode(args):
    """Decode over a KV history in portions (HBM-bound): new tokens per second
    and algorithmic HBM bytes (the whole history's K and V, the new queries,
    out and lse) per call over the HIP-event-timed call."""
    import numpy as np
    import torch

    import cakv_synth as syn
    import context_attention_kv_amd as cakv

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(3)
    torch.cuda.set_device(0)
    w = syn.DECODE_WORKLOADS[args.decode]
    log(f"generating {w.name}")
    q, k, v = syn.make_decode(w)
    qd = torch.from_numpy(q.view(np.int16)).cuda().view(torch.bfloat16)
    kd = torch.from_numpy(k.view(np.int16)).cuda().view(torch.bfloat16)
    vd = torch.from_numpy(v.view(np.int16)).cuda().view(torch.bfloat16)
    del k, v
    bounds = w.portions()
    kp = [kd[:, o:o + l].contiguous() for o, l in bounds]
    vp = [vd[:, o:o + l].contiguous() for o, l in bounds]
    offs = [o for o, _ in bounds]
    out = torch.empty((w.B, w.Tn, w.Hq, w.D), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.B, w.Hq, w.Tn), dtype=torch.float32, device="cuda")
    nbytes = cakv.cakv_decode_workspace_size(w.B, w.Hq, w.Hkv, w.Tn, w.D, [l for _, l in bounds])
    ws = torch.empty(nbytes // 4 + 4, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def call():
        cakv.cakv_decode(qd, kp, vp, offs, w.hist, w.causal, out, lse, workspace=ws)

    steps = max(args.steps, 1) * 10
    for _ in range(max(args.warmup, 1) * 5):
        call()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    ms = sum(a.elapsed_time(b) for a, b in ev) / steps
    kv_bytes = 2 * w.B * w.total * w.Hkv * w.D * 2
    alg = kv_bytes + w.B * w.Tn * w.Hq * w.D * (2 + 4) + w.B * w.Hq * w.Tn * 4
    gbs = alg / (ms * 1e-3) / 1e9
    rec = {
        "metric": "decode over a KV history in portions: algorithmic HBM GB/s",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": max(args.warmup, 1) * 5,
        "ms_per_step": round(wall_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded SplitMix64/Box-Muller inputs of the workload's shape)",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "history": w.hist,
                   "portions": w.N, "new_tokens": w.Tn, "d_k": w.D, "causal": w.causal},
        "new_tokens_per_s": round(w.B * w.Tn / (ms * 1e-3), 1),
        "roofline": {"bound": "hbm", "kernel": "decode_split_kernel + decode_merge_kernel",
                     "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": decode_traffic(w.name),
                     "bytes_per_call": alg, "avg_call_ms": round(ms, 4),
                     "workspace_bytes": nbytes},
    }
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", type=int, default=5, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target wall time of the CPU oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-aux", action="store_true", help="skip finalize/merge timing")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the sustained matrix-core rate measurement")
    ap.add_argument("--per-block", action="store_true",
                    help="time the per-block ring-step calls (state_init, block_update per "
                         "block, finalize) on --config's workload")
    ap.add_argument("--backward", action="store_true",
                    help="time cakv_backward_blocks on the 131,072-token causal context "
                         "(the million-token workload's shape at 1/8 length) instead")
    ap.add_argument("--decode", type=int, default=0, choices=[0, 1, 2], metavar="CFG",
                    help="time cakv_decode on decode workload CFG (2 = million-token "
                         "history) instead of the forward path")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run one plain device-to-device copy of BYTES bytes (the "
                         "known-size reference for HBM byte counters) and exit")
    args = ap.parse_args()
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.decode:
        bench_decode(args)
        return
    if args.backward:
        bench_backward(args)
        return
    if args.per_block:
        bench_per_block(args)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one rank's share on ONE GPU; --gpus {args.gpus} "
              f"(WORLD_SIZE={world}) is not supported: the ring over several GPUs is not "
              "built, only the single-GPU hot path.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import cakv_synth as syn
    import context_attention_kv_amd as cakv

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(3)
    torch.cuda.set_device(0)
    w = syn.WORKLOADS[args.config]
    ranks = list(w.ranks)
    C = w.C

    # ---- inputs: seeded on the host, then resident in HBM -----------------
    t0 = time.time()
    log(f"generating {w.name}")
    k_host = syn.make_kv_full(w, "k")
    v_host = syn.make_kv_full(w, "v")
    q_host = {r: syn.make_q_local(w, r) for r in ranks}

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(a).cuda()

    kd, vd = dev(k_host), dev(v_host)
    if w.B == 1:
        kb = [kd[:, j * C:(j + 1) * C] for j in range(w.N)]
        vb = [vd[:, j * C:(j + 1) * C] for j in range(w.N)]
    else:
        kb = [kd[:, j * C:(j + 1) * C].contiguous() for j in range(w.N)]
        vb = [vd[:, j * C:(j + 1) * C].contiguous() for j in range(w.N)]
        del kd, vd
    qd = {r: dev(q_host[r]) for r in ranks}
    out = {r: torch.empty((w.B, C, w.Hq, w.D), dtype=torch.float32, device="cuda") for r in ranks}
    lse = {r: torch.empty((w.B, w.Hq, C), dtype=torch.float32, device="cuda") for r in ranks}
    torch.cuda.synchronize()
    log(f"inputs ready in {time.time() - t0:.1f}s")

    # caller-owned workspace of the key-split path for small shares (none
    # when the share fills the GPU)
    ws_bytes = cakv.cakv_forward_workspace_size(cakv.CAKV_BF16 if w.dtype == "bf16" else cakv.CAKV_F32,
                                                w.B, w.Hq, w.Hkv, C, w.D)
    ws = torch.empty(ws_bytes // 4 + 4, dtype=torch.float32, device="cuda") if ws_bytes else None
    stream = torch.cuda.current_stream()
    n_launch = len(ranks)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps * n_launch)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps * n_launch)]

    def step(timed_idx=None):
        for i, r in enumerate(ranks):
            if timed_idx is not None:
                starts[timed_idx * n_launch + i].record(stream)
            cakv.cakv_local_shard_forward(qd[r], kb, vb, r, w.causal, out[r], lse[r], workspace=ws)
            if timed_idx is not None:
                ends[timed_idx * n_launch + i].record(stream)

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log(f"warmup {i + 1}/{args.warmup} done")
    torch.cuda.synchronize()
    clock = ClockSampler()
    with clock:
        t_start = time.perf_counter()
        for s in range(args.steps):
            step(s)
        torch.cuda.synchronize()
        t_end = time.perf_counter()
    log("timed steps done")

    ms_per_step = (t_end - t_start) * 1e3 / args.steps
    flops_step = useful_flops(w, ranks)
    value = flops_step / (ms_per_step * 1e-3) / 1e12
    launch_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    # per-launch useful FLOPs: each launch is one rank's shard
    per_launch = [useful_flops(w, [r]) for r in ranks] * args.steps
    achieved = sum(per_launch) / (sum(launch_ms) * 1e-3) / 1e12
    # per-step launch time (all ranks' launches of a step summed)
    step_ms = [sum(launch_ms[i * n_launch:(i + 1) * n_launch]) for i in range(args.steps)]
    st = launch_stats(step_ms)
    is_bf16 = w.dtype == "bf16"
    peak = PEAK_BF16_TFLOPS if is_bf16 else PEAK_F32_VALU_TFLOPS
    traffic = traffic_for(w.name)
    roofline = {
        "bound": "mfma" if is_bf16 else "alu",
        "kernel": forward_kernel_name(w) + (" + split_merge_kernel (key split)" if ws is not None
                                            else ""),
        "achieved": round(achieved, 2),
        "peak": round(peak, 1),
        "unit": "TFLOP/s",
        "frac": round(achieved / peak, 4),
        "traffic": traffic,
        "avg_launch_ms": round(sum(launch_ms) / len(launch_ms), 4),
        "flops_per_launch": per_launch[0] if len(set(per_launch)) == 1 else None,
        # the same rate from the median / fastest / slowest timed step
        "launch_ms": st,
        "achieved_median": round(flops_step / (st["median"] * 1e-3) / 1e12, 2),
        "achieved_range": [round(flops_step / (st["max"] * 1e-3) / 1e12, 2),
                           round(flops_step / (st["min"] * 1e-3) / 1e12, 2)],
        "gfx_clock": clock.summary(),
    }

    # ---- what the matrix cores sustain on this chip (bf16 workloads) -------
    # back-to-back bf16 products from registers on every compute unit: random
    # operands (the practical ceiling: power draw follows the operand bits and
    # the clock settles lower) and zeros
    if is_bf16 and not args.no_ceiling:
        sink = torch.zeros(4, device="cuda")
        cakv.cakv_diag_mfma_burn(False, 20000, sink)
        rates = {}
        for name, zero in (("random_operands", False), ("zero_operands", True)):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            cakv.cakv_diag_mfma_burn(zero, CEILING_ITERS, sink)
            b.record(stream)
            torch.cuda.synchronize()
            rates[name] = round(cakv.diag_mfma_flops(CEILING_ITERS) / (a.elapsed_time(b) * 1e-3)
                                / 1e12, 1)
        roofline["sustained_mfma"] = dict(rates, unit="TFLOP/s", what=(
            "bf16 32x32x16 products back to back from registers on every CU "
            "(cakv_diag_mfma_burn)"))
        roofline["frac_of_sustained"] = round(achieved / rates["random_operands"], 4)
        log("matrix-core ceiling measured")

    # ---- bandwidth-bound kernels at this workload's row count ---------------
    kernels = {}
    if not args.no_aux:
        r = ranks[-1]
        rows = w.B * w.Hq * C
        o_a = out[r]
        o_b = torch.empty_like(o_a).copy_(o_a)
        l_a, l_b = lse[r], lse[r].clone()
        o_o = torch.empty_like(o_a)
        l_o = torch.empty_like(l_a)
        l_state = torch.ones_like(l_a)
        fin = torch.empty_like(o_a)

        def timeit(fn, reps=5):
            fn()
            torch.cuda.synchronize()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(reps)]
            for a, b in ev:
                a.record(stream)
                fn()
                b.record(stream)
            torch.cuda.synchronize()
            return sum(a.elapsed_time(b) for a, b in ev) / reps

        t_fin = timeit(lambda: cakv.cakv_finalize(l_a, l_state, o_a, fin, l_o))
        t_mrg = timeit(lambda: cakv.cakv_lse_merge(o_a, l_a, o_b, l_b, o_o, l_o))
        b_fin = rows * (8 * w.D + 12)
        b_mrg = rows * (12 * w.D + 12)
        kernels = {
            "finalize": {"bound": "hbm", "ms": round(t_fin, 4), "bytes": b_fin,
                         "achieved_GBs": round(b_fin / t_fin / 1e6, 1), "peak_GBs": PEAK_HBM_GBS,
                         "frac": round(b_fin / t_fin / 1e6 / PEAK_HBM_GBS, 4)},
            "lse_merge": {"bound": "hbm", "ms": round(t_mrg, 4), "bytes": b_mrg,
                          "achieved_GBs": round(b_mrg / t_mrg / 1e6, 1), "peak_GBs": PEAK_HBM_GBS,
                          "frac": round(b_mrg / t_mrg / 1e6 / PEAK_HBM_GBS, 4)},
        }
        del o_b, o_o, fin
        log("finalize/merge timed")

    # ---- CPU oracle baseline on a bounded row sample (also a parity check) --
    cpu_baseline = None
    parity = None
    if not args.no_cpu_baseline:
        import oracle

        cores = len(os.sched_getaffinity(0))
        r = ranks[-1]
        sample = syn.sample_rows(w, per_head=16, seed=11)
        rng = np.random.default_rng(11)
        sample = sample[rng.permutation(len(sample))]
        done, spent, flops_cpu = 0, 0.0, 0
        got_o_all, ref_o_all, got_l_all, ref_l_all = [], [], [], []
        o_host = out[r].cpu().numpy()
        l_host = lse[r].cpu().numpy()
        batch = max(cores, 8)
        while done < len(sample) and spent < args.cpu_seconds:
            rows = sample[done:done + batch]
            t = time.perf_counter()
            ro, rl = oracle.attention(q_host[r], k_host, v_host, q_off=r * C, causal=w.causal,
                                      rows=rows, threads=cores)
            spent += time.perf_counter() - t
            for (b, h, i) in rows:
                keys = (r * C + i + 1) if w.causal else w.T
                flops_cpu += 4 * w.D * keys
            got_o_all.append(o_host[rows[:, 0], rows[:, 2], rows[:, 1]])
            got_l_all.append(l_host[rows[:, 0], rows[:, 1], rows[:, 2]])
            ref_o_all.append(ro)
            ref_l_all.append(rl)
            done += len(rows)
        cpu_tflops = flops_cpu / spent / 1e12
        cpu_baseline = {
            "value": cpu_tflops, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{done} query rows (seeded, all heads) of rank {r}'s shard, fp64, "
                      f"{spent:.1f}s; full shard extrapolated "
                      f"{useful_flops(w, [r]) / (cpu_tflops * 1e12):.0f}s",
        }
        go = np.concatenate(got_o_all)
        ro = np.concatenate(ref_o_all)
        gl = np.concatenate(got_l_all)
        rl = np.concatenate(ref_l_all)
        parity = {"rows": int(done), "max_abs_out": float(np.abs(go - ro).max()),
                  "mean_abs_out": float(np.abs(go - ro).mean()),
                  "max_abs_lse": float(np.abs(gl - rl).max())}
        log(f"cpu baseline: {done} rows in {spent:.1f}s")

    rec = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if is_bf16 else "f32",
        "data": "synthetic (seeded SplitMix64/Box-Muller inputs of the workload's shape)",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "T": w.T,
                   "N": w.N, "chunk": C, "d_k": w.D, "causal": w.causal, "ranks": ranks,
                   "parallelism": "one context-parallel rank's share on 1 GPU"},
        "pct_of_peak": round(100 * value / peak, 2),
        "roofline": roofline,
        "cpu_baseline": cpu_baseline,
        "parity": parity,
        "kernels": kernels,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
