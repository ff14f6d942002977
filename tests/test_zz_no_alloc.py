"""GPU check of cakv_decode_noalloc, the decode entry point that allocates
nothing (its split states live in the library's fixed per-GPU scratch array):
through the C ABI its results must equal cakv_decode's (same kernels, same
plan, same arithmetic: bit for bit), on two calls in a row, the second with
a smaller input, so that the second call runs on the array the first left
behind. Both are also held to the oracle's bf16 tolerances."""
import numpy as np
import pytest
import torch

import cakv_synth as syn
import context_attention_kv_amd as cakv
import oracle
from gpu_util import all_rows, compare, gather_rows, say, to_dev

pytestmark = pytest.mark.gpu


def _case(B, Hq, Hkv, hist, Tn, N, D, seed):
    w = syn.DecodeWorkload("noalloc", B=B, Hq=Hq, Hkv=Hkv, hist=hist, N=N, Tn=Tn, D=D,
                           seed=seed)
    q, k, v = syn.make_decode(w)
    bounds = w.portions()
    kd, vd = to_dev(k), to_dev(v)
    kp = [kd[:, o:o + l].contiguous() for o, l in bounds]
    vp = [vd[:, o:o + l].contiguous() for o, l in bounds]
    return w, q, k, v, to_dev(q), kp, vp, [o for o, _ in bounds]


def _both(w, qd, kp, vp, offs):
    shape = (w.B, w.Tn, w.Hq, w.D)
    out_ws = torch.full(shape, float("nan"), device="cuda")
    lse_ws = torch.full((w.B, w.Hq, w.Tn), float("nan"), device="cuda")
    cakv.cakv_decode(qd, kp, vp, offs, w.hist, True, out_ws, lse_ws)
    out_na = torch.full(shape, float("nan"), device="cuda")
    lse_na = torch.full((w.B, w.Hq, w.Tn), float("nan"), device="cuda")
    cakv.cakv_decode_noalloc(qd, kp, vp, offs, w.hist, True, out_na, lse_na)
    torch.cuda.synchronize()
    return out_ws, lse_ws, out_na, lse_na


def test_noalloc_decode_equals_workspace_decode_twice():
    # first call: 4 batch rows, 32 query heads on 8, a 200,000-token history in
    # 8 portions and 3 new tokens (split state ~12.8 MB of the 32 MiB array)
    big = _case(4, 32, 8, 200_000, 3, 8, 128, 2101)
    # second call, smaller: one batch row, 8 heads on 2, 1,000 tokens, d = 64
    small = _case(1, 8, 2, 1000, 2, 3, 64, 2102)
    for tag, (w, q, k, v, qd, kp, vp, offs) in (("large", big), ("smaller", small)):
        need = cakv.cakv_decode_workspace_size(w.B, w.Hq, w.Hkv, w.Tn, w.D,
                                               [t.shape[1] for t in kp])
        say(f"[noalloc {tag}] B={w.B} Hq={w.Hq} Hkv={w.Hkv} hist={w.hist} Tn={w.Tn} D={w.D} "
            f"split state {need} bytes")
        assert 0 < need <= cakv.CAKV_DECODE_SCRATCH_BYTES
        out_ws, lse_ws, out_na, lse_na = _both(w, qd, kp, vp, offs)
        assert torch.equal(out_na, out_ws), f"{tag}: out differs from cakv_decode"
        assert torch.equal(lse_na, lse_ws), f"{tag}: lse differs from cakv_decode"
        rows = all_rows(w.B, w.Hq, w.Tn)
        ro, rl = oracle.attention(q, k, v, q_off=w.hist, k_off=0, causal=True, rows=rows)
        go, gl = gather_rows(out_na, lse_na, rows)
        compare(go, gl, ro, rl, "bf16", f"noalloc decode, {tag}", rows)


def test_noalloc_decode_rejects_sizes_above_its_scratch():
    w = syn.DecodeWorkload("noalloc-big", B=128, Hq=32, Hkv=8, hist=1000, N=2, Tn=16, D=128,
                           seed=2103)
    qd = torch.zeros((w.B, w.Tn, w.Hq, w.D), dtype=torch.bfloat16, device="cuda")
    kp = [torch.zeros((w.B, 500, w.Hkv, w.D), dtype=torch.bfloat16, device="cuda")
          for _ in range(2)]
    out = torch.zeros((w.B, w.Tn, w.Hq, w.D), device="cuda")
    with pytest.raises(cakv.CakvError) as e:
        cakv.cakv_decode_noalloc(qd, kp, kp, [0, 500], 1000, True, out)
    assert e.value.status == cakv.CAKV_ERR_SHAPE
    torch.cuda.synchronize()
    assert float(out.abs().max()) == 0.0   # nothing was launched
