"""Host-only checks of the C ABI (no GPU needed; nothing here launches work).

* libcakv.so loads and exports every function include/*.h declares.
* cakv_schedule reproduces the ring rounds printed on the web page "Sequence
  parallelism -- splitting the token dimension across GPUs" (section "A better
  mental model: move blocks past the queries") and, bit for bit, the block
  classes the oracle's brute-force pair count gives (section "Causal
  attention gives us another optimization").
* every argument error returns its status before anything is enqueued.
"""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import context_attention_kv_amd as cakv
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if h.endswith(".h"):
            text = open(os.path.join(ROOT, "include", h)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(cakv_[a-z_0-9]+)\s*\(", text))
    return sorted(names)


def test_every_declared_symbol_is_exported():
    names = _header_functions()
    assert set(names) == set(cakv.EXPORTED)
    out = subprocess.run(["nm", "-D", "--defined-only", cakv.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for n in names:
        assert n in exported, n
        assert hasattr(cakv.lib(), n)


def test_abi_version_and_status_strings():
    assert cakv.abi_version() == 2
    for code, name in enumerate(["CAKV_OK", "CAKV_ERR_NULL", "CAKV_ERR_SHAPE", "CAKV_ERR_DTYPE",
                                 "CAKV_ERR_ALIGN", "CAKV_ERR_RANGE", "CAKV_ERR_HIP",
                                 "CAKV_ERR_INTERNAL"]):
        assert cakv.status_str(code) == name
    assert cakv.status_str(99) == "CAKV_UNKNOWN_STATUS"


def _golden_rounds():
    path = os.path.join(ROOT, "tests", "golden", "page_ring_rounds_n4.txt")
    rows = [tuple(int(x) for x in l.split()) for l in open(path)
            if l.strip() and not l.startswith("#")]
    return rows


def test_schedule_reproduces_page_ring_rounds():
    rounds = _golden_rounds()
    assert len(rounds) == 12
    for rnd, gpu, kv in rounds:
        blocks, _ = cakv.cakv_schedule(gpu, 4, 8192, False)
        assert blocks[rnd - 1] == kv
    # the unprinted fourth round follows the same rotation
    assert [cakv.cakv_schedule(g, 4, 8192, False)[0][3] for g in range(4)] == [1, 2, 3, 0]


@pytest.mark.parametrize("n", [1, 2, 3, 4, 8, 64])
@pytest.mark.parametrize("chunk", [1, 5, 64, 100])
@pytest.mark.parametrize("causal", [True, False])
def test_schedule_classes_match_brute_force(n, chunk, causal):
    starts = np.arange(n) * chunk
    lens = np.full(n, chunk)
    for r in range(n):
        blocks, classes = cakv.cakv_schedule(r, n, chunk, causal)
        assert sorted(blocks) == list(range(n))
        assert blocks == [(r - k) % n for k in range(n)]
        cls, _, _ = oracle.classify(chunk, r * chunk, starts, lens, causal=causal)
        assert [int(cls[j]) for j in blocks] == classes


def test_classify_block_edges():
    F, Dg, S = cakv.CAKV_FULL, cakv.CAKV_DIAG, cakv.CAKV_SKIP
    assert cakv.cakv_classify_block(5, 1, 5, 1, True) == F       # one query, one key, same pos
    assert cakv.cakv_classify_block(5, 2, 5, 1, True) == F
    assert cakv.cakv_classify_block(5, 1, 5, 2, True) == Dg
    assert cakv.cakv_classify_block(5, 1, 6, 9, True) == S
    assert cakv.cakv_classify_block(5, 0, 0, 9, False) == S      # nothing to pair
    assert cakv.cakv_classify_block(0, 9, 100, 9, False) == F
    for qo, ql, ko, kl in [(0, 7, 3, 11), (10, 5, 0, 10), (10, 5, 0, 11), (3, 3, 5, 1)]:
        cls, _, _ = oracle.classify(ql, qo, [0], [kl], k_off=ko, causal=True)
        assert cakv.cakv_classify_block(qo, ql, ko, kl, True) == int(cls[0])


# --- argument errors: each returns its code and launches nothing ----------------

L = cakv.lib()
NULL = None
FAKE = 0x10000          # aligned, never dereferenced: validation fails first
MIS = 0x10008           # 8-byte aligned only


def _code(ret):
    return ret


def _bu(**kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, dtype=1, B=1, Hq=4, Hkv=2, Tq=8, Tkv=8, D=128,
                qo=0, ko=0, causal=1, scale=0.0, m=FAKE, l=FAKE, o=FAKE, tc=None, st=None)
    args.update(kw)
    return L.cakv_block_update(args["q"], args["k"], args["v"], args["dtype"], args["B"],
                               args["Hq"], args["Hkv"], args["Tq"], args["Tkv"], args["D"],
                               args["qo"], args["ko"], args["causal"], args["scale"],
                               args["m"], args["l"], args["o"], args["tc"], args["st"])


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), 3), (dict(B=-1), 2), (dict(Tq=-2), 2), (dict(Tkv=-1), 2),
    (dict(Hq=3, Hkv=2), 2), (dict(Hkv=0), 2), (dict(D=96), 2), (dict(q=NULL), 1),
    (dict(m=NULL), 1), (dict(k=NULL), 1), (dict(v=NULL), 1), (dict(q=MIS), 4),
    (dict(o=MIS), 4), (dict(k=MIS), 4), (dict(tc=FAKE + 4), 4),
    (dict(Hq=1 << 18, Hkv=2), 2),
    (dict(B=1 << 16, Hq=1 << 10, Hkv=1 << 10, Tq=1 << 20), 2),   # grid above 2^31 - 1
])
def test_block_update_errors(kw, code):
    assert _bu(**kw) == code
    assert L.cakv_last_error().decode() != ""


def test_block_update_noops_launch_nothing():
    # empty or fully masked problems return OK before touching the device
    assert _bu(B=0, q=NULL) == 0
    assert _bu(Tq=0, q=NULL) == 0
    assert _bu(qo=0, ko=8) == 0          # keys all in the future: SKIP
    assert _bu(Tkv=0, k=NULL, v=NULL) == 0


def _fwd(**kw):
    n = kw.pop("n", 4)
    kb = (ctypes.c_void_p * n)(*([FAKE] * n))
    args = dict(q=FAKE, kb=kb, vb=kb, dtype=1, B=1, Hq=8, Hkv=8, C=64, n=n, D=128, rank=3,
                causal=1, scale=0.0, out=FAKE, odt=0, lse=None, ws=None, wsb=0, tc=None,
                st=None)
    args.update(kw)
    return L.cakv_local_shard_forward(args["q"], args["kb"], args["vb"], args["dtype"],
                                      args["B"], args["Hq"], args["Hkv"], args["C"], args["n"],
                                      args["D"], args["rank"], args["causal"], args["scale"],
                                      args["out"], args["odt"], args["lse"], args["ws"],
                                      args["wsb"], args["tc"], args["st"])


@pytest.mark.parametrize("kw,code", [
    (dict(rank=4), 5), (dict(rank=-1), 5), (dict(n=0, rank=0), 5), (dict(n=65, rank=0), 5),
    (dict(dtype=2), 3), (dict(odt=5), 3), (dict(D=32), 2), (dict(Hq=6, Hkv=4), 2),
    (dict(C=-1), 2), (dict(q=NULL), 1), (dict(out=NULL), 1), (dict(kb=None), 1),
    (dict(out=MIS), 4), (dict(q=MIS), 4), (dict(ws=MIS, wsb=1 << 20), 4),
    (dict(ws=FAKE, wsb=-1), 2),
])
def test_local_shard_errors(kw, code):
    assert _fwd(**kw) == code


def test_local_shard_null_block_that_the_schedule_reads():
    n = 4
    kb = (ctypes.c_void_p * n)(FAKE, FAKE, FAKE, None)   # block 3 is read by rank 3
    assert _fwd(kb=kb) == 1
    kb = (ctypes.c_void_p * n)(FAKE, FAKE, FAKE, MIS)
    assert _fwd(kb=kb) == 4


def test_schedule_errors():
    blocks = (ctypes.c_int32 * 4)()
    cls = (ctypes.c_int8 * 4)()
    assert L.cakv_schedule(0, 4, 16, 1, None, cls) == 1
    assert L.cakv_schedule(4, 4, 16, 1, blocks, cls) == 5
    assert L.cakv_schedule(0, 0, 16, 1, blocks, cls) == 5
    assert L.cakv_schedule(0, 4, -1, 1, blocks, cls) == 2


def test_state_finalize_merge_errors():
    assert L.cakv_state_init(None, FAKE, FAKE, 1, 1, 1, 128, None) == 1
    assert L.cakv_state_init(FAKE, FAKE, FAKE, 1, 1, 1, 100, None) == 2
    assert L.cakv_state_init(FAKE, FAKE, MIS, 1, 1, 1, 128, None) == 4
    assert L.cakv_state_init(None, None, None, 0, 1, 1, 128, None) == 0
    assert L.cakv_finalize(FAKE, FAKE, FAKE, FAKE, 9, None, 1, 1, 1, 128, None) == 3
    assert L.cakv_finalize(FAKE, None, FAKE, FAKE, 0, None, 1, 1, 1, 128, None) == 1
    assert L.cakv_finalize(FAKE, FAKE, FAKE, MIS, 0, None, 1, 1, 1, 128, None) == 4
    assert L.cakv_lse_merge(FAKE, FAKE, FAKE, None, FAKE, FAKE, 1, 1, 1, 64, None) == 1
    assert L.cakv_lse_merge(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 1, 48, None) == 2
    assert L.cakv_lse_merge(FAKE, FAKE, MIS, FAKE, FAKE, FAKE, 1, 1, 1, 64, None) == 4


def test_diag_mfma_burn_errors():
    assert L.cakv_diag_mfma_burn(0, -1, FAKE, None) == 2
    assert L.cakv_diag_mfma_burn(0, 1 << 31, FAKE, None) == 2
    assert L.cakv_diag_mfma_burn(0, 5, None, None) == 1
    assert L.cakv_diag_mfma_burn(0, 0, None, None) == 0   # nothing to launch


def test_diag_workgroup_order_range():
    """Orders 0..2 are accepted (the launchers apply them from the next
    call on; the GPU test checks results stay bit-identical); others are
    rejected without changing the setting."""
    for order in (1, 2, 0):
        assert L.cakv_diag_set_workgroup_order(order) == 0
    assert L.cakv_diag_set_workgroup_order(3) == 5    # CAKV_ERR_RANGE
    assert L.cakv_diag_set_workgroup_order(-1) == 5
    assert b"workgroup order" in L.cakv_last_error()


def test_decode_errors_and_workspace_size():
    I64 = ctypes.c_int64
    lens = (I64 * 3)(1000, 0, 64)
    offs = (I64 * 3)(0, 1000, 1000)
    ptrs = (ctypes.c_void_p * 3)(FAKE, None, FAKE)
    nb = I64(0)
    # workspace size: 34 tiles of 32 keys; (B=1, Hkv=2, one 32-row block) -> splits of one tile
    assert L.cakv_decode_workspace_size(1, 8, 2, 4, 128, lens, 3, ctypes.byref(nb)) == 0
    assert nb.value == 34 * 1 * 2 * 1 * 32 * (128 + 2) * 4
    assert L.cakv_decode_workspace_size(0, 8, 2, 4, 128, lens, 3, ctypes.byref(nb)) == 0
    assert nb.value == 0
    assert L.cakv_decode_workspace_size(1, 8, 3, 4, 128, lens, 3, ctypes.byref(nb)) == 2
    assert L.cakv_decode_workspace_size(1, 8, 2, 4, 96, lens, 3, ctypes.byref(nb)) == 2
    assert L.cakv_decode_workspace_size(1, 1 << 18, 2, 4, 128, lens, 3, ctypes.byref(nb)) == 2
    assert L.cakv_decode_workspace_size(1, 8, 2, 4, 128, lens, 0, ctypes.byref(nb)) == 5
    assert L.cakv_decode_workspace_size(1, 8, 2, 4, 128, None, 3, ctypes.byref(nb)) == 1
    bad = (I64 * 1)(-1)
    assert L.cakv_decode_workspace_size(1, 8, 2, 4, 128, bad, 1, ctypes.byref(nb)) == 2
    need = 34 * 2 * 32 * 130 * 4

    def dec(q=FAKE, k=ptrs, v=ptrs, n=3, dtype=1, B=1, D=128, out=FAKE, odt=0, ws=FAKE,
            wsb=need):
        return L.cakv_decode(q, k, v, lens, offs, n, dtype, B, 8, 2, 4, D, 1004, 1, 0.0, out,
                             odt, None, ws, wsb, None)
    assert dec(dtype=0) == 3            # fp32 decode is not provided
    assert dec(dtype=7) == 3
    assert dec(odt=5) == 3
    assert dec(n=0) == 5
    assert dec(D=80) == 2
    assert dec(q=None) == 1
    assert dec(ws=None) == 1
    assert dec(wsb=need - 4) == 2
    assert dec(q=MIS) == 4
    assert dec(k=None) == 1
    assert dec(B=0, q=None, out=None, ws=None) == 0   # nothing to do


def test_decode_noalloc_errors_and_scratch_limit():
    """cakv_decode_noalloc checks exactly what cakv_decode checks (no
    workspace argument), and rejects sizes whose split state exceeds its
    fixed scratch array before touching the device."""
    I64 = ctypes.c_int64
    lens = (I64 * 3)(1000, 0, 64)
    offs = (I64 * 3)(0, 1000, 1000)
    ptrs = (ctypes.c_void_p * 3)(FAKE, None, FAKE)

    def dec(q=FAKE, k=ptrs, v=ptrs, n=3, dtype=1, B=1, Hq=8, Hkv=2, Tn=4, D=128, out=FAKE,
            odt=0):
        return L.cakv_decode_noalloc(q, k, v, lens, offs, n, dtype, B, Hq, Hkv, Tn, D, 1004, 1,
                                     0.0, out, odt, None, None)
    assert dec(dtype=0) == 3
    assert dec(odt=5) == 3
    assert dec(n=0) == 5
    assert dec(D=80) == 2
    assert dec(Hq=8, Hkv=3) == 2
    assert dec(q=None) == 1
    assert dec(out=MIS) == 4
    assert dec(k=None) == 1
    assert dec(B=0, q=None, out=None) == 0   # nothing to do
    nb = I64(0)
    # 128 batch rows x 8 kv heads x two 32-row blocks: one split already needs
    # 2,048 row blocks of state (34 MB)
    assert L.cakv_decode_workspace_size(128, 32, 8, 16, 128, lens, 3, ctypes.byref(nb)) == 0
    assert nb.value > cakv.CAKV_DECODE_SCRATCH_BYTES
    assert dec(B=128, Hq=32, Hkv=8, Tn=16) == 2
    assert "scratch" in L.cakv_last_error().decode()
    # the million-token history (32 query heads on 8, one to sixteen new
    # tokens) fits
    big = (I64 * 8)(*([131072] * 7 + [131073]))
    for tn in (1, 16):
        assert L.cakv_decode_workspace_size(1, 32, 8, tn, 128, big, 8, ctypes.byref(nb)) == 0
        assert nb.value <= cakv.CAKV_DECODE_SCRATCH_BYTES


def test_forward_workspace_size():
    """Small bf16 shares of the four-wave kernel get a split workspace sized
    S x rows x (D + 2) floats (S key parts, partial m, l, o per row); shares
    that fill the GPU, fp32 and grouped-query d = 128 shapes need none."""
    nb = ctypes.c_int64(-1)
    # 8 heads x 2048 rows, d = 128: 128 four-wave workgroups -> 4 parts
    assert L.cakv_forward_workspace_size(1, 1, 8, 8, 2048, 128, ctypes.byref(nb)) == 0
    rows = 8 * 2048
    assert nb.value == (2 * 4 * rows + 4 * rows * 128) * 4
    assert L.cakv_forward_workspace_size(1, 64, 12, 12, 512, 64, ctypes.byref(nb)) == 0
    assert nb.value == 0                        # 3,072 workgroups: no split
    assert L.cakv_forward_workspace_size(0, 1, 8, 8, 2048, 128, ctypes.byref(nb)) == 0
    assert nb.value == 0                        # fp32
    assert L.cakv_forward_workspace_size(1, 1, 32, 8, 4096, 128, ctypes.byref(nb)) == 0
    assert nb.value == 0                        # grouped heads at d = 128 (ping-pong kernel)
    assert L.cakv_forward_workspace_size(1, 1, 8, 8, 0, 128, ctypes.byref(nb)) == 0
    assert nb.value == 0
    assert L.cakv_forward_workspace_size(2, 1, 8, 8, 64, 128, ctypes.byref(nb)) == 3
    assert L.cakv_forward_workspace_size(1, 1, 8, 8, 64, 96, ctypes.byref(nb)) == 2
    assert L.cakv_forward_workspace_size(1, 1, 8, 8, 64, 128, None) == 1


def test_forward_blocks_errors():
    I64 = ctypes.c_int64
    lens = (I64 * 2)(100, 0)
    offs = (I64 * 2)(0, 100)
    ptrs = (ctypes.c_void_p * 2)(FAKE, None)

    def fb(q=FAKE, n=2, dtype=1, B=1, D=128, Hkv=2, out=FAKE, odt=0, ln=lens, k=ptrs):
        return L.cakv_forward_blocks(q, k, ptrs, ln, offs, n, dtype, B, 8, Hkv, 50, D, 100, 1, 0.0,
                                     out, odt, None, None, 0, None, None)
    assert fb(dtype=5) == 3
    assert fb(odt=5) == 3
    assert fb(n=0) == 5
    assert fb(n=65) == 5
    assert fb(D=96) == 2
    assert fb(Hkv=3) == 2
    assert fb(ln=(I64 * 2)(-1, 0)) == 2
    assert fb(q=None) == 1
    assert fb(k=None) == 1
    assert fb(q=MIS) == 4
    assert fb(B=0, q=None, out=None) == 0


def test_backward_errors():
    I64 = ctypes.c_int64
    lens = (I64 * 1)(100)
    offs = (I64 * 1)(0)
    ptrs = (ctypes.c_void_p * 1)(FAKE)
    nb = I64(0)
    assert L.cakv_backward_workspace_size(2, 8, 300, ctypes.byref(nb)) == 0 and nb.value == 2 * 8 * 300 * 8
    assert L.cakv_backward_workspace_size(-1, 8, 300, ctypes.byref(nb)) == 2

    def bw(dtype=1, n=1, D=128, q=FAKE, dout=FAKE, ws=FAKE, wsb=8 * 50 * 8, dk=ptrs):
        return L.cakv_backward_blocks(q, ptrs, ptrs, lens, offs, n, dtype, 1, 8, 2, 50, D, 100, 1,
                                      0.0, FAKE, FAKE, dout, FAKE, dk, ptrs, ws, wsb, None)
    assert bw(dtype=0) == 3
    assert bw(n=0) == 5
    assert bw(D=96) == 2
    assert bw(q=None) == 1
    assert bw(dout=None) == 1
    assert bw(dk=None) == 1
    assert bw(ws=None) == 1
    assert bw(wsb=16) == 2
    assert bw(q=MIS) == 4
