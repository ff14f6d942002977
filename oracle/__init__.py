"""fp64 CPU oracle for one rank's ring attention -- TEST INFRASTRUCTURE.

Only the test-suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import this package. The product library never does, and
this package imports nothing from the product.

The arithmetic lives in ``oracle.c`` (plain C, fp64, OpenMP over rows); this
module only builds it with gcc, loads it with ctypes and marshals numpy
arrays. Every function follows the web page "Sequence parallelism --
splitting the token dimension across GPUs" (llmdaily.org, day 58):

* ``attention``        -- softmax(Q K^T / sqrt(d_k)) V row by row, the plain
                          definition (section "Attention wants keys and values
                          from other tokens"), with the causal rule of section
                          "Causal attention gives us another optimization".
* ``online_blockwise`` -- the running (m, l, o) update of section "But softmax
                          seems to require all attention scores at once",
                          applied block by block in any order.
* ``classify``         -- brute-force count of allowed pairs per block and per
                          tile (section "Causal attention gives us another
                          optimization").
* ``lse_merge``        -- combination of two normalised partials (section
                          "Training and inference stress this dimension
                          differently"; formula read from the rescale rule).

Inputs are numpy arrays: float32, or uint16 holding bfloat16 bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
# CAKV_ORACLE_LIB selects another build of oracle.c (the host-sanitizer test
# build, tests/sanitize/run_host_sanitizers.py)
_LIB_PATH = os.environ.get("CAKV_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (no fast-math, no reassociation)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.run(
            ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
             "-fno-fast-math", "-o", tmp, _SRC, "-lm"],
            check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        I = ctypes.c_int
        D = ctypes.c_double
        lib.oracle_attention_rows.argtypes = [
            P, I, P, P, I, I64, I64, I64, I64, I64, I64, I64, I64, I, D, I64,
            P, P, P, P]
        lib.oracle_attention_rows.restype = I
        lib.oracle_online_blockwise.argtypes = [
            P, I, P, P, I, I64, I64, I64, I64, I64, I64, I64, I64, I, D, I64,
            P, P, P, I64, P, P, P, P, P, P]
        lib.oracle_online_blockwise.restype = I
        lib.oracle_classify.argtypes = [
            I64, I64, I64, I, I64, P, P, I64, I64, I64, I64, P, P, P]
        lib.oracle_classify.restype = I
        lib.oracle_lse_merge.argtypes = [P, P, P, P, I64, I64, P, P]
        lib.oracle_lse_merge.restype = None
        lib.oracle_attention_backward.argtypes = [
            P, I, P, P, I, P, I, I64, I64, I64, I64, I64, I64, I64, I64, I,
            ctypes.c_double, P, P, P]
        lib.oracle_attention_backward.restype = I
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dtype_flag(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return 1
    if a.dtype == np.float32:
        return 0
    raise TypeError(f"oracle inputs are float32 or uint16 (bf16 bits), got {a.dtype}")


def _rows_array(rows, B, H, Tq):
    if rows is None:
        b, h, i = np.meshgrid(np.arange(B), np.arange(H), np.arange(Tq), indexing="ij")
        rows = np.stack([b.ravel(), h.ravel(), i.ravel()], axis=1)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 3))
    return rows


def default_scale(D: int) -> float:
    """1/sqrt(d_k): the scale of section 'Attention wants keys and values...'."""
    return 1.0 / np.sqrt(float(D))


def attention(q, k, v, *, q_off=0, k_off=0, causal=True, scale=None, rows=None,
              return_weights=False, threads=None):
    """O1: fp64 attention of the rows (b, h, i) of q [B,Tq,Hq,D] against
    k, v [B,Tk,Hkv,D]. Query row i sits at global position q_off + i, key j at
    k_off + j. rows=None means every row. Returns (out [n,D], lse [n]) and,
    if asked, the weights [n,Tk]. Row order of the result follows ``rows``
    (for rows=None: b-major, then head, then position)."""
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    B, Tq, Hq, D = q.shape
    Bk, Tk, Hkv, Dk = k.shape
    assert Bk == B and Dk == D and v.shape == k.shape
    fq, fk = _dtype_flag(q), _dtype_flag(k)
    assert _dtype_flag(v) == fk
    rows = _rows_array(rows, B, Hq, Tq)
    n = rows.shape[0]
    out = np.zeros((n, D), np.float64)
    lse = np.zeros((n,), np.float64)
    w = np.zeros((n, Tk), np.float64) if return_weights else None
    if scale is None:
        scale = default_scale(D)
    _set_threads(threads)
    rc = _load().oracle_attention_rows(
        _ptr(q), fq, _ptr(k), _ptr(v), fk, B, Hq, Hkv, Tq, Tk, D, q_off, k_off,
        int(bool(causal)), float(scale), n, _ptr(rows), _ptr(out), _ptr(lse),
        _ptr(w))
    if rc != 0:
        raise ValueError("oracle_attention_rows: bad arguments")
    return (out, lse, w) if return_weights else (out, lse)


def online_blockwise(q, k, v, starts, lens, order, *, q_off=0, k_off=0,
                     causal=True, scale=None, rows=None, return_state=False,
                     threads=None):
    """O2: the page's running-statistics algorithm over key blocks taken in
    ``order``. Returns (out, lse) and optionally the state (m, l, o)."""
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    B, Tq, Hq, D = q.shape
    _, Tk, Hkv, _ = k.shape
    fq, fk = _dtype_flag(q), _dtype_flag(k)
    rows = _rows_array(rows, B, Hq, Tq)
    n = rows.shape[0]
    starts = np.ascontiguousarray(starts, dtype=np.int64)
    lens = np.ascontiguousarray(lens, dtype=np.int64)
    order = np.ascontiguousarray(order, dtype=np.int64)
    assert starts.shape == lens.shape == order.shape
    out = np.zeros((n, D), np.float64)
    lse = np.zeros((n,), np.float64)
    m = np.zeros((n,), np.float64)
    l_ = np.zeros((n,), np.float64)
    o = np.zeros((n, D), np.float64)
    if scale is None:
        scale = default_scale(D)
    _set_threads(threads)
    rc = _load().oracle_online_blockwise(
        _ptr(q), fq, _ptr(k), _ptr(v), fk, B, Hq, Hkv, Tq, Tk, D, q_off, k_off,
        int(bool(causal)), float(scale), len(starts), _ptr(starts), _ptr(lens),
        _ptr(order), n, _ptr(rows), _ptr(out), _ptr(lse), _ptr(m), _ptr(l_),
        _ptr(o))
    if rc != 0:
        raise ValueError("oracle_online_blockwise: bad arguments")
    if return_state:
        return out, lse, (m, l_, o)
    return out, lse


def classify(Tq, q_off, starts, lens, *, k_off=0, causal=True, B=1, Hq=1,
             tile_q=32, tile_k=64):
    """O3: brute-force block classes (0 FULL, 1 DIAG, 2 SKIP), allowed-pair
    counts per block, and tile counts [full, masked, skip] over B*Hq."""
    starts = np.ascontiguousarray(starts, dtype=np.int64)
    lens = np.ascontiguousarray(lens, dtype=np.int64)
    nb = len(starts)
    cls = np.zeros((nb,), np.int8)
    pairs = np.zeros((nb,), np.int64)
    tiles = np.zeros((3,), np.int64)
    rc = _load().oracle_classify(Tq, q_off, k_off, int(bool(causal)), nb,
                                 _ptr(starts), _ptr(lens), B, Hq, tile_q,
                                 tile_k, _ptr(cls), _ptr(pairs), _ptr(tiles))
    if rc != 0:
        raise ValueError("oracle_classify: bad arguments")
    return cls, pairs, tiles


def attention_backward(q, k, v, dout, *, q_off=0, k_off=0, causal=True, scale=None,
                       threads=None):
    """O4: fp64 gradients (dq [B,Tq,Hq,D], dk, dv [B,Tk,Hkv,D]) of
    sum(out * dout) for out = attention(q, k, v) as in O1."""
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    dout = np.ascontiguousarray(dout)
    B, Tq, Hq, D = q.shape
    Bk, Tk, Hkv, Dk = k.shape
    assert Bk == B and Dk == D and v.shape == k.shape and dout.shape == q.shape
    fq, fk, fd = _dtype_flag(q), _dtype_flag(k), _dtype_flag(dout)
    assert _dtype_flag(v) == fk
    if scale is None:
        scale = default_scale(D)
    dq = np.zeros((B, Tq, Hq, D), np.float64)
    dk = np.zeros((B, Tk, Hkv, D), np.float64)
    dv = np.zeros((B, Tk, Hkv, D), np.float64)
    _set_threads(threads)
    rc = _load().oracle_attention_backward(
        _ptr(q), fq, _ptr(k), _ptr(v), fk, _ptr(dout), fd, B, Hq, Hkv, Tq, Tk, D,
        q_off, k_off, int(bool(causal)), float(scale), _ptr(dq), _ptr(dk), _ptr(dv))
    if rc != 0:
        raise ValueError("oracle_attention_backward: bad arguments")
    return dq, dk, dv


def lse_merge(o_a, lse_a, o_b, lse_b):
    """fp64 log-sum-exp merge of two normalised partials (rows x D)."""
    o_a = np.ascontiguousarray(o_a, dtype=np.float64)
    o_b = np.ascontiguousarray(o_b, dtype=np.float64)
    lse_a = np.ascontiguousarray(lse_a, dtype=np.float64)
    lse_b = np.ascontiguousarray(lse_b, dtype=np.float64)
    rows, D = o_a.shape
    o = np.zeros_like(o_a)
    lse = np.zeros_like(lse_a)
    _load().oracle_lse_merge(_ptr(o_a), _ptr(lse_a), _ptr(o_b), _ptr(lse_b),
                             rows, D, _ptr(o), _ptr(lse))
    return o, lse


def _set_threads(threads):
    # OpenMP reads OMP_NUM_THREADS at first use; an explicit count is set
    # through the runtime so later calls can change it.
    if threads is None:
        return
    try:
        gomp = ctypes.CDLL("libgomp.so.1")
        gomp.omp_set_num_threads(int(threads))
    except OSError:
        os.environ["OMP_NUM_THREADS"] = str(int(threads))


def ring_rows_for_rank(rank: int, chunk: int):
    """Global positions owned by `rank` when T is cut into equal chunks of
    `chunk` tokens (section 'Split tokens across four GPUs'), 0-based."""
    return rank * chunk, (rank + 1) * chunk
