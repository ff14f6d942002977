"""Seeded synthetic inputs and the workload table.

This package is shared by the tests, the benchmark and the smoke check. It
holds no attention arithmetic: ``synth.c`` maps (seed, tensor, index) to a
value with SplitMix64 and Box-Muller (see that file), and this module knows
the shapes and value distributions of the five workloads.

Shapes follow the web page "Sequence parallelism -- splitting the token
dimension across GPUs": a hidden state X of shape B x T x d (section "Start
with the hidden-state tensor") cut into N equal contiguous chunks of T/N
tokens, chunk r on rank r (section "Split tokens across four GPUs"). Per head
that is Q, K, V of shape [B, T, H, d_k] with d = H * d_k. The bidirectional
shape (Z = 12 heads, L = 2048) comes from the glossary page "Sequence
Parallelism" (section "Why It Exists").
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
# CAKV_SYNTH_LIB selects another build of synth.c (the host-sanitizer test
# build, tests/sanitize/run_host_sanitizers.py)
_LIB_PATH = os.environ.get("CAKV_SYNTH_LIB") or os.path.join(_HERE, "libcakvsynth.so")
_lib = None

TENSOR_Q, TENSOR_K, TENSOR_V = 0, 1, 2
F32, BF16 = 0, 1
NORMAL, UNIFORM = 0, 1


def build(force: bool = True) -> str:
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                        "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        lib.synth_fill.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_uint64, ctypes.c_uint64,
                                   ctypes.c_int64, ctypes.c_float, ctypes.c_void_p,
                                   ctypes.c_int64, ctypes.c_int64]
        lib.synth_fill.restype = ctypes.c_int
        lib.synth_raw.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        lib.synth_raw.restype = ctypes.c_uint64
        lib.synth_stream_key.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        lib.synth_stream_key.restype = ctypes.c_uint64
        lib.synth_bf16_to_f32.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64]
        lib.synth_bf16_to_f32.restype = None
        _lib = lib
    return _lib


def fill(out: np.ndarray, *, seed: int, tensor: int, n0: int = 0, dist: int = NORMAL,
         mul: float = 1.0, head_mul: Optional[Sequence[float]] = None, H: int = 0,
         D: int = 0) -> np.ndarray:
    """Fill the contiguous array `out` (float32 or uint16 = bf16 bits) with
    stream elements n0, n0+1, ... of (seed, tensor)."""
    assert out.flags["C_CONTIGUOUS"]
    if out.dtype == np.float32:
        dt = F32
    elif out.dtype == np.uint16:
        dt = BF16
    else:
        raise TypeError(out.dtype)
    hm = None
    if head_mul is not None:
        hm = np.ascontiguousarray(head_mul, dtype=np.float32)
        assert len(hm) == H and D > 0
    rc = _load().synth_fill(out.ctypes.data_as(ctypes.c_void_p), out.size, dt, dist,
                            seed, tensor, n0, float(mul),
                            None if hm is None else hm.ctypes.data_as(ctypes.c_void_p),
                            H, D)
    if rc != 0:
        raise ValueError("synth_fill: bad arguments")
    return out


def raw(seed: int, tensor: int, n: int) -> int:
    """Raw 64-bit SplitMix64 output n of the (seed, tensor) stream."""
    lib = _load()
    return int(lib.synth_raw(lib.synth_stream_key(seed, tensor), n))


def bf16_to_f32(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.uint16)
    out = np.empty(a.shape, np.float32)
    _load().synth_bf16_to_f32(a.ctypes.data_as(ctypes.c_void_p),
                              out.ctypes.data_as(ctypes.c_void_p), a.size)
    return out


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: a causal or bidirectional self-attention over
    T tokens cut into N chunks of C = T/N, seen from the given rank(s)."""
    name: str
    B: int
    Hq: int
    Hkv: int
    T: int
    N: int
    D: int
    dtype: str            # "f32" or "bf16" (inputs); accumulation is fp32
    causal: bool
    ranks: tuple          # ranks whose local shard is computed
    q_dist: int = NORMAL
    k_dist: int = NORMAL
    v_dist: int = NORMAL
    qkv_mul: float = 1.0  # multiplier on Q, K and V
    k_head_mul: Optional[tuple] = None  # per-KV-head multiplier on K
    seed: int = 0

    @property
    def C(self) -> int:
        return self.T // self.N

    @property
    def group(self) -> int:
        return self.Hq // self.Hkv


INV_SQRT2 = float(np.float32(1.0 / np.sqrt(2.0)))

WORKLOADS = {
    1: Workload("ring-toy-T1024-N4-d64-f32-causal", B=1, Hq=1, Hkv=1, T=1024, N=4, D=64,
                dtype="f32", causal=True, ranks=(3,), seed=1001),
    2: Workload("sharp-heads-H8-T8192-N4-d128-bf16-causal", B=1, Hq=8, Hkv=8, T=8192, N=4,
                D=128, dtype="bf16", causal=True, ranks=(0, 1, 2, 3),
                k_head_mul=(1.0, 1.0, 1.0, 1.0, 8.0, 8.0, 8.0, 8.0), seed=1002),
    3: Workload("bidir-B64-Z12-L2048-N4-d64-bf16", B=64, Hq=12, Hkv=12, T=2048, N=4, D=64,
                dtype="bf16", causal=False, ranks=(0,), seed=1003),
    4: Workload("hidden-share-B8-H64-T32768-N4-d128-bf16-causal", B=8, Hq=64, Hkv=64,
                T=32768, N=4, D=128, dtype="bf16", causal=True, ranks=(3,),
                qkv_mul=INV_SQRT2, seed=1004),
    5: Workload("million-token-T1048576-N8-Hq32-Hkv8-d128-bf16-causal", B=1, Hq=32, Hkv=8,
                T=1048576, N=8, D=128, dtype="bf16", causal=True, ranks=(7,),
                v_dist=UNIFORM, seed=1005),
}


def _np_dtype(w: Workload):
    return np.float32 if w.dtype == "f32" else np.uint16


def make_q_local(w: Workload, rank: int) -> np.ndarray:
    """Q rows of chunk `rank`: [B, C, Hq, D], elements of the full Q stream."""
    C = w.C
    q = np.empty((w.B, C, w.Hq, w.D), _np_dtype(w))
    for b in range(w.B):
        n0 = ((b * w.T + rank * C) * w.Hq) * w.D
        fill(q[b], seed=w.seed, tensor=TENSOR_Q, n0=n0, dist=w.q_dist, mul=w.qkv_mul)
    return q


def make_kv_full(w: Workload, which: str) -> np.ndarray:
    """The full K or V of the sequence: [B, T, Hkv, D]."""
    tensor = TENSOR_K if which == "k" else TENSOR_V
    dist = w.k_dist if which == "k" else w.v_dist
    hm = w.k_head_mul if which == "k" else None
    a = np.empty((w.B, w.T, w.Hkv, w.D), _np_dtype(w))
    fill(a, seed=w.seed, tensor=tensor, n0=0, dist=dist, mul=w.qkv_mul, head_mul=hm,
         H=w.Hkv, D=w.D)
    return a


def make_q_full(w: Workload) -> np.ndarray:
    a = np.empty((w.B, w.T, w.Hq, w.D), _np_dtype(w))
    fill(a, seed=w.seed, tensor=TENSOR_Q, n0=0, dist=w.q_dist, mul=w.qkv_mul)
    return a


def sample_rows(w: Workload, per_head: int, seed: int = 0, fixed=True) -> np.ndarray:
    """Row sample (b, h, i) for checks at full size: per (b, head) the fixed
    rows 0, 1, 127, 128, 255, 256, C/2, C-2, C-1 (those that exist) plus seeded
    extra rows up to `per_head`."""
    C = w.C
    base = [0, 1, 127, 128, 255, 256, C // 2, C - 2, C - 1] if fixed else []
    base = sorted({i for i in base if 0 <= i < C})
    rows = []
    key = 0
    for b in range(w.B):
        for h in range(w.Hq):
            chosen = list(base[:per_head])
            extra = per_head - len(chosen)
            n = 0
            while extra > 0:
                i = raw(seed + 77, 3, key * 1000003 + n) % C
                n += 1
                if i not in chosen:
                    chosen.append(int(i))
                    extra -= 1
            key += 1
            rows.extend((b, h, i) for i in sorted(chosen))
    return np.asarray(rows, dtype=np.int64)


def scaled(w: Workload, **kw) -> Workload:
    """A copy of `w` with some fields replaced (smaller test variants)."""
    return dataclasses.replace(w, **kw)


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    """Decode over a KV history held in portions: a sequence of `hist` history
    tokens followed by Tn new tokens. The history is cut into N equal portions;
    the new tokens' own keys and values are appended to the last portion (they
    are in the cache when the new queries run, under the causal rule)."""
    name: str
    B: int
    Hq: int
    Hkv: int
    hist: int
    N: int
    Tn: int
    D: int
    causal: bool = True
    v_dist: int = NORMAL
    seed: int = 0

    @property
    def total(self) -> int:
        return self.hist + self.Tn

    def portions(self):
        """(offset, length) of each portion, in position order."""
        P = self.hist // self.N
        out = [(j * P, P) for j in range(self.N)]
        o, l = out[-1]
        out[-1] = (o, self.total - o)
        return out


DECODE_WORKLOADS = {
    1: DecodeWorkload("decode-small-B2-Hq8-Hkv2-hist1000-N4-Tn4-d128", B=2, Hq=8, Hkv=2,
                      hist=1000, N=4, Tn=4, D=128, seed=2001),
    2: DecodeWorkload("decode-million-token-hist1048576-N8-Hq32-Hkv8-Tn1-d128-bf16", B=1, Hq=32,
                      Hkv=8, hist=1048576, N=8, Tn=1, D=128, v_dist=UNIFORM, seed=2002),
}


def make_decode(w: DecodeWorkload):
    """(q [B, Tn, Hq, D], k [B, total, Hkv, D], v) as bf16 bits: the Tn new
    queries are rows hist .. hist+Tn-1 of the sequence's Q stream, k and v the
    whole sequence's K and V streams."""
    q = np.empty((w.B, w.Tn, w.Hq, w.D), np.uint16)
    for b in range(w.B):
        fill(q[b], seed=w.seed, tensor=TENSOR_Q, n0=((b * w.total + w.hist) * w.Hq) * w.D)
    k = np.empty((w.B, w.total, w.Hkv, w.D), np.uint16)
    v = np.empty((w.B, w.total, w.Hkv, w.D), np.uint16)
    fill(k, seed=w.seed, tensor=TENSOR_K)
    fill(v, seed=w.seed, tensor=TENSOR_V, dist=w.v_dist)
    return q, k, v
