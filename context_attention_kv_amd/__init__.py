"""Python binding of libcakv: local-shard ring attention on MI355X (gfx950).

Argument marshalling only. Every function here has the name and meaning of a
C entry point declared in include/cakv.h; it turns torch tensors into device
pointers and the current HIP stream into a handle, calls libcakv.so through
ctypes, and raises CakvError on a non-zero status. All device work happens in
the library's HIP kernels; there is no fallback. If libcakv.so is missing the
import fails: build it with ``python -m context_attention_kv_amd.build``.

Layouts (contiguous, innermost last): Q/out/o [B, T, Hq, D]; K/V blocks
[B, T, Hkv, D]; m/l/lse [B, Hq, T].
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
# CAKV_LIB_PATH selects another build of the same library: the host-only
# sanitizer build of the C ABI layer, whose launchers all return an error
# (tests/sanitize/run_host_sanitizers.py)
LIB_PATH = os.environ.get("CAKV_LIB_PATH") or os.path.join(_HERE, "libcakv.so")

CAKV_OK = 0
CAKV_ERR_NULL, CAKV_ERR_SHAPE, CAKV_ERR_DTYPE, CAKV_ERR_ALIGN, CAKV_ERR_RANGE, CAKV_ERR_HIP = 1, 2, 3, 4, 5, 6
CAKV_F32, CAKV_BF16 = 0, 1
CAKV_FULL, CAKV_DIAG, CAKV_SKIP = 0, 1, 2
CAKV_MAX_CHUNKS = 64
CAKV_TILE_Q, CAKV_TILE_K = 32, 64

# every symbol include/cakv.h declares
EXPORTED = (
    "cakv_abi_version", "cakv_status_str", "cakv_last_error", "cakv_classify_block",
    "cakv_schedule", "cakv_state_init", "cakv_block_update", "cakv_finalize",
    "cakv_lse_merge", "cakv_local_shard_forward", "cakv_diag_mfma_burn", "cakv_decode",
    "cakv_decode_workspace_size", "cakv_forward_blocks", "cakv_backward_blocks",
    "cakv_backward_workspace_size", "cakv_decode_noalloc", "cakv_forward_workspace_size",
    "cakv_diag_set_workgroup_order",
)
CAKV_DECODE_SCRATCH_BYTES = 32 << 20   # scratch array behind cakv_decode_noalloc
DIAG_MFMA_WG = 2048   # workgroups of one cakv_diag_mfma_burn launch (include/cakv_diag.h)


class CakvError(RuntimeError):
    def __init__(self, status: int, func: str, detail: str):
        self.status = status
        super().__init__(f"{func}: {status_str(status)}: {detail}")


def _load_lib():
    # torch ships its own HIP runtime under the same soname; loading it first
    # makes libcakv bind to that one instance, so tensors, streams and kernels
    # all live in a single runtime.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"libcakv.so not found at {LIB_PATH}; build it with "
            "`python -m context_attention_kv_amd.build` (needs ROCm hipcc)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, I64, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
    sig = {
        "cakv_abi_version": ([], I),
        "cakv_status_str": ([I], ctypes.c_char_p),
        "cakv_last_error": ([], ctypes.c_char_p),
        "cakv_classify_block": ([I64, I64, I64, I64, I, P], I),
        "cakv_schedule": ([I, I, I64, I, P, P], I),
        "cakv_state_init": ([P, P, P, I, I, I, I, P], I),
        "cakv_block_update": ([P, P, P, I, I, I, I, I, I, I, I64, I64, I, F, P, P, P, P, P], I),
        "cakv_finalize": ([P, P, P, P, I, P, I, I, I, I, P], I),
        "cakv_lse_merge": ([P, P, P, P, P, P, I, I, I, I, P], I),
        "cakv_local_shard_forward": ([P, P, P, I, I, I, I, I, I, I, I, I, F, P, I, P, P, I64, P, P],
                                     I),
        "cakv_diag_mfma_burn": ([I, I64, P, P], I),
        "cakv_diag_set_workgroup_order": ([I], I),
        "cakv_decode": ([P, P, P, P, P, I, I, I, I, I, I, I, I64, I, F, P, I, P, P, I64, P], I),
        "cakv_forward_blocks": ([P, P, P, P, P, I, I, I, I, I, I, I, I64, I, F, P, I, P, P, I64, P,
                                 P], I),
        "cakv_forward_workspace_size": ([I, I, I, I, I, I, P], I),
        "cakv_backward_blocks": ([P, P, P, P, P, I, I, I, I, I, I, I, I64, I, F, P, P, P, P, P, P,
                                  P, I64, P], I),
        "cakv_backward_workspace_size": ([I, I, I, P], I),
        "cakv_decode_workspace_size": ([I, I, I, I, I, P, I, P], I),
        "cakv_decode_noalloc": ([P, P, P, P, P, I, I, I, I, I, I, I, I64, I, F, P, I, P, P], I),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


_lib = _load_lib()


def lib() -> ctypes.CDLL:
    return _lib


def status_str(status: int) -> str:
    return _lib.cakv_status_str(status).decode()


def _check(status: int, func: str):
    if status != CAKV_OK:
        raise CakvError(status, func, _lib.cakv_last_error().decode())


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(int(stream))
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return CAKV_BF16
    if t.dtype == torch.float32:
        return CAKV_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _contig(*ts):
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _counters(tc) -> Optional[int]:
    """Device pointer of a tile-counter tensor: int64 with the three entries
    (full, masked, skipped) the library adds to."""
    if tc is None:
        return None
    import torch
    if tc.dtype != torch.int64 or tc.numel() < 3 or not tc.is_contiguous():
        raise ValueError("tile_counters must be a contiguous int64 tensor of 3 entries")
    return tc.data_ptr()


def abi_version() -> int:
    return _lib.cakv_abi_version()


def cakv_classify_block(q_offset: int, q_len: int, kv_offset: int, kv_len: int,
                        causal: bool) -> int:
    out = ctypes.c_int8()
    _check(_lib.cakv_classify_block(q_offset, q_len, kv_offset, kv_len, int(causal),
                                    ctypes.byref(out)), "cakv_classify_block")
    return out.value


def cakv_schedule(rank: int, n_chunks: int, chunk_len: int, causal: bool):
    """Ring order and per-block class for one rank (host only)."""
    n = max(int(n_chunks), 0)
    blocks = (ctypes.c_int32 * max(n, 1))()
    classes = (ctypes.c_int8 * max(n, 1))()
    _check(_lib.cakv_schedule(rank, n_chunks, chunk_len, int(causal), blocks, classes),
           "cakv_schedule")
    return list(blocks[:n]), list(classes[:n])


def cakv_state_init(m, l, o, stream=None):
    _contig(m, l, o)
    B, Tq, Hq, D = o.shape
    _check(_lib.cakv_state_init(_ptr(m), _ptr(l), _ptr(o), B, Hq, Tq, D, _stream(stream)),
           "cakv_state_init")


def cakv_block_update(q, k, v, q_offset: int, kv_offset: int, causal: bool, m, l, o,
                      scale: float = 0.0, tile_counters=None, stream=None):
    _contig(q, k, v, m, l, o)
    B, Tq, Hq, D = q.shape
    Bk, Tkv, Hkv, Dk = k.shape
    if Bk != B or Dk != D or tuple(v.shape) != tuple(k.shape) or v.dtype != k.dtype \
            or q.dtype != k.dtype:
        raise ValueError("q/k/v shapes or dtypes disagree")
    if tuple(o.shape) != (B, Tq, Hq, D) or tuple(m.shape) != (B, Hq, Tq) \
            or tuple(l.shape) != (B, Hq, Tq):
        raise ValueError("state shapes disagree with q")
    _check(_lib.cakv_block_update(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), B, Hq, Hkv, Tq,
                                  Tkv, D, q_offset, kv_offset, int(causal), float(scale),
                                  _ptr(m), _ptr(l), _ptr(o), _counters(tile_counters),
                                  _stream(stream)), "cakv_block_update")


def cakv_finalize(m, l, o, out, lse=None, stream=None):
    _contig(m, l, o, out, lse)
    B, Tq, Hq, D = o.shape
    if tuple(out.shape) != tuple(o.shape):
        raise ValueError("out shape disagrees with o")
    _check(_lib.cakv_finalize(_ptr(m), _ptr(l), _ptr(o), _ptr(out), _dtype_code(out),
                              _ptr(lse), B, Hq, Tq, D, _stream(stream)), "cakv_finalize")


def cakv_lse_merge(o_a, lse_a, o_b, lse_b, o_out, lse_out, stream=None):
    _contig(o_a, lse_a, o_b, lse_b, o_out, lse_out)
    B, Tq, Hq, D = o_a.shape
    for t in (o_b, o_out):
        if tuple(t.shape) != tuple(o_a.shape):
            raise ValueError("merge operand shapes disagree")
    _check(_lib.cakv_lse_merge(_ptr(o_a), _ptr(lse_a), _ptr(o_b), _ptr(lse_b), _ptr(o_out),
                               _ptr(lse_out), B, Hq, Tq, D, _stream(stream)), "cakv_lse_merge")


def cakv_forward_workspace_size(dtype_code: int, B: int, Hq: int, Hkv: int, Tq: int,
                                D: int) -> int:
    """Bytes of workspace that lets the whole-shard forward split a small
    share's key range (0 when it is not split)."""
    out = ctypes.c_int64(0)
    _check(_lib.cakv_forward_workspace_size(dtype_code, B, Hq, Hkv, Tq, D, ctypes.byref(out)),
           "cakv_forward_workspace_size")
    return out.value


def _fwd_workspace(workspace, q, Hkv: int, Tq: int):
    """(pointer, bytes, tensor) of the forward workspace: "auto" allocates
    what cakv_forward_workspace_size asks for (nothing when it is 0), None
    passes none, a tensor is passed as given."""
    if workspace is None:
        return None, 0, None
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError('workspace must be "auto", None or a device tensor')
        B, _, Hq, D = q.shape
        nbytes = cakv_forward_workspace_size(_dtype_code(q), B, Hq, Hkv, Tq, D)
        if nbytes == 0:
            return None, 0, None
        import torch
        workspace = torch.empty(nbytes // 4 + 4, dtype=torch.float32, device=q.device)
    return workspace.data_ptr(), workspace.numel() * workspace.element_size(), workspace


def cakv_local_shard_forward(q_local, k_blocks: Sequence, v_blocks: Sequence, rank: int,
                             causal: bool, out, lse=None, scale: float = 0.0,
                             tile_counters=None, workspace="auto", stream=None):
    """One rank's share: q_local [B, C, Hq, D] against N blocks [B, C, Hkv, D]
    in ring order rank, rank-1, ...; writes out [B, C, Hq, D] and lse [B, Hq, C].
    workspace: "auto" (allocate cakv_forward_workspace_size bytes when a small
    share can use them), None, or a device tensor."""
    _contig(q_local, out, lse, *k_blocks, *v_blocks)
    B, C, Hq, D = q_local.shape
    n = len(k_blocks)
    if len(v_blocks) != n or n == 0:
        raise ValueError("need the same positive number of K and V blocks")
    Hkv = k_blocks[0].shape[2]
    for t in list(k_blocks) + list(v_blocks):
        if tuple(t.shape) != (B, C, Hkv, D) or t.dtype != q_local.dtype:
            raise ValueError("every block must be [B, C, Hkv, D] with the query dtype")
    karr = (ctypes.c_void_p * n)(*[t.data_ptr() for t in k_blocks])
    varr = (ctypes.c_void_p * n)(*[t.data_ptr() for t in v_blocks])
    wp, wb, _keep = _fwd_workspace(workspace, q_local, Hkv, C)
    _check(_lib.cakv_local_shard_forward(_ptr(q_local), karr, varr, _dtype_code(q_local), B,
                                         Hq, Hkv, C, n, D, rank, int(causal), float(scale),
                                         _ptr(out), _dtype_code(out), _ptr(lse), wp, wb,
                                         _counters(tile_counters), _stream(stream)),
           "cakv_local_shard_forward")


def cakv_diag_mfma_burn(zero_operands: bool, iters: int, sink, stream=None):
    """Measurement aid: back-to-back bf16 matrix-core products on every compute
    unit (random or zero operands); FLOPs = diag_mfma_flops(iters)."""
    _check(_lib.cakv_diag_mfma_burn(int(bool(zero_operands)), int(iters), _ptr(sink),
                                    _stream(stream)), "cakv_diag_mfma_burn")


def cakv_diag_set_workgroup_order(order: int):
    """Permute the logical workgroup ids of every later launch (0 none, 1
    scrambled, 2 reversed): an ordering check for tests; results must stay
    bit-identical."""
    _check(_lib.cakv_diag_set_workgroup_order(int(order)), "cakv_diag_set_workgroup_order")


def diag_mfma_flops(iters: int) -> float:
    return float(DIAG_MFMA_WG) * 4 * iters * 16 * 32768


def cakv_decode_workspace_size(B: int, Hq: int, Hkv: int, Tn: int, D: int,
                               kv_lens: Sequence[int]) -> int:
    """Bytes of workspace cakv_decode needs for these sizes."""
    n = len(kv_lens)
    lens = (ctypes.c_int64 * max(n, 1))(*[int(x) for x in kv_lens])
    out = ctypes.c_int64(0)
    _check(_lib.cakv_decode_workspace_size(B, Hq, Hkv, Tn, D, lens, n, ctypes.byref(out)),
           "cakv_decode_workspace_size")
    return out.value


def cakv_decode(q, k_portions: Sequence, v_portions: Sequence, kv_offsets: Sequence[int],
                q_offset: int, causal: bool, out, lse=None, workspace=None, scale: float = 0.0,
                stream=None):
    """New queries q [B, Tn, Hq, D] (positions q_offset ...) against KV history
    portions k/v [B, L_j, Hkv, D] at global offsets kv_offsets[j]; writes out
    [B, Tn, Hq, D] and lse [B, Hq, Tn]. workspace: a device tensor of at least
    cakv_decode_workspace_size bytes (allocated here when None)."""
    _contig(q, out, lse, *k_portions, *v_portions)
    B, Tn, Hq, D = q.shape
    n = len(k_portions)
    if len(v_portions) != n or len(kv_offsets) != n or n == 0:
        raise ValueError("need the same positive number of K portions, V portions and offsets")
    Hkv = k_portions[0].shape[2]
    lens = []
    for kp, vp in zip(k_portions, v_portions):
        if kp.shape != vp.shape or kp.shape[0] != B or kp.shape[2] != Hkv or kp.shape[3] != D:
            raise ValueError("every portion must be [B, L_j, Hkv, D] for K and V alike")
        lens.append(int(kp.shape[1]))
    if workspace is None:
        import torch
        nbytes = cakv_decode_workspace_size(B, Hq, Hkv, Tn, D, lens)
        workspace = torch.empty(max(nbytes, 16) // 4 + 4, dtype=torch.float32, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    karr = (ctypes.c_void_p * n)(*[t.data_ptr() if t.numel() else None for t in k_portions])
    varr = (ctypes.c_void_p * n)(*[t.data_ptr() if t.numel() else None for t in v_portions])
    larr = (ctypes.c_int64 * n)(*lens)
    oarr = (ctypes.c_int64 * n)(*[int(x) for x in kv_offsets])
    _check(_lib.cakv_decode(_ptr(q), karr, varr, larr, oarr, n, _dtype_code(q), B, Hq, Hkv, Tn,
                            D, int(q_offset), int(causal), float(scale), _ptr(out),
                            _dtype_code(out), _ptr(lse), _ptr(workspace), ws_bytes,
                            _stream(stream)), "cakv_decode")


def cakv_decode_noalloc(q, k_portions: Sequence, v_portions: Sequence,
                        kv_offsets: Sequence[int], q_offset: int, causal: bool, out, lse=None,
                        scale: float = 0.0, stream=None):
    """cakv_decode with the splits' states in the library's fixed per-GPU
    scratch array (CAKV_DECODE_SCRATCH_BYTES) instead of a workspace: no device
    memory is allocated, here or in the library. Calls that overlap on one GPU
    share that array and must be ordered by the caller."""
    _contig(q, out, lse, *k_portions, *v_portions)
    B, Tn, Hq, D = q.shape
    n = len(k_portions)
    if len(v_portions) != n or len(kv_offsets) != n or n == 0:
        raise ValueError("need the same positive number of K portions, V portions and offsets")
    Hkv = k_portions[0].shape[2]
    lens = []
    for kp, vp in zip(k_portions, v_portions):
        if kp.shape != vp.shape or kp.shape[0] != B or kp.shape[2] != Hkv or kp.shape[3] != D:
            raise ValueError("every portion must be [B, L_j, Hkv, D] for K and V alike")
        lens.append(int(kp.shape[1]))
    karr = (ctypes.c_void_p * n)(*[t.data_ptr() if t.numel() else None for t in k_portions])
    varr = (ctypes.c_void_p * n)(*[t.data_ptr() if t.numel() else None for t in v_portions])
    larr = (ctypes.c_int64 * n)(*lens)
    oarr = (ctypes.c_int64 * n)(*[int(x) for x in kv_offsets])
    _check(_lib.cakv_decode_noalloc(_ptr(q), karr, varr, larr, oarr, n, _dtype_code(q), B, Hq,
                                    Hkv, Tn, D, int(q_offset), int(causal), float(scale),
                                    _ptr(out), _dtype_code(out), _ptr(lse), _stream(stream)),
           "cakv_decode_noalloc")


def cakv_forward_blocks(q, k_blocks: Sequence, v_blocks: Sequence, kv_offsets: Sequence[int],
                        q_offset: int, causal: bool, out, lse=None, scale: float = 0.0,
                        tile_counters=None, workspace="auto", stream=None):
    """Queries q [B, Tq, Hq, D] at positions q_offset ... against blocks
    [B, L_t, Hkv, D] of any lengths at global offsets kv_offsets[t], in the
    order given; writes out [B, Tq, Hq, D] and lse [B, Hq, Tq]."""
    _contig(q, out, lse, *k_blocks, *v_blocks)
    B, Tq, Hq, D = q.shape
    n = len(k_blocks)
    if len(v_blocks) != n or len(kv_offsets) != n or n == 0:
        raise ValueError("need the same positive number of K blocks, V blocks and offsets")
    Hkv = k_blocks[0].shape[2]
    lens = []
    for kb, vb in zip(k_blocks, v_blocks):
        if kb.shape != vb.shape or kb.shape[0] != B or kb.shape[2] != Hkv or kb.shape[3] != D \
                or kb.dtype != q.dtype or vb.dtype != q.dtype:
            raise ValueError("every block must be [B, L_t, Hkv, D] with the query dtype")
        lens.append(int(kb.shape[1]))
    karr = (ctypes.c_void_p * n)(*[t.data_ptr() if t.numel() else None for t in k_blocks])
    varr = (ctypes.c_void_p * n)(*[t.data_ptr() if t.numel() else None for t in v_blocks])
    larr = (ctypes.c_int64 * n)(*lens)
    oarr = (ctypes.c_int64 * n)(*[int(x) for x in kv_offsets])
    wp, wb, _keep = _fwd_workspace(workspace, q, Hkv, Tq)
    _check(_lib.cakv_forward_blocks(_ptr(q), karr, varr, larr, oarr, n, _dtype_code(q), B, Hq,
                                    Hkv, Tq, D, int(q_offset), int(causal), float(scale),
                                    _ptr(out), _dtype_code(out), _ptr(lse), wp, wb,
                                    _counters(tile_counters), _stream(stream)),
           "cakv_forward_blocks")


def cakv_backward_workspace_size(B: int, Hq: int, Tq: int) -> int:
    """Bytes of workspace cakv_backward_blocks needs for these sizes."""
    out = ctypes.c_int64()
    _check(_lib.cakv_backward_workspace_size(B, Hq, Tq, ctypes.byref(out)),
           "cakv_backward_workspace_size")
    return int(out.value)


def cakv_backward_blocks(q, k_blocks: Sequence, v_blocks: Sequence, kv_offsets: Sequence[int],
                         q_offset: int, causal: bool, out, lse, dout, dq, dk_blocks: Sequence,
                         dv_blocks: Sequence, workspace=None, scale: float = 0.0, stream=None):
    """Gradients of cakv_forward_blocks: dq [B, Tq, Hq, D], dk/dv blocks
    [B, L_t, Hkv, D] (fp32, overwritten) from out/lse of the forward and the
    bf16 upstream gradient dout."""
    _contig(q, out, lse, dout, dq, *k_blocks, *v_blocks, *dk_blocks, *dv_blocks)
    B, Tq, Hq, D = q.shape
    n = len(k_blocks)
    if not (len(v_blocks) == len(kv_offsets) == len(dk_blocks) == len(dv_blocks) == n) or n == 0:
        raise ValueError("need the same positive number of blocks, offsets and gradient blocks")
    Hkv = k_blocks[0].shape[2]
    lens = [int(t.shape[1]) for t in k_blocks]
    for kb, vb, gk, gv in zip(k_blocks, v_blocks, dk_blocks, dv_blocks):
        if not (kb.shape == vb.shape == gk.shape == gv.shape) or kb.shape[0] != B \
                or kb.shape[2] != Hkv or kb.shape[3] != D:
            raise ValueError("blocks and their gradients must all be [B, L_t, Hkv, D]")
    if workspace is None:
        import torch
        nbytes = cakv_backward_workspace_size(B, Hq, Tq)
        workspace = torch.empty(max(nbytes // 4, 4), dtype=torch.float32, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()

    def arr(ts):
        return (ctypes.c_void_p * n)(*[t.data_ptr() if t.numel() else None for t in ts])
    larr = (ctypes.c_int64 * n)(*lens)
    oarr = (ctypes.c_int64 * n)(*[int(x) for x in kv_offsets])
    _check(_lib.cakv_backward_blocks(_ptr(q), arr(k_blocks), arr(v_blocks), larr, oarr, n,
                                     _dtype_code(q), B, Hq, Hkv, Tq, D, int(q_offset),
                                     int(causal), float(scale), _ptr(out), _ptr(lse), _ptr(dout),
                                     _ptr(dq), arr(dk_blocks), arr(dv_blocks), _ptr(workspace),
                                     ws_bytes, _stream(stream)), "cakv_backward_blocks")
