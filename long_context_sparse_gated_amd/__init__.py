"""Python binding of libcsa, the MI355X compressed-attention core of DeepSeek-V4.

Argument marshalling only: every function checks the torch tensors it is
given (device, dtype, contiguity, shape), passes their device pointers and
the current HIP stream to the C entry point of the same name
(``include/csa.h``), and raises ``RuntimeError`` with the library's status
string when the call is rejected.  No arithmetic happens here; if the shared
library is missing the import of a function fails loudly (there is no other
code path).

Build the library with ``python -m long_context_sparse_gated_amd.build``.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
from typing import Optional

__all__ = [
    "Layer", "load_library", "library_path", "csa_window_append", "csa_rope", "csa_compress",
    "csa_index_topk", "csa_attend", "hca_attend", "csa_workspace_bytes", "csa_status_str",
    "CSA_OP_INDEX_TOPK", "CSA_OP_ATTEND", "CSA_OP_HCA_ATTEND", "EXPORTED_SYMBOLS",
    "csa_output_projection", "csa_project", "csa_index_topk_noalloc",
    "CSA_NOALLOC_SCRATCH_BYTES", "Paged", "csa_cache_update",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
CSA_OP_INDEX_TOPK, CSA_OP_ATTEND, CSA_OP_HCA_ATTEND = 1, 2, 3
CSA_NOALLOC_SCRATCH_BYTES = 32 << 20    # CSA_NOALLOC_SCRATCH_BYTES of csa.h
EXPORTED_SYMBOLS = ("csa_window_append", "csa_rope", "csa_compress", "csa_index_topk",
                    "csa_attend", "hca_attend", "csa_workspace_bytes", "csa_status_str",
                    "csa_version", "csa_output_projection", "csa_output_projection_workspace_bytes",
                    "csa_project", "csa_project_workspace_bytes", "csa_index_topk_noalloc",
                    "csa_cache_update")


class _CLayer(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("qk_rope_head_dim", ctypes.c_int32),
                ("rope_theta", ctypes.c_double), ("sliding_window", ctypes.c_int32),
                ("compress_ratio", ctypes.c_int32), ("overlap", ctypes.c_int32),
                ("index_n_heads", ctypes.c_int32), ("index_head_dim", ctypes.c_int32),
                ("index_rope_dim", ctypes.c_int32), ("index_topk", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("rope_factor", ctypes.c_double),
                ("rope_original_context", ctypes.c_double), ("rope_beta_fast", ctypes.c_double),
                ("rope_beta_slow", ctypes.c_double)]


class _COproj(ctypes.Structure):
    _fields_ = [("tokens", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("o_groups", ctypes.c_int32),
                ("o_lora_rank", ctypes.c_int32), ("hidden_size", ctypes.c_int32)]


class _CProj(ctypes.Structure):
    _fields_ = [("tokens", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("q_lora_rank", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("comp_dim", ctypes.c_int32),
                ("index_dim", ctypes.c_int32), ("index_heads", ctypes.c_int32),
                ("eps", ctypes.c_float), ("q_head_norm", ctypes.c_int32)]


class _CBatch(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_new", ctypes.c_int32),
                ("pos0", ctypes.c_void_p), ("pos0_max", ctypes.c_int64),
                ("n_valid", ctypes.c_void_p), ("cu_seqlens", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("block_entries", ctypes.c_int32),
                ("block_table_stride", ctypes.c_int32), ("pool_blocks", ctypes.c_int64)]


@dataclasses.dataclass(frozen=True)
class Layer:
    """Mirror of ``csa_layer``; dtype is ``"bf16"`` or ``"f32"``."""
    dtype: str
    num_heads: int
    head_dim: int
    qk_rope_head_dim: int
    rope_theta: float
    sliding_window: int
    compress_ratio: int
    overlap: int
    index_n_heads: int = 0
    index_head_dim: int = 0
    index_rope_dim: int = 0
    index_topk: int = 0
    softmax_scale: float = 0.0
    rope_factor: float = 0.0            # YaRN scale; 0: none
    rope_original_context: float = 0.0
    rope_beta_fast: float = 0.0
    rope_beta_slow: float = 0.0

    @classmethod
    def from_spec(cls, spec) -> "Layer":
        """From a ``synth.LayerSpec``-like object (field names of the workloads)."""
        return cls(dtype=spec.dtype, num_heads=spec.num_heads, head_dim=spec.head_dim,
                   qk_rope_head_dim=spec.rope_dim, rope_theta=spec.rope_theta,
                   sliding_window=spec.window, compress_ratio=spec.ratio, overlap=spec.overlap,
                   index_n_heads=spec.index_heads if spec.kind == "csa" else 0,
                   index_head_dim=spec.index_dim if spec.kind == "csa" else 0,
                   index_rope_dim=spec.index_rope_dim if spec.kind == "csa" else 0,
                   index_topk=spec.topk if spec.kind == "csa" else 0,
                   rope_factor=getattr(spec, "rope_factor", 0.0),
                   rope_original_context=getattr(spec, "rope_original_context", 0.0),
                   rope_beta_fast=getattr(spec, "rope_beta_fast", 0.0),
                   rope_beta_slow=getattr(spec, "rope_beta_slow", 0.0))

    def _c(self) -> _CLayer:
        return _CLayer(1 if self.dtype == "bf16" else (0 if self.dtype == "f32" else 99),
                       self.num_heads, self.head_dim, self.qk_rope_head_dim, self.rope_theta,
                       self.sliding_window, self.compress_ratio, self.overlap,
                       self.index_n_heads, self.index_head_dim, self.index_rope_dim,
                       self.index_topk, self.softmax_scale, self.rope_factor,
                       self.rope_original_context, self.rope_beta_fast, self.rope_beta_slow)


_lib = None


def library_path() -> str:
    return os.path.join(_PKG, "libcsa.so")


def load_library():
    """Load libcsa.so from the package directory (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    # torch first: the library then binds to the HIP runtime torch already
    # loaded (same soname), so device memory, streams and launches share one
    # runtime in the process.
    _torch()
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m long_context_sparse_gated_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    LP, BP = ctypes.POINTER(_CLayer), ctypes.POINTER(_CBatch)
    sig = {
        "csa_window_append": [LP, BP, P, P, I64, P],
        "csa_rope": [LP, BP, P, I32, I32, I32, I32, P],
        "csa_compress": [LP, BP, I32, I32, P, P, P, ctypes.c_float, P, P, P, I64, P],
        "csa_cache_update": [LP, BP, P, P, I64, P, P, P, P, P, P, P, P, P, P, P, P, I64,
                             ctypes.c_float, P],
        "csa_index_topk": [LP, BP, P, P, P, I64, P, P, P, SZ, P],
        "csa_index_topk_noalloc": [LP, BP, P, P, P, I64, P, P, P],
        "csa_attend": [LP, BP, P, P, I64, P, I64, P, P, P, P, SZ, P],
        "hca_attend": [LP, BP, P, P, I64, P, I64, P, P, P, SZ, P],
        "csa_output_projection": [ctypes.POINTER(_COproj), P, P, P, P, P, SZ, P],
        "csa_project": [ctypes.POINTER(_CProj), P, P, P, P, P, P, P, P, P, P, P, P, P, P, SZ,
                        P],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.csa_workspace_bytes.argtypes = [LP, I32, I32, I64, I32]
    lib.csa_workspace_bytes.restype = SZ
    lib.csa_status_str.argtypes = [ctypes.c_int]
    lib.csa_status_str.restype = ctypes.c_char_p
    lib.csa_version.argtypes = []
    lib.csa_version.restype = I32
    lib.csa_output_projection_workspace_bytes.argtypes = [ctypes.POINTER(_COproj)]
    lib.csa_output_projection_workspace_bytes.restype = SZ
    lib.csa_project_workspace_bytes.argtypes = [ctypes.POINTER(_CProj)]
    lib.csa_project_workspace_bytes.restype = SZ
    _lib = lib
    return lib


def csa_status_str(status: int) -> str:
    return load_library().csa_status_str(status).decode()


def _check(status: int, what: str):
    if status != 0:
        raise RuntimeError(f"{what}: {csa_status_str(status)}")


def _torch():
    import torch
    return torch


def _ptr(t, name, dtype=None):
    if t is None:
        return None
    torch = _torch()
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _store_dtype(layer: Layer):
    torch = _torch()
    return torch.bfloat16 if layer.dtype == "bf16" else torch.float32


@dataclasses.dataclass(frozen=True)
class Paged:
    """Block table of one layer's paged pools (``csa_batch.block_table``):
    entry w of sequence b is row ``block_table[b, w // block_entries] *
    block_entries + w % block_entries`` of each pool tensor, which is
    ``[blocks * block_entries, width]``; ``pool_cap`` entries per sequence."""
    block_table: object     # int32 [B, stride] device tensor
    block_entries: int
    pool_cap: int


def _batch(pos0, pos0_max, B, n, n_valid=None, cu_seqlens=None, paged=None, pool=None):
    torch = _torch()
    _ptr(pos0, "pos0", torch.int64)
    if pos0.numel() != B:
        raise ValueError("pos0 must hold one position per sequence")
    nv = cu = None
    if n_valid is not None:
        nv = _ptr(n_valid, "n_valid", torch.int32)
        if n_valid.numel() != B:
            raise ValueError("n_valid must hold one count per sequence")
    if cu_seqlens is not None:
        cu = _ptr(cu_seqlens, "cu_seqlens", torch.int32)
        if cu_seqlens.numel() != B + 1:
            raise ValueError("cu_seqlens must hold B + 1 row offsets")
    tab, E, stride, blocks = None, 0, 0, 0
    if paged is not None:
        tab = _ptr(paged.block_table, "block_table", torch.int32)
        if paged.block_table.dim() != 2 or paged.block_table.shape[0] != B:
            raise ValueError("block_table must be [B, blocks per sequence]")
        E, stride = int(paged.block_entries), int(paged.block_table.shape[1])
        if pool is None or pool.dim() != 2 or pool.shape[0] % E:
            raise ValueError("a paged pool is [blocks * block_entries, width]")
        blocks = pool.shape[0] // E
    return _CBatch(B, n, pos0.data_ptr(), int(pos0_max), nv, cu, tab, E, stride, blocks)


def _lead(x, nd_tail, cu_seqlens, n_new, pos0):
    """(B, n) of a per-token tensor: [B, n, *tail] padded, [rows, *tail] packed."""
    if cu_seqlens is None:
        if x.dim() != 2 + nd_tail:
            raise ValueError("per-token tensors are [B, n_new, ...] (padded rows)")
        return x.shape[0], x.shape[1]
    if n_new is None or x.dim() != 1 + nd_tail:
        raise ValueError("packed calls take [rows, ...] tensors and n_new (longest sequence)")
    return pos0.numel(), int(n_new)


def _pool_cap(pool, paged):
    if pool is None:
        return 0
    return int(paged.pool_cap) if paged is not None else pool.shape[1]


def _stream():
    return _torch().cuda.current_stream().cuda_stream


def csa_workspace_bytes(layer: Layer, batch: int, n_new: int, pool_cap: int, op: int) -> int:
    lay = layer._c()
    n = load_library().csa_workspace_bytes(ctypes.byref(lay), batch, n_new, pool_cap, op)
    if n == ctypes.c_size_t(-1).value:
        raise RuntimeError("csa_workspace_bytes: invalid layer or op")
    return int(n)


def _workspace(layer, B, n, pool_cap, op, ws, device):
    need = csa_workspace_bytes(layer, B, n, pool_cap, op)
    if ws is None:
        if need == 0:
            return None, 0
        torch = _torch()
        ws = torch.empty(need, dtype=torch.uint8, device=device)
    return ws, ws.numel() * ws.element_size()


def csa_window_append(layer: Layer, pos0, pos0_max: int, kv, ring, n_valid=None,
                      cu_seqlens=None, n_new=None):
    """kv [B, n_new, D] (packed: [rows, D]) -> ring [B, cap, D] at slot position % cap,
    rotated.  n_valid (int32 [B], optional): only the first n_valid[b] rows are appended."""
    dt = _store_dtype(layer)
    B, n = _lead(kv, 1, cu_seqlens, n_new, pos0)
    bt = _batch(pos0, pos0_max, B, n, n_valid, cu_seqlens)
    lay = layer._c()
    _check(load_library().csa_window_append(
        ctypes.byref(lay), ctypes.byref(bt), _ptr(kv, "kv", dt), _ptr(ring, "ring", dt),
        ring.shape[1], _stream()), "csa_window_append")


def csa_rope(layer: Layer, pos0, pos0_max: int, x, rope_dim: int, sign: int = 1, n_valid=None,
             cu_seqlens=None, n_new=None):
    """x [B, n_new, rows, width] (packed: [rows, rows_per_token, width]) rotated in place
    at sign * position."""
    dt = _store_dtype(layer)
    B, n = _lead(x, 2, cu_seqlens, n_new, pos0)
    rows, width = x.shape[-2], x.shape[-1]
    bt = _batch(pos0, pos0_max, B, n, n_valid, cu_seqlens)
    lay = layer._c()
    _check(load_library().csa_rope(ctypes.byref(lay), ctypes.byref(bt), _ptr(x, "x", dt), rows,
                                   width, rope_dim, sign, _stream()), "csa_rope")


def csa_compress(layer: Layer, pos0, pos0_max: int, kv, gate, state_kv, state_gate, pool,
                 rope_dim: int, norm_weight=None, norm_eps: float = 1e-6, n_valid=None,
                 cu_seqlens=None, n_new=None, paged: Optional[Paged] = None):
    """kv, gate [B, n_new, width] (packed: [rows, width]); state_* [B, (1+overlap)m, width];
    pool [B, cap, width] (paged: [blocks * block_entries, width]).
    n_valid (int32 [B], optional): only the first n_valid[b] rows are pooled and kept."""
    torch = _torch()
    dt = _store_dtype(layer)
    B, n = _lead(kv, 1, cu_seqlens, n_new, pos0)
    width = kv.shape[-1]
    bt = _batch(pos0, pos0_max, B, n, n_valid, cu_seqlens, paged, pool)
    lay = layer._c()
    _check(load_library().csa_compress(
        ctypes.byref(lay), ctypes.byref(bt), width, rope_dim, _ptr(kv, "kv", dt),
        _ptr(gate, "gate", dt), _ptr(norm_weight, "norm_weight", torch.float32), norm_eps,
        _ptr(state_kv, "state_kv", dt), _ptr(state_gate, "state_gate", dt),
        _ptr(pool, "pool", dt), _pool_cap(pool, paged), _stream()), "csa_compress")


def csa_cache_update(layer: Layer, pos0, pos0_max: int, kv, ring, ckv=None, cgate=None,
                     state_kv=None, state_gate=None, pool=None, ikv=None, igate=None,
                     istate_kv=None, istate_gate=None, ipool=None, norm_weight=None,
                     inorm_weight=None, norm_eps: float = 1e-6, n_valid=None, cu_seqlens=None,
                     n_new=None, paged: Optional[Paged] = None):
    """The window append and the compressor(s) of one layer call in one call (one
    launch for a decode step): as csa_window_append(kv, ring), then csa_compress of
    (ckv, cgate) into (state_kv, state_gate, pool) and of (ikv, igate) into the
    indexer's state and ipool, for the streams the layer has."""
    torch = _torch()
    dt = _store_dtype(layer)
    B, n = _lead(kv, 1, cu_seqlens, n_new, pos0)
    bt = _batch(pos0, pos0_max, B, n, n_valid, cu_seqlens, paged, pool)
    lay = layer._c()
    f32 = torch.float32
    _check(load_library().csa_cache_update(
        ctypes.byref(lay), ctypes.byref(bt), _ptr(kv, "kv", dt), _ptr(ring, "ring", dt),
        ring.shape[1], _ptr(ckv, "ckv", dt), _ptr(cgate, "cgate", dt),
        _ptr(norm_weight, "norm_weight", f32), _ptr(state_kv, "state_kv", dt),
        _ptr(state_gate, "state_gate", dt), _ptr(pool, "pool", dt), _ptr(ikv, "ikv", dt),
        _ptr(igate, "igate", dt), _ptr(inorm_weight, "inorm_weight", f32),
        _ptr(istate_kv, "istate_kv", dt), _ptr(istate_gate, "istate_gate", dt),
        _ptr(ipool, "ipool", dt), _pool_cap(pool, paged) if pool is not None else 0, norm_eps,
        _stream()), "csa_cache_update")


def csa_index_topk(layer: Layer, pos0, pos0_max: int, q_idx, weights, k_pool, topk_idx,
                   scores_out=None, workspace=None, n_valid=None, cu_seqlens=None, n_new=None,
                   paged: Optional[Paged] = None):
    """q_idx [B,n,H_I,D_I], weights [B,n,H_I], k_pool [B,cap,D_I] -> topk_idx [B,n,k] int32
    (packed: leading [rows] instead of [B, n]; paged: k_pool [blocks * block_entries, D_I])."""
    torch = _torch()
    dt = _store_dtype(layer)
    B, n = _lead(q_idx, 2, cu_seqlens, n_new, pos0)
    bt = _batch(pos0, pos0_max, B, n, n_valid, cu_seqlens, paged, k_pool)
    pcap = _pool_cap(k_pool, paged)
    ws, wsb = _workspace(layer, B, n, pcap, CSA_OP_INDEX_TOPK, workspace, q_idx.device)
    lay = layer._c()
    _check(load_library().csa_index_topk(
        ctypes.byref(lay), ctypes.byref(bt), _ptr(q_idx, "q_idx", dt), _ptr(weights, "weights", dt),
        _ptr(k_pool, "k_pool", dt), pcap, _ptr(topk_idx, "topk_idx", torch.int32),
        _ptr(scores_out, "scores_out", torch.float32), _ptr(ws, "workspace"), wsb, _stream()),
        "csa_index_topk")


def csa_index_topk_noalloc(layer: Layer, pos0, pos0_max: int, q_idx, weights, k_pool, topk_idx,
                           scores_out=None, n_valid=None, cu_seqlens=None, n_new=None,
                           paged: Optional[Paged] = None):
    """csa_index_topk on the library's static scratch (no workspace argument,
    nothing allocated); calls overlapping on one device race on it."""
    torch = _torch()
    dt = _store_dtype(layer)
    B, n = _lead(q_idx, 2, cu_seqlens, n_new, pos0)
    bt = _batch(pos0, pos0_max, B, n, n_valid, cu_seqlens, paged, k_pool)
    lay = layer._c()
    _check(load_library().csa_index_topk_noalloc(
        ctypes.byref(lay), ctypes.byref(bt), _ptr(q_idx, "q_idx", dt), _ptr(weights, "weights", dt),
        _ptr(k_pool, "k_pool", dt), _pool_cap(k_pool, paged),
        _ptr(topk_idx, "topk_idx", torch.int32), _ptr(scores_out, "scores_out", torch.float32),
        _stream()), "csa_index_topk_noalloc")


def csa_attend(layer: Layer, pos0, pos0_max: int, q, win, pool, topk_idx, sinks, out,
               workspace=None, n_valid=None, cu_seqlens=None, n_new=None,
               paged: Optional[Paged] = None):
    """q [B,n,H,D], win [B,cap,D], pool [B,pcap,D], topk_idx [B,n,k], sinks [H] -> out
    (packed: leading [rows] instead of [B, n]; paged: pool [blocks * block_entries, D])."""
    torch = _torch()
    dt = _store_dtype(layer)
    B, n = _lead(q, 2, cu_seqlens, n_new, pos0)
    bt = _batch(pos0, pos0_max, B, n, n_valid, cu_seqlens, paged, pool)
    pcap = _pool_cap(pool, paged)
    ws, wsb = _workspace(layer, B, n, pcap, CSA_OP_ATTEND, workspace, q.device)
    lay = layer._c()
    _check(load_library().csa_attend(
        ctypes.byref(lay), ctypes.byref(bt), _ptr(q, "q", dt), _ptr(win, "win", dt), win.shape[1],
        _ptr(pool, "pool", dt), pcap, _ptr(topk_idx, "topk_idx", torch.int32),
        _ptr(sinks, "sinks", torch.float32), _ptr(out, "out", dt), _ptr(ws, "workspace"), wsb,
        _stream()), "csa_attend")


def hca_attend(layer: Layer, pos0, pos0_max: int, q, win, pool, sinks, out, workspace=None,
               n_valid=None, cu_seqlens=None, n_new=None, paged: Optional[Paged] = None):
    """As csa_attend with every visible entry (compress_ratio 0: window only; pool may be None)."""
    torch = _torch()
    dt = _store_dtype(layer)
    B, n = _lead(q, 2, cu_seqlens, n_new, pos0)
    bt = _batch(pos0, pos0_max, B, n, n_valid, cu_seqlens, paged if pool is not None else None,
                pool)
    pcap = _pool_cap(pool, paged)
    ws, wsb = _workspace(layer, B, n, pcap, CSA_OP_HCA_ATTEND, workspace, q.device)
    lay = layer._c()
    _check(load_library().hca_attend(
        ctypes.byref(lay), ctypes.byref(bt), _ptr(q, "q", dt), _ptr(win, "win", dt), win.shape[1],
        _ptr(pool, "pool", dt), pcap, _ptr(sinks, "sinks", torch.float32), _ptr(out, "out", dt),
        _ptr(ws, "workspace"), wsb, _stream()), "hca_attend")


def csa_output_projection(attn_out, w_a, w_b, out, o_groups: int, workspace=None):
    """attn_out [T, H, D], w_a [G*R, (H/G)*D], w_b [hidden, G*R] (bf16) -> out [T, hidden]."""
    torch = _torch()
    T, H, D = attn_out.shape
    R = w_a.shape[0] // o_groups
    shape = _COproj(T, H, D, o_groups, R, w_b.shape[0])
    if tuple(w_a.shape) != (o_groups * R, (H // o_groups) * D) or w_b.shape[1] != o_groups * R \
            or tuple(out.shape) != (T, w_b.shape[0]):
        raise ValueError("csa_output_projection: inconsistent shapes")
    lib = load_library()
    need = lib.csa_output_projection_workspace_bytes(ctypes.byref(shape))
    if need == ctypes.c_size_t(-1).value:
        raise RuntimeError("csa_output_projection: invalid sizes")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=attn_out.device)
    bf = torch.bfloat16
    _check(lib.csa_output_projection(
        ctypes.byref(shape), _ptr(attn_out, "attn_out", bf), _ptr(w_a, "w_a", bf),
        _ptr(w_b, "w_b", bf), _ptr(out, "out", bf), _ptr(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream()), "csa_output_projection")


def csa_project(x, w_x, g_qa, g_kv, w_q, outs: dict, *, q_lora_rank: int, num_heads: int,
                head_dim: int, comp_dim: int, index_dim: int, index_heads: int,
                eps: float = 1e-6, q_head_norm: bool = True, workspace=None):
    """Producer projections.  x [T, hidden], w_x and w_q stacked (out, in) bf16
    weights, g_qa / g_kv float32 norm weights; ``outs`` holds the device
    tensors q, kv and (as the layer has them) ckv, cgate, ikv, igate, qi, wi."""
    torch = _torch()
    T, hidden = x.shape
    shape = _CProj(T, hidden, q_lora_rank, num_heads, head_dim, comp_dim, index_dim,
                   index_heads, eps, 1 if q_head_norm else 0)
    nx = q_lora_rank + head_dim + 2 * comp_dim + 2 * index_dim + index_heads
    nq = num_heads * head_dim + index_heads * index_dim
    want = {"q": (T, num_heads, head_dim), "kv": (T, head_dim), "ckv": (T, comp_dim),
            "cgate": (T, comp_dim), "ikv": (T, index_dim), "igate": (T, index_dim),
            "qi": (T, index_heads, index_dim), "wi": (T, index_heads)}
    if tuple(w_x.shape) != (nx, hidden) or tuple(w_q.shape) != (nq, q_lora_rank) or \
            tuple(g_qa.shape) != (q_lora_rank,) or tuple(g_kv.shape) != (head_dim,):
        raise ValueError("csa_project: inconsistent weight shapes")
    for k, shp in want.items():
        if k in outs and outs[k] is not None and tuple(outs[k].shape) != shp:
            raise ValueError(f"csa_project: {k} must be {shp}")
    lib = load_library()
    need = lib.csa_project_workspace_bytes(ctypes.byref(shape))
    if need == ctypes.c_size_t(-1).value:
        raise RuntimeError("csa_project: invalid sizes")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    bf, f32 = torch.bfloat16, torch.float32
    o = {k: _ptr(outs.get(k), k, bf) for k in want}
    _check(lib.csa_project(
        ctypes.byref(shape), _ptr(x, "x", bf), _ptr(w_x, "w_x", bf), _ptr(g_qa, "g_qa", f32),
        _ptr(g_kv, "g_kv", f32), _ptr(w_q, "w_q", bf), o["q"], o["kv"], o["ckv"], o["cgate"],
        o["ikv"], o["igate"], o["qi"], o["wi"], _ptr(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream()), "csa_project")

