"""One attention layer's hot path as a sequence of libcsa calls.

``LayerCache`` owns the per-layer device buffers the pages put in the layer's
cache [Transformers DeepSeek-V4 model page, "Cache layers": the K=V window,
the compressor's buffer / pool / counter / overlap state, and for CSA the
indexer's own buffer / pool at index_head_dim].  Pools are contiguous
``[B, pool_cap, width]`` tensors, or paged: ``[blocks * block_entries,
width]`` tensors addressed through a per-sequence block table of the layer
(each layer has its own table and block count, since the layers' pools
differ in ratio and size).  ``layer_step`` runs one call of the layer: window
append, compressor(s), indexer + top-k (CSA), attention.  It only orders
calls; all arithmetic is in libcsa.  The window append and the compressors
go through csa_cache_update (one launch for a decode step).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

from . import (CSA_OP_ATTEND, CSA_OP_HCA_ATTEND, CSA_OP_INDEX_TOPK, Layer, Paged, csa_attend,
               csa_cache_update, csa_index_topk, csa_workspace_bytes, hca_attend)

__all__ = ["LayerCache", "layer_step"]


@dataclasses.dataclass
class LayerCache:
    layer: Layer
    batch: int
    win_cap: int
    pool_cap: int
    device: str = "cuda"
    # paged pools: entries per block, blocks in each pool tensor, and the
    # int32 [batch, blocks per sequence] block table (device)
    block_entries: int = 0
    pool_blocks: int = 0
    block_table: object = None

    def __post_init__(self):
        import torch
        L = self.layer
        dt = torch.bfloat16 if L.dtype == "bf16" else torch.float32
        B, dev = self.batch, self.device
        z = lambda *s: torch.zeros(*s, dtype=dt, device=dev)
        self.ring = z(B, self.win_cap, L.head_dim)
        self.pool = self.ipool = None
        self.paged = None
        if L.compress_ratio > 0:
            Ls = (1 + L.overlap) * L.compress_ratio
            if self.block_entries:
                rows = self.pool_blocks * self.block_entries
                self.paged = Paged(self.block_table, self.block_entries, self.pool_cap)
                self.pool = z(rows, L.head_dim)
            else:
                self.pool = z(B, self.pool_cap, L.head_dim)
            self.cstate_kv, self.cstate_gate = z(B, Ls, L.head_dim), z(B, Ls, L.head_dim)
            if L.index_topk > 0:
                self.ipool = (z(rows, L.index_head_dim) if self.block_entries else
                              z(B, self.pool_cap, L.index_head_dim))
                self.istate_kv = z(B, Ls, L.index_head_dim)
                self.istate_gate = z(B, Ls, L.index_head_dim)
        self._ws = {}

    def workspace(self, n_new: int, op: int):
        import torch
        key = (n_new, op)
        if key not in self._ws:
            need = csa_workspace_bytes(self.layer, self.batch, n_new,
                                       self.pool_cap if self.layer.compress_ratio > 0 else 0, op)
            self._ws[key] = torch.empty(max(need, 256), dtype=torch.uint8, device=self.device)
        return self._ws[key]


def layer_step(cache: LayerCache, pos0, pos0_max: int, q, kv, ckv=None, cgate=None, ikv=None,
               igate=None, qi=None, wi=None, sinks=None, out=None, topk_idx=None,
               norm_weight=None, inorm_weight=None, norm_eps: float = 1e-6, n_valid=None,
               cu_seqlens=None, n_new: Optional[int] = None):
    """One call of the layer for q [B,n,H,D] and the new tokens' streams.

    n_valid (int32 [B] on the device, optional) makes it a padded
    variable-length call: sequence b has n_valid[b] valid tokens, the first of
    its n rows; the caches advance by those only and the output rows of the
    padding are unspecified.  cu_seqlens (int32 [B + 1] on the device) with
    n_new (the longest sequence) makes it a packed call: every per-token
    tensor is [rows, ...] with sequence b in rows cu_seqlens[b] ..
    cu_seqlens[b + 1] - 1.  Returns (out, topk_idx or None), shaped like q.
    """
    import torch
    L = cache.layer
    if cu_seqlens is None:
        B, n = q.shape[:2]
        lead = (B, n)
    else:
        B, n = pos0.numel(), int(n_new)
        lead = (q.shape[0],)
    geo = dict(n_valid=n_valid, cu_seqlens=cu_seqlens, n_new=n_new)
    if out is None:
        out = torch.empty_like(q)
    # the window append and the compressor(s): one launch for a decode step
    pg = dict(geo, paged=cache.paged)
    if L.compress_ratio == 0:
        csa_cache_update(L, pos0, pos0_max, kv, cache.ring, **geo)
        hca_attend(L, pos0, pos0_max, q, cache.ring, None, sinks, out,
                   cache.workspace(n, CSA_OP_HCA_ATTEND), **geo)
        return out, None
    idx_streams = {}
    if L.index_topk > 0:
        idx_streams = dict(ikv=ikv, igate=igate, istate_kv=cache.istate_kv,
                           istate_gate=cache.istate_gate, ipool=cache.ipool,
                           inorm_weight=inorm_weight)
    csa_cache_update(L, pos0, pos0_max, kv, cache.ring, ckv, cgate, cache.cstate_kv,
                     cache.cstate_gate, cache.pool, norm_weight=norm_weight, norm_eps=norm_eps,
                     **idx_streams, **pg)
    if L.index_topk == 0:
        hca_attend(L, pos0, pos0_max, q, cache.ring, cache.pool, sinks, out,
                   cache.workspace(n, CSA_OP_HCA_ATTEND), **pg)
        return out, None
    if topk_idx is None:
        topk_idx = torch.empty(*lead, L.index_topk, dtype=torch.int32, device=q.device)
    csa_index_topk(L, pos0, pos0_max, qi, wi, cache.ipool, topk_idx,
                   workspace=cache.workspace(n, CSA_OP_INDEX_TOPK), **pg)
    csa_attend(L, pos0, pos0_max, q, cache.ring, cache.pool, topk_idx, sinks, out,
               cache.workspace(n, CSA_OP_ATTEND), **pg)
    return out, topk_idx
