"""One attention layer's hot path as a sequence of libcsa calls.

``LayerCache`` owns the per-layer device buffers the pages put in the layer's
cache [Transformers DeepSeek-V4 model page, "Cache layers": the K=V window,
the compressor's buffer / pool / counter / overlap state, and for CSA the
indexer's own buffer / pool at index_head_dim].  ``layer_step`` runs one
call of n_new tokens per sequence: window append, compressor(s), indexer +
top-k (CSA), attention.  It only orders calls; all arithmetic is in libcsa.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

from . import (CSA_OP_ATTEND, CSA_OP_HCA_ATTEND, CSA_OP_INDEX_TOPK, Layer, csa_attend,
               csa_compress, csa_index_topk, csa_window_append, csa_workspace_bytes, hca_attend)

__all__ = ["LayerCache", "layer_step"]


@dataclasses.dataclass
class LayerCache:
    layer: Layer
    batch: int
    win_cap: int
    pool_cap: int
    device: str = "cuda"

    def __post_init__(self):
        import torch
        L = self.layer
        dt = torch.bfloat16 if L.dtype == "bf16" else torch.float32
        B, dev = self.batch, self.device
        z = lambda *s: torch.zeros(*s, dtype=dt, device=dev)
        self.ring = z(B, self.win_cap, L.head_dim)
        self.pool = self.ipool = None
        if L.compress_ratio > 0:
            Ls = (1 + L.overlap) * L.compress_ratio
            self.pool = z(B, self.pool_cap, L.head_dim)
            self.cstate_kv, self.cstate_gate = z(B, Ls, L.head_dim), z(B, Ls, L.head_dim)
            if L.index_topk > 0:
                self.ipool = z(B, self.pool_cap, L.index_head_dim)
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
               norm_weight=None, inorm_weight=None, norm_eps: float = 1e-6, n_valid=None):
    """One call of the layer for q [B,n,H,D] and the new tokens' streams.

    n_valid (int32 [B] on the device, optional) makes it a variable-length
    call: sequence b has n_valid[b] valid tokens, the first of its n rows; the
    caches advance by those only and the output rows of the padding are
    unspecified.  Returns (out [B,n,H,D], topk_idx [B,n,k] or None).
    """
    import torch
    L = cache.layer
    B, n = q.shape[:2]
    if out is None:
        out = torch.empty_like(q)
    csa_window_append(L, pos0, pos0_max, kv, cache.ring, n_valid)
    if L.compress_ratio == 0:
        hca_attend(L, pos0, pos0_max, q, cache.ring, None, sinks, out,
                   cache.workspace(n, CSA_OP_HCA_ATTEND), n_valid=n_valid)
        return out, None
    csa_compress(L, pos0, pos0_max, ckv, cgate, cache.cstate_kv, cache.cstate_gate, cache.pool,
                 L.qk_rope_head_dim, norm_weight, norm_eps, n_valid)
    if L.index_topk == 0:
        hca_attend(L, pos0, pos0_max, q, cache.ring, cache.pool, sinks, out,
                   cache.workspace(n, CSA_OP_HCA_ATTEND), n_valid=n_valid)
        return out, None
    csa_compress(L, pos0, pos0_max, ikv, igate, cache.istate_kv, cache.istate_gate, cache.ipool,
                 L.index_rope_dim, inorm_weight, norm_eps, n_valid)
    if topk_idx is None:
        topk_idx = torch.empty(B, n, L.index_topk, dtype=torch.int32, device=q.device)
    csa_index_topk(L, pos0, pos0_max, qi, wi, cache.ipool, topk_idx,
                   workspace=cache.workspace(n, CSA_OP_INDEX_TOPK), n_valid=n_valid)
    csa_attend(L, pos0, pos0_max, q, cache.ring, cache.pool, topk_idx, sinks, out,
               cache.workspace(n, CSA_OP_ATTEND), n_valid=n_valid)
    return out, topk_idx
