"""Seeded synthetic inputs for the compressed-attention layer workloads.

This module only draws random numbers and stores them in the layer's storage
dtype.  It holds none of the layer's arithmetic: RoPE, pooling, scoring,
selection and attention live in ``oracle/`` (CPU definition) and in the HIP
library, and neither of those is imported here.

Every tensor is drawn in blocks of 256 rows (first axis), block k of
sequence b from ``numpy.random.default_rng([seed, tensor_id, b, k])`` (PCG64)
as float32 normals, scaled, and rounded to bfloat16 with round-to-nearest-
even when the workload is bf16.  Seeding per (tensor, sequence, block) lets a
test redraw just the rows the oracle needs (``draw_rows``) and lets the full
draw run on several threads.  bf16 tensors are returned as ``uint16`` bit patterns;
``bf16_bits_to_f32`` / ``to_f64`` decode them exactly.

Workloads (names used by tests and the benchmark):

* ``tiny_csa``      fp32, B=1, S=256, H=8, D=64, R=16, W=32, m=4 overlapping,
                    indexer 4x32, top-k 16, base 10000.
* ``csa_prefill``   bf16, B=1, S=8192, H=64, D=512, R=64, W=128, m=4
                    overlapping, indexer 64x128, top-k 512, base 160000.
* ``hca_prefill``   bf16, B=1, S=65536, H=64, D=512, R=64, W=128, m=128,
                    no indexer, base 160000.
* ``csa_decode``    bf16, 64 sequences x 1 token at position 131072; caches of
                    32768 pooled entries, 32768 indexer keys, 128 window rows.
* ``mixed_decode``  bf16, 4 sequences x 1 token at position 1048576; a CSA layer
                    (262144 entries), an HCA layer (8192 entries) and a
                    sliding-only layer (base 10000).

Smaller variants (``scaled``) keep the per-layer shapes and shrink S or the
context so the CPU oracle finishes in seconds.
"""
from __future__ import annotations

import dataclasses
import math
import os
from typing import Dict, List, Optional

import numpy as np

__all__ = [
    "LayerSpec", "Workload", "WORKLOADS", "workload", "prefill_inputs",
    "decode_inputs", "bf16_bits_to_f32", "f32_to_bf16_bits", "to_f64",
    "grid_index_inputs", "OPROJ_SHAPE", "oproj_inputs", "PROJ_SHAPE", "proj_inputs",
]

# Tensor ids keep streams independent of draw order.
_TID = {
    "q": 1, "kv": 2, "ckv": 3, "cgate": 4, "ikv": 5, "igate": 6, "qi": 7,
    "wi": 8, "sinks": 9, "pool": 10, "ipool": 11, "win": 12, "cstate_kv": 13,
    "cstate_gate": 14, "istate_kv": 15, "istate_gate": 16, "norm": 17,
    "attn_out": 18, "o_a": 19, "o_b": 20, "hidden": 21, "w_x": 22, "w_q": 23, "g_qa": 24,
    "g_kv": 25,
}


@dataclasses.dataclass(frozen=True)
class LayerSpec:
    kind: str                 # "csa" | "hca" | "sliding"
    dtype: str                # "bf16" | "f32"
    num_heads: int = 64
    head_dim: int = 512
    rope_dim: int = 64
    rope_theta: float = 160000.0
    window: int = 128
    ratio: int = 4            # 0 for sliding-only
    overlap: int = 1
    index_heads: int = 64
    index_dim: int = 128
    index_rope_dim: int = 64
    topk: int = 512
    # YaRN rope scaling of every rope of the layer (0: none)
    rope_factor: float = 0.0
    rope_original_context: float = 65536.0
    rope_beta_fast: float = 32.0
    rope_beta_slow: float = 1.0

    @property
    def has_indexer(self) -> bool:
        return self.kind == "csa"


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    layers: List[LayerSpec]
    batch: int
    n_new: int                # tokens per sequence in this call
    pos0: int                 # absolute position of the first new token
    # distribution knobs (standard deviations)
    q_std: float = 1.0
    kv_std: float = 1.0
    qi_std: float = 1.0
    ikv_std: float = 1.0
    wi_std: float = 1.0
    cache_std: float = 1.0
    sink_std: float = 1.0

    @property
    def decode(self) -> bool:
        return self.pos0 > 0


def _tiny_layer() -> LayerSpec:
    return LayerSpec(kind="csa", dtype="f32", num_heads=8, head_dim=64, rope_dim=16,
                     rope_theta=10000.0, window=32, ratio=4, overlap=1,
                     index_heads=4, index_dim=32, index_rope_dim=16, topk=16)


# The V4-shaped layers scale every rope with YaRN, factor 16 over a 65536-token
# original context (optimum-intel issue 1748, "What V4-Flash adds vs V3").
_V4_YARN = dict(rope_factor=16.0, rope_original_context=65536.0)


def _csa_layer(dtype="bf16") -> LayerSpec:
    return LayerSpec(kind="csa", dtype=dtype, **_V4_YARN)


def _hca_layer(dtype="bf16") -> LayerSpec:
    return LayerSpec(kind="hca", dtype=dtype, ratio=128, overlap=0, **_V4_YARN)


def _sliding_layer(dtype="bf16") -> LayerSpec:
    return LayerSpec(kind="sliding", dtype=dtype, ratio=0, overlap=0, rope_theta=10000.0,
                     **_V4_YARN)


def _prefill(name, layer, S, batch=1):
    D, Di = layer.head_dim, layer.index_dim
    return Workload(name=name, layers=[layer], batch=batch, n_new=S, pos0=0,
                    q_std=1 / math.sqrt(D), kv_std=1 / math.sqrt(D),
                    qi_std=1 / math.sqrt(Di), ikv_std=1 / math.sqrt(Di),
                    wi_std=1 / math.sqrt(layer.index_heads), cache_std=1.0)


def _decode(name, layers, batch, pos):
    D, Di = 512, 128
    return Workload(name=name, layers=layers, batch=batch, n_new=1, pos0=pos,
                    q_std=1 / math.sqrt(D), kv_std=1 / math.sqrt(D),
                    qi_std=1 / math.sqrt(Di), ikv_std=1 / math.sqrt(Di),
                    wi_std=1 / 8, cache_std=1.0)


WORKLOADS: Dict[str, Workload] = {
    "tiny_csa": dataclasses.replace(
        _prefill("tiny_csa", _tiny_layer(), 256), q_std=1 / 8, kv_std=1 / 8,
        qi_std=1 / math.sqrt(32), ikv_std=1 / math.sqrt(32), wi_std=0.5),
    "csa_prefill": dataclasses.replace(_prefill("csa_prefill", _csa_layer(), 8192), wi_std=1 / 8),
    "hca_prefill": _prefill("hca_prefill", _hca_layer(), 65536),
    "csa_decode": _decode("csa_decode", [_csa_layer()], 64, 131072),
    "mixed_decode": _decode("mixed_decode", [_csa_layer(), _hca_layer(), _sliding_layer()],
                            4, 1048576),
}


def workload(name: str, *, S: Optional[int] = None, batch: Optional[int] = None,
             pos0: Optional[int] = None, variant: str = "plain") -> Workload:
    """A named workload, optionally rescaled.

    ``variant``: ``"plain"`` (the stated distributions) or ``"peaked"`` (q and
    window/compressor kv drawn at unit scale and sinks at 4x, so that logits
    spread over several units and softmax weights are far from uniform).
    """
    w = WORKLOADS[name]
    kw = {}
    if S is not None:
        kw["n_new"] = S
    if batch is not None:
        kw["batch"] = batch
    if pos0 is not None:
        kw["pos0"] = pos0
    if variant == "peaked":
        kw.update(q_std=1.0, kv_std=1.0 if w.layers[0].dtype == "bf16" else 0.5,
                  sink_std=4.0)
    elif variant != "plain":
        raise ValueError(variant)
    return dataclasses.replace(w, **kw) if kw else w


# ----------------------------------------------------------------------------
# storage conversions (no layer arithmetic)

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f64(a: np.ndarray) -> np.ndarray:
    """Exact decode of a stored tensor (uint16 = bf16 bits, else float) to float64."""
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


ROW_BLOCK = 256   # rows per independently seeded block


def _draw_block(seed, name, b, blk, nrows, tail, std, dtype):
    rng = np.random.default_rng([seed, _TID[name], b, blk])
    x = rng.standard_normal((nrows,) + tuple(tail), dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    return x


_POOL = None


def _pool():
    global _POOL
    if _POOL is None:
        from concurrent.futures import ThreadPoolExecutor
        _POOL = ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1))
    return _POOL


def _draw(seed: int, name: str, b: int, shape, std: float, dtype: str) -> np.ndarray:
    """Tensor `name` of sequence b: rows drawn in blocks of ROW_BLOCK rows, block k
    from default_rng([seed, tensor id, b, k]) (so any row subset can be redrawn)."""
    shape = tuple(shape)
    rows, tail = shape[0], shape[1:]
    nblk = (rows + ROW_BLOCK - 1) // ROW_BLOCK
    parts = list(_pool().map(
        lambda k: _draw_block(seed, name, b, k, min(ROW_BLOCK, rows - k * ROW_BLOCK), tail, std,
                              dtype), range(nblk)))
    if not parts:
        return np.zeros(shape, dtype=np.uint16 if dtype == "bf16" else np.float32)
    return np.concatenate(parts, axis=0)


def draw_rows(seed: int, name: str, b: int, shape, std: float, dtype: str, rows) -> np.ndarray:
    """Rows `rows` (indices along the first axis) of the tensor _draw would return."""
    shape = tuple(shape)
    rows = np.asarray(rows, dtype=np.int64)
    out = np.zeros((len(rows),) + shape[1:], dtype=np.uint16 if dtype == "bf16" else np.float32)
    for k in np.unique(rows // ROW_BLOCK):
        n = min(ROW_BLOCK, shape[0] - k * ROW_BLOCK)
        blk = _draw_block(seed, name, b, int(k), n, shape[1:], std, dtype)
        sel = np.nonzero(rows // ROW_BLOCK == k)[0]
        out[sel] = blk[rows[sel] - k * ROW_BLOCK]
    return out


def _stack(seed, name, batch, shape, std, dtype):
    return np.stack([_draw(seed, name, b, shape, std, dtype) for b in range(batch)])


def prefill_inputs(w: Workload, seed: int = 0, layer: int = 0) -> Dict[str, np.ndarray]:
    """Inputs of one prefill call of ``w.n_new`` tokens per sequence.

    Keys: q [B,S,H,D]; kv [B,S,D] (window stream, un-rotated); ckv, cgate
    [B,S,D] (compressor stream and per-channel gate logits); ikv, igate
    [B,S,D_I]; qi [B,S,H_I,D_I] (un-rotated); wi [B,S,H_I]; sinks [H] float32.
    """
    L = w.layers[layer]
    s = seed * 16 + layer
    out = {k: _stack(s, k, w.batch, *v) for k, v in prefill_shapes(w, layer).items()}
    out["sinks"] = _draw(s, "sinks", 0, (L.num_heads,), w.sink_std, "f32")
    return out


def prefill_shapes(w: Workload, layer: int = 0):
    """name -> (shape per sequence, std, dtype) of the prefill tensors."""
    L = w.layers[layer]
    S, H, D, dt = w.n_new, L.num_heads, L.head_dim, L.dtype
    out = {"q": ((S, H, D), w.q_std, dt), "kv": ((S, D), w.kv_std, dt)}
    if L.ratio > 0:
        out["ckv"] = ((S, D), w.kv_std, dt)
        out["cgate"] = ((S, D), 1.0, dt)
    if L.has_indexer:
        Hi, Di = L.index_heads, L.index_dim
        out["ikv"] = ((S, Di), w.ikv_std, dt)
        out["igate"] = ((S, Di), 1.0, dt)
        out["qi"] = ((S, Hi, Di), w.qi_std, dt)
        out["wi"] = ((S, Hi), w.wi_std, dt)
    return out


def prefill_rows(w: Workload, seed: int, layer: int, b: int, name: str, rows) -> np.ndarray:
    """Rows of one prefill tensor of sequence b (same values as prefill_inputs)."""
    shape, std, dt = prefill_shapes(w, layer)[name]
    return draw_rows(seed * 16 + layer, name, b, shape, std, dt, rows)


def cache_shapes(w: Workload, layer: int = 0):
    """name -> (shape per sequence, std, dtype) of a decode workload's caches."""
    L = w.layers[layer]
    D, dt, std = L.head_dim, L.dtype, w.cache_std
    out = {"win": ((L.window, D), std, dt)}
    if L.ratio > 0:
        P = w.pos0 // L.ratio
        Ls = (1 + L.overlap) * L.ratio
        out["pool"] = ((P, D), std, dt)
        out["cstate_kv"] = ((Ls, D), w.kv_std, dt)
        out["cstate_gate"] = ((Ls, D), 1.0, dt)
        if L.has_indexer:
            Di = L.index_dim
            out["ipool"] = ((P, Di), std, dt)
            out["istate_kv"] = ((Ls, Di), w.ikv_std, dt)
            out["istate_gate"] = ((Ls, Di), 1.0, dt)
    return out


def cache_rows(w: Workload, seed: int, layer: int, b: int, name: str, rows) -> np.ndarray:
    """Rows of one cache tensor of sequence b (same values as decode_cache_seq)."""
    shape, std, dt = cache_shapes(w, layer)[name]
    return draw_rows(seed * 16 + layer, name, b, shape, std, dt, rows)


def decode_cache_seq(w: Workload, seed: int, layer: int, b: int,
                     names: Optional[List[str]] = None) -> Dict[str, np.ndarray]:
    """Cache contents of one sequence for a decode workload.

    pool [P,D] and ipool [P,D_I] hold rotated pooled entries 0..P-1 with
    P = pos0//m (the entries closed before the new token); win [W,D] holds rotated window rows for positions
    pos0-W .. pos0-1 at ring slot (position mod W); cstate_* / istate_* hold
    the raw compressor tokens of the (1+overlap)*m positions before pos0 at
    slot (position mod (1+overlap)*m).
    """
    shapes = cache_shapes(w, layer)
    names = list(shapes) if names is None else names
    return {k: _draw(seed * 16 + layer, k, b, *shapes[k]) for k in names}


def decode_inputs(w: Workload, seed: int = 0, layer: int = 0,
                  seqs: Optional[List[int]] = None) -> Dict[str, np.ndarray]:
    """New-token inputs (prefill_inputs with S=1) plus per-sequence caches.

    ``seqs`` restricts the cache draw to those sequences (the new-token
    tensors always cover the whole batch); cache arrays are then stacked in
    the order of ``seqs``.
    """
    assert w.n_new == 1
    out = prefill_inputs(w, seed, layer)
    seqs = list(range(w.batch)) if seqs is None else list(seqs)
    caches = [decode_cache_seq(w, seed, layer, b) for b in seqs]
    for k in caches[0]:
        out[k] = np.stack([c[k] for c in caches])
    return out


def grid_index_inputs(n_q: int, pool: int, Hi: int, Di: int, Ri: int, seed: int = 0,
                      distinct_rows: int = 0):
    """Indexer inputs on exact grids: q, k in (1/8)Z and w in (1/4)Z, all in [-1, 1].

    The rope channels of the keys are zero, so the rotated query's rope part
    never contributes.  Every product, ReLU, weighted sum and partial sum of
    the index score is then an exact float32 value whatever the summation
    order, so any correct implementation selects bit-identical top-k sets.
    ``distinct_rows`` > 0 builds the keys from that many distinct rows
    (repeated at random), so equal scores occur between different entries and
    the lowest-index tie-break decides.  Returns float32 arrays (all values
    exact in bf16).
    """
    rng = np.random.default_rng([seed, 99])
    q = rng.integers(-8, 9, size=(n_q, Hi, Di)).astype(np.float32) / 8
    k = rng.integers(-8, 9, size=(pool, Di)).astype(np.float32) / 8
    if distinct_rows > 0:
        k = k[rng.integers(0, distinct_rows, size=pool)]
    k[:, Di - Ri:] = 0
    wt = rng.integers(-4, 5, size=(n_q, Hi)).astype(np.float32) / 4
    return q, k, wt


# Output projection after the attention of the csa_prefill workload: 8192
# tokens x 64 heads x 512, eight groups of eight heads, rank 1024 per group,
# hidden size 4096 (sizes chosen here; the pages name the fields only).
OPROJ_SHAPE = dict(T=8192, H=64, D=512, G=8, R=1024, hidden=4096)


def oproj_inputs(T: int, H: int, D: int, G: int, R: int, hidden: int, seed: int = 0,
                 rows=None) -> Dict[str, np.ndarray]:
    """bf16 bits of the output projection's inputs: x [T, H, D] ~ N(0, 1),
    w_a [G R, (H/G) D] ~ N(0, 1/((H/G) D)), w_b [hidden, G R] ~ N(0, 1/(G R))
    (so that both products stay near unit scale).  ``rows`` draws only those
    token rows of x (the weights are always whole)."""
    ig = (H // G) * D
    if rows is None:
        x = _draw(seed, "attn_out", 0, (T, H, D), 1.0, "bf16")
    else:
        x = draw_rows(seed, "attn_out", 0, (T, H, D), 1.0, "bf16", rows)
    return {"x": x,
            "w_a": _draw(seed, "o_a", 0, (G * R, ig), 1.0 / math.sqrt(ig), "bf16"),
            "w_b": _draw(seed, "o_b", 0, (hidden, G * R), 1.0 / math.sqrt(G * R), "bf16")}


# Producer projections of the csa_prefill layer: 8192 tokens, hidden size
# 4096, query latent of rank 1024 (sizes chosen here; the pages name the
# modules only), 64 heads x 512, compressor width 512, indexer 64 x 128.
PROJ_SHAPE = dict(T=8192, hidden=4096, q_lora=1024, H=64, D=512, comp=512, Di=128, Hi=64)


def proj_inputs(T: int, hidden: int, q_lora: int, H: int, D: int, comp: int, Di: int, Hi: int,
                seed: int = 0, rows=None) -> Dict[str, np.ndarray]:
    """x [T, hidden] ~ N(0, 1) (bf16 bits), stacked weights w_x ~ N(0, 1/hidden)
    and w_q ~ N(0, 1/q_lora) (bf16 bits), norm weights g_qa, g_kv ~ 1 + N(0, 0.1^2)
    (float32).  ``rows`` draws only those token rows of x."""
    nx = q_lora + D + 2 * comp + 2 * Di + Hi
    nq = H * D + Hi * Di
    if rows is None:
        x = _draw(seed, "hidden", 0, (T, hidden), 1.0, "bf16")
    else:
        x = draw_rows(seed, "hidden", 0, (T, hidden), 1.0, "bf16", rows)
    return {"x": x,
            "w_x": _draw(seed, "w_x", 0, (nx, hidden), 1.0 / math.sqrt(hidden), "bf16"),
            "w_q": _draw(seed, "w_q", 0, (nq, q_lora), 1.0 / math.sqrt(q_lora), "bf16"),
            "g_qa": np.float32(1.0) + _draw(seed, "g_qa", 0, (q_lora,), 0.1, "f32"),
            "g_kv": np.float32(1.0) + _draw(seed, "g_kv", 0, (D,), 0.1, "f32")}

