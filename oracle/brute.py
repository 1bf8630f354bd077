"""Dense-mask brute force of the same layer, for tiny shapes only.

TEST INFRASTRUCTURE ONLY (same rule as ``csa_oracle``).  This is a second,
independent formulation used to pin the per-query oracle: it shares no code
with ``csa_oracle`` and builds everything as whole-sequence tensors, the way
the model page describes the eager layer [Transformers DeepSeek-V4 model page,
"Attention mask layout"]:

* the key axis is cat([window rows (S columns), compressor columns]) and the
  mask is cat([sliding causal mask, block_bias]);
* CSA: the compressor gathers k entries per query, unrolled to S*k columns;
  query t may use only columns S + t*k + j whose index is not -1;
* HCA: S + T_total columns, entry w open to query t iff w < (t+1)//m;
* the sink is one more logit column per head that carries no value;
* RoPE uses real cos/sin tables and the interleaved "rotate every two" form
  instead of complex multiplication; pooling uses a dense membership matrix;
  top-k uses rank counting instead of sorting.

Everything is float64 with no rounding to a storage dtype.
"""
from __future__ import annotations

import numpy as np

__all__ = ["rope_tables", "apply_rope", "dense_compress", "dense_index_scores",
           "rank_topk", "dense_attention"]


def rope_tables(pos, rope_dim: int, base: float):
    """cos/sin per channel of the rope slice, each frequency repeated for its pair."""
    inv = 1.0 / (base ** (np.arange(0, rope_dim, 2, dtype=np.float64) / rope_dim))
    ang = np.outer(np.asarray(pos, np.float64), inv)           # [n, R/2]
    ang = np.repeat(ang, 2, axis=-1)                             # [n, R]
    return np.cos(ang), np.sin(ang)


def apply_rope(x, cos, sin):
    """x [..., n, D] (positions on axis -2): rotate the last R channels in interleaved pairs."""
    x = np.array(x, dtype=np.float64, copy=True)
    R = cos.shape[-1]
    r = x[..., -R:]
    swapped = np.empty_like(r)
    swapped[..., 0::2] = -r[..., 1::2]
    swapped[..., 1::2] = r[..., 0::2]
    x[..., -R:] = r * cos + swapped * sin
    return x


def dense_compress(kv, gate, ratio, overlap, rope_dim, base):
    """All entries of a sequence from position 0 via a membership matrix [n_entries, S]."""
    kv = np.asarray(kv, np.float64)
    gate = np.asarray(gate, np.float64)
    S = kv.shape[0]
    P = S // ratio
    s = np.arange(S)[None, :]
    w = np.arange(P)[:, None]
    member = ((s >= (w - overlap) * ratio) & (s < (w + 1) * ratio)).astype(np.float64)
    e = np.exp(gate - gate.max(axis=0, keepdims=True))           # [S, C]
    num = member @ (e * kv)
    den = member @ e
    pooled = num / den
    cos, sin = rope_tables(np.arange(P) * ratio, rope_dim, base)
    return apply_rope(pooled, cos, sin)


def dense_index_scores(qi, wi, ikeys, ratio, rope_dim, base):
    """scores[t, w] for every query and entry, -inf where entry w is not yet closed."""
    S = qi.shape[0]
    cos, sin = rope_tables(np.arange(S), rope_dim, base)
    q = apply_rope(np.swapaxes(qi, 0, 1), cos, sin)              # [Hi, S, Di]
    dots = np.einsum("hsd,wd->hsw", q, np.asarray(ikeys, np.float64))
    sc = np.einsum("sh,hsw->sw", np.asarray(wi, np.float64), np.maximum(dots, 0))
    t = np.arange(S)[:, None]
    wcol = np.arange(ikeys.shape[0])[None, :]
    return np.where(wcol < (t + 1) // ratio, sc, -np.inf)


def rank_topk(scores_row, k):
    """Selection by rank counting: entry w is kept iff fewer than k entries beat it."""
    s = np.asarray(scores_row, np.float64)
    valid = np.isfinite(s)
    n = s.shape[0]
    keep = []
    for w in range(n):
        if not valid[w]:
            continue
        better = 0
        for v in range(n):
            if valid[v] and (s[v] > s[w] or (s[v] == s[w] and v < w)):
                better += 1
        if better < k:
            keep.append(w)
    out = -np.ones(k, dtype=np.int64)
    out[:len(keep)] = keep
    return out


def dense_attention(q, win_kv, comp_kv, comp_mask, window, sinks, scale, rope_dim, base):
    """Eager-style attention over cat([window keys, compressor keys]) with one mask.

    q [S,H,D] un-rotated; win_kv [S,D] un-rotated window rows (rotated here at
    their positions); comp_kv [C,D] compressor columns (already rotated);
    comp_mask [S,C] True where query t may use column c.  Returns the output
    after the -t rotation, float64.
    """
    S, H, D = q.shape
    cos, sin = rope_tables(np.arange(S), rope_dim, base)
    qr = apply_rope(np.swapaxes(q, 0, 1), cos, sin)              # [H, S, D]
    kw = apply_rope(win_kv, cos, sin)                            # [S, D]
    keys = np.concatenate([kw, np.asarray(comp_kv, np.float64)], axis=0)
    t = np.arange(S)[:, None]
    s = np.arange(S)[None, :]
    slide = (s <= t) & (s > t - window)
    mask = np.concatenate([slide, comp_mask], axis=1)            # [S, S+C]
    logits = scale * np.einsum("hsd,cd->hsc", qr, keys)
    logits = np.where(mask[None], logits, -np.inf)
    if sinks is not None:
        sink_col = np.broadcast_to(np.asarray(sinks, np.float64)[:, None, None], (H, S, 1))
        logits = np.concatenate([logits, sink_col], axis=-1)
    mx = logits.max(axis=-1, keepdims=True)
    p = np.exp(logits - mx)
    p = p / p.sum(axis=-1, keepdims=True)
    if sinks is not None:
        p = p[..., :-1]
    o = np.einsum("hsc,cd->hsd", p, keys)                         # [H, S, D]
    ci, si = rope_tables(-np.arange(S), rope_dim, base)
    o = apply_rope(o, ci, si)
    return np.swapaxes(o, 0, 1)                                    # [S, H, D]
