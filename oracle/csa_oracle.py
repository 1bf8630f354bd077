"""CPU oracle for the DeepSeek-V4 compressed attention core (CSA / HCA layers).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module; the HIP library never
does, and this module imports nothing from it.

Plain float64 numpy, one query at a time, in the order the pages state the
layer.  Stored intermediates (rotated queries, pooled entries, window rows and
the layer output) are rounded to the storage dtype with round-to-nearest-even
where the layer stores them; ``dtype="f64"`` turns every rounding off (used by
the invariance pins).

Sources (titles and sections of the pages this follows):

* [HF-doc] Transformers documentation, DeepSeek-V4 model page, sections
  "Hybrid attention (sec. 2.3)", "Attention mask layout" and "Cache layers".
* [HF-PR] huggingface/transformers pull request 45616 (DeepSeek-V4 port),
  commit notes on RoPE apply, the attention sink, stateless compressor /
  indexer and the output-rope un-rotation comment.
* [TL] TransformerLens ``deepseek_v4.py`` adapter, ``_compressor_bridge``
  (compressor and indexer submodule lists).
* [OV] optimum-intel issue 1748, "What V4-Flash adds vs V3".
* [MLX] mlx-lm pull request 1797, architecture list.

Readings where the pages are silent (each is also listed in the design doc):

* gate logits are per channel; the pooling softmax runs over the window's
  tokens separately for every channel;
* CSA entry w pools tokens [(w-1)m, (w+1)m) (windows of 2m, stride m), HCA
  entry w pools [wm, (w+1)m); tokens before position 0 do not exist and are
  left out of the softmax;
* a pooled entry is rotated at position w*m (parity unpinned by the pages:
  no printed value fixes it);
* the indexer score is sum_h w[t,h] * ReLU(rot(q_I[t,h]) . k_I[w]) (the
  paper's formulas are referenced, not printed: parity unpinned by the pages);
* top-k ranks by score descending then entry index ascending, -0 == +0, and
  is emitted in ascending index order padded with -1;
* softmax scale 1/sqrt(D) on the logits, the sink logit unscaled.
"""
from __future__ import annotations

import math
from typing import Dict, Iterable, NamedTuple, Optional

import numpy as np

__all__ = [
    "round_to", "Yarn", "yarn_correction_index", "rope_frequencies", "rope_base", "rope",
    "pool_entry", "compress", "visible_entries",
    "window_positions", "index_scores", "topk_select", "attend",
    "csa_prefill", "hca_prefill", "sliding_prefill", "decode_step", "output_projection",
    "ProjSizes", "project_inputs", "paged_rows", "PagedPool", "page_pool",
]

_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def round_to(x, dtype: str) -> np.ndarray:
    """Round float64 values to the storage dtype, nearest-even, in one step.

    "bf16": 8 significant bits, exponent range of float32 (subnormal quantum
    2^-133); "f32": IEEE single; "f64": unchanged.
    """
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f64":
        return x.copy()
    if dtype == "f32":
        return x.astype(np.float32).astype(np.float64)
    if dtype != "bf16":
        raise ValueError(dtype)
    _, e = np.frexp(x)
    e = np.maximum(e, -125)           # below 2^-126 the quantum stays 2^-133
    q = np.ldexp(np.round(np.ldexp(x, 8 - e)), e - 8)   # np.round: half to even
    return np.where(np.abs(q) > _BF16_MAX, np.copysign(np.inf, x), q)


class Yarn(NamedTuple):
    """YaRN-scaled rope frequencies [OV "What V4-Flash adds vs V3": YaRN RoPE
    scaling, factor 16, 65k -> 1M context].  The pages name the method and the
    factor only; the ramp below is the YaRN method's (its published default
    turn counts beta_fast = 32, beta_slow = 1 are the layer spec's defaults)."""
    base: float
    factor: float
    original_context: float
    beta_fast: float
    beta_slow: float


def yarn_correction_index(n_turns: float, rope_dim: int, base: float, context: float) -> float:
    """The (real) pair index j at which theta_j = base^(-2j/rope_dim) makes
    ``n_turns`` full turns over ``context`` positions: context theta_j / (2 pi)
    = n_turns, i.e. j = rope_dim ln(context / (2 pi n_turns)) / (2 ln base)."""
    return rope_dim * math.log(context / (2.0 * math.pi * n_turns)) / (2.0 * math.log(base))


def rope_frequencies(rope_dim: int, base) -> np.ndarray:
    """theta_j for the rope_dim/2 pairs: base^(-2j/rope_dim) for a float base.

    For a ``Yarn`` base with factor s > 1: pairs up to lo (those turning at
    least beta_fast times over the original context) keep theta_j, pairs from
    hi on (at most beta_slow turns) are slowed to theta_j / s, and in between
    theta_j (1 - r) + (theta_j / s) r with r rising linearly in j; lo and hi
    are the correction indices of beta_fast and beta_slow rounded down and up
    and clamped to [0, rope_dim - 1].
    """
    j = np.arange(rope_dim // 2, dtype=np.float64)
    if not isinstance(base, Yarn):
        return base ** (-2.0 * j / rope_dim)
    theta = base.base ** (-2.0 * j / rope_dim)
    if not base.factor > 1.0:
        return theta
    lo = math.floor(yarn_correction_index(base.beta_fast, rope_dim, base.base,
                                          base.original_context))
    hi = math.ceil(yarn_correction_index(base.beta_slow, rope_dim, base.base,
                                         base.original_context))
    lo, hi = max(lo, 0), min(hi, rope_dim - 1)
    if hi == lo:
        hi += 0.001
    r = np.clip((j - lo) / (hi - lo), 0.0, 1.0)
    return theta * (1.0 - r) + (theta / base.factor) * r


def rope_base(L):
    """The rope frequency spec of a layer spec: its base, or a ``Yarn``."""
    f = getattr(L, "rope_factor", 0.0)
    if f > 1.0:
        return Yarn(L.rope_theta, f, L.rope_original_context, L.rope_beta_fast,
                    L.rope_beta_slow)
    return L.rope_theta


def rope(x, pos, rope_dim: int, base, sign: int = 1) -> np.ndarray:
    """Partial interleaved-pair rotary embedding [HF-PR RoPE apply; HF-doc sec. 2.3].

    The last ``rope_dim`` channels of each row, taken as pairs (c, c+1), are a
    complex number x_c + i x_{c+1} multiplied by exp(i * sign * pos * theta_j),
    theta_j = base^(-2j/rope_dim) for pair j (``rope_frequencies``; ``base``
    may be a ``Yarn``); other channels pass unchanged.  ``pos`` broadcasts
    against the leading axes of ``x``.
    """
    x = np.array(x, dtype=np.float64, copy=True)
    if rope_dim == 0:
        return x
    D = x.shape[-1]
    theta = rope_frequencies(rope_dim, base)
    ang = sign * np.asarray(pos, dtype=np.float64)[..., None] * theta
    z = x[..., D - rope_dim::2] + 1j * x[..., D - rope_dim + 1::2]
    z = z * np.exp(1j * ang)
    x[..., D - rope_dim::2] = z.real
    x[..., D - rope_dim + 1::2] = z.imag
    return x


def pool_entry(kv, gate, pos: int, rope_dim: int, base: float,
               norm_weight=None, eps: float = 1e-6) -> np.ndarray:
    """One compressed entry from its window's tokens [HF-doc sec. 2.3; TL compressor].

    Learned gated pooling: for every channel, softmax of the gate logits over
    the window's tokens, then the weighted sum of the kv values.  The
    compressor's submodules are kv_proj, gate_proj, kv_norm, rotary_emb: after
    pooling come the optional RMSNorm and the rotation at ``pos``.  Returns
    float64, unrounded.
    """
    kv = np.asarray(kv, dtype=np.float64)
    g = np.asarray(gate, dtype=np.float64)
    g = g - g.max(axis=0, keepdims=True)
    e = np.exp(g)
    alpha = e / e.sum(axis=0, keepdims=True)
    pooled = (alpha * kv).sum(axis=0)
    if norm_weight is not None:
        pooled = pooled / np.sqrt(np.mean(pooled * pooled) + eps) * np.asarray(norm_weight, np.float64)
    return rope(pooled, pos, rope_dim, base, +1)


def entry_tokens(w: int, ratio: int, overlap: int, p0: int = 0):
    """Token positions [lo, hi) pooled into entry w (tokens before p0 do not exist)."""
    return max((w - overlap) * ratio, p0), (w + 1) * ratio


def compress(kv, gate, ratio: int, overlap: int, rope_dim: int, base: float, dtype: str,
             norm_weight=None, eps: float = 1e-6, p0: int = 0) -> np.ndarray:
    """All entries that close inside a sequence of tokens at positions p0..p0+S-1.

    CSA (overlap=1): entry w covers tokens [(w-1)m, (w+1)m); HCA (overlap=0):
    [wm, (w+1)m).  Entry w closes at token (w+1)m-1 [HF-doc, attention mask
    layout: entry w is visible to query t iff w < (t+1)//m].  ``p0`` must be a
    multiple of ``ratio``; row i of the result is entry p0/ratio + i, rounded
    to ``dtype`` (the pool is stored).
    """
    kv = np.asarray(kv, dtype=np.float64)
    gate = np.asarray(gate, dtype=np.float64)
    S = kv.shape[0]
    assert p0 % ratio == 0
    w0, w1 = p0 // ratio, (p0 + S) // ratio
    out = np.zeros((w1 - w0, kv.shape[1]))
    for w in range(w0, w1):
        lo, hi = entry_tokens(w, ratio, overlap, p0)
        out[w - w0] = pool_entry(kv[lo - p0:hi - p0], gate[lo - p0:hi - p0], w * ratio,
                                 rope_dim, base, norm_weight, eps)
    return round_to(out, dtype)


def visible_entries(t: int, ratio: int, p0: int = 0) -> range:
    """Entries query t may use: w < (t+1)//m [HF-doc, attention mask layout, HCA]."""
    if ratio == 0:
        return range(0)
    return range(p0 // ratio, (t + 1) // ratio)


def window_positions(t: int, window: int, p0: int = 0) -> range:
    """Key positions of the sliding branch for query t: t-W < s <= t [HF-doc, mask layout]."""
    return range(max(p0, t - window + 1), t + 1)


def index_scores(qi_t, wi_t, keys, t: int, rope_dim: int, base: float, dtype: str) -> np.ndarray:
    """Lightning Indexer scores of query t against pooled indexer keys [HF-doc sec. 2.3 CSA; TL indexer].

    The indexer owns q_b_proj, a scorer with per-head weights_proj and a
    rotary embedding; its query is rotated at t (stored at the storage dtype)
    and each head's dot product with a key passes a ReLU before the weighted
    sum over heads.  ``keys`` are the visible keys, already rotated.
    """
    q = round_to(rope(qi_t, t, rope_dim, base, +1), dtype)          # [Hi, Di]
    dots = q @ np.asarray(keys, dtype=np.float64).T                   # [Hi, n]
    return (np.asarray(wi_t, np.float64)[:, None] * np.maximum(dots, 0.0)).sum(axis=0)


def topk_select(scores, k: int, first: int = 0) -> np.ndarray:
    """Per-query top-k block selection [HF-doc sec. 2.3 CSA and mask layout].

    Candidates are entries first..first+n-1 with the given scores.  If n <= k
    all are selected; otherwise the k best under (score descending, index
    ascending).  Emitted ascending, then -1 for every empty slot (the
    indexer's sentinel passed straight into the mask).
    """
    s = np.asarray(scores, dtype=np.float64)
    n = s.shape[0]
    if n <= k:
        sel = np.arange(n)
    else:
        order = np.lexsort((np.arange(n), -s))
        sel = np.sort(order[:k])
    out = np.full(k, -1, dtype=np.int64)
    out[:len(sel)] = sel + first
    return out


def attend(q_t, t: int, rows, sinks, scale: float, rope_dim: int, base: float,
           dtype: str) -> np.ndarray:
    """Attention of query t's heads over one row list (K = V) [HF-doc sec. 2.3; HF-PR].

    Shared K=V MQA: each row is both key and value.  The query is rotated at
    t; per head the sink logit joins the softmax as one more column with no
    value (GPT-OSS eager form); the output's rope slice is rotated back at -t
    (eq. 26 of the paper, per the model page) and stored.
    """
    rows = np.asarray(rows, dtype=np.float64)
    q = round_to(rope(q_t, t, rope_dim, base, +1), dtype)              # [H, D]
    logits = scale * (q @ rows.T)                                       # [H, n]
    M = logits.max(axis=1)
    if sinks is not None:
        sinks = np.asarray(sinks, dtype=np.float64)
        M = np.maximum(M, sinks)
    e = np.exp(logits - M[:, None])
    Z = e.sum(axis=1)
    if sinks is not None:
        Z = Z + np.exp(sinks - M)
    o = (e @ rows) / Z[:, None]
    o = rope(o, t, rope_dim, base, -1)
    return round_to(o, dtype)


# ----------------------------------------------------------------------------
# layer drivers: the steps above in the layer's order, over chosen queries

def _spec_scale(L, scale):
    return 1.0 / math.sqrt(L.head_dim) if scale is None else scale


def _window_rows(kv, L, p0, dtype):
    S = kv.shape[0]
    return round_to(rope(kv, np.arange(p0, p0 + S), L.rope_dim, rope_base(L), +1), dtype)


def csa_prefill(L, inp: Dict[str, np.ndarray], queries: Optional[Iterable[int]] = None,
                p0: int = 0, dtype: Optional[str] = None, scale: Optional[float] = None,
                norm_weight=None, inorm_weight=None, eps: float = 1e-6):
    """One sequence of a CSA layer, prefilled from position p0 (inputs float64).

    inp: q [S,H,D], kv [S,D], ckv/cgate [S,D], ikv/igate [S,Di], qi [S,Hi,Di],
    wi [S,Hi], sinks [H] (or None).  Returns dict with pool, ipool, win (the
    stored rotated window rows), idx [nq,k] (absolute entry ids) and out
    [nq,H,D] for the chosen queries (indices into the sequence).
    """
    dt = L.dtype if dtype is None else dtype
    S = inp["q"].shape[0]
    qs = range(S) if queries is None else list(queries)
    pool = compress(inp["ckv"], inp["cgate"], L.ratio, L.overlap, L.rope_dim, rope_base(L),
                    dt, norm_weight, eps, p0)
    ipool = compress(inp["ikv"], inp["igate"], L.ratio, L.overlap, L.index_rope_dim,
                     rope_base(L), dt, inorm_weight, eps, p0)
    win = _window_rows(inp["kv"], L, p0, dt)
    w0 = p0 // L.ratio
    sc_ = _spec_scale(L, scale)
    idx = np.zeros((len(qs), L.topk), dtype=np.int64)
    out = np.zeros((len(qs), L.num_heads, L.head_dim))
    for n, i in enumerate(qs):
        t = p0 + i
        vis = visible_entries(t, L.ratio, p0)
        sc = index_scores(inp["qi"][i], inp["wi"][i], ipool[vis.start - w0:vis.stop - w0], t,
                          L.index_rope_dim, rope_base(L), dt)
        idx[n] = topk_select(sc, L.topk, first=vis.start)
        wp = window_positions(t, L.window, p0)
        rows = np.concatenate([win[wp.start - p0:wp.stop - p0],
                               pool[idx[n][idx[n] >= 0] - w0]])
        out[n] = attend(inp["q"][i], t, rows, inp["sinks"], sc_, L.rope_dim, rope_base(L), dt)
    return {"pool": pool, "ipool": ipool, "win": win, "idx": idx, "out": out}


def hca_prefill(L, inp, queries=None, p0: int = 0, dtype=None, scale=None,
                norm_weight=None, eps: float = 1e-6):
    """One sequence of an HCA layer: every visible entry plus the window [HF-doc sec. 2.3 HCA]."""
    dt = L.dtype if dtype is None else dtype
    S = inp["q"].shape[0]
    qs = range(S) if queries is None else list(queries)
    pool = compress(inp["ckv"], inp["cgate"], L.ratio, L.overlap, L.rope_dim, rope_base(L),
                    dt, norm_weight, eps, p0)
    win = _window_rows(inp["kv"], L, p0, dt)
    w0 = p0 // L.ratio
    sc_ = _spec_scale(L, scale)
    out = np.zeros((len(qs), L.num_heads, L.head_dim))
    for n, i in enumerate(qs):
        t = p0 + i
        vis = visible_entries(t, L.ratio, p0)
        wp = window_positions(t, L.window, p0)
        rows = np.concatenate([win[wp.start - p0:wp.stop - p0], pool[vis.start - w0:vis.stop - w0]])
        out[n] = attend(inp["q"][i], t, rows, inp["sinks"], sc_, L.rope_dim, rope_base(L), dt)
    return {"pool": pool, "win": win, "out": out}


def sliding_prefill(L, inp, queries=None, p0: int = 0, dtype=None, scale=None):
    """Sliding-only layer: the window branch alone [HF-doc sec. 2.3, sliding_attention]."""
    dt = L.dtype if dtype is None else dtype
    S = inp["q"].shape[0]
    qs = range(S) if queries is None else list(queries)
    win = _window_rows(inp["kv"], L, p0, dt)
    sc_ = _spec_scale(L, scale)
    out = np.zeros((len(qs), L.num_heads, L.head_dim))
    for n, i in enumerate(qs):
        t = p0 + i
        wp = window_positions(t, L.window, p0)
        out[n] = attend(inp["q"][i], t, win[wp.start - p0:wp.stop - p0], inp["sinks"], sc_,
                        L.rope_dim, rope_base(L), dt)
    return {"win": win, "out": out}


# ----------------------------------------------------------------------------
# paged pools [HF-doc "Cache layers": one cache per layer, each holding its own
# pool; OV "What native registration would touch": the cache layout is not
# uniform across layers].  The pages define no paging; the reading taken: a
# sequence's pooled entries live in fixed-size blocks of a shared pool tensor,
# block j of sequence b at block table[b][j].  Paging moves rows only; every
# value is the contiguous pool's.

def paged_rows(ids, table, block_entries: int) -> np.ndarray:
    """Rows of the paged pool tensor holding entries ``ids`` of one sequence:
    table[w // E] * E + w % E for entry w (E = block_entries)."""
    ids = np.asarray(ids, dtype=np.int64)
    table = np.asarray(table, dtype=np.int64)
    return table[ids // block_entries] * block_entries + ids % block_entries


def page_pool(pool, table, block_entries: int, blocks: int) -> np.ndarray:
    """The paged pool tensor [blocks * E, width] holding one sequence's
    contiguous pool [n, width] (rows of unused blocks are zero)."""
    pool = np.asarray(pool, dtype=np.float64)
    out = np.zeros((blocks * block_entries, pool.shape[1]))
    out[paged_rows(np.arange(pool.shape[0]), table, block_entries)] = pool
    return out


class PagedPool:
    """Read view of one sequence's entries 0 .. n-1 in a paged pool tensor, for
    ``decode_step`` (which indexes its pool caches with id arrays)."""

    def __init__(self, rows, table, block_entries: int, n: int):
        self.rows = rows
        self.table = np.asarray(table, dtype=np.int64)
        self.E = block_entries
        self.shape = (n, np.asarray(rows).shape[1])

    def __getitem__(self, ids):
        if isinstance(ids, slice):
            ids = np.arange(*ids.indices(self.shape[0]))
        ids = np.asarray(ids, dtype=np.int64)
        assert ids.size == 0 or (ids.min() >= 0 and ids.max() < self.shape[0])
        return np.asarray(self.rows, dtype=np.float64)[paged_rows(ids, self.table, self.E)]


def decode_step(L, t: int, new: Dict[str, np.ndarray], cache: Dict[str, np.ndarray],
                dtype=None, scale=None, norm_weight=None, inorm_weight=None, eps=1e-6):
    """One new token at position t of one sequence, against its caches.

    new: q [H,D], kv [D], ckv/cgate [D], ikv/igate [Di], qi [Hi,Di], wi [Hi],
    sinks.  cache: win [W,D] (rotated rows of positions t-W..t-1 at slot
    position mod W), pool [P,D], ipool [P,Di] (entries 0..P-1), and the raw
    compressor tokens of the positions before t (cstate_* / istate_*, slot
    position mod (1+overlap)m).  P = t // m: the entries closed before t.  The caches are updated the way the layer's
    cache would be [HF-doc, cache layers; HF-PR stateless compressor]: the
    window gains row t, and an entry closes when (t+1) % m == 0.  Returns
    idx (CSA), out [H,D], and the new entries (if any).
    """
    dt = L.dtype if dtype is None else dtype
    W = L.window
    res = {}
    win = np.array(cache["win"], dtype=np.float64, copy=True)
    cap = win.shape[0]
    win[t % cap] = round_to(rope(new["kv"], t, L.rope_dim, rope_base(L), +1), dt)
    wrows = np.stack([win[s % cap] for s in window_positions(t, W)])
    rows = [wrows]
    if L.ratio > 0:
        m, ov = L.ratio, L.overlap
        Ls = (1 + ov) * m
        streams = [("pool", "ckv", "cgate", "cstate_kv", "cstate_gate", L.rope_dim, norm_weight)]
        if L.has_indexer:
            streams.append(("ipool", "ikv", "igate", "istate_kv", "istate_gate",
                            L.index_rope_dim, inorm_weight))
        pools, fresh = {}, {}
        for pk, kk, gk, sk, sg, rd, nw in streams:
            pool = cache[pk]          # entries 0 .. t//m - 1 (any array-like)
            if (t + 1) % m == 0:
                w = (t + 1) // m - 1
                lo, hi = entry_tokens(w, m, ov)
                toks = list(range(lo, hi))
                kvs = np.stack([new[kk] if s == t else cache[sk][s % Ls] for s in toks])
                gts = np.stack([new[gk] if s == t else cache[sg][s % Ls] for s in toks])
                ent = round_to(pool_entry(kvs, gts, w * m, rd, rope_base(L), nw, eps), dt)
                assert pool.shape[0] == w, "cache must hold the entries closed before t"
                fresh[pk] = ent
                res["new_" + pk] = ent
            pools[pk] = pool

        def gather(pk, ids):
            """Rows `ids` of pool pk, the entry closing at t (if any) last."""
            ids = np.asarray(ids, dtype=np.int64)
            P = pools[pk].shape[0]
            old = np.asarray(pools[pk][ids[ids < P]], dtype=np.float64)
            if pk in fresh and np.any(ids >= P):
                old = np.concatenate([old, fresh[pk][None]])
            return old.reshape(len(ids), -1)

        vis = visible_entries(t, m)
        if L.has_indexer:
            keys = gather("ipool", np.arange(vis.start, vis.stop))
            sc = index_scores(new["qi"], new["wi"], keys, t, L.index_rope_dim, rope_base(L), dt)
            idx = topk_select(sc, L.topk, first=vis.start)
            res["idx"] = idx
            rows.append(gather("pool", idx[idx >= 0]))
        else:
            rows.append(gather("pool", np.arange(vis.start, vis.stop)))
    rows = np.concatenate(rows)
    res["out"] = attend(new["q"], t, rows, new["sinks"], _spec_scale(L, scale), L.rope_dim,
                        rope_base(L), dt)
    return res


def output_projection(attn_out, w_a, w_b, o_groups: int, dtype: str) -> np.ndarray:
    """Grouped low-rank output projection [HF-doc sec. 2.3, "Grouped Output
    Projection"; HF-PR notes on DeepseekV4GroupedLinear].

    attn_out [T, H, D] (the attention output after the -t rotation); w_a
    [G R, (H / G) D], o_a_proj's (out, in) weight, rows g R .. g R + R - 1 for
    group g; w_b [hidden, G R], o_b_proj's weight.  Group g takes the heads
    g H/G .. (g+1) H/G - 1 of a token: y[t, g] = w_a[g] x[t, g], stored at
    ``dtype`` like the module output; out[t] = w_b y[t], stored at ``dtype``.
    The pages give no bias; none is added.
    """
    x = np.asarray(attn_out, dtype=np.float64)
    T, H, D = x.shape
    G = o_groups
    ig = (H // G) * D
    R = np.asarray(w_a).shape[0] // G
    xg = x.reshape(T, G, ig)
    wa = np.asarray(w_a, dtype=np.float64).reshape(G, R, ig)
    y = np.empty((T, G, R))
    for g in range(G):
        y[:, g, :] = xg[:, g, :] @ wa[g].T
    y = round_to(y, dtype)
    return round_to(y.reshape(T, G * R) @ np.asarray(w_b, dtype=np.float64).T, dtype)


class ProjSizes(NamedTuple):
    """Widths of the producer projections (0 drops a stream: a layer without
    compressor has comp = 0, one without indexer index_dim = index_heads = 0)."""
    q_lora: int
    heads: int
    head_dim: int
    comp: int
    index_dim: int
    index_heads: int


def _rms_rows(y, weight, eps):
    y = np.asarray(y, dtype=np.float64)
    out = y / np.sqrt(np.mean(y * y, axis=-1, keepdims=True) + eps)
    return out if weight is None else out * np.asarray(weight, dtype=np.float64)


def project_inputs(x, w_x, g_qa, g_kv, w_q, sz: ProjSizes, eps: float, q_head_norm: bool,
                   dtype: str) -> dict:
    """Producer side of the attention block [TL, the adapter's self_attn
    module list (q_a_proj, q_a_norm, q_b_proj, q_b_norm, kv_proj, kv_norm,
    compressor) and ``_compressor_bridge`` (compressor kv_proj / gate_proj,
    indexer kv_proj / gate_proj / q_b_proj / scorer.weights_proj); HF-doc
    sec. 2.3: kv_proj makes the single shared K=V head].

    x [T, hidden] are the block's normalised hidden states.  w_x stacks the
    (out, in) weights read from x, in this row order: q_a_proj (q_lora rows),
    kv_proj (D), compressor kv_proj (comp), compressor gate_proj (comp),
    indexer kv_proj (index_dim), indexer gate_proj (index_dim),
    weights_proj (index_heads).  w_q stacks the weights read from the query
    latent: q_b_proj (H D rows) then the indexer's q_b_proj (H_I D_I rows).

    Every projection output is stored at ``dtype``; the two RMSNorms
    (q_a_norm with weight g_qa, kv_norm with weight g_kv) read the stored
    projection and are stored in turn; with ``q_head_norm`` each head of q
    is divided by its RMS over D (q_b_norm, read as carrying no weight), else
    q is the stored projection.  The compressor's own kv_norm acts on pooled
    entries (``compress``), not here.
    """
    x = np.asarray(x, dtype=np.float64)
    T = x.shape[0]
    y = round_to(x @ np.asarray(w_x, dtype=np.float64).T, dtype)
    cuts = np.cumsum([0, sz.q_lora, sz.head_dim, sz.comp, sz.comp, sz.index_dim, sz.index_dim,
                      sz.index_heads])
    seg = [y[:, cuts[i]:cuts[i + 1]] for i in range(7)]
    latent = round_to(_rms_rows(seg[0], g_qa, eps), dtype)
    out = {"latent": latent, "kv": round_to(_rms_rows(seg[1], g_kv, eps), dtype),
           "ckv": seg[2], "cgate": seg[3], "ikv": seg[4], "igate": seg[5], "wi": seg[6]}
    yq = round_to(latent @ np.asarray(w_q, dtype=np.float64).T, dtype)
    hd = sz.heads * sz.head_dim
    q = yq[:, :hd].reshape(T, sz.heads, sz.head_dim)
    if q_head_norm:
        q = round_to(_rms_rows(q, None, eps), dtype)
    out["q"] = q
    out["qi"] = yq[:, hd:].reshape(T, sz.index_heads, sz.index_dim)
    return out

