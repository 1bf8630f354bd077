"""Shared plumbing of the GPU parity tests: device upload/download of the
synthetic inputs, the oracle over chosen queries, and comparison rules.

Tolerances (from the arithmetic; written in each comparison):
* bf16 outputs: |gpu - ref| <= 2e-3 + 2e-2 |ref| element-wise;
* float32 outputs: |gpu - ref| <= 1e-5 + 1e-5 |ref|;
* stored rows computed in float64 on both sides and rounded once (pooled
  entries, window rows): identical bits, except a float64 result lying within
  a few ulps of a rounding midpoint, which the two sides' float64 libraries
  may round apart (at most one storage ulp, on a vanishing fraction);
* top-k ids: identical, or every differing id is a provable near tie: its
  exact score lies within the float32 forward-error bounds of the k-th score
  (gamma_n * sum|terms|, n = D_I + H_I + 1, u = 2^-24).
"""
from __future__ import annotations

import sys

import numpy as np

import synth
from synth import to_f64

TOL = {"bf16": (2e-3, 2e-2), "f32": (1e-5, 1e-5)}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(arr, device="cuda"):
    """Stored numpy tensor (uint16 = bf16 bits, float32) -> device tensor."""
    import torch
    if arr.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)


def host(t) -> np.ndarray:
    """Device tensor -> float64 numpy (exact)."""
    import torch
    if t.dtype == torch.bfloat16:
        return to_f64(t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
    return t.detach().cpu().numpy().astype(np.float64)


def assert_close(gpu, ref, dtype, what=""):
    a, r = TOL[dtype]
    gpu, ref = np.asarray(gpu, np.float64), np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    err = np.abs(gpu - ref)
    bad = err > a + r * np.abs(ref)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; first at "
                             f"{tuple(i)} gpu={gpu[tuple(i)]} ref={ref[tuple(i)]} "
                             f"max_err={err.max():.3e}")
    return float(err.max())


def ulp_diff_ok(gpu, ref, dtype, what="", max_frac=1e-4):
    """Stored-row comparison: identical bits except rare one-ulp midpoint cases."""
    gpu, ref = np.asarray(gpu, np.float64), np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    diff = gpu != ref
    if not diff.any():
        return 0
    ulp = np.abs(ref) * (2.0 ** -7 if dtype == "bf16" else 2.0 ** -23)
    far = np.abs(gpu - ref) > ulp + 1e-300
    assert not far.any(), f"{what}: {far.sum()} values differ by more than one ulp"
    assert diff.mean() <= max_frac, f"{what}: {diff.sum()} one-ulp differences"
    return int(diff.sum())


def index_exact(spec, qi_t, wi_t, keys, t, dtype=None):
    """Exact (float64) index scores of query t against ``keys`` and the sum of
    |terms| of each score, for the float32 error bound of ``audit_topk``.

    Both use the layer's own rope frequencies (``O.rope_base(spec)``: the
    plain base, or the YaRN-scaled frequencies the layer's keys were rotated
    with), so the exact scores are those of the stored keys."""
    from oracle import csa_oracle as O
    dt = spec.dtype if dtype is None else dtype
    base = O.rope_base(spec)
    keys = np.asarray(keys, dtype=np.float64)
    sc = O.index_scores(qi_t, wi_t, keys, t, spec.index_rope_dim, base, dt)
    q = O.round_to(O.rope(qi_t, t, spec.index_rope_dim, base, +1), dt)
    ab = (np.abs(wi_t)[:, None] * (np.abs(q) @ np.abs(keys).T)).sum(axis=0)
    return sc, ab


def audit_topk(gpu_idx, ref_idx, scores, absterms, Di, Hi):
    """Differences between two top-k id lists must be provable near ties.

    scores / absterms: exact scores and sum|terms| of the visible entries
    (index = entry id).  Returns the number of differing ids.
    """
    g = set(int(x) for x in gpu_idx if x >= 0)
    r = set(int(x) for x in ref_idx if x >= 0)
    assert len(g) == len(r), "different numbers of selected entries"
    assert list(gpu_idx[:len(g)]) == sorted(g) and all(x == -1 for x in gpu_idx[len(g):]), \
        "gpu ids must be ascending then -1"
    if g == r:
        return 0
    u = 2.0 ** -24
    n = Di + Hi + 1
    gamma = n * u / (1 - n * u)
    sel = sorted(r, key=lambda w: (-scores[w], w))
    kth = sel[-1]
    for w in g.symmetric_difference(r):
        lim = gamma * (absterms[w] + absterms[kth]) * 1.0001 + 1e-30
        assert abs(scores[w] - scores[kth]) <= lim, \
            f"entry {w}: score {scores[w]} vs k-th {scores[kth]} exceeds near-tie bound {lim}"
    return len(g.symmetric_difference(r))


def seq_f64(inp, b):
    """Sequence b of prefill inputs as float64 (sinks shared)."""
    return {k: (v if v is None else to_f64(v) if k == "sinks" else to_f64(v[b]))
            for k, v in inp.items()}


class LazyF64:
    """Read-only float64 view of a stored tensor, decoded only where indexed.

    Lets the oracle walk a full-size sequence while converting just the rows
    it touches (sampled queries, gathered cache rows)."""

    def __init__(self, arr):
        self.arr = arr
        self.shape = arr.shape

    def __getitem__(self, i):
        return to_f64(self.arr[i])

    def __len__(self):
        return self.shape[0]
