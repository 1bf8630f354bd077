"""The near-tie audit of top-k ids (tests/helpers.audit_topk) on the CPU.

The GPU parity tests accept an id that differs from the oracle's only when
its exact score lies within the float32 forward-error bound of the k-th
score.  These checks make sure that audit is sound on a YaRN layer (the
V4-shaped workloads scale every rope by factor 16): the exact scores must be
those of the layer's own rope frequencies, a planted wrong id must be
rejected, and a true tie must be accepted.
"""
import dataclasses

import numpy as np
import pytest

import synth
from oracle import csa_oracle as O
from synth import to_f64
from tests.helpers import audit_topk, index_exact


def _yarn_case(S=600, k=32, seed=3):
    w = synth.workload("csa_prefill", S=S)
    spec = dataclasses.replace(w.layers[0], topk=k)
    assert spec.rope_factor > 1.0, "the V4-shaped layer runs YaRN"
    inp = synth.prefill_inputs(w, seed)
    x = {k_: (to_f64(v) if k_ == "sinks" else to_f64(v[0])) for k_, v in inp.items()
         if k_ in ("qi", "wi", "ikv", "igate")}
    ipool = O.compress(x["ikv"], x["igate"], spec.ratio, spec.overlap, spec.index_rope_dim,
                       O.rope_base(spec), spec.dtype)
    return spec, x, ipool


def test_exact_scores_use_the_layers_yarn_frequencies():
    spec, x, ipool = _yarn_case()
    t = 599
    keys = ipool[:(t + 1) // 4]
    sc, ab = index_exact(spec, x["qi"][t], x["wi"][t], keys, t)
    want = O.index_scores(x["qi"][t], x["wi"][t], keys, t, spec.index_rope_dim,
                          O.rope_base(spec), spec.dtype)
    assert np.array_equal(sc, want)
    assert np.all(ab >= np.abs(sc))
    # the plain base gives other scores and another selection: scoring the
    # audit with it would judge ids against the wrong numbers
    plain = O.index_scores(x["qi"][t], x["wi"][t], keys, t, spec.index_rope_dim,
                           spec.rope_theta, spec.dtype)
    assert np.abs(plain - sc).max() > 1e-3
    assert not np.array_equal(O.topk_select(plain, spec.topk), O.topk_select(sc, spec.topk))


@pytest.mark.parametrize("t", [300, 599])
def test_audit_rejects_a_planted_wrong_id(t):
    spec, x, ipool = _yarn_case()
    keys = ipool[:(t + 1) // 4]
    sc, ab = index_exact(spec, x["qi"][t], x["wi"][t], keys, t)
    ref = O.topk_select(sc, spec.topk)
    assert audit_topk(ref.copy(), ref, sc, ab, spec.index_dim, spec.index_heads) == 0
    # swap the weakest selected id for the weakest unselected one: far from a tie
    sel = set(int(v) for v in ref if v >= 0)
    out = [w for w in range(len(sc)) if w not in sel]
    weakest_in = min(sel, key=lambda w: (sc[w], -w))
    weakest_out = min(out, key=lambda w: (sc[w], -w))
    bad = np.array(sorted((sel - {weakest_in}) | {weakest_out}) +
                   [-1] * (spec.topk - len(sel)), dtype=np.int64)
    with pytest.raises(AssertionError, match="near-tie bound"):
        audit_topk(bad, ref, sc, ab, spec.index_dim, spec.index_heads)


def test_audit_rejects_a_dropped_or_unordered_selection():
    spec, x, ipool = _yarn_case()
    t = 599
    keys = ipool[:(t + 1) // 4]
    sc, ab = index_exact(spec, x["qi"][t], x["wi"][t], keys, t)
    ref = O.topk_select(sc, spec.topk)
    short = ref.copy()
    short[-1] = -1
    with pytest.raises(AssertionError, match="different numbers"):
        audit_topk(short, ref, sc, ab, spec.index_dim, spec.index_heads)
    shuffled = ref.copy()
    shuffled[[0, 1]] = shuffled[[1, 0]]
    with pytest.raises(AssertionError, match="ascending"):
        audit_topk(shuffled, ref, sc, ab, spec.index_dim, spec.index_heads)


def test_audit_accepts_an_exact_tie_taken_the_other_way():
    # entries 2 and 5 tie exactly at the k-th place; the lowest id (2) wins,
    # a selection holding 5 instead differs only by that tie
    sc = np.array([9.0, 8.0, 1.5, 7.0, 0.5, 1.5, 0.25])
    ab = np.abs(sc) + 1.0
    ref = O.topk_select(sc, 4)
    assert list(ref) == [0, 1, 2, 3]
    other = np.array([0, 1, 3, 5])
    assert audit_topk(other, ref, sc, ab, 128, 64) == 2
