"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each test ties one oracle function to a closed form, a library routine, an
invariant of the mathematics, the pages' worked example, or the independent
dense-mask formulation in ``oracle.brute``.  A plausible slip in the oracle
(a dropped term, a wrong sign or index, a transposed operand, a half-split
instead of interleaved rotation, a wrong window edge) fails at least one.
"""
import math
import os

import numpy as np
import pytest

from oracle import brute
from oracle import csa_oracle as O
from synth import LayerSpec, f32_to_bf16_bits, bf16_bits_to_f32

HERE = os.path.dirname(os.path.abspath(__file__))


def small_layer(kind="csa", **kw):
    base = dict(kind=kind, dtype="f64", num_heads=4, head_dim=16, rope_dim=8, rope_theta=10000.0,
                window=8, ratio=4 if kind == "csa" else (8 if kind == "hca" else 0),
                overlap=1 if kind == "csa" else 0, index_heads=3, index_dim=12,
                index_rope_dim=4, topk=2)
    base.update(kw)
    return LayerSpec(**base)


def rand_inputs(L, S, seed=0, q_scale=1.0):
    rng = np.random.default_rng(seed)
    H, D, Hi, Di = L.num_heads, L.head_dim, L.index_heads, L.index_dim
    return {
        "q": rng.standard_normal((S, H, D)) * q_scale,
        "kv": rng.standard_normal((S, D)),
        "ckv": rng.standard_normal((S, D)),
        "cgate": rng.standard_normal((S, D)),
        "ikv": rng.standard_normal((S, Di)),
        "igate": rng.standard_normal((S, Di)),
        "qi": rng.standard_normal((S, Hi, Di)),
        "wi": rng.standard_normal((S, Hi)),
        "sinks": rng.standard_normal(H),
    }


# ----------------------------------------------------------------------------
# rounding to the storage dtype

def _bf16_neighbours(x):
    """The two bf16 values around x, found by walking float32 bit patterns."""
    f = np.float32(x)
    bits = np.array([f], np.float32).view(np.uint32)[0] & np.uint32(0xFFFF0000)
    lo = np.array([bits], np.uint32).view(np.float32)[0]
    up = np.array([bits + np.uint32(0x10000)], np.uint32).view(np.float32)[0]
    return sorted([float(lo), float(up)], key=lambda v: v)


def test_round_bf16_is_nearest_even_single_rounding():
    rng = np.random.default_rng(1)
    xs = np.concatenate([rng.standard_normal(3000) * 10.0 ** rng.integers(-6, 6, 3000),
                         [1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 1 + 2 ** -8 + 2 ** -30]])
    r = O.round_to(xs, "bf16")
    for x, y in zip(xs, r):
        a, b = sorted(_bf16_neighbours(x))
        if not (a <= x <= b):
            a, b = sorted(_bf16_neighbours(np.nextafter(np.float32(x), np.float32(0))))
        assert y in (a, b)
        da, db = abs(x - a), abs(x - b)
        if da != db:
            assert y == (a if da < db else b)
        else:   # tie: even significand (low bit of the bf16 pattern is 0)
            bits = int(np.array([y], np.float32).view(np.uint32)[0]) >> 16
            assert bits & 1 == 0
    # exact ties and a value just above a tie that float32 rounding would move onto it
    assert O.round_to(1 + 2 ** -8, "bf16") == 1.0
    assert O.round_to(1 + 3 * 2 ** -8, "bf16") == 1 + 2 ** -6
    assert O.round_to(1 + 2 ** -8 + 2 ** -30, "bf16") == 1 + 2 ** -7


def test_round_bf16_matches_storage_conversion_on_float32_inputs():
    # the generator's float32 -> bf16 conversion is the same rounding on float32 inputs
    rng = np.random.default_rng(2)
    x = rng.standard_normal(10000).astype(np.float32)
    assert np.array_equal(O.round_to(x.astype(np.float64), "bf16"),
                          bf16_bits_to_f32(f32_to_bf16_bits(x)).astype(np.float64))


# ----------------------------------------------------------------------------
# RoPE

def test_rope_unit_vectors_closed_form():
    D, R, base, p = 16, 8, 10000.0, 37
    for j in range(R // 2):
        x = np.zeros(D)
        x[D - R + 2 * j] = 1.0
        y = O.rope(x, p, R, base, +1)
        th = p * base ** (-2 * j / R)
        expect = np.zeros(D)
        expect[D - R + 2 * j] = math.cos(th)
        expect[D - R + 2 * j + 1] = math.sin(th)
        assert np.allclose(y, expect, atol=1e-14)


def test_rope_identity_inverse_norm_and_untouched_channels():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 32))
    p = np.array([0, 1, 100, 65535, 1048576])
    R = 16
    assert np.array_equal(O.rope(x[:1], 0, R, 1e4, +1), x[:1])
    y = O.rope(x, p, R, 1e4, +1)
    assert np.array_equal(y[:, :32 - R], x[:, :32 - R])
    assert np.allclose(O.rope(y, p, R, 1e4, -1), x, atol=1e-12)
    pn = lambda a: a[:, 32 - R::2] ** 2 + a[:, 32 - R + 1::2] ** 2
    assert np.allclose(pn(y), pn(x), atol=1e-12)


def test_rope_relative_position_property():
    rng = np.random.default_rng(4)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    a = O.rope(q, 1000, 64, 160000.0) @ O.rope(k, 900, 64, 160000.0)
    b = O.rope(q, 1000 + 4096, 64, 160000.0) @ O.rope(k, 900 + 4096, 64, 160000.0)
    assert abs(a - b) < 1e-10


def test_rope_matches_independent_table_form():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((7, 24))
    pos = np.arange(7) * 13
    c, s = brute.rope_tables(pos, 8, 500.0)
    assert np.allclose(O.rope(x, pos, 8, 500.0, +1), brute.apply_rope(x, c, s), atol=1e-13)


# ----------------------------------------------------------------------------
# YaRN frequencies (the pages name YaRN and factor 16 over a 65k context; the
# ramp is the method's, so these pins rest on the turn-count definitions)

_YARN = dict(factor=16.0, original_context=65536.0, beta_fast=32.0, beta_slow=1.0)


def test_yarn_factor_one_is_plain_rope():
    for R, base in ((64, 10000.0), (64, 160000.0), (16, 10000.0)):
        plain = O.rope_frequencies(R, base)
        assert np.array_equal(plain, base ** (-2.0 * np.arange(R // 2) / R))
        y = O.rope_frequencies(R, O.Yarn(base, 1.0, 65536.0, 32.0, 1.0))
        assert np.array_equal(plain, y)


def test_yarn_correction_index_counts_turns():
    # at the real index c(n), theta = base^(-2c/R) makes n turns over the context
    for n in (1.0, 5.0, 32.0):
        for R, base, ctx in ((64, 10000.0, 65536.0), (64, 160000.0, 65536.0),
                             (128, 500000.0, 4096.0)):
            c = O.yarn_correction_index(n, R, base, ctx)
            theta = base ** (-2.0 * c / R)
            assert abs(ctx * theta / (2 * math.pi) - n) < 1e-9 * n


@pytest.mark.parametrize("base", [10000.0, 160000.0])
def test_yarn_frequencies_by_turn_count(base):
    R, s = 64, _YARN["factor"]
    plain = base ** (-2.0 * np.arange(R // 2) / R)
    y = O.rope_frequencies(R, O.Yarn(base, **_YARN))
    turns = _YARN["original_context"] * plain / (2 * math.pi)
    # exactly the pairs that turn at least beta_fast times keep their frequency
    assert np.array_equal(y == plain, turns >= _YARN["beta_fast"])
    ratio = y / plain
    assert np.all(np.diff(ratio) <= 1e-15) and ratio.min() >= 1 / s - 1e-15
    slowed = np.isclose(ratio, 1 / s, rtol=0, atol=1e-15)
    ramp = ~(turns >= _YARN["beta_fast"]) & ~slowed
    # on the ramp the ratio falls linearly in the pair index
    rj = np.nonzero(ramp)[0]
    assert len(rj) >= 3 and np.allclose(np.diff(ratio[rj], 2), 0.0, atol=1e-13)
    if base == 160000.0:
        # the ramp ends inside the 32 pairs: exactly those turning at most
        # beta_slow times (rounded to whole pair indices) run s times slower
        assert np.array_equal(slowed, turns <= _YARN["beta_slow"])
        assert slowed.sum() >= 2 and np.array_equal(y[slowed], plain[slowed] / s)
    else:
        assert not slowed.any()  # the ramp would end past the last pair


def test_yarn_slowed_pairs_at_s_times_the_position_turn_like_plain_rope():
    rng = np.random.default_rng(6)
    R, base, s = 64, 160000.0, _YARN["factor"]
    x = rng.standard_normal(R)
    y = O.rope_frequencies(R, O.Yarn(base, **_YARN))
    slowed = np.isclose(y, base ** (-2.0 * np.arange(R // 2) / R) / s, rtol=0, atol=1e-18)
    a = O.rope(x, 1000 * s, R, O.Yarn(base, **_YARN))
    b = O.rope(x, 1000, R, base)
    ch = np.repeat(slowed, 2)
    assert ch.sum() >= 4 and np.allclose(a[ch], b[ch], atol=1e-9)
    # the pairs that keep their frequency turn like plain rope at the same position
    kept = np.repeat(y == base ** (-2.0 * np.arange(R // 2) / R), 2)
    assert kept.sum() >= 4 and np.allclose(O.rope(x, 777, R, O.Yarn(base, **_YARN))[kept],
                                           O.rope(x, 777, R, base)[kept], atol=1e-12)


def test_yarn_layer_spec_selects_the_scaled_frequencies():
    L = LayerSpec(kind="csa", dtype="f64", rope_factor=16.0)
    assert isinstance(O.rope_base(L), O.Yarn) and O.rope_base(L).factor == 16.0
    assert O.rope_base(LayerSpec(kind="csa", dtype="f64")) == 160000.0


# ----------------------------------------------------------------------------
# compressor

def test_pool_equal_gates_is_mean_over_window_tokens():
    rng = np.random.default_rng(6)
    S, C, m = 32, 6, 4
    kv = rng.standard_normal((S, C))
    gate = np.zeros((S, C))
    for overlap in (0, 1):
        pool = O.compress(kv, gate, m, overlap, 0, 1e4, "f64")
        assert pool.shape == (S // m, C)
        for w in range(S // m):
            lo = max((w - overlap) * m, 0)
            assert np.allclose(pool[w], kv[lo:(w + 1) * m].mean(axis=0), atol=1e-14)
    # the first CSA entry has only m tokens (nothing before position 0)
    pool = O.compress(kv, gate, m, 1, 0, 1e4, "f64")
    assert np.allclose(pool[0], kv[:4].mean(axis=0))
    assert np.allclose(pool[1], kv[:8].mean(axis=0))


def test_pool_dominant_gate_selects_that_token_per_channel():
    rng = np.random.default_rng(7)
    S, C, m = 16, 5, 4
    kv = rng.standard_normal((S, C))
    gate = rng.standard_normal((S, C))
    # channel c of entry 2 (tokens 4..11) is dominated by token 4 + c
    for c in range(C):
        gate[4 + c, c] = 60.0
    pool = O.compress(kv, gate, m, 1, 0, 1e4, "f64")
    for c in range(C):
        assert abs(pool[2, c] - kv[4 + c, c]) < 1e-20 + 1e-12 * abs(kv[4 + c, c])


def test_pool_ratio_one_without_overlap_or_rope_is_identity():
    rng = np.random.default_rng(8)
    kv, gate = rng.standard_normal((9, 4)), rng.standard_normal((9, 4))
    assert np.allclose(O.compress(kv, gate, 1, 0, 0, 1e4, "f64"), kv, atol=1e-15)


def test_pool_rmsnorm_closed_form():
    kv = np.full((4, 6), -2.5)
    g = np.linspace(0.5, 1.5, 6)
    out = O.pool_entry(kv, np.zeros((4, 6)), 0, 0, 1e4, norm_weight=g, eps=1e-6)
    assert np.allclose(out, -g / math.sqrt(1 + 1e-6 / 6.25), atol=1e-14)


def test_pool_locality_of_overlapping_windows():
    rng = np.random.default_rng(9)
    S, m = 32, 4
    kv, gate = rng.standard_normal((S, 3)), rng.standard_normal((S, 3))
    base = O.compress(kv, gate, m, 1, 2, 1e4, "f64")
    for s in range(S):
        kv2 = kv.copy()
        kv2[s] += 1.0
        changed = np.nonzero(np.any(O.compress(kv2, gate, m, 1, 2, 1e4, "f64") != base, axis=1))[0]
        expect = [w for w in range(S // m) if (w - 1) * m <= s < (w + 1) * m]
        assert list(changed) == expect, s


def test_compress_matches_dense_membership_formulation():
    rng = np.random.default_rng(10)
    for m, ov in ((4, 1), (8, 0), (2, 1)):
        kv, gate = rng.standard_normal((40, 10)), rng.standard_normal((40, 10))
        a = O.compress(kv, gate, m, ov, 6, 300.0, "f64")
        b = brute.dense_compress(kv, gate, m, ov, 6, 300.0)
        assert np.allclose(a, b, atol=1e-13)


# ----------------------------------------------------------------------------
# indexer and top-k

def test_index_score_single_head_is_relu_of_key_channel():
    rng = np.random.default_rng(11)
    keys = rng.standard_normal((20, 8))
    q = np.zeros((3, 8))
    q[1, 0] = 1.0                       # channel 0 is not a rope channel (R=4)
    w = np.array([0.0, 1.0, 0.0])
    sc = O.index_scores(q, w, keys, 77, 4, 1e4, "f64")
    assert np.allclose(sc, np.maximum(keys[:, 0], 0.0), atol=1e-15)
    sc2 = O.index_scores(q, -2.0 * w, keys, 77, 4, 1e4, "f64")
    assert np.allclose(sc2, -2.0 * np.maximum(keys[:, 0], 0.0))


def test_index_scores_match_dense_formulation():
    L = small_layer()
    inp = rand_inputs(L, 40, seed=12)
    ik = O.compress(inp["ikv"], inp["igate"], 4, 1, L.index_rope_dim, L.rope_theta, "f64")
    dense = brute.dense_index_scores(inp["qi"], inp["wi"], ik, 4, L.index_rope_dim, L.rope_theta)
    for t in range(40):
        n = (t + 1) // 4
        sc = O.index_scores(inp["qi"][t], inp["wi"][t], ik[:n], t, L.index_rope_dim,
                            L.rope_theta, "f64")
        assert np.allclose(sc, dense[t, :n], atol=1e-12)
        assert np.all(np.isinf(dense[t, n:]))


def test_topk_matches_rank_counting_with_ties():
    rng = np.random.default_rng(13)
    for trial in range(60):
        n = int(rng.integers(0, 40))
        k = int(rng.integers(1, 12))
        if trial % 2:
            s = rng.integers(-3, 4, n).astype(np.float64)      # many exact ties
        else:
            s = rng.standard_normal(n)
        got = O.topk_select(s, k)
        assert np.array_equal(got, brute.rank_topk(s, k))
        v = got[got >= 0]
        assert np.all(np.diff(v) > 0) and np.all(got[len(v):] == -1)
        assert len(v) == min(n, k)


def test_topk_signed_zero_ties_break_by_index():
    s = np.array([0.0, -0.0, 0.0, -0.0, -1.0, 0.0])
    assert list(O.topk_select(s, 3)) == [0, 1, 2]
    s = np.array([-0.0, 0.0, 5.0])
    assert list(O.topk_select(s, 2)) == [0, 2]


def test_topk_offset_entries_keep_absolute_ids():
    s = np.array([1.0, 3.0, 2.0])
    assert list(O.topk_select(s, 2, first=10)) == [11, 12]
    assert list(O.topk_select(s, 5, first=10)) == [10, 11, 12, -1, -1]


# ----------------------------------------------------------------------------
# attention

def test_attend_first_token_closed_form():
    rng = np.random.default_rng(14)
    H, D = 4, 16
    q, kv = rng.standard_normal((H, D)), rng.standard_normal(D)
    sinks = rng.standard_normal(H)
    scale = 0.3
    out = O.attend(q, 0, kv[None], sinks, scale, 8, 1e4, "f64")
    l = scale * q @ kv
    expect = (1 / (1 + np.exp(sinks - l)))[:, None] * kv[None]
    assert np.allclose(out, expect, atol=1e-14)
    assert np.allclose(O.attend(q, 0, kv[None], None, scale, 8, 1e4, "f64"), kv[None], atol=1e-15)


def test_attend_zero_query_is_sink_damped_mean_then_unrotated():
    rng = np.random.default_rng(15)
    rows = rng.standard_normal((7, 16))
    sinks = np.array([0.0, 1.0, -2.0])
    t = 55
    out = O.attend(np.zeros((3, 16)), t, rows, sinks, 0.25, 8, 1e4, "f64")
    mean = rows.sum(axis=0)[None] / (7 + np.exp(sinks))[:, None]
    assert np.allclose(out, O.rope(mean, t, 8, 1e4, -1), atol=1e-14)
    # a sink far above every logit empties the output
    out = O.attend(rng.standard_normal((3, 16)), t, rows, np.full(3, 60.0), 0.25, 8, 1e4, "f64")
    assert np.max(np.abs(out)) < 1e-20


def test_attend_without_sink_matches_torch_sdpa_with_v_equal_k_copy():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(16)
    H, D, n, t = 5, 32, 11, 300
    q, rows = rng.standard_normal((H, D)), rng.standard_normal((n, D))
    ref = O.attend(q, t, rows, np.full(H, -np.inf), 0.2, 16, 1e4, "f64")
    ref2 = O.attend(q, t, rows, None, 0.2, 16, 1e4, "f64")
    qr = torch.from_numpy(O.rope(q, t, 16, 1e4, +1))[None, :, None, :]        # [1,H,1,D]
    k = torch.from_numpy(rows)[None, None].expand(1, H, n, D)
    v = k.clone()
    o = torch.nn.functional.scaled_dot_product_attention(qr, k, v, scale=0.2)[0, :, 0].numpy()
    o = O.rope(o, t, 16, 1e4, -1)
    assert np.allclose(ref, o, atol=1e-13) and np.allclose(ref2, o, atol=1e-13)


def test_attend_invariant_to_row_order():
    rng = np.random.default_rng(17)
    q, rows, sinks = rng.standard_normal((4, 16)), rng.standard_normal((9, 16)), rng.standard_normal(4)
    a = O.attend(q, 40, rows, sinks, 0.5, 8, 1e4, "f64")
    b = O.attend(q, 40, rows[rng.permutation(9)], sinks, 0.5, 8, 1e4, "f64")
    assert np.allclose(a, b, atol=1e-14)


# ----------------------------------------------------------------------------
# whole layer

def test_worked_mask_example_from_the_model_page():
    rows = []
    with open(os.path.join(HERE, "golden", "mask_example.txt")) as f:
        for line in f:
            if line.startswith("#") or line.startswith("t "):
                continue
            t, lo, hi, filled, hca = line.split()
            rows.append((int(t), int(lo), int(hi), int(filled), hca))
    assert len(rows) == 16
    csa = small_layer("csa", window=8, ratio=4, topk=2)
    inp = rand_inputs(csa, 16, seed=18)
    res = O.csa_prefill(csa, inp)
    for t, lo, hi, filled, hca in rows:
        wp = O.window_positions(t, 8)
        assert (wp.start, wp.stop - 1) == (lo, hi)
        assert int(np.sum(res["idx"][t] >= 0)) == filled
        vis = list(O.visible_entries(t, 8))
        assert vis == ([] if hca == "-" else [int(v) for v in hca.split(",")])


def _dense_csa_mask(idx, S, P):
    k = idx.shape[1]
    comp_cols = np.zeros((S, S * k), dtype=bool)
    for t in range(S):
        for j in range(k):
            comp_cols[t, t * k + j] = idx[t, j] >= 0
    return comp_cols


@pytest.mark.parametrize("sinks_on", [True, False])
def test_csa_layer_matches_dense_mask_formulation(sinks_on):
    L = small_layer("csa", window=8, ratio=4, topk=3)
    S = 36
    inp = rand_inputs(L, S, seed=19, q_scale=2.0)
    if not sinks_on:
        inp["sinks"] = None
    res = O.csa_prefill(L, inp, dtype="f64")
    # independent pieces: dense pooling, dense scores + rank selection, one big mask
    pool = brute.dense_compress(inp["ckv"], inp["cgate"], 4, 1, L.rope_dim, L.rope_theta)
    ik = brute.dense_compress(inp["ikv"], inp["igate"], 4, 1, L.index_rope_dim, L.rope_theta)
    sc = brute.dense_index_scores(inp["qi"], inp["wi"], ik, 4, L.index_rope_dim, L.rope_theta)
    idx = np.stack([brute.rank_topk(sc[t], L.topk) for t in range(S)])
    assert np.array_equal(idx, res["idx"])
    gathered = np.concatenate([pool[np.maximum(idx[t], 0)] for t in range(S)])
    o = brute.dense_attention(inp["q"], inp["kv"], gathered, _dense_csa_mask(idx, S, len(pool)),
                              8, inp["sinks"], 1 / math.sqrt(L.head_dim), L.rope_dim,
                              L.rope_theta)
    assert np.allclose(res["out"], o, atol=1e-12)


def test_hca_layer_matches_dense_mask_formulation():
    L = small_layer("hca", window=8, ratio=8)
    S = 40
    inp = rand_inputs(L, S, seed=20, q_scale=2.0)
    res = O.hca_prefill(L, inp, dtype="f64")
    pool = brute.dense_compress(inp["ckv"], inp["cgate"], 8, 0, L.rope_dim, L.rope_theta)
    t = np.arange(S)[:, None]
    mask = np.arange(len(pool))[None, :] < (t + 1) // 8
    o = brute.dense_attention(inp["q"], inp["kv"], pool, mask, 8, inp["sinks"],
                              1 / math.sqrt(L.head_dim), L.rope_dim, L.rope_theta)
    assert np.allclose(res["out"], o, atol=1e-12)


def test_sliding_layer_matches_dense_mask_formulation():
    L = small_layer("sliding", window=5)
    S = 17
    inp = rand_inputs(L, S, seed=21, q_scale=2.0)
    res = O.sliding_prefill(L, inp, dtype="f64")
    o = brute.dense_attention(inp["q"], inp["kv"], np.zeros((0, L.head_dim)),
                              np.zeros((S, 0), bool), 5, inp["sinks"], 1 / math.sqrt(L.head_dim),
                              L.rope_dim, L.rope_theta)
    assert np.allclose(res["out"], o, atol=1e-12)


def test_csa_with_topk_covering_every_entry_equals_dense_over_pool_and_window():
    L = small_layer("csa", window=6, ratio=4, topk=64)
    S = 48
    inp = rand_inputs(L, S, seed=22, q_scale=2.0)
    csa = O.csa_prefill(L, inp, dtype="f64")
    Lh = small_layer("hca", window=6, ratio=4, overlap=1)
    hca = O.hca_prefill(Lh, inp, dtype="f64")
    assert np.allclose(csa["out"], hca["out"], atol=1e-13)


@pytest.mark.parametrize("kind", ["csa", "hca"])
def test_position_shift_leaves_outputs_unchanged(kind):
    L = small_layer(kind, window=8)
    S = 32
    inp = rand_inputs(L, S, seed=23, q_scale=2.0)
    run = O.csa_prefill if kind == "csa" else O.hca_prefill
    a = run(L, inp, dtype="f64")
    b = run(L, inp, dtype="f64", p0=L.ratio * 1000)
    assert np.allclose(a["out"], b["out"], atol=1e-9)
    if kind == "csa":
        sel_a = a["idx"]
        sel_b = np.where(b["idx"] >= 0, b["idx"] - 1000, -1)
        assert np.array_equal(sel_a, sel_b)


@pytest.mark.parametrize("kind", ["csa", "hca", "sliding"])
def test_decode_step_equals_prefill_row(kind):
    L = small_layer(kind, window=8)
    S = 48
    inp = rand_inputs(L, S, seed=24, q_scale=2.0)
    run = {"csa": O.csa_prefill, "hca": O.hca_prefill, "sliding": O.sliding_prefill}[kind]
    for t in (S - 1, S - 2, S - 5, 31):
        full = run(L, {k: (v[:t + 1] if k != "sinks" else v) for k, v in inp.items()}, dtype="f64")
        cap = L.window
        win = np.zeros((cap, L.head_dim))
        for s in range(max(0, t - cap), t):
            win[s % cap] = full["win"][s]
        cache = {"win": win}
        new = {k: (v[t] if k != "sinks" else v) for k, v in inp.items()}
        if L.ratio > 0:
            m, Ls = L.ratio, (1 + L.overlap) * L.ratio
            P = t // m
            cache["pool"] = full["pool"][:P]
            for pre, kk, gk in (("c", "ckv", "cgate"), ("i", "ikv", "igate")):
                st_kv, st_g = np.zeros((Ls, inp[kk].shape[1])), np.zeros((Ls, inp[kk].shape[1]))
                for s in range(max(0, t - Ls), t):
                    st_kv[s % Ls], st_g[s % Ls] = inp[kk][s], inp[gk][s]
                cache[pre + "state_kv"], cache[pre + "state_gate"] = st_kv, st_g
            if L.has_indexer:
                cache["ipool"] = full["ipool"][:P]
        res = O.decode_step(L, t, new, cache, dtype="f64")
        assert np.allclose(res["out"], full["out"][t], atol=1e-13)
        if L.has_indexer:
            assert np.array_equal(res["idx"], full["idx"][t])
        if L.ratio > 0 and (t + 1) % L.ratio == 0:
            assert np.allclose(res["new_pool"], full["pool"][(t + 1) // L.ratio - 1], atol=1e-15)


# ----------------------------------------------------------------------------
# paged pools

def test_paged_rows_is_a_bijection_onto_the_sequences_blocks():
    E, table = 4, np.array([5, 0, 3])
    rows = O.paged_rows(np.arange(12), table, E)
    assert list(rows[:4]) == [20, 21, 22, 23] and list(rows[4:8]) == [0, 1, 2, 3]
    assert sorted(rows) == sorted(set(rows))                 # no two entries share a row
    assert set(rows // E) == set(table)                        # exactly the table's blocks
    assert np.array_equal(rows % E, np.arange(12) % E)         # offsets within a block kept
    # two sequences with disjoint tables never share a row
    other = O.paged_rows(np.arange(12), np.array([1, 2, 4]), E)
    assert not set(rows) & set(other)


@pytest.mark.parametrize("kind", ["csa", "hca"])
def test_decode_step_on_paged_pools_equals_contiguous(kind):
    """A decode step reading its pools through a shuffled block table gives the
    contiguous result exactly (ids, output, the entry that closes)."""
    L = small_layer(kind, window=8)
    S = 63 if kind == "csa" else 47          # an entry closes at t = S (csa: 64 % 4, hca: 48 % 8)
    inp = rand_inputs(L, S + 1, seed=31, q_scale=2.0)
    full = {"csa": O.csa_prefill, "hca": O.hca_prefill}[kind](
        L, {k: (v[:S] if k != "sinks" else v) for k, v in inp.items()}, dtype="f64")
    t = S
    m, Ls = L.ratio, (1 + L.overlap) * L.ratio
    P = t // m
    win = np.zeros((L.window, L.head_dim))
    for s_ in range(t - L.window, t):
        win[s_ % L.window] = full["win"][s_]
    cache = {"win": win}
    for pre, kk, gk in (("c", "ckv", "cgate"), ("i", "ikv", "igate")):
        st_kv, st_g = np.zeros((Ls, inp[kk].shape[1])), np.zeros((Ls, inp[kk].shape[1]))
        for s_ in range(t - Ls, t):
            st_kv[s_ % Ls], st_g[s_ % Ls] = inp[kk][s_], inp[gk][s_]
        cache[pre + "state_kv"], cache[pre + "state_gate"] = st_kv, st_g
    new = {k: (v[t] if k != "sinks" else v) for k, v in inp.items()}
    E = 4
    nblk = (P + E - 1) // E
    rng = np.random.default_rng(5)
    table = rng.permutation(3 * nblk)[:nblk]                  # shuffled, sparse blocks
    cont = dict(cache, pool=full["pool"][:P])
    paged = dict(cache, pool=O.PagedPool(O.page_pool(full["pool"][:P], table, E, 3 * nblk),
                                         table, E, P))
    if L.has_indexer:
        cont["ipool"] = full["ipool"][:P]
        paged["ipool"] = O.PagedPool(O.page_pool(full["ipool"][:P], table, E, 3 * nblk),
                                     table, E, P)
    a = O.decode_step(L, t, new, cont, dtype="f64")
    b = O.decode_step(L, t, new, paged, dtype="f64")
    assert np.array_equal(a["out"], b["out"])
    assert np.array_equal(a["new_pool"], b["new_pool"])
    if L.has_indexer:
        assert np.array_equal(a["idx"], b["idx"])
    # a wrong table (the block of an attended entry pointing at an unused
    # block) reads other rows and changes the result
    if nblk > 0:
        bad = table.copy()
        j0 = int(a["idx"][0]) // E if L.has_indexer else 0
        bad[j0] = [j for j in range(3 * nblk) if j not in set(table)][0]
        c = dict(paged, pool=O.PagedPool(paged["pool"].rows, bad, E, P))
        if L.has_indexer:
            c["ipool"] = O.PagedPool(paged["ipool"].rows, bad, E, P)
        assert not np.array_equal(O.decode_step(L, t, new, c, dtype="f64")["out"], a["out"])


# ----------------------------------------------------------------------------
# grouped output projection

def _oproj_inputs(T, H, D, G, R, hidden, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H, D))
    wa = rng.standard_normal((G * R, (H // G) * D))
    wb = rng.standard_normal((hidden, G * R))
    return x, wa, wb


def test_output_projection_matches_loops_on_tiny_sizes():
    T, H, D, G, R, hidden = 3, 4, 2, 2, 3, 5
    x, wa, wb = _oproj_inputs(T, H, D, G, R, hidden, 11)
    out = O.output_projection(x, wa, wb, G, "f64")
    ref = np.zeros((T, hidden))
    hp = H // G
    for t in range(T):
        y = np.zeros(G * R)
        for g in range(G):
            for r in range(R):
                for hh in range(hp):
                    for d in range(D):
                        y[g * R + r] += x[t, g * hp + hh, d] * wa[g * R + r, hh * D + d]
        for o in range(hidden):
            ref[t, o] = sum(y[j] * wb[o, j] for j in range(G * R))
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_output_projection_equals_dense_block_diagonal_product():
    T, H, D, G, R, hidden = 7, 8, 4, 4, 5, 6
    x, wa, wb = _oproj_inputs(T, H, D, G, R, hidden, 12)
    ig = (H // G) * D
    full = np.zeros((G * R, H * D))
    for g in range(G):
        full[g * R:(g + 1) * R, g * ig:(g + 1) * ig] = wa[g * R:(g + 1) * R]
    dense = (x.reshape(T, H * D) @ full.T) @ wb.T
    assert np.allclose(O.output_projection(x, wa, wb, G, "f64"), dense, rtol=1e-12, atol=1e-12)
    # one group is two plain products
    assert np.allclose(O.output_projection(x, full, wb, 1, "f64"), dense, rtol=1e-12, atol=1e-12)


def test_output_projection_group_locality_and_stored_intermediate():
    T, H, D, G, R, hidden = 4, 6, 3, 3, 2, 5
    x, wa, wb = _oproj_inputs(T, H, D, G, R, hidden, 13)
    g = 1
    wb_g = np.zeros_like(wb)
    wb_g[:, g * R:(g + 1) * R] = wb[:, g * R:(g + 1) * R]
    x2 = x.copy()
    hp = H // G
    x2[:, :g * hp] += 1.0
    x2[:, (g + 1) * hp:] -= 2.0
    # only group g's heads reach the output through group g's block of w_b
    assert np.allclose(O.output_projection(x, wa, wb_g, G, "f64"),
                       O.output_projection(x2, wa, wb_g, G, "f64"), atol=1e-12)
    assert not np.allclose(O.output_projection(x, wa, wb, G, "f64"),
                           O.output_projection(x2, wa, wb, G, "f64"))
    # the intermediate is stored at the dtype: rounding it first is the same result
    xb = O.round_to(x, "bf16")
    out = O.output_projection(xb, wa, wb, G, "bf16")
    y = O.round_to(np.einsum("tgi,gri->tgr", xb.reshape(T, G, hp * D), wa.reshape(G, R, hp * D)),
                   "bf16")
    assert np.array_equal(out, O.round_to(y.reshape(T, G * R) @ wb.T, "bf16"))



# ----------------------------------------------------------------------------
# producer projections

def _proj_case(seed, T=3, hidden=6, sz=None):
    sz = sz or O.ProjSizes(q_lora=4, heads=2, head_dim=3, comp=2, index_dim=2, index_heads=2)
    rng = np.random.default_rng(seed)
    nx = sz.q_lora + sz.head_dim + 2 * sz.comp + 2 * sz.index_dim + sz.index_heads
    nq = sz.heads * sz.head_dim + sz.index_heads * sz.index_dim
    return (sz, rng.standard_normal((T, hidden)), rng.standard_normal((nx, hidden)),
            rng.uniform(0.5, 1.5, sz.q_lora), rng.uniform(0.5, 1.5, sz.head_dim),
            rng.standard_normal((nq, sz.q_lora)))


def test_project_inputs_matches_loops_on_tiny_sizes():
    sz, x, wx, gqa, gkv, wq = _proj_case(21)
    eps = 1e-6
    out = O.project_inputs(x, wx, gqa, gkv, wq, sz, eps, True, "f64")
    T, hidden = x.shape

    def dot_rows(a, w, r0, n):
        return [[sum(a[t][i] * w[r0 + o][i] for i in range(len(a[t]))) for o in range(n)]
                for t in range(len(a))]

    def rms(v, g):
        r = (sum(e * e for e in v) / len(v) + eps) ** 0.5
        return [v[i] / r * (1.0 if g is None else g[i]) for i in range(len(v))]

    xl = x.tolist()
    qa = dot_rows(xl, wx, 0, sz.q_lora)
    lat = [rms(r, gqa) for r in qa]
    kv = [rms(r, gkv) for r in dot_rows(xl, wx, sz.q_lora, sz.head_dim)]
    off = sz.q_lora + sz.head_dim
    ckv = dot_rows(xl, wx, off, sz.comp)
    cg = dot_rows(xl, wx, off + sz.comp, sz.comp)
    ikv = dot_rows(xl, wx, off + 2 * sz.comp, sz.index_dim)
    ig = dot_rows(xl, wx, off + 2 * sz.comp + sz.index_dim, sz.index_dim)
    wi = dot_rows(xl, wx, off + 2 * sz.comp + 2 * sz.index_dim, sz.index_heads)
    qfull = dot_rows(lat, wq, 0, sz.heads * sz.head_dim)
    q = [[rms(r[h * sz.head_dim:(h + 1) * sz.head_dim], None) for h in range(sz.heads)]
         for r in qfull]
    qi = dot_rows(lat, wq, sz.heads * sz.head_dim, sz.index_heads * sz.index_dim)
    for name, ref in [("latent", lat), ("kv", kv), ("ckv", ckv), ("cgate", cg), ("ikv", ikv),
                      ("igate", ig), ("wi", wi), ("q", q)]:
        assert np.allclose(out[name], np.array(ref), rtol=1e-12, atol=1e-12), name
    assert np.allclose(out["qi"], np.array(qi).reshape(T, sz.index_heads, sz.index_dim),
                       rtol=1e-12, atol=1e-12)


def test_project_inputs_norm_properties():
    sz, x, wx, gqa, gkv, wq = _proj_case(22, T=5, hidden=8,
                                         sz=O.ProjSizes(6, 3, 4, 2, 2, 3))
    ones = np.ones
    out = O.project_inputs(x, wx, ones(sz.q_lora), ones(sz.head_dim), wq, sz, 0.0, True, "f64")
    # unit-weight RMSNorm rows and per-head q rows have unit RMS
    for name in ("latent", "kv"):
        assert np.allclose(np.sqrt(np.mean(out[name] ** 2, axis=-1)), 1.0, rtol=1e-12)
    assert np.allclose(np.sqrt(np.mean(out["q"] ** 2, axis=-1)), 1.0, rtol=1e-12)
    # scaling x: the normalised streams do not move, the plain ones scale with it
    out3 = O.project_inputs(3.0 * x, wx, ones(sz.q_lora), ones(sz.head_dim), wq, sz, 0.0, True,
                            "f64")
    for name in ("latent", "kv", "q", "qi"):
        assert np.allclose(out3[name], out[name], rtol=1e-11, atol=1e-12), name
    for name in ("ckv", "cgate", "ikv", "igate", "wi"):
        assert np.allclose(out3[name], 3.0 * out[name], rtol=1e-12), name
    # without q_b_norm q is the plain product of the latent
    raw = O.project_inputs(x, wx, ones(sz.q_lora), ones(sz.head_dim), wq, sz, 0.0, False, "f64")
    hd = sz.heads * sz.head_dim
    assert np.allclose(raw["q"].reshape(x.shape[0], hd), raw["latent"] @ wq[:hd].T, rtol=1e-12)


def test_project_inputs_streams_are_separate_rows_of_the_stacked_weight():
    sz, x, wx, gqa, gkv, wq = _proj_case(23)
    base = O.project_inputs(x, wx, gqa, gkv, wq, sz, 1e-6, True, "f64")
    off = sz.q_lora + sz.head_dim + sz.comp  # the compressor gate rows
    wx2 = wx.copy()
    wx2[off:off + sz.comp] *= -2.0
    moved = O.project_inputs(x, wx2, gqa, gkv, wq, sz, 1e-6, True, "f64")
    for name in base:
        if name == "cgate":
            assert np.allclose(moved[name], -2.0 * base[name], rtol=1e-12)
        else:
            assert np.array_equal(moved[name], base[name]), name
    # no indexer and no compressor: those outputs are empty, the rest unchanged
    sz0 = O.ProjSizes(sz.q_lora, sz.heads, sz.head_dim, 0, 0, 0)
    keep = np.r_[0:sz.q_lora + sz.head_dim]
    out0 = O.project_inputs(x, wx[keep], gqa, gkv, wq[:sz.heads * sz.head_dim], sz0, 1e-6, True,
                            "f64")
    for name in ("latent", "kv", "q"):
        assert np.array_equal(out0[name], base[name]), name
    assert out0["ckv"].shape == (x.shape[0], 0) and out0["qi"].shape == (x.shape[0], 0, 0)


def test_project_inputs_stored_points_at_bf16():
    sz, x, wx, gqa, gkv, wq = _proj_case(24, T=6, hidden=16, sz=O.ProjSizes(16, 2, 8, 4, 4, 2))
    xb = O.round_to(x, "bf16")
    out = O.project_inputs(xb, wx, gqa, gkv, wq, sz, 1e-6, False, "bf16")
    # q reads the stored latent; the latent reads the stored projection
    hd = sz.heads * sz.head_dim
    assert np.array_equal(out["q"].reshape(x.shape[0], hd),
                          O.round_to(out["latent"] @ wq[:hd].T, "bf16"))
    y = O.round_to(xb @ wx[:sz.q_lora].T, "bf16")
    lat = O.round_to(y / np.sqrt(np.mean(y * y, axis=-1, keepdims=True) + 1e-6) * gqa, "bf16")
    assert np.array_equal(out["latent"], lat)
    for name in ("latent", "kv", "ckv", "q", "qi"):
        assert np.array_equal(out[name], O.round_to(out[name], "bf16")), name
