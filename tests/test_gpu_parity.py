"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Every case prints its name before touching the GPU.  Sizes here let the
oracle finish in seconds while spanning several tiles with ragged tails;
the full-size workloads are in test_gpu_fullsize.py.
"""
import numpy as np
import pytest

import synth
from oracle import csa_oracle as O
from synth import to_f64
from tests.helpers import (assert_close, audit_topk, dev, host, index_exact, say, seq_f64,
                           ulp_diff_ok)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def csa():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import long_context_sparse_gated_amd as m
    m.load_library()
    return m


def _prefill_gpu(m, spec, inp, B, S):
    import torch
    from long_context_sparse_gated_amd.layer import LayerCache, layer_step
    L = m.Layer.from_spec(spec)
    pool_cap = max(1, S // spec.ratio) if spec.ratio else 0
    cache = LayerCache(L, B, S, pool_cap)
    pos0 = torch.zeros(B, dtype=torch.int64, device="cuda")
    args = {k: dev(v) for k, v in inp.items() if k != "sinks"}
    sinks = None if inp["sinks"] is None else dev(inp["sinks"])
    out, idx = layer_step(cache, pos0, 0, args["q"], args["kv"], args.get("ckv"), args.get("cgate"),
                          args.get("ikv"), args.get("igate"), args.get("qi"), args.get("wi"), sinks)
    torch.cuda.synchronize()
    return L, cache, pos0, args, sinks, out, idx


def _check_csa_prefill(m, spec, w, seed, queries_per_seq=None, sinks=True):
    import torch
    inp = synth.prefill_inputs(w, seed)
    if not sinks:
        inp["sinks"] = None
    B, S = w.batch, w.n_new
    L, cache, pos0, args, sinks, out, idx = _prefill_gpu(m, spec, inp, B, S)
    gidx = idx.cpu().numpy()
    ndiff = 0
    for b in range(B):
        x = seq_f64(inp, b)
        qs = list(range(S)) if queries_per_seq is None else queries_per_seq
        ref = O.csa_prefill(spec, x, queries=qs)
        ulp_diff_ok(host(cache.pool[b]), ref["pool"], spec.dtype, "pool")
        ulp_diff_ok(host(cache.ipool[b]), ref["ipool"], spec.dtype, "ipool")
        ulp_diff_ok(host(cache.ring[b]), ref["win"], spec.dtype, "window rows")
        for n, t in enumerate(qs):
            nv = (t + 1) // spec.ratio
            keys = ref["ipool"][:nv]
            sc, ab = index_exact(spec, x["qi"][t], x["wi"][t], keys, t)
            ndiff += audit_topk(gidx[b, t], ref["idx"][n], sc, ab, spec.index_dim,
                                spec.index_heads)
        go = host(out[b])[qs]
        same = [n for n, t in enumerate(qs) if np.array_equal(gidx[b, t], ref["idx"][n])]
        assert_close(go[same], ref["out"][same], spec.dtype, "attention output (same ids)")
        # attention with the oracle's ids on both sides
        if len(same) < len(qs):
            idx2 = idx.clone()
            idx2[b, qs] = torch.from_numpy(ref["idx"].astype(np.int32)).cuda()
            out2 = torch.empty_like(out)
            m.csa_attend(L, pos0, 0, args["q"], cache.ring, cache.pool, idx2, sinks, out2,
                         cache.workspace(S, m.CSA_OP_ATTEND))
            torch.cuda.synchronize()
            assert_close(host(out2[b])[qs], ref["out"], spec.dtype, "attention output (oracle ids)")
    say(f"  near-tie id differences: {ndiff}")
    return ndiff


def test_tiny_csa_layer_f32(csa):
    say("case: tiny_csa f32 S=256 (generic kernels)")
    w = synth.workload("tiny_csa")
    for seed in (0, 1):
        _check_csa_prefill(csa, w.layers[0], w, seed)


def test_csa_layer_f32_medium(csa):
    # float32 through the generic kernels beyond the tiny shape: 16 heads x 128
    # (rope 32), window 64, indexer 8 x 64 (rope 32), top-32, S = 400 (no tile
    # divides it), a sample of queries
    import dataclasses
    say("case: csa f32 H=16 D=128 W=64 S=400 (generic kernels)")
    w = synth.workload("tiny_csa", S=400)
    spec = dataclasses.replace(w.layers[0], num_heads=16, head_dim=128, rope_dim=32, window=64,
                               index_heads=8, index_dim=64, index_rope_dim=32, topk=32)
    w = dataclasses.replace(w, layers=[spec])
    _check_csa_prefill(csa, spec, w, 4, queries_per_seq=[0, 3, 63, 64, 200, 255, 256, 399])


def test_tiny_csa_layer_f32_peaked(csa):
    say("case: tiny_csa f32 peaked")
    w = synth.workload("tiny_csa", variant="peaked")
    _check_csa_prefill(csa, w.layers[0], w, 2)


def test_tiny_csa_layer_f32_yarn(csa):
    say("case: tiny_csa f32 with YaRN (factor 16 over a 64-token original context)")
    import dataclasses
    w = synth.workload("tiny_csa")
    spec = dataclasses.replace(w.layers[0], rope_factor=16.0, rope_original_context=64.0)
    w = dataclasses.replace(w, layers=[spec])
    _check_csa_prefill(csa, spec, w, 3)


def test_csa_prefill_bf16_plain_rope(csa):
    say("case: csa_prefill bf16 S=700 without YaRN")
    import dataclasses
    w = synth.workload("csa_prefill", S=700)
    spec = dataclasses.replace(w.layers[0], rope_factor=0.0, topk=64)
    w = dataclasses.replace(w, layers=[spec])
    _check_csa_prefill(csa, spec, w, 6, queries_per_seq=[0, 3, 64, 300, 699])


def test_csa_prefill_bf16_small_topk(csa):
    say("case: csa_prefill bf16 S=1000 k=64 B=2 (mfma kernels)")
    import dataclasses
    w = synth.workload("csa_prefill", S=1000, batch=2)
    spec = dataclasses.replace(w.layers[0], topk=64)
    w = dataclasses.replace(w, layers=[spec])
    _check_csa_prefill(csa, spec, w, 0, queries_per_seq=[0, 1, 2, 3, 4, 7, 100, 255, 256, 257,
                                                        500, 777, 998, 999])


def test_csa_prefill_bf16_rope_width_32(csa):
    """A CSA layer with 32 rope channels (attention and indexer): the indexer
    runs its kernel for rope widths other than 64, the attention its R=32
    instance."""
    say("case: csa_prefill bf16 S=1000 k=64 B=2, rope width 32")
    import dataclasses
    w = synth.workload("csa_prefill", S=1000, batch=2)
    spec = dataclasses.replace(w.layers[0], topk=64, rope_dim=32, index_rope_dim=32)
    w = dataclasses.replace(w, layers=[spec])
    _check_csa_prefill(csa, spec, w, 5, queries_per_seq=[0, 3, 4, 63, 64, 255, 256, 511, 700, 999])


@pytest.mark.parametrize("name,S,pos0", [("csa_prefill", 600, 0), ("csa_prefill", 301, 1000),
                                         ("hca_prefill", 700, 0), ("tiny_csa", 200, 37)])
def test_compress_with_rmsnorm(csa, name, S, pos0):
    """The compressor's optional RMSNorm (both streams of a CSA layer, HCA, float32) against
    the oracle, also from a nonzero position with the state ring carrying earlier tokens."""
    import torch
    say(f"case: compress with RMSNorm {name} S={S} pos0={pos0}")
    m = csa
    w = synth.workload(name, S=S + pos0)
    spec = w.layers[0]
    inp = synth.prefill_inputs(w, 9)
    x = seq_f64(inp, 0)
    L = m.Layer.from_spec(spec)
    rng = np.random.default_rng(10)
    streams = [("ckv", "cgate", spec.head_dim, spec.rope_dim)]
    if spec.kind == "csa":
        streams.append(("ikv", "igate", spec.index_dim, spec.index_rope_dim))
    for kk, gk, width, rd in streams:
        nw = (1.0 + 0.25 * rng.standard_normal(width)).astype(np.float32)
        cap = (S + pos0) // spec.ratio
        Ls = (1 + spec.overlap) * spec.ratio
        tdt = torch.bfloat16 if spec.dtype == "bf16" else torch.float32
        st_kv = torch.zeros(1, Ls, width, dtype=tdt, device="cuda")
        st_g = torch.zeros(1, Ls, width, dtype=tdt, device="cuda")
        pool = torch.zeros(1, cap, width, dtype=tdt, device="cuda")
        kv_all, g_all = dev(inp[kk][:1]), dev(inp[gk][:1])
        nwd = torch.from_numpy(nw).cuda()
        # the earlier tokens (if any) in one call, then the S new ones
        for a, n in ((0, pos0), (pos0, S)):
            if n == 0:
                continue
            p0 = torch.full((1,), a, dtype=torch.int64, device="cuda")
            m.csa_compress(L, p0, a, kv_all[:, a:a + n].contiguous(), g_all[:, a:a + n].contiguous(),
                           st_kv, st_g, pool, rd, norm_weight=nwd, norm_eps=1e-6)
        torch.cuda.synchronize()
        ref = O.compress(x[kk], x[gk], spec.ratio, spec.overlap, rd, O.rope_base(spec),
                         spec.dtype, nw.astype(np.float64), 1e-6, 0)
        ulp_diff_ok(host(pool[0]), ref, spec.dtype, f"{kk} pool with RMSNorm")


def test_csa_prefill_bf16_k512(csa):
    say("case: csa_prefill bf16 S=2600 k=512 (mfma kernels)")
    w = synth.workload("csa_prefill", S=2600)
    _check_csa_prefill(csa, w.layers[0], w, 3,
                       queries_per_seq=[0, 3, 127, 128, 2046, 2047, 2048, 2100, 2555, 2598, 2599])


def test_csa_prefill_bf16_peaked(csa):
    say("case: csa_prefill bf16 peaked S=2200")
    w = synth.workload("csa_prefill", S=2200, variant="peaked")
    _check_csa_prefill(csa, w.layers[0], w, 4, queries_per_seq=[5, 600, 2047, 2100, 2199])


def _check_dense_prefill(m, kind, S, seed, queries, variant="plain", sinks=True):
    import torch
    name = "hca_prefill"
    w = synth.workload(name, S=S, variant=variant)
    spec = w.layers[0]
    if kind == "sliding":
        import dataclasses
        spec = synth.LayerSpec(kind="sliding", dtype="bf16", ratio=0, overlap=0, rope_theta=10000.0,
                               rope_factor=16.0, rope_original_context=65536.0)
        w = dataclasses.replace(w, layers=[spec])
    inp = synth.prefill_inputs(w, seed)
    if not sinks:
        inp["sinks"] = None
    L, cache, pos0, args, sk, out, _ = _prefill_gpu(m, spec, inp, w.batch, S)
    x = seq_f64(inp, 0)
    if kind == "sliding":
        ref = O.sliding_prefill(spec, x, queries=queries)
    else:
        ref = O.hca_prefill(spec, x, queries=queries)
        ulp_diff_ok(host(cache.pool[0]), ref["pool"], "bf16", "pool")
    ulp_diff_ok(host(cache.ring[0]), ref["win"], "bf16", "window rows")
    err = assert_close(host(out[0])[queries], ref["out"], "bf16", f"{kind} output")
    say(f"  max abs err {err:.3e}")


def test_hca_prefill_bf16(csa):
    say("case: hca_prefill bf16 S=4200")
    _check_dense_prefill(csa, "hca", 4200, 0, [0, 1, 126, 127, 128, 255, 1000, 4095, 4096, 4199])


def test_hca_prefill_bf16_peaked(csa):
    say("case: hca_prefill bf16 peaked S=3000")
    _check_dense_prefill(csa, "hca", 3000, 1, [0, 127, 1500, 2999], variant="peaked")


def test_csa_prefill_without_sinks(csa):
    """No sink through the prefill attention kernel (one block per query, no
    split): plain softmax over window and selected rows."""
    say("case: csa_prefill bf16 S=1000 k=64 sinks=None")
    import dataclasses
    w = synth.workload("csa_prefill", S=1000)
    spec = dataclasses.replace(w.layers[0], topk=64)
    w = dataclasses.replace(w, layers=[spec])
    _check_csa_prefill(csa, spec, w, 15, queries_per_seq=[0, 1, 5, 127, 128, 600, 999],
                       sinks=False)


def test_hca_prefill_without_sinks(csa):
    say("case: hca_prefill bf16 S=1500 sinks=None")
    _check_dense_prefill(csa, "hca", 1500, 16, [0, 127, 128, 700, 1499], sinks=False)


def test_sliding_prefill_bf16(csa):
    say("case: sliding prefill bf16 S=700")
    _check_dense_prefill(csa, "sliding", 700, 2, [0, 1, 64, 127, 128, 129, 699])


def _decode_case(m, name, pos0, batch, seed, layers=None, valid=None, variant="plain",
                 sinks=True):
    """One decode step at pos0 for every sequence and layer, against the oracle.
    sinks=False runs the layer without a sink (the oracle with none)."""
    import torch
    from long_context_sparse_gated_amd.layer import LayerCache, layer_step
    w = synth.workload(name, pos0=pos0, batch=batch, variant=variant)
    for li, spec in enumerate(w.layers):
        if layers is not None and li not in layers:
            continue
        say(f"  layer {li} {spec.kind}")
        inp = synth.decode_inputs(w, seed, li)
        L = m.Layer.from_spec(spec)
        pool_cap = (pos0 + 1) // spec.ratio if spec.ratio else 0
        cache = LayerCache(L, batch, spec.window, max(pool_cap, 1))
        cache.ring.copy_(dev(inp["win"]))
        if spec.ratio:
            P = pos0 // spec.ratio
            cache.pool[:, :P].copy_(dev(inp["pool"]))
            cache.cstate_kv.copy_(dev(inp["cstate_kv"]))
            cache.cstate_gate.copy_(dev(inp["cstate_gate"]))
            if spec.has_indexer:
                cache.ipool[:, :P].copy_(dev(inp["ipool"]))
                cache.istate_kv.copy_(dev(inp["istate_kv"]))
                cache.istate_gate.copy_(dev(inp["istate_gate"]))
        p0 = torch.full((batch,), pos0, dtype=torch.int64, device="cuda")
        a = {k: dev(inp[k]) for k in ("q", "kv", "ckv", "cgate", "ikv", "igate", "qi", "wi")
             if k in inp}
        nvd = None if valid is None else torch.tensor(valid, dtype=torch.int32, device="cuda")
        sk = dev(inp["sinks"]) if sinks else None
        out, idx = layer_step(cache, p0, pos0, a["q"], a["kv"], a.get("ckv"), a.get("cgate"),
                              a.get("ikv"), a.get("igate"), a.get("qi"), a.get("wi"),
                              sk, n_valid=nvd)
        torch.cuda.synchronize()
        for b in range(batch):
            if valid is not None and valid[b] == 0:
                # a padding token: every cache of the sequence is as it was
                assert torch.equal(cache.ring[b], dev(inp["win"])[b]), f"seq {b}: ring"
                if spec.ratio:
                    P = pos0 // spec.ratio
                    assert torch.equal(cache.pool[b, :P], dev(inp["pool"])[b]), f"seq {b}: pool"
                    assert not cache.pool[b, P:].any(), f"seq {b}: no new entry"
                    assert torch.equal(cache.cstate_kv[b], dev(inp["cstate_kv"])[b])
                    if spec.has_indexer:
                        assert torch.equal(cache.istate_gate[b], dev(inp["istate_gate"])[b])
                        assert not cache.ipool[b, P:].any(), f"seq {b}: no new key"
                continue
            new = {k: (to_f64(inp[k]) if k == "sinks" else to_f64(inp[k][b, 0]))
                   for k in ("q", "kv", "ckv", "cgate", "ikv", "igate", "qi", "wi", "sinks")
                   if k in inp}
            if not sinks:
                new["sinks"] = None
            cch = {k: to_f64(inp[k][b]) for k in ("win", "pool", "ipool", "cstate_kv",
                                                  "cstate_gate", "istate_kv", "istate_gate")
                   if k in inp}
            ref = O.decode_step(spec, pos0, new, cch)
            if "new_pool" in ref:
                w_new = (pos0 + 1) // spec.ratio - 1
                ulp_diff_ok(host(cache.pool[b, w_new]), ref["new_pool"], "bf16", "new entry")
            if spec.has_indexer:
                nv = (pos0 + 1) // spec.ratio
                keys = to_f64(inp["ipool"][b])
                if "new_ipool" in ref:
                    keys = np.concatenate([keys, ref["new_ipool"][None]])
                keys = keys[:nv]
                sc, ab = index_exact(spec, new["qi"], new["wi"], keys, pos0)
                gi = idx[b, 0].cpu().numpy()
                nd = audit_topk(gi, ref["idx"], sc, ab, spec.index_dim, spec.index_heads)
                if nd:
                    say(f"  seq {b}: {nd} near-tie id differences; re-attend with oracle ids")
                    idx2 = idx.clone()
                    idx2[b, 0] = torch.from_numpy(ref["idx"].astype(np.int32)).cuda()
                    m.csa_attend(L, p0, pos0, a["q"], cache.ring, cache.pool, idx2,
                                 sk, out, cache.workspace(1, m.CSA_OP_ATTEND))
                    torch.cuda.synchronize()
            assert_close(host(out[b, 0]), ref["out"], "bf16", f"decode out seq {b}")


def test_csa_decode_small(csa):
    say("case: csa decode B=3 pos0=5000")
    _decode_case(csa, "csa_decode", 5000, 3, 0)


def test_csa_decode_entry_closes(csa):
    say("case: csa decode B=2 pos0=4099 (entry closes at t)")
    _decode_case(csa, "csa_decode", 4099, 2, 1)


def test_varlen_decode_step_skips_padding(csa):
    """A one-token call where some sequences have no token: their caches stay
    as they were, the others match the oracle (an entry closes at 4099)."""
    say("case: varlen decode csa_decode pos0=4099 B=4 valid (1, 0, 1, 0)")
    _decode_case(csa, "csa_decode", 4099, 4, 7, valid=(1, 0, 1, 0))


def test_csa_decode_b20_head_group_path(csa):
    say("case: csa decode B=20 pos0=3001 (row slices x head groups, merged)")
    _decode_case(csa, "csa_decode", 3001, 20, 5)


def test_hca_decode_b16(csa):
    say("case: mixed decode B=16 pos0=40000, HCA layer only (row slices x head groups)")
    _decode_case(csa, "mixed_decode", 40000, 16, 6, layers=[1])


def test_mixed_decode_small(csa):
    say("case: mixed decode B=2 pos0=40959 (HCA entry closes) three layers")
    _decode_case(csa, "mixed_decode", 40959, 2, 2)


def test_mixed_decode_long_topk_path(csa):
    say("case: mixed decode B=2 pos0=70001, CSA layer only (1024-thread top-k)")
    _decode_case(csa, "mixed_decode", 70001, 2, 3, layers=[0])


def test_csa_decode_peaked(csa):
    say("case: csa decode peaked B=3 pos0=6001 (split rows, merged)")
    _decode_case(csa, "csa_decode", 6001, 3, 8, variant="peaked")


def test_csa_decode_peaked_b20(csa):
    say("case: csa decode peaked B=20 pos0=3003 (row slices x head groups)")
    _decode_case(csa, "csa_decode", 3003, 20, 9, variant="peaked")


def test_mixed_decode_peaked(csa):
    say("case: mixed decode peaked B=2 pos0=40959 three layers")
    _decode_case(csa, "mixed_decode", 40959, 2, 10, variant="peaked")


def test_decode_without_sinks_split_rows(csa):
    """No sink: the split partials of a few tokens with long row lists
    (attend_mfma with row splits, then the merge) against plain softmax."""
    say("case: csa decode B=3 pos0=5000 sinks=None (split rows, merged)")
    _decode_case(csa, "csa_decode", 5000, 3, 11, sinks=False)
    say("case: mixed decode B=2 pos0=40000 HCA layer sinks=None (split rows, merged)")
    _decode_case(csa, "mixed_decode", 40000, 2, 12, layers=[1], sinks=False)


def test_decode_without_sinks_head_groups(csa):
    """No sink through the decode attention kernel (16..255 tokens) and its merge."""
    say("case: csa decode B=20 pos0=3001 sinks=None (row slices x head groups)")
    _decode_case(csa, "csa_decode", 3001, 20, 13, sinks=False)
    say("case: sliding layer B=24 sinks=None (one slice)")
    _decode_case(csa, "mixed_decode", 40000, 24, 14, layers=[2], sinks=False)


def test_decode_graph_replay_matches_eager(csa):
    """A captured decode step (all three layers) replays bit-identically to the eager calls,
    with eager work and synchronisations between the replays."""
    import torch
    from long_context_sparse_gated_amd.layer import LayerCache, layer_step
    say("case: decode step as a HIP graph, mixed_decode B=2 pos0=40959")
    m = csa
    w = synth.workload("mixed_decode", pos0=40959, batch=2)
    pos0, B = w.pos0, w.batch
    p0 = torch.full((B,), pos0, dtype=torch.int64, device="cuda")
    layers = []
    for li, spec in enumerate(w.layers):
        inp = synth.decode_inputs(w, 4, li)
        L = m.Layer.from_spec(spec)
        pool_cap = (pos0 + 1) // spec.ratio if spec.ratio else 1
        cache = LayerCache(L, B, spec.window, pool_cap)
        cache.ring.copy_(dev(inp["win"]))
        if spec.ratio:
            P = pos0 // spec.ratio
            cache.pool[:, :P].copy_(dev(inp["pool"]))
            cache.cstate_kv.copy_(dev(inp["cstate_kv"]))
            cache.cstate_gate.copy_(dev(inp["cstate_gate"]))
            if spec.has_indexer:
                cache.ipool[:, :P].copy_(dev(inp["ipool"]))
                cache.istate_kv.copy_(dev(inp["istate_kv"]))
                cache.istate_gate.copy_(dev(inp["istate_gate"]))
        a = {k: dev(inp[k]) for k in ("q", "kv", "ckv", "cgate", "ikv", "igate", "qi", "wi",
                                       "sinks") if k in inp}
        out = torch.empty_like(a["q"])
        idx = (torch.empty(B, 1, spec.topk, dtype=torch.int32, device="cuda")
               if spec.has_indexer else None)
        layers.append((cache, a, out, idx))

    def step():
        for cache, a, out, idx in layers:
            layer_step(cache, p0, pos0, a["q"], a["kv"], a.get("ckv"), a.get("cgate"),
                       a.get("ikv"), a.get("igate"), a.get("qi"), a.get("wi"), a["sinks"],
                       out=out, topk_idx=idx)

    step()
    torch.cuda.synchronize()
    ref = [(o.clone(), None if ix is None else ix.clone()) for _, _, o, ix in layers]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for _, _, o, ix in layers:  # clobber the outputs eagerly between replays
            o.fill_(0)
            if ix is not None:
                ix.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for (o_ref, ix_ref), (_, _, o, ix) in zip(ref, layers):
            assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), rep
            if ix is not None:
                assert torch.equal(ix, ix_ref), rep
        step()  # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("n_q,pool,distinct,pos0", [
    (37, 700, 0, 2700), (64, 900, 5, 3000), (9, 300, 0, 0), (1, 5000, 0, 19999),
    (1, 30000, 7, 119999), (3, 2048, 3, 8191), (7, 12000, 0, 47990), (5, 600, 0, 2048),
    (2, 3001, 0, 11990), (1, 32768, 2, 131071),
    # the mixed long-context decode row length (262144 keys), plain and tie-heavy
    (1, 262144, 0, 1048575), (2, 262144, 3, 1048574),
    # every key equal, so every score ties and the lowest ids win: prefill
    # (one-wave and block selection) and decode (one block, and slices)
    (37, 700, 1, 2700), (8, 12000, 1, 47990), (1, 32768, 1, 131071), (1, 262144, 1, 1048575)])
def test_topk_bit_exact_on_grid_inputs(csa, n_q, pool, distinct, pos0):
    """Exact-arithmetic scores: both sides must select identical ids (ties: lowest id)."""
    _grid_topk_case(csa, n_q, pool, distinct, pos0)


def _grid_topk_case(m, n_q, pool, distinct, pos0):
    import torch
    say(f"case: grid top-k n_q={n_q} pool={pool} distinct={distinct} pos0={pos0}")
    spec = synth.LayerSpec(kind="csa", dtype="bf16")
    L = m.Layer.from_spec(spec)
    k = spec.topk
    q, keys, wt = synth.grid_index_inputs(n_q, pool, 64, 128, 64, seed=n_q + pool,
                                          distinct_rows=distinct)
    B = 1
    pos0_t = torch.full((B,), pos0, dtype=torch.int64, device="cuda")
    assert (pos0 + n_q) // 4 <= pool
    qd = torch.from_numpy(q[None]).to(torch.bfloat16).cuda()
    kd = torch.from_numpy(keys[None]).to(torch.bfloat16).cuda()
    wd = torch.from_numpy(wt[None]).to(torch.bfloat16).cuda()
    idx = torch.empty(B, n_q, k, dtype=torch.int32, device="cuda")
    sc_out = torch.full((B, n_q, pool), float("nan"), dtype=torch.float32, device="cuda")
    m.csa_index_topk(L, pos0_t, pos0, qd, wd, kd, idx, scores_out=sc_out)
    torch.cuda.synchronize()
    gi, gs = idx.cpu().numpy()[0], sc_out.cpu().numpy()[0]
    for i in range(n_q):
        t = pos0 + i
        nv = (t + 1) // 4
        sc = O.index_scores(q[i].astype(np.float64), wt[i].astype(np.float64),
                            keys[:nv].astype(np.float64), t, 64, O.rope_base(spec), "bf16")
        assert np.array_equal(gs[i, :nv].astype(np.float64), sc), "scores must be exact"
        ref = O.topk_select(sc, k)
        assert np.array_equal(gi[i], ref), f"query {i}: ids differ"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("yarn", [False, True])
@pytest.mark.parametrize("sign", [1, -1])
def test_csa_rope_matches_oracle(csa, dtype, yarn, sign):
    """csa_rope rotates the last rope_dim channels of every row in place at
    sign * position; stored bits equal the oracle's float64 rotation rounded
    once (rows of 96 channels, 32 rope channels, three rows per token, two
    sequences at distant positions)."""
    import torch
    m = csa
    say(f"case: csa_rope dtype={dtype} yarn={yarn} sign={sign}")
    B, n, rows, width, rd = 2, 37, 3, 96, 32
    spec = synth.LayerSpec(kind="sliding", dtype=dtype, num_heads=4, head_dim=64, rope_dim=16,
                           rope_theta=160000.0, ratio=0, overlap=0,
                           rope_factor=16.0 if yarn else 0.0, rope_original_context=4096.0)
    L = m.Layer.from_spec(spec)
    rng = np.random.default_rng([17, sign + 1, int(yarn)])
    x = rng.standard_normal((B, n, rows, width)).astype(np.float32)
    if dtype == "bf16":
        x = to_f64(synth.f32_to_bf16_bits(x))
    x = x.astype(np.float64)
    pos = np.array([5, 250000], dtype=np.int64)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    xd = torch.from_numpy(x).to(torch.float32).to(tdt).cuda()
    p0 = torch.from_numpy(pos).cuda()
    m.csa_rope(L, p0, int(pos.max()), xd, rd, sign)
    torch.cuda.synchronize()
    got = host(xd)
    t = pos[:, None] + np.arange(n)[None, :]                       # [B, n]
    ref = O.round_to(O.rope(x, sign * t[:, :, None], rd, O.rope_base(spec), +1), dtype)
    assert np.array_equal(got[..., :width - rd], x[..., :width - rd]), "channels before the slice"
    ulp_diff_ok(got, ref, dtype, "rotated rows")
    if yarn:  # the scaled frequencies differ from the plain ones on these positions
        plain = O.round_to(O.rope(x, sign * t[:, :, None], rd, spec.rope_theta, +1), dtype)
        assert not np.array_equal(plain, ref)


def test_chunked_prefill_equals_one_shot(csa):
    """Streaming state: prefill in chunks (including a single-token call) matches one call.

    Caches and top-k ids must match bitwise.  Outputs of calls of >= 256
    tokens match bitwise too (such calls never split a query's rows across
    blocks); the single-token calls do split, which changes the order of the
    float32 sums, so they are held to the bf16 tolerance."""
    import torch
    from long_context_sparse_gated_amd.layer import LayerCache, layer_step
    say("case: chunked prefill vs one-shot, csa bf16 S=1030")
    m = csa
    w = synth.workload("csa_prefill", S=1030)
    spec = w.layers[0]
    inp = synth.prefill_inputs(w, 5)
    L = m.Layer.from_spec(spec)
    S = w.n_new
    a = {k: dev(v) for k, v in inp.items() if k != "sinks"}
    sinks = dev(inp["sinks"])
    one = LayerCache(L, 1, S, S // 4)
    p = torch.zeros(1, dtype=torch.int64, device="cuda")
    out1, idx1 = layer_step(one, p, 0, a["q"], a["kv"], a["ckv"], a["cgate"], a["ikv"], a["igate"],
                            a["qi"], a["wi"], sinks)
    ch = LayerCache(L, 1, S, S // 4)
    outs, idxs = [], []
    for lo, hi in ((0, 301), (301, 302), (302, 303), (303, 771), (771, 1030)):  # as `chunks`
        p = torch.full((1,), lo, dtype=torch.int64, device="cuda")
        sl = {k: v[:, lo:hi].contiguous() for k, v in a.items()}
        o, ix = layer_step(ch, p, lo, sl["q"], sl["kv"], sl["ckv"], sl["cgate"], sl["ikv"],
                           sl["igate"], sl["qi"], sl["wi"], sinks)
        outs.append(o)
        idxs.append(ix)
    torch.cuda.synchronize()
    assert torch.equal(one.pool, ch.pool) and torch.equal(one.ipool, ch.ipool)
    assert torch.equal(one.ring, ch.ring)
    assert torch.equal(idx1, torch.cat(idxs, 1))
    chunks = ((0, 301), (301, 302), (302, 303), (303, 771), (771, 1030))
    for (lo, hi), o in zip(chunks, outs):
        if hi - lo >= 256:
            assert torch.equal(out1[:, lo:hi].view(torch.int16), o.view(torch.int16)), (lo, hi)
        else:
            assert_close(host(o[0]), host(out1[0, lo:hi]).astype(np.float64), "bf16",
                         f"chunk {lo}:{hi}")


def test_repeat_runs_are_bitwise_identical(csa):
    import torch
    say("case: determinism, csa bf16 S=900 twice")
    w = synth.workload("csa_prefill", S=900)
    inp = synth.prefill_inputs(w, 6)
    r1 = _prefill_gpu(csa, w.layers[0], inp, 1, 900)
    r2 = _prefill_gpu(csa, w.layers[0], inp, 1, 900)
    assert torch.equal(r1[6], r2[6])
    assert torch.equal(r1[5].view(torch.int16), r2[5].view(torch.int16))


# ----------------------------------------------------------------------------
# grouped output projection

def _oproj_gpu(m, inp, G, T, hidden):
    import torch
    x, wa, wb = dev(inp["x"]), dev(inp["w_a"]), dev(inp["w_b"])
    out = torch.full((T, hidden), float("nan"), dtype=torch.bfloat16, device="cuda")
    m.csa_output_projection(x, wa, wb, out, G)
    torch.cuda.synchronize()
    return host(out)


@pytest.mark.parametrize("T,H,D,G,R,hidden", [
    (300, 8, 64, 2, 96, 200),      # ragged in every dimension of both products
    (1, 4, 64, 4, 32, 256),        # one token
    (129, 16, 32, 1, 64, 513),     # one group: two plain products
    (257, 8, 64, 4, 40, 96),       # rank below one tile, G R = 160
    (64, 4, 64, 4, 8, 96),         # one head per group, the smallest G R (32)
])
def test_output_projection_small(csa, T, H, D, G, R, hidden):
    say(f"output projection T={T} H={H} D={D} G={G} R={R} hidden={hidden}")
    inp = synth.oproj_inputs(T, H, D, G, R, hidden, seed=5)
    got = _oproj_gpu(csa, inp, G, T, hidden)
    ref = O.output_projection(to_f64(inp["x"]), to_f64(inp["w_a"]), to_f64(inp["w_b"]), G, "bf16")
    assert np.isfinite(got).all()
    assert_close(got, ref, "bf16", "output projection")


def test_output_projection_full_size_sampled(csa):
    s = synth.OPROJ_SHAPE
    T, H, D, G, R, hidden = s["T"], s["H"], s["D"], s["G"], s["R"], s["hidden"]
    say(f"output projection full size {s}, sampled rows")
    inp = synth.oproj_inputs(T, H, D, G, R, hidden, seed=7)
    got = _oproj_gpu(csa, inp, G, T, hidden)
    assert np.isfinite(got).all()
    rows = np.r_[0:3, 127:130, 4095:4097, T - 3:T, np.random.default_rng(3).integers(0, T, 40)]
    ref = O.output_projection(to_f64(inp["x"][rows]), to_f64(inp["w_a"]), to_f64(inp["w_b"]), G,
                              "bf16")
    assert_close(got[rows], ref, "bf16", "output projection rows")
    # the same rows drawn alone match the whole draw
    part = synth.oproj_inputs(T, H, D, G, R, hidden, seed=7, rows=rows)
    assert np.array_equal(part["x"], inp["x"][rows])


# ----------------------------------------------------------------------------
# producer projections

def _proj_gpu(m, inp, T, hidden, q_lora, H, D, comp, Di, Hi, qn, q_offset=0):
    import torch
    bf = torch.bfloat16
    shapes = {"q": (T, H, D), "kv": (T, D), "ckv": (T, comp), "cgate": (T, comp),
              "ikv": (T, Di), "igate": (T, Di), "qi": (T, Hi, Di), "wi": (T, Hi)}
    outs = {k: torch.full(v, float("nan"), dtype=bf, device="cuda") for k, v in shapes.items()
            if (k in ("q", "kv")) or (k in ("ckv", "cgate") and comp) or
            (k in ("ikv", "igate", "qi", "wi") and Di)}
    if q_offset:  # q as a contiguous view q_offset elements into its buffer
        buf = torch.full((T * H * D + q_offset,), float("nan"), dtype=bf, device="cuda")
        outs["q"] = buf[q_offset:].view(T, H, D)
    need = m.load_library().csa_project_workspace_bytes(
        m._CProj(T, hidden, q_lora, H, D, comp, Di, Hi, 1e-6, 1 if qn else 0))
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    m.csa_project(dev(inp["x"]), dev(inp["w_x"]), dev(inp["g_qa"]), dev(inp["g_kv"]),
                  dev(inp["w_q"]), outs, q_lora_rank=q_lora, num_heads=H, head_dim=D,
                  comp_dim=comp, index_dim=Di, index_heads=Hi, eps=1e-6, q_head_norm=qn,
                  workspace=ws)
    torch.cuda.synchronize()
    got = {k: host(v) for k, v in outs.items()}
    got["latent"] = host(ws.view(torch.bfloat16)[:T * q_lora].view(T, q_lora))
    return got


def _proj_check(got, ref, rows=None):
    for k, g in got.items():
        r = ref[k]
        g = g if rows is None else g[rows]
        assert np.isfinite(g).all(), k
        assert_close(g, r.reshape(g.shape), "bf16", f"projection {k}")


@pytest.mark.parametrize("T,hidden,q_lora,H,D,comp,Di,Hi,qn", [
    (300, 256, 96, 4, 64, 64, 32, 8, True),      # ragged rows, every stream
    (129, 128, 64, 2, 128, 0, 0, 0, False),      # sliding-only layer, no q_b_norm
    (1, 64, 32, 3, 32, 32, 0, 0, True),          # one token, compressor without indexer
    (77, 96, 32, 2, 36, 20, 12, 4, True),        # stream widths off 8-column pieces
    (300, 128, 96, 3, 512, 32, 40, 3, True),     # heads of 512: q_b_norm in the product's
                                                 # epilogue; ragged rows, q_I's 120 columns
                                                 # a partial last tile
    (65, 64, 32, 2, 512, 0, 0, 0, False),        # heads of 512 without q_b_norm
])
def test_project_small(csa, T, hidden, q_lora, H, D, comp, Di, Hi, qn):
    say(f"projections T={T} hidden={hidden} q_lora={q_lora} H={H} D={D} comp={comp} "
        f"Di={Di} Hi={Hi} q_head_norm={qn}")
    inp = synth.proj_inputs(T, hidden, q_lora, H, D, comp, Di, Hi, seed=9)
    got = _proj_gpu(csa, inp, T, hidden, q_lora, H, D, comp, Di, Hi, qn)
    ref = O.project_inputs(to_f64(inp["x"]), to_f64(inp["w_x"]), inp["g_qa"], inp["g_kv"],
                           to_f64(inp["w_q"]), O.ProjSizes(q_lora, H, D, comp, Di, Hi), 1e-6,
                           qn, "bf16")
    _proj_check(got, ref)


def test_project_unaligned_q_heads_of_512(csa):
    # q two bytes off a 16-byte boundary: the per-head norm cannot be fused
    # into the product's 16-byte stores and runs as a pass of its own
    T, hidden, q_lora, H, D, comp, Di, Hi = 130, 64, 32, 2, 512, 16, 24, 2
    say(f"projections, q at a 2-byte offset, T={T} H={H} D={D}")
    inp = synth.proj_inputs(T, hidden, q_lora, H, D, comp, Di, Hi, seed=11)
    got = _proj_gpu(csa, inp, T, hidden, q_lora, H, D, comp, Di, Hi, True, q_offset=1)
    ref = O.project_inputs(to_f64(inp["x"]), to_f64(inp["w_x"]), inp["g_qa"], inp["g_kv"],
                           to_f64(inp["w_q"]), O.ProjSizes(q_lora, H, D, comp, Di, Hi), 1e-6,
                           True, "bf16")
    _proj_check(got, ref)


def test_project_full_size_sampled(csa):
    s = synth.PROJ_SHAPE
    args = (s["T"], s["hidden"], s["q_lora"], s["H"], s["D"], s["comp"], s["Di"], s["Hi"])
    say(f"projections full size {s}, sampled rows")
    inp = synth.proj_inputs(*args, seed=4)
    got = _proj_gpu(csa, inp, *args, True)
    T = s["T"]
    rows = np.r_[0:2, 255:257, T - 2:T, np.random.default_rng(8).integers(0, T, 26)]
    ref = O.project_inputs(to_f64(inp["x"][rows]), to_f64(inp["w_x"]), inp["g_qa"], inp["g_kv"],
                           to_f64(inp["w_q"]),
                           O.ProjSizes(s["q_lora"], s["H"], s["D"], s["comp"], s["Di"], s["Hi"]),
                           1e-6, True, "bf16")
    _proj_check(got, ref, rows)


# ----------------------------------------------------------------------------
# variable-length batched prefill

def test_varlen_prefill_matches_separate_calls(csa):
    """A padded batch with per-sequence valid lengths (700, 413, 0): the caches
    advance by the valid tokens only.  Valid rows, top-k ids and caches equal
    each sequence run alone (ids and caches bitwise); a second, full call then
    equals a one-shot run over each sequence's concatenated tokens; one
    sequence is also held against the oracle."""
    import torch
    from long_context_sparse_gated_amd.layer import LayerCache, layer_step
    say("case: varlen prefill, csa bf16, B=3, n_new=700, lens (700, 413, 0), then 300 more")
    m = csa
    S, S2, lens = 700, 300, (700, 413, 0)
    w = synth.workload("csa_prefill", S=S, batch=3)
    spec = w.layers[0]
    inp = synth.prefill_inputs(w, 11)
    inp2 = synth.prefill_inputs(synth.workload("csa_prefill", S=S2, batch=3), 12)
    L = m.Layer.from_spec(spec)
    cap, pcap = S + S2, (S + S2) // 4
    keys = ("q", "kv", "ckv", "cgate", "ikv", "igate", "qi", "wi")
    a = {k: dev(inp[k]) for k in keys}
    a2 = {k: dev(inp2[k]) for k in keys}
    sinks = dev(inp["sinks"])
    cache = LayerCache(L, 3, cap, pcap)
    p0 = torch.zeros(3, dtype=torch.int64, device="cuda")
    nv = torch.tensor(lens, dtype=torch.int32, device="cuda")
    out, idx = layer_step(cache, p0, 0, *(a[k] for k in keys), sinks, n_valid=nv)
    torch.cuda.synchronize()
    out, idx = out.clone(), idx.clone()
    # an empty sequence leaves its caches untouched (they start at zero)
    assert not cache.ring[2].any() and not cache.pool[2].any() and not cache.ipool[2].any()
    assert not cache.cstate_kv[2].any() and not cache.istate_kv[2].any()
    # second call: every sequence continues with 300 valid tokens
    p1 = torch.tensor(lens, dtype=torch.int64, device="cuda")
    out2, idx2 = layer_step(cache, p1, max(lens), *(a2[k] for k in keys), sinks)
    torch.cuda.synchronize()
    for b, n in enumerate(lens):
        # the sequence alone: its valid tokens, then the same 300
        one = LayerCache(L, 1, cap, pcap)
        z = torch.zeros(1, dtype=torch.int64, device="cuda")
        cat = {k: torch.cat([a[k][b:b + 1, :n], a2[k][b:b + 1]], 1).contiguous() for k in keys}
        o1, i1 = layer_step(one, z, 0, *(cat[k] for k in keys), sinks)
        torch.cuda.synchronize()
        if n:
            assert torch.equal(idx[b, :n], i1[0, :n]), f"sequence {b}: first-call ids"
            assert_close(host(out[b, :n]), host(o1[0, :n]), "bf16", f"sequence {b} first call")
        assert torch.equal(idx2[b], i1[0, n:]), f"sequence {b}: second-call ids"
        assert_close(host(out2[b]), host(o1[0, n:]), "bf16", f"sequence {b} second call")
        ne = (n + S2) // 4
        assert torch.equal(cache.pool[b, :ne], one.pool[0, :ne]), f"sequence {b}: pool"
        assert torch.equal(cache.ipool[b, :ne], one.ipool[0, :ne]), f"sequence {b}: indexer pool"
        assert torch.equal(cache.ring[b], one.ring[0]), f"sequence {b}: window ring"
        assert torch.equal(cache.cstate_kv[b], one.cstate_kv[0]), f"sequence {b}: state"
        assert torch.equal(cache.istate_gate[b], one.istate_gate[0]), f"sequence {b}: state"
    # the 413-token sequence against the oracle on sampled queries
    x = seq_f64(inp, 1)
    x = {k: (v if k == "sinks" else v[:lens[1]]) for k, v in x.items()}
    qs = [0, 3, 4, 130, 255, 300, 411, 412]
    ref = O.csa_prefill(spec, x, queries=qs)
    gi = idx[1].cpu().numpy()
    nd = 0
    for j, t in enumerate(qs):
        sc, ab = index_exact(spec, x["qi"][t], x["wi"][t], ref["ipool"][:(t + 1) // 4], t)
        nd += audit_topk(gi[t], ref["idx"][j], sc, ab, spec.index_dim, spec.index_heads)
    say(f"  near-tie id differences: {nd}")
    same = [j for j, t in enumerate(qs) if np.array_equal(gi[t], ref["idx"][j])]
    assert_close(host(out[1])[qs][same], ref["out"][same], "bf16", "varlen rows vs oracle")
    # every sampled row again with the oracle's ids (the second call appended
    # positions 413..712 of this sequence: ring slots and pool rows the first
    # call's queries read are unchanged)
    idx_o = idx.clone()
    idx_o[1, qs] = torch.from_numpy(ref["idx"].astype(np.int32)).cuda()
    out_o = torch.empty_like(out)
    m.csa_attend(L, p0, 0, a["q"], cache.ring, cache.pool, idx_o, sinks, out_o,
                 cache.workspace(S, m.CSA_OP_ATTEND), n_valid=nv)
    torch.cuda.synchronize()
    assert_close(host(out_o[1])[qs], ref["out"], "bf16", "varlen rows vs oracle (oracle ids)")


@pytest.mark.parametrize("kind", ["hca", "sliding"])
def test_varlen_prefill_dense_layers(csa, kind):
    """Variable-length prefill through an HCA layer (compressor, no indexer)
    and a sliding-only layer (window only): caches bitwise equal to each
    sequence run alone, outputs within tolerance, an empty sequence leaves
    its caches untouched, one sequence against the oracle."""
    import dataclasses
    import torch
    from long_context_sparse_gated_amd.layer import LayerCache, layer_step
    say(f"case: varlen prefill, {kind} bf16, B=3, n_new=700, lens (700, 413, 0), then 300 more")
    m = csa
    S, S2, lens = 700, 300, (700, 413, 0)
    w = synth.workload("hca_prefill", S=S, batch=3)
    w2 = synth.workload("hca_prefill", S=S2, batch=3)
    if kind == "sliding":
        spec = synth.LayerSpec(kind="sliding", dtype="bf16", ratio=0, overlap=0,
                               rope_theta=10000.0, rope_factor=16.0,
                               rope_original_context=65536.0)
        w = dataclasses.replace(w, layers=[spec])
        w2 = dataclasses.replace(w2, layers=[spec])
    spec = w.layers[0]
    inp, inp2 = synth.prefill_inputs(w, 13), synth.prefill_inputs(w2, 14)
    keys = ("q", "kv") if kind == "sliding" else ("q", "kv", "ckv", "cgate")
    a = {k: dev(inp[k]) for k in keys}
    a2 = {k: dev(inp2[k]) for k in keys}
    sinks = dev(inp["sinks"])
    L = m.Layer.from_spec(spec)
    cap = S + S2
    pcap = cap // spec.ratio if spec.ratio else 1

    def run(cache, p0, pmax, t, nv=None):
        return layer_step(cache, p0, pmax, t["q"], t["kv"], t.get("ckv"), t.get("cgate"),
                          sinks=sinks, n_valid=nv)[0]

    cache = LayerCache(L, 3, cap, pcap)
    p0 = torch.zeros(3, dtype=torch.int64, device="cuda")
    nv = torch.tensor(lens, dtype=torch.int32, device="cuda")
    out = run(cache, p0, 0, a, nv).clone()
    torch.cuda.synchronize()
    assert not cache.ring[2].any()
    if spec.ratio:
        assert not cache.pool[2].any() and not cache.cstate_kv[2].any()
    p1 = torch.tensor(lens, dtype=torch.int64, device="cuda")
    out2 = run(cache, p1, max(lens), a2)
    torch.cuda.synchronize()
    for b, n in enumerate(lens):
        one = LayerCache(L, 1, cap, pcap)
        z = torch.zeros(1, dtype=torch.int64, device="cuda")
        cat = {k: torch.cat([a[k][b:b + 1, :n], a2[k][b:b + 1]], 1).contiguous() for k in keys}
        o1 = run(one, z, 0, cat)
        torch.cuda.synchronize()
        if n:
            assert_close(host(out[b, :n]), host(o1[0, :n]), "bf16", f"sequence {b} first call")
        assert_close(host(out2[b]), host(o1[0, n:]), "bf16", f"sequence {b} second call")
        assert torch.equal(cache.ring[b], one.ring[0]), f"sequence {b}: window ring"
        if spec.ratio:
            ne = (n + S2) // spec.ratio
            assert torch.equal(cache.pool[b, :ne], one.pool[0, :ne]), f"sequence {b}: pool"
            assert torch.equal(cache.cstate_kv[b], one.cstate_kv[0]), f"sequence {b}: state"
            assert torch.equal(cache.cstate_gate[b], one.cstate_gate[0]), f"sequence {b}: state"
    x = seq_f64(inp, 1)
    x = {k: (v if k == "sinks" else v[:lens[1]]) for k, v in x.items()}
    qs = [0, 1, 127, 128, 255, 256, 400, 412]
    ref = O.sliding_prefill(spec, x, queries=qs) if kind == "sliding" else \
        O.hca_prefill(spec, x, queries=qs)
    assert_close(host(out[1])[qs], ref["out"], "bf16", f"varlen {kind} rows vs oracle")


# ----------------------------------------------------------------------------
# paged pools and packed variable-length rows

def _shuffled_table(B, per_seq, spare, seed):
    """int32 [B, per_seq] device block table over B * per_seq + spare blocks,
    shuffled (no two sequences share a block) -> (table, host copy, blocks)."""
    import torch
    rng = np.random.default_rng(seed)
    nb = B * per_seq + spare
    ids = rng.permutation(nb)[:B * per_seq].reshape(B, per_seq).astype(np.int32)
    return torch.from_numpy(ids).cuda(), ids, nb


def _gather_paged(pool_rows, table_host, E, n):
    """Entries 0..n-1 of each sequence from a paged pool tensor (host float64)."""
    rows = host(pool_rows)
    return np.stack([rows[O.paged_rows(np.arange(n), table_host[b], E)]
                     for b in range(table_host.shape[0])])


def test_paged_prefill_matches_contiguous(csa):
    """A CSA prefill in two chunks with both pools paged through a shuffled
    block table (128 entries per block): ids, outputs and every pooled entry
    bitwise equal to the contiguous run; sampled queries of one sequence
    against the oracle."""
    import torch
    from long_context_sparse_gated_amd.layer import LayerCache, layer_step
    say("case: paged prefill, csa bf16 B=2 S=1000 in chunks (0, 600), (600, 1000), E=128")
    m = csa
    B, S, E = 2, 1000, 128
    w = synth.workload("csa_prefill", S=S, batch=B)
    spec = w.layers[0]
    inp = synth.prefill_inputs(w, 21)
    L = m.Layer.from_spec(spec)
    keys = ("q", "kv", "ckv", "cgate", "ikv", "igate", "qi", "wi")
    a = {k: dev(inp[k]) for k in keys}
    sinks = dev(inp["sinks"])
    pcap = S // 4
    per = (pcap + E - 1) // E
    tab, tab_h, nb = _shuffled_table(B, per, 3, seed=4)
    cont = LayerCache(L, B, S, pcap)
    paged = LayerCache(L, B, S, pcap, block_entries=E, pool_blocks=nb, block_table=tab)
    for lo, hi in ((0, 600), (600, S)):
        p = torch.full((B,), lo, dtype=torch.int64, device="cuda")
        sl = {k: v[:, lo:hi].contiguous() for k, v in a.items()}
        o1, i1 = layer_step(cont, p, lo, *(sl[k] for k in keys), sinks)
        o2, i2 = layer_step(paged, p, lo, *(sl[k] for k in keys), sinks)
        torch.cuda.synchronize()
        assert torch.equal(i1, i2), f"chunk {lo}: ids"
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), f"chunk {lo}: output"
    assert np.array_equal(_gather_paged(paged.pool, tab_h, E, pcap), host(cont.pool))
    assert np.array_equal(_gather_paged(paged.ipool, tab_h, E, pcap), host(cont.ipool))
    # rows of blocks no sequence owns stay untouched
    unused = sorted(set(range(nb)) - set(tab_h.ravel().tolist()))
    prow = host(paged.pool).reshape(nb, E, -1)
    assert not prow[unused].any()
    # one sequence against the oracle (the last chunk's queries)
    x = seq_f64(inp, 1)
    qs = [600, 601, 777, 999]
    ref = O.csa_prefill(spec, x, queries=qs)
    assert np.array_equal(_gather_paged(paged.pool, tab_h, E, pcap)[1], ref["pool"])
    gi = i2[1].cpu().numpy()
    for j, t in enumerate(qs):
        sc, ab = index_exact(spec, x["qi"][t], x["wi"][t], ref["ipool"][:(t + 1) // 4], t)
        audit_topk(gi[t - 600], ref["idx"][j], sc, ab, spec.index_dim, spec.index_heads)
    same = [j for j, t in enumerate(qs) if np.array_equal(gi[t - 600], ref["idx"][j])]
    assert_close(host(o2[1])[[t - 600 for t in qs]][same], ref["out"][same], "bf16",
                 "paged prefill vs oracle")


def test_paged_decode_matches_contiguous(csa):
    """One decode step of the mixed three-layer model (entries close in the
    CSA and HCA layers at this position) with each layer's pools paged
    through its own shuffled table (CSA: 256 entries per block, HCA: 128):
    outputs, ids and the new entries bitwise equal to the contiguous run; one
    sequence against the oracle reading the paged rows."""
    import torch
    from long_context_sparse_gated_amd.layer import LayerCache, layer_step
    m = csa
    pos0, B = 40959, 3
    say(f"case: paged decode, mixed_decode B={B} pos0={pos0}")
    w = synth.workload("mixed_decode", pos0=pos0, batch=B)
    for li, spec in enumerate(w.layers):
        say(f"  layer {li} {spec.kind}")
        inp = synth.decode_inputs(w, 22, li)
        L = m.Layer.from_spec(spec)
        pcap = (pos0 + 1) // spec.ratio if spec.ratio else 1
        kw = {}
        if spec.ratio:
            E = 256 if spec.has_indexer else 128
            tab, tab_h, nb = _shuffled_table(B, (pcap + E - 1) // E, 5, seed=li)
            kw = dict(block_entries=E, pool_blocks=nb, block_table=tab)
        cont = LayerCache(L, B, spec.window, pcap)
        paged = LayerCache(L, B, spec.window, pcap, **kw)
        P = pos0 // spec.ratio if spec.ratio else 0
        for c in (cont, paged):
            c.ring.copy_(dev(inp["win"]))
            if spec.ratio:
                c.cstate_kv.copy_(dev(inp["cstate_kv"]))
                c.cstate_gate.copy_(dev(inp["cstate_gate"]))
                if spec.has_indexer:
                    c.istate_kv.copy_(dev(inp["istate_kv"]))
                    c.istate_gate.copy_(dev(inp["istate_gate"]))
        if spec.ratio:
            cont.pool[:, :P].copy_(dev(inp["pool"]))
            for b in range(B):
                rows = torch.from_numpy(O.paged_rows(np.arange(P), tab_h[b], E)).cuda()
                paged.pool[rows] = dev(inp["pool"][b])
                if spec.has_indexer:
                    paged.ipool[rows] = dev(inp["ipool"][b])
            if spec.has_indexer:
                cont.ipool[:, :P].copy_(dev(inp["ipool"]))
        p0 = torch.full((B,), pos0, dtype=torch.int64, device="cuda")
        args = [dev(inp[k]) if k in inp else None
                for k in ("q", "kv", "ckv", "cgate", "ikv", "igate", "qi", "wi")]
        sk = dev(inp["sinks"])
        o1, i1 = layer_step(cont, p0, pos0, *args, sk)
        o2, i2 = layer_step(paged, p0, pos0, *args, sk)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), "output"
        if spec.has_indexer:
            assert torch.equal(i1, i2), "ids"
        if spec.ratio:
            n = pcap
            assert np.array_equal(_gather_paged(paged.pool, tab_h, E, n), host(cont.pool[:, :n]))
        # sequence 2 against the oracle, its pools read through the table
        b = 2
        new = {k: (to_f64(inp[k]) if k == "sinks" else to_f64(inp[k][b, 0]))
               for k in ("q", "kv", "ckv", "cgate", "ikv", "igate", "qi", "wi", "sinks")
               if k in inp}
        cch = {k: to_f64(inp[k][b]) for k in ("win", "cstate_kv", "cstate_gate", "istate_kv",
                                              "istate_gate") if k in inp}
        if spec.ratio:  # the paged rows as they were before the step
            rows_before = np.zeros((nb * E, spec.head_dim))
            rows_before[O.paged_rows(np.arange(P), tab_h[b], E)] = to_f64(inp["pool"][b])
            cch["pool"] = O.PagedPool(rows_before, tab_h[b], E, P)
            if spec.has_indexer:
                irows = np.zeros((nb * E, spec.index_dim))
                irows[O.paged_rows(np.arange(P), tab_h[b], E)] = to_f64(inp["ipool"][b])
                cch["ipool"] = O.PagedPool(irows, tab_h[b], E, P)
        ref = O.decode_step(spec, pos0, new, cch)
        if spec.has_indexer:
            keys = np.concatenate([cch["ipool"][np.arange(P)], ref["new_ipool"][None]])
            sc, ab = index_exact(spec, new["qi"], new["wi"], keys, pos0)
            nd = audit_topk(i2[b, 0].cpu().numpy(), ref["idx"], sc, ab, spec.index_dim,
                            spec.index_heads)
            if nd:  # a proven near tie: outputs differ by the rows chosen
                say(f"  seq {b}: {nd} near-tie id differences")
                continue
        assert_close(host(o2[b, 0]), ref["out"], "bf16", f"layer {li} seq {b} vs oracle")


@pytest.mark.parametrize("kind", ["csa", "hca", "sliding"])
def test_packed_varlen_prefill_matches_padded(csa, kind):
    """Packed rows (cu_seqlens, no padding rows) against the padded
    variable-length call of the same sequences (700, 413 and 0 tokens, then
    300 more each): ids, outputs and caches bitwise equal."""
    import dataclasses
    import torch
    from long_context_sparse_gated_amd.layer import LayerCache, layer_step
    say(f"case: packed varlen prefill, {kind} bf16, lens (700, 413, 0) then 300 each")
    m = csa
    S, S2, lens = 700, 300, (700, 413, 0)
    name = "csa_prefill" if kind == "csa" else "hca_prefill"
    w, w2 = synth.workload(name, S=S, batch=3), synth.workload(name, S=S2, batch=3)
    if kind == "sliding":
        spec = synth.LayerSpec(kind="sliding", dtype="bf16", ratio=0, overlap=0,
                               rope_theta=10000.0, rope_factor=16.0,
                               rope_original_context=65536.0)
        w, w2 = dataclasses.replace(w, layers=[spec]), dataclasses.replace(w2, layers=[spec])
    spec = w.layers[0]
    inp, inp2 = synth.prefill_inputs(w, 23), synth.prefill_inputs(w2, 24)
    keys = [k for k in ("q", "kv", "ckv", "cgate", "ikv", "igate", "qi", "wi") if k in inp]
    a = {k: dev(inp[k]) for k in keys}
    a2 = {k: dev(inp2[k]) for k in keys}
    sinks = dev(inp["sinks"])
    L = m.Layer.from_spec(spec)
    cap = S + S2
    pcap = cap // spec.ratio if spec.ratio else 1

    def run(cache, p0, pmax, t, **geo):
        return layer_step(cache, p0, pmax, t["q"], t["kv"], t.get("ckv"), t.get("cgate"),
                          t.get("ikv"), t.get("igate"), t.get("qi"), t.get("wi"), sinks, **geo)

    pad, pk = LayerCache(L, 3, cap, pcap), LayerCache(L, 3, cap, pcap)
    p0 = torch.zeros(3, dtype=torch.int64, device="cuda")
    nv = torch.tensor(lens, dtype=torch.int32, device="cuda")
    cu = torch.tensor(np.r_[0, np.cumsum(lens)], dtype=torch.int32, device="cuda")
    packed = {k: torch.cat([v[b, :n] for b, n in enumerate(lens)]).contiguous()
              for k, v in a.items()}
    o1, i1 = run(pad, p0, 0, a, n_valid=nv)
    o2, i2 = run(pk, p0, 0, packed, cu_seqlens=cu, n_new=S)
    torch.cuda.synchronize()
    for b, n in enumerate(lens):
        r = int(sum(lens[:b]))
        assert torch.equal(o1[b, :n].view(torch.int16), o2[r:r + n].view(torch.int16)), b
        if i1 is not None:
            assert torch.equal(i1[b, :n], i2[r:r + n]), b
    # second call: 300 more tokens each, packed as three equal runs
    p1 = torch.tensor(lens, dtype=torch.int64, device="cuda")
    cu2 = torch.tensor([0, S2, 2 * S2, 3 * S2], dtype=torch.int32, device="cuda")
    packed2 = {k: v.reshape(3 * S2, *v.shape[2:]).contiguous() for k, v in a2.items()}
    o3, i3 = run(pad, p1, max(lens), a2)
    o4, i4 = run(pk, p1, max(lens), packed2, cu_seqlens=cu2, n_new=S2)
    torch.cuda.synchronize()
    assert torch.equal(o3.reshape(3 * S2, *o3.shape[2:]).view(torch.int16),
                       o4.view(torch.int16))
    if i3 is not None:
        assert torch.equal(i3.reshape(3 * S2, -1), i4)
    assert torch.equal(pad.ring, pk.ring)
    if spec.ratio:
        assert torch.equal(pad.pool, pk.pool) and torch.equal(pad.cstate_kv, pk.cstate_kv)
        if spec.has_indexer:
            assert torch.equal(pad.ipool, pk.ipool) and torch.equal(pad.istate_gate,
                                                                     pk.istate_gate)


def test_packed_paged_decode_skips_absent_sequences(csa):
    """One-token calls with packed rows (sequence 1 has no token) on
    paged pools, against the padded call on contiguous pools: outputs and ids
    bitwise equal, the absent sequences' caches untouched (an entry closes at
    4099)."""
    import torch
    from long_context_sparse_gated_amd.layer import LayerCache, layer_step
    m = csa
    pos0, B, E = 4099, 4, 128
    lens = (1, 0, 1, 1)
    say(f"case: packed + paged decode, csa_decode B={B} pos0={pos0} lens {lens}")
    w = synth.workload("csa_decode", pos0=pos0, batch=B)
    spec = w.layers[0]
    inp = synth.decode_inputs(w, 25, 0)
    L = m.Layer.from_spec(spec)
    pcap = (pos0 + 1) // 4
    P = pos0 // 4
    tab, tab_h, nb = _shuffled_table(B, (pcap + E - 1) // E, 2, seed=9)
    pad = LayerCache(L, B, spec.window, pcap)
    pk = LayerCache(L, B, spec.window, pcap, block_entries=E, pool_blocks=nb, block_table=tab)
    for c in (pad, pk):
        c.ring.copy_(dev(inp["win"]))
        for k in ("cstate_kv", "cstate_gate", "istate_kv", "istate_gate"):
            getattr(c, k).copy_(dev(inp[k]))
    pad.pool[:, :P].copy_(dev(inp["pool"]))
    pad.ipool[:, :P].copy_(dev(inp["ipool"]))
    for b in range(B):
        rows = torch.from_numpy(O.paged_rows(np.arange(P), tab_h[b], E)).cuda()
        pk.pool[rows] = dev(inp["pool"][b])
        pk.ipool[rows] = dev(inp["ipool"][b])
    keys = ("q", "kv", "ckv", "cgate", "ikv", "igate", "qi", "wi")
    a = {k: dev(inp[k]) for k in keys}
    present = [b for b in range(B) if lens[b]]
    packed = {k: v[present, 0].contiguous() for k, v in a.items()}
    p0 = torch.full((B,), pos0, dtype=torch.int64, device="cuda")
    nv = torch.tensor(lens, dtype=torch.int32, device="cuda")
    cu = torch.tensor(np.r_[0, np.cumsum(lens)], dtype=torch.int32, device="cuda")
    sk = dev(inp["sinks"])
    o1, i1 = layer_step(pad, p0, pos0, *(a[k] for k in keys), sk, n_valid=nv)
    o2, i2 = layer_step(pk, p0, pos0, *(packed[k] for k in keys), sk, cu_seqlens=cu, n_new=1)
    torch.cuda.synchronize()
    for r, b in enumerate(present):
        assert torch.equal(o1[b, 0].view(torch.int16), o2[r].view(torch.int16)), b
        assert torch.equal(i1[b, 0], i2[r]), b
    got = _gather_paged(pk.pool, tab_h, E, pcap)
    assert np.array_equal(got, host(pad.pool))
    for b in [b for b in range(B) if lens[b] == 0]:  # absent: no new entry, state as it was
        assert not got[b, P:].any()
        assert torch.equal(pk.cstate_kv[b], dev(inp["cstate_kv"])[b])


@pytest.mark.parametrize("kind,n,pos,paged", [
    ("csa", 1, 131071, False),   # a decode step that closes an entry ((p + 1) % 4 == 0)
    ("csa", 1, 131072, False),   # one that does not
    ("csa", 1, 5003, True),      # paged pools (shuffled block table)
    ("hca", 1, 8191, False),
    ("sliding", 1, 777, False),
    ("csa", 37, 3001, False),    # a prefill chunk: the separate kernels behind the same call
])
def test_cache_update_matches_separate_calls(csa, kind, n, pos, paged):
    """csa_cache_update (one launch for a decode step) writes the window ring, the
    compressor states and the pools bit for bit as csa_window_append and csa_compress
    called one after the other."""
    import torch
    from long_context_sparse_gated_amd.layer import LayerCache
    say(f"case: cache update {kind} n={n} pos={pos} paged={paged}")
    m = csa
    spec = {"csa": synth.workload("csa_decode").layers[0],
            "hca": synth.workload("mixed_decode").layers[1],
            "sliding": synth.workload("mixed_decode").layers[2]}[kind]
    L = m.Layer.from_spec(spec)
    B, W = 3, spec.window
    ratio = spec.ratio
    pool_cap = (pos + n) // ratio + 1 if ratio else 0
    g = torch.Generator(device="cuda").manual_seed(11)
    bf = torch.bfloat16

    def rnd(*shape):
        return torch.randn(*shape, generator=g, device="cuda").to(bf)

    kw = {}
    if paged and ratio:
        E = 256
        per = (pool_cap + E - 1) // E
        perm = torch.randperm(B * per, generator=torch.Generator().manual_seed(3))
        kw = dict(block_entries=E, pool_blocks=B * per,
                  block_table=perm.view(B, per).to(torch.int32).cuda())
    caches = [LayerCache(L, B, W + n, max(pool_cap, 1), **kw) for _ in range(2)]
    # the same random cache contents in both
    for name in ("ring", "pool", "ipool", "cstate_kv", "cstate_gate", "istate_kv", "istate_gate"):
        a = getattr(caches[0], name, None)
        if a is not None:
            a.copy_(torch.randn(a.shape, generator=g, device="cuda").to(a.dtype))
            getattr(caches[1], name).copy_(a)
    D, Di = spec.head_dim, spec.index_dim
    kv, ckv, cgate = rnd(B, n, D), rnd(B, n, D), rnd(B, n, D)
    ikv, igate = rnd(B, n, Di), rnd(B, n, Di)
    nw = torch.rand(D, generator=g, device="cuda") + 0.5
    inw = torch.rand(Di, generator=g, device="cuda") + 0.5
    p0 = torch.tensor([pos, pos + 1, pos + 2], dtype=torch.int64, device="cuda")
    pm = pos + 2
    c0, c1 = caches
    # separate calls
    m.csa_window_append(L, p0, pm, kv, c0.ring)
    if ratio:
        m.csa_compress(L, p0, pm, ckv, cgate, c0.cstate_kv, c0.cstate_gate, c0.pool,
                       spec.rope_dim, nw, 1e-6, paged=c0.paged)
        if spec.has_indexer:
            m.csa_compress(L, p0, pm, ikv, igate, c0.istate_kv, c0.istate_gate, c0.ipool,
                           spec.index_rope_dim, inw, 1e-6, paged=c0.paged)
    # one call
    if not ratio:
        m.csa_cache_update(L, p0, pm, kv, c1.ring)
    elif not spec.has_indexer:
        m.csa_cache_update(L, p0, pm, kv, c1.ring, ckv, cgate, c1.cstate_kv, c1.cstate_gate,
                           c1.pool, norm_weight=nw, paged=c1.paged)
    else:
        m.csa_cache_update(L, p0, pm, kv, c1.ring, ckv, cgate, c1.cstate_kv, c1.cstate_gate,
                           c1.pool, ikv, igate, c1.istate_kv, c1.istate_gate, c1.ipool,
                           norm_weight=nw, inorm_weight=inw, paged=c1.paged)
    torch.cuda.synchronize()
    for name in ("ring", "pool", "ipool", "cstate_kv", "cstate_gate", "istate_kv", "istate_gate"):
        a = getattr(c0, name, None)
        if a is not None:
            assert torch.equal(a.view(torch.int16), getattr(c1, name).view(torch.int16)), name
