"""Parity at the full workload sizes, in the launch configuration the
benchmark times (same entry points, shapes and capacities).  The oracle runs
on sampled queries / sequences only; sampled rows include the first and last
tokens, the window and top-k boundaries, and a random spread."""
import numpy as np
import pytest

import synth
from oracle import csa_oracle as O
from synth import to_f64
from tests.helpers import (LazyF64, assert_close, audit_topk, dev, host, index_exact, say,
                           ulp_diff_ok)

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(scope="module")
def csa():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import long_context_sparse_gated_amd as m
    m.load_library()
    return m


def _sample(S, extra, n_random, seed):
    rng = np.random.default_rng(seed)
    qs = set(i for i in extra if 0 <= i < S)
    qs.update(int(x) for x in rng.integers(0, S, n_random))
    return sorted(qs)


def _lazy_seq(inp, b, eager=()):
    out = {}
    for k, v in inp.items():
        if k == "sinks":
            out[k] = to_f64(v)
        elif k in eager:
            out[k] = to_f64(v[b])
        else:
            out[k] = LazyF64(v[b])
    return out


def test_csa_prefill_full_s8192(csa):
    import torch
    from long_context_sparse_gated_amd.layer import LayerCache, layer_step
    say("case: csa_prefill full S=8192 (benchmark launch configuration)")
    m = csa
    w = synth.workload("csa_prefill")
    spec, S = w.layers[0], w.n_new
    inp = synth.prefill_inputs(w, 0)
    L = m.Layer.from_spec(spec)
    cache = LayerCache(L, 1, S, S // spec.ratio)
    a = {k: dev(v) for k, v in inp.items()}
    pos0 = torch.zeros(1, dtype=torch.int64, device="cuda")
    out, idx = layer_step(cache, pos0, 0, a["q"], a["kv"], a["ckv"], a["cgate"], a["ikv"],
                          a["igate"], a["qi"], a["wi"], a["sinks"])
    torch.cuda.synchronize()
    qs = _sample(S, [0, 1, 2, 3, 127, 128, 2046, 2047, 2048, 4095, 4096, 8190, 8191], 11, 7)
    x = _lazy_seq(inp, 0, eager=("kv", "ckv", "cgate", "ikv", "igate"))
    ref = O.csa_prefill(spec, x, queries=qs)
    ulp_diff_ok(host(cache.pool[0]), ref["pool"], "bf16", "pool")
    ulp_diff_ok(host(cache.ipool[0]), ref["ipool"], "bf16", "ipool")
    ulp_diff_ok(host(cache.ring[0]), ref["win"], "bf16", "window rows")
    gi = idx[0].cpu().numpy()
    nd = 0
    for n, t in enumerate(qs):
        keys = ref["ipool"][:(t + 1) // spec.ratio]
        sc, ab = index_exact(spec, x["qi"][t], x["wi"][t], keys, t)
        nd += audit_topk(gi[t], ref["idx"][n], sc, ab, spec.index_dim, spec.index_heads)
    say(f"  near-tie id differences: {nd} over {len(qs)} queries")
    idx2 = idx.clone()
    idx2[0, qs] = torch.from_numpy(ref["idx"].astype(np.int32)).cuda()
    out2 = torch.empty_like(out)
    m.csa_attend(L, pos0, 0, a["q"], cache.ring, cache.pool, idx2, a["sinks"], out2,
                 cache.workspace(S, m.CSA_OP_ATTEND))
    torch.cuda.synchronize()
    err = assert_close(host(out2[0, qs]), ref["out"], "bf16", "csa attention output")
    say(f"  max abs err {err:.3e}")


def test_hca_prefill_full_s65536(csa):
    import torch
    from long_context_sparse_gated_amd.layer import LayerCache, layer_step
    say("case: hca_prefill full S=65536")
    m = csa
    w = synth.workload("hca_prefill")
    spec, S = w.layers[0], w.n_new
    inp = synth.prefill_inputs(w, 0)
    L = m.Layer.from_spec(spec)
    cache = LayerCache(L, 1, S, S // spec.ratio)
    a = {k: dev(v) for k, v in inp.items()}
    del inp["q"]
    pos0 = torch.zeros(1, dtype=torch.int64, device="cuda")
    out, _ = layer_step(cache, pos0, 0, a["q"], a["kv"], a["ckv"], a["cgate"], sinks=a["sinks"])
    torch.cuda.synchronize()
    qs = _sample(S, [0, 1, 126, 127, 128, 255, 32767, 65407, 65408, 65534, 65535], 9, 8)
    x = _lazy_seq(inp, 0, eager=("kv", "ckv", "cgate"))
    # q rows of the sampled queries only (redrawn from their seeded blocks)
    qrows = synth.prefill_rows(w, 0, 0, 0, "q", qs)

    class QRows:
        shape = (S,) + qrows.shape[1:]

        def __getitem__(self, i):
            return to_f64(qrows[qs.index(i)])

    x["q"] = QRows()
    ref = O.hca_prefill(spec, x, queries=qs)
    ulp_diff_ok(host(cache.pool[0]), ref["pool"], "bf16", "pool")
    ulp_diff_ok(host(cache.ring[0, :256]), ref["win"][:256], "bf16", "window rows (head)")
    ulp_diff_ok(host(cache.ring[0, -256:]), ref["win"][-256:], "bf16", "window rows (tail)")
    err = assert_close(host(out[0, qs]), ref["out"], "bf16", "hca attention output")
    say(f"  max abs err {err:.3e}")


def _decode_full(m, name, seqs_checked, layers=None):
    import torch
    from long_context_sparse_gated_amd.layer import LayerCache, layer_step
    w = synth.workload(name)
    pos0, B = w.pos0, w.batch
    for li, spec in enumerate(w.layers):
        if layers is not None and li not in layers:
            continue
        say(f"  layer {li} ({spec.kind}) B={B} t={pos0}")
        L = m.Layer.from_spec(spec)
        pool_cap = (pos0 + 1) // spec.ratio if spec.ratio else 1
        cache = LayerCache(L, B, spec.window, pool_cap)
        names = list(synth.cache_shapes(w, li))
        for b in range(B):  # one sequence at a time keeps host memory bounded
            c = synth.decode_cache_seq(w, 0, li, b)
            cache.ring[b].copy_(dev(c["win"]))
            if spec.ratio:
                P = pos0 // spec.ratio
                cache.pool[b, :P].copy_(dev(c["pool"]))
                cache.cstate_kv[b].copy_(dev(c["cstate_kv"]))
                cache.cstate_gate[b].copy_(dev(c["cstate_gate"]))
                if spec.has_indexer:
                    cache.ipool[b, :P].copy_(dev(c["ipool"]))
                    cache.istate_kv[b].copy_(dev(c["istate_kv"]))
                    cache.istate_gate[b].copy_(dev(c["istate_gate"]))
            del c
        new = synth.prefill_inputs(w, 0, li)
        a = {k: dev(v) for k, v in new.items()}
        p0 = torch.full((B,), pos0, dtype=torch.int64, device="cuda")
        out, idx = layer_step(cache, p0, pos0, a["q"], a["kv"], a.get("ckv"), a.get("cgate"),
                              a.get("ikv"), a.get("igate"), a.get("qi"), a.get("wi"), a["sinks"])
        torch.cuda.synchronize()
        for b in seqs_checked:
            nb = {k: (to_f64(v) if k == "sinks" else to_f64(v[b, 0])) for k, v in new.items()}
            c = synth.decode_cache_seq(w, 0, li, b, names=[n for n in names if n != "pool"])
            cc = {k: to_f64(v) for k, v in c.items()}
            if spec.ratio:
                cc["pool"] = LazyF64(synth.decode_cache_seq(w, 0, li, b, names=["pool"])["pool"])
            ref = O.decode_step(spec, pos0, nb, cc)
            if spec.has_indexer:
                nv = (pos0 + 1) // spec.ratio
                keys = cc["ipool"][:nv]
                sc, ab = index_exact(spec, nb["qi"], nb["wi"], keys, pos0)
                nd = audit_topk(idx[b, 0].cpu().numpy(), ref["idx"], sc, ab, spec.index_dim,
                                spec.index_heads)
                if nd:
                    say(f"    seq {b}: {nd} near-tie differences; re-attend with oracle ids")
                    idx2 = idx.clone()
                    idx2[b, 0] = torch.from_numpy(ref["idx"].astype(np.int32)).cuda()
                    m.csa_attend(L, p0, pos0, a["q"], cache.ring, cache.pool, idx2, a["sinks"],
                                 out, cache.workspace(1, m.CSA_OP_ATTEND))
                    torch.cuda.synchronize()
            err = assert_close(host(out[b, 0]), ref["out"], "bf16", f"decode seq {b}")
            say(f"    seq {b}: max abs err {err:.3e}")
        del cache, a


def test_csa_decode_full_b64_t131072(csa):
    say("case: csa_decode full B=64 t=131072")
    _decode_full(csa, "csa_decode", [0, 37, 63])


def test_mixed_decode_full_b4_t1m(csa):
    say("case: mixed_decode full B=4 t=1048576 (CSA, HCA, sliding)")
    _decode_full(csa, "mixed_decode", [0, 3])
