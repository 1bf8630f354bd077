"""Throughput of the compressed-attention layer hot path on one MI355X.

Headline (``value``): the CSA prefill layer, bf16, B=1, S=8192, 64 query
heads, one shared K=V head, head_dim 512 (64 rope channels, base 160000),
window 128, compressor m=4 with overlapping windows (2048 entries), indexer
64 heads x 128 with top-512.  One step = the whole hot path for the 8192
tokens: window append (RoPE of the K=V rows), the main and indexer
compressors, indexer scores + top-k, and the sparse attention with sink and
output un-rotation.

The same JSON line carries, under ``workloads``, the other layer shapes timed
the same way (one step = every call of the layer(s) for one batch):

* ``hca_prefill``  S=65536, m'=128 non-overlapping pooling, dense attention
                   over the window and every visible entry;
* ``csa_decode``   64 sequences x 1 token at position 131072 (32768 entries);
* ``mixed_decode`` 4 sequences x 1 token at position 1048576 through a CSA
                   layer (262144 entries), an HCA layer (8192 entries) and a
                   sliding-only layer;
* ``output_projection`` the grouped low-rank output projection of the 8192
                   prefill tokens (8 groups of 8 heads x 512 -> rank 1024 each
                   -> hidden 4096), priced in its two products' MFMA FLOPs;
* ``projections`` the producer projections of the same 8192 tokens (hidden
                   4096 -> query latent 1024, kv 512, compressor 2 x 512, indexer
                   2 x 128 + 64 head weights; latent -> 64 x 512 queries and 64 x
                   128 indexer queries; the norms), priced in MFMA FLOPs;
* ``varlen_prefill`` a padded batch of four CSA sequences of 2048, 1536, 768
                   and 256 valid tokens (padded to 2048), in valid tokens/s.

Prefill steps are priced in MFMA FLOPs (4 H D per attended (query, row)
pair, plus 2 H_I D_I per scored (query, key) pair); decode steps in the HBM
bytes the step must move at least once (new-token inputs and outputs, cache
rows read, cache slots written).  A decode step is replayed as one captured
HIP graph (its eager time is reported beside it).  Inputs are seeded synthetic tensors
(``synth``), resident in HBM before timing starts.  The attention launch of
the headline step is timed with HIP events on its stream inside the timed
region (``roofline``); ``cpu_baseline`` is the CPU oracle's rate on a bounded
sample of the headline workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E


def attended_rows(S, W, m, k):
    """Sum over queries t < S of (window rows + attended entries); k=0: all visible."""
    tot = 0
    for t in range(S):
        nv = (t + 1) // m if m else 0
        tot += min(W, t + 1) + (min(k, nv) if k else nv)
    return tot


def scored_pairs(S, m):
    return sum((t + 1) // m for t in range(S))


def prefill_flops(spec, S):
    attn = 4.0 * spec.num_heads * spec.head_dim * attended_rows(
        S, spec.window, spec.ratio, spec.topk if spec.has_indexer else 0)
    idx = (2.0 * spec.index_heads * spec.index_dim * scored_pairs(S, spec.ratio)
           if spec.has_indexer else 0.0)
    return attn, idx


def decode_bytes(spec, B, t):
    """HBM bytes one decode call of one token per sequence must move."""
    e = 2 if spec.dtype == "bf16" else 4
    H, D = spec.num_heads, spec.head_dim
    per = 2 * H * D * e + 2 * D * e + min(spec.window, t + 1) * D * e + H * 4
    if spec.ratio:
        Ls = (1 + spec.overlap) * spec.ratio
        emit = (t + 1) % spec.ratio == 0
        widths = [D] + ([spec.index_dim] if spec.has_indexer else [])
        for wd in widths:
            per += 4 * wd * e                       # new kv+gate read, state slot written
            if emit:
                per += 2 * (Ls - 1) * wd * e + wd * e   # state rows read, entry written
        nv = (t + 1) // spec.ratio
        if spec.has_indexer:
            Hi, Di = spec.index_heads, spec.index_dim
            per += Hi * Di * e + Hi * e + nv * Di * e   # indexer query, weights, keys
            per += 2 * spec.topk * 4                    # ids written, read back
            per += min(spec.topk, nv) * D * e          # selected entries
        else:
            per += nv * D * e                          # every visible entry
    return B * per


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attend_mfma_csa_prefill_S8192_traffic.json")


def measured_traffic():
    """HBM bytes per attention launch from the committed counter profile, or None
    when the kernel sources changed since the counters were taken."""
    import hashlib
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
        h = hashlib.sha256()
        for src in rec["sources"]:
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
        if h.hexdigest() != rec["sources_sha256"]:
            return None
        return rec["read_bytes"] + rec["write_bytes"]
    except (OSError, KeyError, ValueError):
        return None


def host_info():
    """The host cores this process may use, the CPU model and numpy's BLAS."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas, threads = "unknown", 1
    try:
        from threadpoolctl import threadpool_info
        info = [d for d in threadpool_info() if d.get("user_api") == "blas"]
        if info:
            blas = f"{info[0].get('internal_api')} {info[0].get('version')}"
            threads = max(d.get("num_threads", 1) for d in info)
    except Exception:  # pragma: no cover
        pass
    return {"cpu_model": model, "host_cores": len(os.sched_getaffinity(0)), "blas": blas,
            "blas_threads": int(threads)}


def _baseline(value, unit, dt, sample):
    h = host_info()
    return {"value": value, "unit": unit, "cores": h["blas_threads"], "kind": "oracle",
            "sample": f"{sample}; {dt:.1f} s of oracle time", **h}


def cpu_baseline(spec, inp, stride):
    """The oracle as it stands, on every `stride`-th query of the same layer."""
    from oracle import csa_oracle as O
    from synth import to_f64
    x = {k: (to_f64(v) if k == "sinks" else to_f64(v[0])) for k, v in inp.items()}
    S = x["q"].shape[0]
    qs = list(range(S - 1, -1, -stride))
    t0 = time.perf_counter()
    O.csa_prefill(spec, x, queries=qs)
    dt = time.perf_counter() - t0
    return _baseline(len(qs) / dt, "tokens/s", dt,
                     f"csa_prefill S={S}: full compressor passes + every {stride}-th query "
                     f"({len(qs)} queries, incl. the last)")


class _Rows:
    """Float64 view of a stored tensor, decoded where indexed (bounded memory)."""

    def __init__(self, arr):
        self.arr, self.shape = arr, arr.shape

    def __getitem__(self, i):
        from synth import to_f64
        return to_f64(self.arr[i])


def cpu_baseline_hca(spec, inp, nq=256):
    """The oracle on the HCA S=65536 layer: full compressor and window passes,
    then nq queries spread over the sequence (rows decoded as gathered)."""
    import numpy as np
    from oracle import csa_oracle as O
    from synth import to_f64
    S = inp["q"].shape[1]
    x = {"q": _Rows(inp["q"][0]), "kv": to_f64(inp["kv"][0]), "ckv": to_f64(inp["ckv"][0]),
         "cgate": to_f64(inp["cgate"][0]), "sinks": to_f64(inp["sinks"])}
    qs = sorted(set(np.linspace(0, S - 1, nq).astype(int).tolist()))
    t0 = time.perf_counter()
    O.hca_prefill(spec, x, queries=qs)
    dt = time.perf_counter() - t0
    return _baseline(len(qs) / dt, "tokens/s", dt,
                     f"hca_prefill S={S}: full compressor and window passes + {len(qs)} "
                     "queries spread over the sequence")


def cpu_baseline_decode(name, seqs):
    """The oracle's decode step of the first `seqs` sequences of a decode
    workload, every layer; the cache draws are not timed."""
    import synth
    from oracle import csa_oracle as O
    from synth import to_f64
    w = synth.workload(name)
    t, dt = w.pos0, 0.0
    for li, spec in enumerate(w.layers):
        new_all = synth.prefill_inputs(w, 0, li)
        for b in range(seqs):
            names = list(synth.cache_shapes(w, li))
            c = synth.decode_cache_seq(w, 0, li, b, names=[n for n in names if n != "pool"])
            cache = {k: to_f64(v) for k, v in c.items()}
            if spec.ratio:
                cache["pool"] = _Rows(synth.decode_cache_seq(w, 0, li, b, names=["pool"])["pool"])
            new = {k: (to_f64(v) if k == "sinks" else to_f64(v[b, 0]))
                   for k, v in new_all.items()}
            t0 = time.perf_counter()
            O.decode_step(spec, t, new, cache)
            dt += time.perf_counter() - t0
            del c, cache
    return _baseline(seqs / dt, "tokens/s", dt,
                     f"{name}: {seqs} of {w.batch} sequences at t={t}, every layer")


def _dev(torch, a):
    import numpy as np
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def _time_steps(torch, step, steps, warmup, attn_events=False):
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        step(None)
    torch.cuda.synchronize()
    evs = ([(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(steps)] if attn_events else [None] * steps)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(steps):
        step(evs[i])
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    attn = (sum(a.elapsed_time(b) for a, b in evs) / steps) if attn_events else None
    return ms, attn


def prefill_leg(torch, m, name, steps, warmup, attn_events=False):
    import synth
    from long_context_sparse_gated_amd.layer import LayerCache
    w = synth.workload(name)
    spec, S = w.layers[0], w.n_new
    inp = synth.prefill_inputs(w, 0)
    L = m.Layer.from_spec(spec)
    a = {k: _dev(torch, v) for k, v in inp.items()}
    cache = LayerCache(L, 1, S, S // spec.ratio)
    pos0 = torch.zeros(1, dtype=torch.int64, device="cuda")
    out = torch.empty_like(a["q"])
    stream = torch.cuda.current_stream()
    if spec.has_indexer:
        idx = torch.empty(1, S, spec.topk, dtype=torch.int32, device="cuda")
        ws_i = cache.workspace(S, m.CSA_OP_INDEX_TOPK)
        ws_a = cache.workspace(S, m.CSA_OP_ATTEND)
    else:
        ws_a = cache.workspace(S, m.CSA_OP_HCA_ATTEND)

    # every step prefills the same sequence from position 0 (a prefill from 0
    # never reads the compressor state, so steps are identical)
    # the caches' update (window append, the compressor of each stream) is
    # one call, as in the layer step
    istreams = {}
    if spec.has_indexer:
        istreams = dict(ikv=a["ikv"], igate=a["igate"], istate_kv=cache.istate_kv,
                        istate_gate=cache.istate_gate, ipool=cache.ipool)

    def step(ev):
        m.csa_cache_update(L, pos0, 0, a["kv"], cache.ring, a["ckv"], a["cgate"], cache.cstate_kv,
                           cache.cstate_gate, cache.pool, **istreams)
        if spec.has_indexer:
            m.csa_index_topk(L, pos0, 0, a["qi"], a["wi"], cache.ipool, idx, workspace=ws_i)
        if ev is not None:
            ev[0].record(stream)
        if spec.has_indexer:
            m.csa_attend(L, pos0, 0, a["q"], cache.ring, cache.pool, idx, a["sinks"], out, ws_a)
        else:
            m.hca_attend(L, pos0, 0, a["q"], cache.ring, cache.pool, a["sinks"], out, ws_a)
        if ev is not None:
            ev[1].record(stream)

    ms, attn_ms = _time_steps(torch, step, steps, warmup, attn_events)
    f_attn, f_idx = prefill_flops(spec, S)
    res = {"ms_per_step": ms, "tokens_per_s": S / (ms * 1e-3),
           "step_tflops": (f_attn + f_idx) / (ms * 1e-3) / 1e12,
           "step_frac_bf16_peak": (f_attn + f_idx) / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
           "attend_flop": f_attn, "index_flop": f_idx}
    if attn_ms is not None:
        res["attend_ms"] = attn_ms
    del a, cache, out
    return spec, inp, res


def _block_table(torch, B, per_seq, seed):
    """A shuffled block table: B sequences x per_seq blocks over B per_seq blocks."""
    import numpy as np
    ids = np.random.default_rng(seed).permutation(B * per_seq).reshape(B, per_seq)
    return torch.from_numpy(ids.astype(np.int32)).cuda(), ids


def decode_leg(torch, m, name, steps, warmup, paged=False):
    """One decode step of every layer of the workload, replayed as a HIP graph.
    paged: each layer's pools live in blocks (256 entries for CSA layers, 128
    for HCA layers) of one tensor per layer, mapped by a shuffled table."""
    import numpy as np
    import synth
    from long_context_sparse_gated_amd.layer import LayerCache, layer_step
    w = synth.workload(name)
    t, B = w.pos0, w.batch
    layers, total_bytes = [], 0
    for li, spec in enumerate(w.layers):
        L = m.Layer.from_spec(spec)
        pool_cap = (t + 1) // spec.ratio if spec.ratio else 1
        kw, tab_h, E = {}, None, 0
        if paged and spec.ratio:
            E = 256 if spec.has_indexer else 128
            per = (pool_cap + E - 1) // E
            tab, tab_h = _block_table(torch, B, per, seed=li)
            kw = dict(block_entries=E, pool_blocks=B * per, block_table=tab)
        cache = LayerCache(L, B, spec.window, pool_cap, **kw)
        for b in range(B):  # one sequence at a time keeps host memory bounded
            c = synth.decode_cache_seq(w, 0, li, b)
            cache.ring[b].copy_(_dev(torch, c["win"]))
            if spec.ratio:
                P = t // spec.ratio
                if tab_h is not None:
                    j = np.arange(P)
                    rows = torch.from_numpy(tab_h[b][j // E] * E + j % E).cuda()
                    cache.pool[rows] = _dev(torch, c["pool"])
                    if spec.has_indexer:
                        cache.ipool[rows] = _dev(torch, c["ipool"])
                    del rows
                else:
                    cache.pool[b, :P].copy_(_dev(torch, c["pool"]))
                    if spec.has_indexer:
                        cache.ipool[b, :P].copy_(_dev(torch, c["ipool"]))
                cache.cstate_kv[b].copy_(_dev(torch, c["cstate_kv"]))
                cache.cstate_gate[b].copy_(_dev(torch, c["cstate_gate"]))
                if spec.has_indexer:
                    cache.istate_kv[b].copy_(_dev(torch, c["istate_kv"]))
                    cache.istate_gate[b].copy_(_dev(torch, c["istate_gate"]))
            del c
        a = {k: _dev(torch, v) for k, v in synth.prefill_inputs(w, 0, li).items()}
        out = torch.empty_like(a["q"])
        idx = (torch.empty(B, 1, spec.topk, dtype=torch.int32, device="cuda")
               if spec.has_indexer else None)
        layers.append((cache, a, out, idx))
        total_bytes += decode_bytes(spec, B, t)
    p0 = torch.full((B,), t, dtype=torch.int64, device="cuda")

    # every step decodes the same token at the same position: the window slot,
    # the compressor state slot and (when an entry closes) the pool entry are
    # rewritten with the same values, so steps are identical
    def step(_ev):
        for cache, a, out, idx in layers:
            layer_step(cache, p0, t, a["q"], a["kv"], a.get("ckv"), a.get("cgate"),
                       a.get("ikv"), a.get("igate"), a.get("qi"), a.get("wi"), a["sinks"],
                       out=out, topk_idx=idx)

    eager_ms, _ = _time_steps(torch, step, steps, warmup)
    # a decode step is a short chain of small launches: replay it as one HIP
    # graph (captured after the warmup above, which also sized the workspaces)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(None)
    torch.cuda.synchronize()
    ms, _ = _time_steps(torch, lambda _ev: graph.replay(), steps, warmup)
    gbs = total_bytes / (ms * 1e-3) / 1e9
    del graph, layers
    torch.cuda.empty_cache()
    res = {"ms_per_step": ms, "tokens_per_s": B / (ms * 1e-3), "algorithmic_bytes": total_bytes,
           "achieved_GBs": gbs, "frac_hbm_peak": gbs / PEAK_HBM_GBS, "hip_graph": True,
           "eager_ms_per_step": eager_ms}
    if paged:
        res["paged"] = "pools in shuffled blocks: 256 entries (CSA layers), 128 (HCA layers)"
    return res


def oproj_leg(torch, m, steps, warmup):
    import synth
    s = synth.OPROJ_SHAPE
    T, H, D, G, R, hidden = s["T"], s["H"], s["D"], s["G"], s["R"], s["hidden"]
    inp = synth.oproj_inputs(T, H, D, G, R, hidden, seed=0)
    x, wa, wb = (_dev(torch, inp[k]) for k in ("x", "w_a", "w_b"))
    out = torch.empty(T, hidden, dtype=torch.bfloat16, device="cuda")
    need = m.load_library().csa_output_projection_workspace_bytes(
        m._COproj(T, H, D, G, R, hidden))
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    ms, _ = _time_steps(torch, lambda _ev: m.csa_output_projection(x, wa, wb, out, G, ws), steps,
                        warmup)
    flop = 2.0 * T * G * R * ((H // G) * D + hidden)
    tf = flop / (ms * 1e-3) / 1e12
    del x, wa, wb, out, ws
    return {"ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3), "algorithmic_flop": flop,
            "achieved_TFLOPs": tf, "frac_bf16_peak": tf / PEAK_BF16_TFLOPS, **s}


VARLEN_LENS = (2048, 1536, 768, 256)


def varlen_leg(torch, m, steps, warmup):
    """A padded batch of four CSA sequences of different valid lengths (one
    layer call each step, from position 0), priced in valid tokens."""
    import synth
    from long_context_sparse_gated_amd.layer import LayerCache, layer_step
    S, B = max(VARLEN_LENS), len(VARLEN_LENS)
    w = synth.workload("csa_prefill", S=S, batch=B)
    spec = w.layers[0]
    inp = synth.prefill_inputs(w, 0)
    L = m.Layer.from_spec(spec)
    keys = ("q", "kv", "ckv", "cgate", "ikv", "igate", "qi", "wi")
    a = {k: _dev(torch, inp[k]) for k in keys}
    sinks = _dev(torch, inp["sinks"])
    cache = LayerCache(L, B, S, S // spec.ratio)
    p0 = torch.zeros(B, dtype=torch.int64, device="cuda")
    nv = torch.tensor(VARLEN_LENS, dtype=torch.int32, device="cuda")
    out = torch.empty_like(a["q"])
    idx = torch.empty(B, S, spec.topk, dtype=torch.int32, device="cuda")
    ms, _ = _time_steps(torch, lambda _ev: layer_step(
        cache, p0, 0, *(a[k] for k in keys), sinks, out=out, topk_idx=idx, n_valid=nv), steps,
        warmup)
    valid = sum(VARLEN_LENS)
    del a, cache, out, idx
    return {"ms_per_step": ms, "valid_tokens_per_s": valid / (ms * 1e-3),
            "lens": list(VARLEN_LENS), "padded_to": S,
            "note": "the prefill scoring, selection and attention kernels skip padding rows "
                    "(left unspecified); the caches advance by the valid tokens"}


def packed_leg(torch, m, steps, warmup):
    """The same four CSA sequences as varlen_prefill with packed rows
    (cu_seqlens, no padding rows), priced in tokens."""
    import numpy as np
    import synth
    from long_context_sparse_gated_amd.layer import LayerCache, layer_step
    S, B = max(VARLEN_LENS), len(VARLEN_LENS)
    w = synth.workload("csa_prefill", S=S, batch=B)
    spec = w.layers[0]
    inp = synth.prefill_inputs(w, 0)
    L = m.Layer.from_spec(spec)
    keys = ("q", "kv", "ckv", "cgate", "ikv", "igate", "qi", "wi")
    a = {k: torch.cat([_dev(torch, inp[k][b, :n]) for b, n in enumerate(VARLEN_LENS)])
         for k in keys}
    sinks = _dev(torch, inp["sinks"])
    cache = LayerCache(L, B, S, S // spec.ratio)
    p0 = torch.zeros(B, dtype=torch.int64, device="cuda")
    cu = torch.tensor(np.r_[0, np.cumsum(VARLEN_LENS)], dtype=torch.int32, device="cuda")
    out = torch.empty_like(a["q"])
    idx = torch.empty(a["q"].shape[0], spec.topk, dtype=torch.int32, device="cuda")
    ms, _ = _time_steps(torch, lambda _ev: layer_step(
        cache, p0, 0, *(a[k] for k in keys), sinks, out=out, topk_idx=idx, cu_seqlens=cu,
        n_new=S), steps, warmup)
    valid = sum(VARLEN_LENS)
    del a, cache, out, idx
    return {"ms_per_step": ms, "tokens_per_s": valid / (ms * 1e-3), "lens": list(VARLEN_LENS),
            "note": "packed rows: every per-token tensor holds the sequences back to back"}


def proj_leg(torch, m, steps, warmup):
    import synth
    s = synth.PROJ_SHAPE
    T, hid, ql, H, D, comp, Di, Hi = (s[k] for k in ("T", "hidden", "q_lora", "H", "D", "comp",
                                                     "Di", "Hi"))
    inp = synth.proj_inputs(T, hid, ql, H, D, comp, Di, Hi, seed=0)
    a = {k: _dev(torch, v) for k, v in inp.items()}
    bf = torch.bfloat16
    outs = {"q": torch.empty(T, H, D, dtype=bf, device="cuda"),
            "kv": torch.empty(T, D, dtype=bf, device="cuda"),
            "ckv": torch.empty(T, comp, dtype=bf, device="cuda"),
            "cgate": torch.empty(T, comp, dtype=bf, device="cuda"),
            "ikv": torch.empty(T, Di, dtype=bf, device="cuda"),
            "igate": torch.empty(T, Di, dtype=bf, device="cuda"),
            "qi": torch.empty(T, Hi, Di, dtype=bf, device="cuda"),
            "wi": torch.empty(T, Hi, dtype=bf, device="cuda")}
    need = m.load_library().csa_project_workspace_bytes(
        m._CProj(T, hid, ql, H, D, comp, Di, Hi, 1e-6, 1))
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")

    def step(_ev):
        m.csa_project(a["x"], a["w_x"], a["g_qa"], a["g_kv"], a["w_q"], outs, q_lora_rank=ql,
                      num_heads=H, head_dim=D, comp_dim=comp, index_dim=Di, index_heads=Hi,
                      eps=1e-6, q_head_norm=True, workspace=ws)

    ms, _ = _time_steps(torch, step, steps, warmup)
    nx = ql + D + 2 * comp + 2 * Di + Hi
    nq = H * D + Hi * Di
    flop = 2.0 * T * (nx * hid + nq * ql)
    tf = flop / (ms * 1e-3) / 1e12
    del a, outs, ws
    return {"ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3), "algorithmic_flop": flop,
            "achieved_TFLOPs": tf, "frac_bf16_peak": tf / PEAK_BF16_TFLOPS, **s}


def calib_copy(torch, mib):
    if mib <= 0:
        return
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


BASELINE_SEQS = {"csa_decode": 16, "mixed_decode": 2}   # sequences the oracle decodes
_HCA_INPUTS = []


def run_leg(torch, m, name, args):
    if name in ("csa_prefill", "hca_prefill"):
        steps = args.steps if name == "csa_prefill" else max(2, args.steps // 4)
        spec, inp, r = prefill_leg(torch, m, name, steps, min(args.warmup, 1 if
                                   name == "hca_prefill" else args.warmup), attn_events=True)
        if name == "hca_prefill" and not args.no_cpu_baseline:
            _HCA_INPUTS.append((spec, inp))
        del inp
        r["roofline"] = {"bound": "mfma", "kernel": "attend_mfma",
                         "achieved": r["attend_flop"] / (r["attend_ms"] * 1e-3) / 1e12,
                         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
        r["roofline"]["frac"] = r["roofline"]["achieved"] / PEAK_BF16_TFLOPS
        return r
    if name in ("csa_decode", "mixed_decode"):
        return decode_leg(torch, m, name, 5 * args.steps, args.warmup)
    if name in ("csa_decode_paged", "mixed_decode_paged"):
        return decode_leg(torch, m, name[:-len("_paged")], 5 * args.steps, args.warmup,
                          paged=True)
    if name == "packed_prefill":
        return packed_leg(torch, m, args.steps, args.warmup)
    if name == "output_projection":
        return oproj_leg(torch, m, args.steps, args.warmup)
    if name == "projections":
        return proj_leg(torch, m, args.steps, args.warmup)
    if name == "varlen_prefill":
        return varlen_leg(torch, m, args.steps, args.warmup)
    raise SystemExit(f"unknown workload {name}")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-stride", type=int, default=1)
    ap.add_argument("--legs",
                    default="hca_prefill,csa_decode,mixed_decode,mixed_decode_paged,"
                            "output_projection,projections,varlen_prefill,packed_prefill",
                    help="comma list of further workloads to time after the headline "
                         "(hca_prefill, csa_decode, mixed_decode, csa_decode_paged, "
                         "mixed_decode_paged, output_projection, projections, varlen_prefill, "
                         "packed_prefill; empty for none)")
    ap.add_argument("--only", default="",
                    help="time just this one workload and print its object (profiling runs)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (untimed), so a "
                         "counter run can scale HBM byte counters against a known size")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the path has no "
              "multi-GPU mode in this library", file=sys.stderr)
        sys.exit(2)

    import torch
    import long_context_sparse_gated_amd as m
    m.load_library()

    if args.only:
        r = run_leg(torch, m, args.only, args)
        calib_copy(torch, args.calib_copy_mib)
        print(json.dumps({"workload": args.only, **r}), flush=True)
        return

    spec, inp, head = prefill_leg(torch, m, "csa_prefill", args.steps, args.warmup,
                                  attn_events=True)
    calib_copy(torch, args.calib_copy_mib)
    torch.cuda.empty_cache()

    legs = {}
    for name in [x for x in args.legs.split(",") if x]:
        legs[name] = run_leg(torch, m, name, args)
        torch.cuda.empty_cache()
        if not args.no_cpu_baseline and name in BASELINE_SEQS:
            legs[name]["cpu_baseline"] = cpu_baseline_decode(name, BASELINE_SEQS[name])
        if not args.no_cpu_baseline and name == "hca_prefill":
            legs[name]["cpu_baseline"] = cpu_baseline_hca(*_HCA_INPUTS.pop())

    S = 8192
    achieved = head["attend_flop"] / (head["attend_ms"] * 1e-3) / 1e12
    res = {
        "metric": "CSA prefill tokens/s @S=8192",
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "csa_prefill", "batch": 1, "seq_len": S, "heads": 64,
                   "head_dim": 512, "rope_dim": 64, "window": 128, "compress_ratio": 4,
                   "index_heads": 64, "index_dim": 128, "index_topk": 512,
                   "rope_theta": spec.rope_theta, "rope_factor": spec.rope_factor,
                   "rope_original_context": spec.rope_original_context},
        "roofline": {"bound": "mfma", "kernel": "attend_mfma", "achieved": achieved,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": measured_traffic(),
                     "launch_ms": head["attend_ms"], "algorithmic_flop": head["attend_flop"]},
        "attend_share_of_step": head["attend_ms"] / head["ms_per_step"],
        "step_frac_bf16_peak": head["step_frac_bf16_peak"],
        "workloads": legs,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(spec, inp, args.cpu_stride)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
