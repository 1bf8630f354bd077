"""Throughput of the CSA layer hot path on one MI355X.

Workload: the CSA prefill layer, bf16, B=1, S=8192, 64 query heads, one shared
K=V head, head_dim 512 (64 rope channels, base 160000), window 128,
compressor m=4 with overlapping windows (2048 entries), indexer 64 heads x
128 with top-512.  Inputs are seeded synthetic tensors (synth.prefill_inputs,
seed 0), resident in HBM before timing starts.

One step = the whole hot path for the 8192 tokens: window append (RoPE of the
K=V rows), the main and indexer compressors, indexer scores + top-k, and the
sparse attention with sink and output un-rotation.

Printed JSON (one line): tokens/s of the step; the roofline of the dominant
kernel (the attention launch, timed with HIP events on its stream inside the
timed region; algorithmic FLOPs = 4 * H * D * sum over queries of attended
rows); the CPU oracle's rate on a bounded sample (``cpu_baseline``).
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
    """Sum over queries t < S of (window rows + selected entries)."""
    tot = 0
    for t in range(S):
        tot += min(W, t + 1) + min(k, (t + 1) // m)
    return tot


def cpu_baseline(spec, inp, stride):
    """The oracle as it stands, on every `stride`-th query of the same layer."""
    from oracle import csa_oracle as O
    from synth import to_f64
    try:
        from threadpoolctl import threadpool_info
        blas = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas = 1
    x = {k: (to_f64(v) if k == "sinks" else to_f64(v[0])) for k, v in inp.items()}
    S = x["q"].shape[0]
    qs = list(range(S - 1, -1, -stride))
    t0 = time.perf_counter()
    O.csa_prefill(spec, x, queries=qs)
    dt = time.perf_counter() - t0
    return {"value": len(qs) / dt, "unit": "tokens/s", "cores": int(blas),
            "kind": "oracle",
            "sample": f"csa_prefill S={S}: full compressor passes + every {stride}-th query "
                      f"({len(qs)} queries, incl. the last), {dt:.1f} s on "
                      f"{len(os.sched_getaffinity(0))} host cores"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-stride", type=int, default=1)
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (untimed), so a "
                         "counter run can scale HBM byte counters against a known size")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the path has no "
              "multi-GPU mode in this library", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import long_context_sparse_gated_amd as m
    from long_context_sparse_gated_amd.layer import LayerCache, layer_step

    w = synth.workload("csa_prefill")
    spec = w.layers[0]
    S = w.n_new
    inp = synth.prefill_inputs(w, 0)
    m.load_library()
    L = m.Layer.from_spec(spec)

    def dev(a):
        import numpy as np
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(a).cuda()

    a = {k: dev(v) for k, v in inp.items()}
    cache = LayerCache(L, 1, S, S // spec.ratio)
    pos0 = torch.zeros(1, dtype=torch.int64, device="cuda")
    out = torch.empty_like(a["q"])
    idx = torch.empty(1, S, spec.topk, dtype=torch.int32, device="cuda")
    ws_i = cache.workspace(S, m.CSA_OP_INDEX_TOPK)
    ws_a = cache.workspace(S, m.CSA_OP_ATTEND)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        m.csa_window_append(L, pos0, 0, a["kv"], cache.ring)
        m.csa_compress(L, pos0, 0, a["ckv"], a["cgate"], cache.cstate_kv, cache.cstate_gate,
                       cache.pool, spec.rope_dim)
        m.csa_compress(L, pos0, 0, a["ikv"], a["igate"], cache.istate_kv, cache.istate_gate,
                       cache.ipool, spec.index_rope_dim)
        m.csa_index_topk(L, pos0, 0, a["qi"], a["wi"], cache.ipool, idx, workspace=ws_i)
        if ev is not None:
            ev[0].record(stream)
        m.csa_attend(L, pos0, 0, a["q"], cache.ring, cache.pool, idx, a["sinks"], out, ws_a)
        if ev is not None:
            ev[1].record(stream)

    # every step prefills the same sequence from position 0 (a prefill from 0
    # never reads the compressor state, so steps are identical)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        step(evs[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_step = total_ms / args.steps
    attn_ms = sum(e0.elapsed_time(e1) for e0, e1 in evs) / args.steps

    rows = attended_rows(S, spec.window, spec.ratio, spec.topk)
    flops = 4.0 * spec.num_heads * spec.head_dim * rows
    achieved = flops / (attn_ms * 1e-3) / 1e12
    res = {
        "metric": "CSA prefill tokens/s @S=8192",
        "value": S / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "csa_prefill", "batch": 1, "seq_len": S, "heads": 64,
                   "head_dim": 512, "rope_dim": 64, "window": 128, "compress_ratio": 4,
                   "index_heads": 64, "index_dim": 128, "index_topk": 512},
        "roofline": {"bound": "mfma", "kernel": "attend_mfma", "achieved": achieved,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": None,
                     "launch_ms": attn_ms, "algorithmic_flop": flops},
        "attend_share_of_step": attn_ms / ms_step,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(spec, inp, args.cpu_stride)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
