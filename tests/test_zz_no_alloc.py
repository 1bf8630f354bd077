"""csa_index_topk_noalloc (the entry point for callers that cannot allocate:
HIP graph capture, tight serving loops) against csa_index_topk with a
workspace, through the C ABI: identical ids and scores on consecutive calls
that share the library's static scratch, each smaller than the one before,
on the decode paths (rows beyond 32768 keys, the one-launch selection) and
the prefill path; a call needing more than the scratch is refused."""
import numpy as np
import pytest

import synth
from tests.helpers import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def csa():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import long_context_sparse_gated_amd as m
    m.load_library()
    return m


def _inputs(B, n, pool, distinct, seed):
    import torch
    qs, ks, ws = [], [], []
    for b in range(B):
        q, k, w = synth.grid_index_inputs(n, pool, 64, 128, 64, seed=seed + 31 * b,
                                          distinct_rows=distinct)
        qs.append(q)
        ks.append(k)
        ws.append(w)
    bf = torch.bfloat16
    return (torch.from_numpy(np.stack(qs)).to(bf).cuda(),
            torch.from_numpy(np.stack(ws)).to(bf).cuda(),
            torch.from_numpy(np.stack(ks)).to(bf).cuda())


# (B, n_new, pool entries, pos0, distinct key rows): each call smaller than the last
CALLS = [(4, 1, 262144, 1048575, 0),   # rows beyond 32768 keys: collect + final selection
         (8, 1, 30000, 119999, 5),     # one-launch selection, tie-heavy keys
         (2, 1, 5000, 19999, 0),       # one-launch selection
         (1, 300, 75, 0, 0)]           # prefill scoring and selection


def test_noalloc_index_topk_matches_workspace_entry(csa):
    import torch
    m = csa
    spec = synth.LayerSpec(kind="csa", dtype="bf16")
    L = m.Layer.from_spec(spec)
    for B, n, pool, pos0, distinct in CALLS:
        say(f"case: noalloc index_topk B={B} n={n} pool={pool} pos0={pos0} distinct={distinct}")
        need = m.csa_workspace_bytes(L, B, n, pool, m.CSA_OP_INDEX_TOPK)
        assert need <= m.CSA_NOALLOC_SCRATCH_BYTES
        q, w, k = _inputs(B, n, pool, distinct, seed=B * 1000 + n)
        p0 = torch.full((B,), pos0, dtype=torch.int64, device="cuda")
        ref = torch.full((B, n, spec.topk), -7, dtype=torch.int32, device="cuda")
        got = torch.full_like(ref, -9)
        sref = torch.zeros(B, n, pool, dtype=torch.float32, device="cuda")
        sgot = torch.ones_like(sref)
        m.csa_index_topk(L, p0, pos0, q, w, k, ref, scores_out=sref)
        m.csa_index_topk_noalloc(L, p0, pos0, q, w, k, got, scores_out=sgot)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), "ids differ from the workspace entry point"
        for b in range(B):
            for i in range(n):
                nv = min((pos0 + i + 1) // 4, pool)
                assert torch.equal(sgot[b, i, :nv], sref[b, i, :nv]), "scores differ"
        # without scores_out the scores live in the scratch as well
        got2 = torch.full_like(ref, -9)
        m.csa_index_topk_noalloc(L, p0, pos0, q, w, k, got2)
        torch.cuda.synchronize()
        assert torch.equal(got2, ref), "ids differ (scores in the scratch)"
        del q, w, k, sref, sgot


def test_noalloc_refuses_calls_beyond_the_scratch(csa):
    import torch
    m = csa
    spec = synth.LayerSpec(kind="csa", dtype="bf16")
    L = m.Layer.from_spec(spec)
    B, n, pool = 1, 8192, 2048           # prefill of 8192 tokens: 64 MiB of scores
    assert m.csa_workspace_bytes(L, B, n, pool, m.CSA_OP_INDEX_TOPK) > m.CSA_NOALLOC_SCRATCH_BYTES
    say("case: noalloc index_topk beyond the scratch is refused")
    q = torch.zeros(B, n, 64, 128, dtype=torch.bfloat16, device="cuda")
    w = torch.zeros(B, n, 64, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(B, pool, 128, dtype=torch.bfloat16, device="cuda")
    idx = torch.full((B, n, spec.topk), -5, dtype=torch.int32, device="cuda")
    p0 = torch.zeros(B, dtype=torch.int64, device="cuda")
    with pytest.raises(RuntimeError, match="CSA_ERR_SCRATCH"):
        m.csa_index_topk_noalloc(L, p0, 0, q, w, k, idx)
    torch.cuda.synchronize()
    assert bool((idx == -5).all()), "a refused call writes nothing"
