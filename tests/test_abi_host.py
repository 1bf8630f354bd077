"""Host-side checks of the C ABI: the library loads, exports every entry point
include/csa.h declares, sizes workspaces, and rejects bad arguments before any
launch.  Every call here fails validation or computes a size, so nothing
reaches a device (the pointers passed are never dereferenced)."""
import ctypes
import os
import re

import pytest

import long_context_sparse_gated_amd as m
from long_context_sparse_gated_amd import _CBatch, _CLayer

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: each call below is rejected first


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(m.library_path()):
        pytest.skip("libcsa.so not built")
    return m.load_library()


def declared_functions():
    src = open(os.path.join(ROOT, "include", "csa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:csa_status|size_t|const char\*|int32_t)\s+(\w+)\s*\(",
                                 src, flags=re.M)))


def test_every_declared_entry_point_is_exported(lib):
    names = declared_functions()
    assert set(names) == set(m.EXPORTED_SYMBOLS), names
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version(lib):
    for code in range(8):
        assert m.csa_status_str(code).startswith("CSA_")
    assert lib.csa_version() >= 400


def csa_layer(**kw):
    base = dict(dtype=1, num_heads=64, head_dim=512, qk_rope_head_dim=64, rope_theta=160000.0,
                sliding_window=128, compress_ratio=4, overlap=1, index_n_heads=64,
                index_head_dim=128, index_rope_dim=64, index_topk=512, softmax_scale=0.0)
    base.update(kw)
    return _CLayer(**base)


def batch(**kw):
    base = dict(batch=1, n_new=8192, pos0=FAKE.value, pos0_max=0)
    base.update(kw)
    return _CBatch(**base)


def test_workspace_sizes(lib):
    L = csa_layer()
    assert lib.csa_workspace_bytes(ctypes.byref(L), 1, 8192, 2048, m.CSA_OP_INDEX_TOPK) >= 8192 * 2048 * 4
    assert lib.csa_workspace_bytes(ctypes.byref(L), 1, 8192, 2048, m.CSA_OP_ATTEND) == 0
    # 64 one-token sequences fill the chip without splitting a row list; four
    # of them split each list over several blocks (float32 partials)
    assert lib.csa_workspace_bytes(ctypes.byref(L), 64, 1, 32768, m.CSA_OP_ATTEND) == 0
    assert lib.csa_workspace_bytes(ctypes.byref(L), 4, 1, 262144, m.CSA_OP_ATTEND) >= 4 * 2 * 64 * 516 * 4
    assert lib.csa_workspace_bytes(ctypes.byref(L), 1, 1, 1, 99) == ctypes.c_size_t(-1).value
    bad = csa_layer(dtype=7)
    assert lib.csa_workspace_bytes(ctypes.byref(bad), 1, 1, 1, 1) == ctypes.c_size_t(-1).value


def call_attend(lib, L, B, win_cap=8192, pool_cap=2048, idx=FAKE, ws=None, wsb=0, q=FAKE):
    return lib.csa_attend(ctypes.byref(L), ctypes.byref(B), q, FAKE, win_cap, FAKE, pool_cap,
                          idx, None, FAKE, ws, wsb, None)


def test_rejections_return_before_launch(lib):
    L, B = csa_layer(), batch()
    NULL, SHAPE, DTYPE, WS, UNSUP = 1, 2, 3, 5, 4
    assert lib.csa_attend(None, ctypes.byref(B), FAKE, FAKE, 8192, FAKE, 2048, FAKE, None, FAKE,
                          None, 0, None) == NULL
    assert call_attend(lib, L, batch(pos0=None)) == NULL
    assert call_attend(lib, L, B, q=None) == NULL
    assert call_attend(lib, L, B, idx=None) == NULL
    assert call_attend(lib, csa_layer(dtype=5), B) == DTYPE
    assert call_attend(lib, csa_layer(qk_rope_head_dim=63), B) == SHAPE
    assert call_attend(lib, csa_layer(qk_rope_head_dim=514), B) == SHAPE
    assert call_attend(lib, csa_layer(index_topk=5000), B) == SHAPE
    assert call_attend(lib, csa_layer(overlap=2), B) == SHAPE
    # YaRN fields: a factor below 1, or a factor > 1 without a valid context or turn counts
    assert call_attend(lib, csa_layer(rope_factor=0.5), B) == SHAPE
    assert call_attend(lib, csa_layer(rope_factor=16.0), B) == SHAPE
    assert call_attend(lib, csa_layer(rope_factor=16.0, rope_original_context=65536.0,
                                      rope_beta_fast=1.0, rope_beta_slow=32.0), B) == SHAPE
    assert call_attend(lib, csa_layer(rope_factor=float("nan")), B) == SHAPE
    assert call_attend(lib, L, B, pool_cap=2047) == SHAPE          # entries (0+8192)/4 = 2048
    assert call_attend(lib, L, B, win_cap=8191) == SHAPE           # needs min(128+8191, 8192)
    assert call_attend(lib, L, batch(n_new=0)) == SHAPE
    # decode shapes need split partials: missing workspace
    Bd = batch(batch=4, n_new=1, pos0_max=1048576)
    assert call_attend(lib, L, Bd, win_cap=128, pool_cap=262144) == WS
    # generic path limits: a large float32 layer is not implemented
    assert call_attend(lib, csa_layer(dtype=0), B) == UNSUP
    # compressor
    assert lib.csa_compress(ctypes.byref(L), ctypes.byref(B), 512, 64, FAKE, FAKE, None,
                            ctypes.c_float(1e-6), FAKE, FAKE, FAKE, 2047, None) == SHAPE
    assert lib.csa_compress(ctypes.byref(L), ctypes.byref(B), 513, 64, FAKE, FAKE, None,
                            ctypes.c_float(1e-6), FAKE, FAKE, FAKE, 2048, None) == SHAPE
    assert lib.csa_compress(ctypes.byref(L), ctypes.byref(B), 512, 64, None, FAKE, None,
                            ctypes.c_float(1e-6), FAKE, FAKE, FAKE, 2048, None) == NULL
    assert lib.csa_compress(ctypes.byref(csa_layer(compress_ratio=0)), ctypes.byref(B), 512, 64,
                            FAKE, FAKE, None, ctypes.c_float(1e-6), FAKE, FAKE, FAKE, 2048,
                            None) == SHAPE
    # indexer
    assert lib.csa_index_topk(ctypes.byref(L), ctypes.byref(B), FAKE, FAKE, FAKE, 2048, FAKE, None,
                              None, 0, None) == WS
    assert lib.csa_index_topk(ctypes.byref(L), ctypes.byref(B), FAKE, FAKE, FAKE, 2048, FAKE, None,
                              ctypes.c_void_p(0x1010), 1 << 40, None) == WS   # misaligned
    assert lib.csa_index_topk(ctypes.byref(csa_layer(index_rope_dim=200)), ctypes.byref(B), FAKE,
                              FAKE, FAKE, 2048, FAKE, None, FAKE, 1 << 40, None) == SHAPE
    # the allocation-free indexer: argument errors first, then the scratch limit,
    # all before any HIP call (a prefill of 8192 tokens needs 64 MiB of scores)
    NOALLOC = lib.csa_index_topk_noalloc
    assert NOALLOC(ctypes.byref(L), ctypes.byref(B), None, FAKE, FAKE, 2048, FAKE, None,
                   None) == NULL
    assert NOALLOC(ctypes.byref(L), ctypes.byref(B), FAKE, FAKE, FAKE, 2047, FAKE, None,
                   None) == SHAPE
    assert NOALLOC(ctypes.byref(L), ctypes.byref(B), FAKE, FAKE, FAKE, 2048, FAKE, None,
                   None) == 7   # CSA_ERR_SCRATCH
    assert m.csa_workspace_bytes(m.Layer("bf16", 64, 512, 64, 160000.0, 128, 4, 1, 64, 128, 64,
                                         512), 1, 8192, 2048, m.CSA_OP_INDEX_TOPK) > \
        m.CSA_NOALLOC_SCRATCH_BYTES
    # packed rows and paged pools: one layout per call, block sizes a power of
    # two of at least 128 entries, a table covering pool_cap, row ids in int32
    assert call_attend(lib, L, batch(n_valid=FAKE.value, cu_seqlens=FAKE.value)) == SHAPE
    for E in (64, 192, 0):
        assert call_attend(lib, L, batch(block_table=FAKE.value, block_entries=E,
                                         block_table_stride=16, pool_blocks=16)) == SHAPE
    assert call_attend(lib, L, batch(block_table=FAKE.value, block_entries=128,
                                     block_table_stride=15, pool_blocks=16)) == SHAPE  # 1920 < 2048
    assert call_attend(lib, L, batch(block_table=FAKE.value, block_entries=128,
                                     block_table_stride=16, pool_blocks=0)) == SHAPE
    assert call_attend(lib, L, batch(block_table=FAKE.value, block_entries=1 << 20,
                                     block_table_stride=1, pool_blocks=4096)) == UNSUP
    assert lib.csa_compress(ctypes.byref(L), ctypes.byref(
        batch(block_table=FAKE.value, block_entries=128, block_table_stride=15, pool_blocks=16)),
        512, 64, FAKE, FAKE, None, ctypes.c_float(1e-6), FAKE, FAKE, FAKE, 2048, None) == SHAPE
    # the fused cache update: the window's and each compressor's checks
    def cache_update(layer=L, b=B, kv=FAKE, ring=FAKE, win_cap=8192, ckv=FAKE, ikv=FAKE,
                     ipool=FAKE, pool_cap=2048, eps=1e-6):
        return lib.csa_cache_update(ctypes.byref(layer), ctypes.byref(b), kv, ring, win_cap, ckv,
                                    FAKE, None, FAKE, FAKE, FAKE, ikv, FAKE, None, FAKE, FAKE,
                                    ipool, pool_cap, ctypes.c_float(eps), None)
    assert cache_update(kv=None) == NULL
    assert cache_update(win_cap=100) == SHAPE
    assert cache_update(ckv=None) == NULL
    assert cache_update(ikv=None) == NULL
    assert cache_update(ipool=None) == NULL
    assert cache_update(pool_cap=2047) == SHAPE
    assert cache_update(eps=-1.0) == SHAPE
    assert cache_update(layer=csa_layer(index_rope_dim=200)) == SHAPE
    assert cache_update(b=batch(block_table=FAKE.value, block_entries=128, block_table_stride=15,
                                pool_blocks=16)) == SHAPE
    # an HCA layer needs no indexer pointers (the call fails on the pool capacity, after the
    # pointers were accepted); a sliding-only layer none of the compressors' (window capacity)
    assert cache_update(layer=csa_layer(compress_ratio=0, overlap=0, index_topk=0), ckv=None,
                        ikv=None, ipool=None, win_cap=100) == SHAPE
    assert cache_update(layer=csa_layer(compress_ratio=128, overlap=0, index_topk=0), ikv=None,
                        ipool=None, pool_cap=63) == SHAPE
    # rope / window
    assert lib.csa_rope(ctypes.byref(L), ctypes.byref(B), FAKE, 1, 512, 64, 2, None) == SHAPE
    assert lib.csa_rope(ctypes.byref(L), ctypes.byref(B), FAKE, 1, 512, 65, 1, None) == SHAPE
    assert lib.csa_window_append(ctypes.byref(L), ctypes.byref(B), FAKE, FAKE, 100, None) == SHAPE
    assert lib.hca_attend(ctypes.byref(csa_layer(compress_ratio=128, overlap=0)), ctypes.byref(B),
                          FAKE, FAKE, 8192, FAKE, 63, None, FAKE, None, 0, None) == SHAPE


def test_binding_rejects_host_tensors():
    torch = pytest.importorskip("torch")
    L = m.Layer("bf16", 64, 512, 64, 160000.0, 128, 4, 1, 64, 128, 64, 512)
    x = torch.zeros(1, 4, 512, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        m.csa_window_append(L, torch.zeros(1, dtype=torch.int64), 0, x, x)


def test_output_projection_sizes_and_rejections(lib):
    NULL, SHAPE, WS, UNSUP = 1, 2, 5, 4
    P = m._COproj(300, 8, 64, 2, 96, 200)
    assert lib.csa_output_projection_workspace_bytes(ctypes.byref(P)) == 300 * 2 * 96 * 2

    def call(p, x=FAKE, wa=FAKE, ws=FAKE, wsb=1 << 40):
        return lib.csa_output_projection(ctypes.byref(p), x, wa, FAKE, FAKE, ws, wsb, None)

    assert lib.csa_output_projection(None, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == NULL
    assert call(P, x=None) == NULL
    assert call(m._COproj(300, 8, 64, 3, 96, 200)) == SHAPE          # 3 does not divide 8
    assert call(m._COproj(0, 8, 64, 2, 96, 200)) == SHAPE
    assert call(m._COproj(300, 8, 60, 2, 96, 200)) == UNSUP          # 4 * 60 not a multiple of 32
    assert call(m._COproj(300, 8, 64, 2, 95, 200)) == UNSUP          # 2 * 95 not a multiple of 32
    assert lib.csa_output_projection_workspace_bytes(
        ctypes.byref(m._COproj(300, 8, 64, 3, 96, 200))) == ctypes.c_size_t(-1).value
    assert call(P, x=ctypes.c_void_p(0x1008)) == UNSUP               # not 16-byte aligned
    assert call(P, ws=None) == WS
    assert call(P, wsb=300 * 2 * 96 * 2 - 1) == WS
    assert call(P, ws=ctypes.c_void_p(0x1010)) == WS                  # not 256-byte aligned


def test_project_sizes_and_rejections(lib):
    NULL, SHAPE, WS, UNSUP = 1, 2, 5, 4
    P = m._CProj(300, 256, 96, 4, 64, 64, 32, 8, 1e-6, 1)
    assert lib.csa_project_workspace_bytes(ctypes.byref(P)) == 300 * 96 * 2

    def call(p, x=FAKE, ckv=FAKE, qi=FAKE, ws=FAKE, wsb=1 << 40):
        return lib.csa_project(ctypes.byref(p), x, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ckv, FAKE,
                               FAKE, FAKE, qi, FAKE, ws, wsb, None)

    assert call(P, x=None) == NULL
    assert call(P, ckv=None) == NULL                                        # compressor present
    assert call(P, qi=None) == NULL                                         # indexer present
    # a layer without compressor and indexer may pass NULL for those streams:
    # the call then gets as far as the workspace check
    assert call(m._CProj(300, 256, 96, 4, 64, 0, 0, 0, 1e-6, 1), ckv=None, qi=None,
                ws=None) == WS
    assert call(m._CProj(300, 250, 96, 4, 64, 64, 32, 8, 1e-6, 1)) == UNSUP  # hidden % 32
    assert call(m._CProj(300, 256, 100, 4, 64, 64, 32, 8, 1e-6, 1)) == UNSUP  # q_lora % 32
    assert call(m._CProj(300, 256, 96, 4, 64, 64, 32, 0, 1e-6, 1)) == SHAPE  # D_I without H_I
    assert call(m._CProj(300, 256, 96, 4, 64, 64, 32, 8, -1.0, 1)) == SHAPE  # negative eps
    assert call(m._CProj(0, 256, 96, 4, 64, 64, 32, 8, 1e-6, 1)) == SHAPE
    assert call(m._CProj(300, 256, 96, 4, 64, 64, 32, 8, 1e-6, 2)) == SHAPE
    assert call(P, x=ctypes.c_void_p(0x1008)) == UNSUP                      # not 16-byte aligned
    assert call(P, ws=None) == WS
    assert call(P, wsb=300 * 96 * 2 - 1) == WS
    assert call(P, ws=ctypes.c_void_p(0x1010)) == WS


def test_binding_checks_variable_length_counts():
    torch = pytest.importorskip("torch")
    # host tensors are refused before any call; a wrong dtype or count too
    pos0 = torch.zeros(2, dtype=torch.int64)
    with pytest.raises(ValueError):
        m._batch(pos0, 0, 2, 8, torch.zeros(2, dtype=torch.int32))      # not on the device
    assert m._CBatch(2, 8, 0x1000, 0).n_valid is None                  # NULL by default
