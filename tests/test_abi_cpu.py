"""The C ABI without a GPU: the library loads, exports what the header
declares, and every host-only function behaves (no kernel is launched)."""
import ctypes
import os
import re

import pytest

import latency_decode_gemm_amd as skg
from latency_decode_gemm_amd import _capi
from latency_decode_gemm_amd.inputs import all_points

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "skinny_gemm.h")


def _header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(skinny_gemm_\w+)\s*\(", text)))


def test_header_declares_expected_api():
    fns = _header_functions()
    for name in ("skinny_gemm_bf16", "skinny_gemm_dispatch", "skinny_gemm_warmup",
                 "skinny_gemm_bf16_with_config", "skinny_gemm_warmup_keys"):
        assert name in fns


def test_library_exports_every_declared_symbol():
    lib = _capi.lib()
    for name in _header_functions():
        assert hasattr(lib, name), name
        assert name in _capi.SIGNATURES, f"{name} has no ctypes signature"


def test_python_binding_has_same_names():
    for name in _header_functions():
        assert callable(getattr(skg, name)), name


def test_struct_layout_matches_header():
    assert ctypes.sizeof(_capi.SkgConfig) == 8 * 4


def test_strerror_covers_codes():
    for code in range(8):
        assert skg.skinny_gemm_strerror(code) != "unknown status"
    assert skg.skinny_gemm_strerror(99) == "unknown status"


def test_dispatch_is_pure_and_deterministic():
    for p in all_points():
        first = skg.skinny_gemm_dispatch(p["M"], p["K"], p["N"])
        assert skg.skinny_gemm_check_config(p["M"], p["K"], p["N"], first)
        for _ in range(200):
            assert skg.skinny_gemm_dispatch(p["M"], p["K"], p["N"]) == first


def test_dispatch_valid_on_a_shape_grid():
    for M in list(range(1, 18)) + [24, 31, 32, 33, 40, 48, 56, 63, 64]:
        for K in (1, 7, 8, 9, 64, 100, 1000, 1536, 2048, 2880, 4096, 7168, 14336, 20000):
            for N in (1, 3, 16, 128, 129, 2112, 24576):
                cfg = skg.skinny_gemm_dispatch(M, K, N)
                assert skg.skinny_gemm_check_config(M, K, N, cfg), (M, K, N, cfg)
                if cfg.backend == skg.SKG_BACKEND_DOT:
                    assert cfg.split_k == 1
                elif cfg.backend != skg.SKG_BACKEND_EVEN:
                    assert cfg.split_k >= 2


def test_dispatch_rejects():
    lib = _capi.lib()
    cfg = _capi.SkgConfig()
    assert lib.skinny_gemm_dispatch(65, 7168, 256, ctypes.byref(cfg)) == skg.SKG_ERR_UNSUPPORTED
    assert lib.skinny_gemm_f32w_dispatch(17, 7168, 256, ctypes.byref(cfg)) == \
        skg.SKG_ERR_UNSUPPORTED
    assert lib.skinny_gemm_dispatch(0, 7168, 256, ctypes.byref(cfg)) == skg.SKG_ERR_INVALID_ARG
    assert lib.skinny_gemm_dispatch(1, -1, 256, ctypes.byref(cfg)) == skg.SKG_ERR_INVALID_ARG
    assert lib.skinny_gemm_dispatch(1, 7168, 256, None) == skg.SKG_ERR_INVALID_ARG


def test_check_config_rules():
    mk = _capi.SkgConfig.make
    ok = mk(inner=skg.SKG_INNER_VALU, split_k=1, row_tiles=1, waves_n=1, waves_k=4, depth=4)
    assert skg.skinny_gemm_check_config(4, 7168, 256, ok)
    bad = [
        mk(backend=skg.SKG_BACKEND_DOT, split_k=2, row_tiles=1, waves_k=4),     # dot with split
        mk(backend=skg.SKG_BACKEND_SPLITK, split_k=1, row_tiles=1, waves_k=4),  # split-K of 1
        mk(row_tiles=3, waves_k=4),                                              # no such variant
        mk(row_tiles=1, depth=5, waves_k=4),
        mk(row_tiles=1, waves_n=4, waves_k=4),                                   # 16 waves
        mk(row_tiles=1, waves_n=0, waves_k=1),
        mk(split_k=4096, row_tiles=1, waves_k=1),                                # empty splits
    ]
    for b in bad:
        assert not skg.skinny_gemm_check_config(4, 7168, 256, b), b
    # the staged A slice must fit in 160 KB of LDS: 16 x 7168 x 2 B = 224 KB
    big = mk(inner=skg.SKG_INNER_MFMA, split_k=1, row_tiles=1, waves_k=4, depth=4)
    assert not skg.skinny_gemm_check_config(16, 7168, 256, big)
    assert skg.skinny_gemm_check_config(16, 7168, 256, mk(inner=skg.SKG_INNER_MFMA, split_k=2,
                                                          row_tiles=1, waves_k=4, depth=4))
    # activations in the load ring: M <= 8 and M * depth <= 32
    ga = dict(inner=skg.SKG_INNER_VALU_GA, split_k=1, row_tiles=1, waves_k=4)
    assert skg.skinny_gemm_check_config(8, 7168, 256, mk(depth=4, **ga))
    assert not skg.skinny_gemm_check_config(9, 7168, 256, mk(depth=4, **ga))
    assert not skg.skinny_gemm_check_config(8, 7168, 256, mk(depth=8, **ga))
    assert skg.skinny_gemm_check_config(2, 7168, 256, mk(depth=12, **ga))
    assert not skg.skinny_gemm_check_config(4, 7168, 256, mk(inner=8, waves_k=4))  # no such inner


def test_even_backend_rules():
    """SKG_BACKEND_EVEN without a K split: min(N, 256 x rb_per_wg) workgroups
    of floor/ceil(N / G) rows, which the waves must cover; no workspace."""
    mk = _capi.SkgConfig.make
    ev = dict(backend=skg.SKG_BACKEND_EVEN, split_k=1, waves_k=2, depth=4)
    # 2112 rows over 256 workgroups: up to 9 rows, 12 covered by 3 VALU waves
    c = mk(inner=skg.SKG_INNER_VALU, row_tiles=1, waves_n=3, rb_per_wg=1, **ev)
    assert skg.skinny_gemm_check_config(2, 7168, 2112, c)
    assert skg.skinny_gemm_workspace_bytes(2, 7168, 2112, c) == 0
    # 8 rows cannot hold 9
    assert not skg.skinny_gemm_check_config(
        2, 7168, 2112, mk(inner=skg.SKG_INNER_VALU, row_tiles=1, waves_n=2, rb_per_wg=1, **ev))
    # 512 workgroups: 5 rows each, 8 covered
    assert skg.skinny_gemm_check_config(
        2, 7168, 2112, mk(inner=skg.SKG_INNER_VALU, row_tiles=1, waves_n=2, rb_per_wg=2, **ev))
    # 7168 rows over 256: 28 each, a 32-row MFMA wave covers them, a 16-row one does not
    mf = dict(backend=skg.SKG_BACKEND_EVEN, split_k=1, waves_n=1, waves_k=2, rb_per_wg=1)
    assert skg.skinny_gemm_check_config(16, 14336, 7168, mk(inner=skg.SKG_INNER_MFMA_GA,
                                                            row_tiles=2, depth=3, **mf))
    assert not skg.skinny_gemm_check_config(16, 14336, 7168, mk(inner=skg.SKG_INNER_MFMA_GA,
                                                                row_tiles=1, depth=4, **mf))
    # fewer rows than workgroups: one row each
    assert skg.skinny_gemm_check_config(
        1, 64, 100, mk(inner=skg.SKG_INNER_VALU, row_tiles=1, waves_n=1, rb_per_wg=1, **ev))
    # at most 64 workgroups per CU
    assert not skg.skinny_gemm_check_config(
        2, 7168, 2112, mk(inner=skg.SKG_INNER_VALU, row_tiles=1, waves_n=3, rb_per_wg=65, **ev))


def test_even_backend_with_k_split():
    """SKG_BACKEND_EVEN with split_k = S: 256 x rb_per_wg workgroups are
    256 x rb_per_wg / S row blocks times S K slices (S must divide the
    workgroup count); each row block holds floor/ceil(N / blocks) rows; the
    slices' partials meet in the workspace's tree slots (S - 1 per output)."""
    mk = _capi.SkgConfig.make
    lib = _capi.lib()

    def geom(M, K, N, cfg):
        st = lib.skinny_gemm_check_config(M, K, N, ctypes.byref(cfg))
        return st == 0

    # 7168 rows, split 2: 128 row blocks of 56 rows; 64-row MFMA waves cover them
    c = mk(backend=skg.SKG_BACKEND_EVEN, inner=skg.SKG_INNER_MFMA_RING_GA, split_k=2,
           row_tiles=4, waves_n=1, waves_k=2, depth=2, rb_per_wg=1)
    assert geom(16, 14336, 7168, c)
    # tree slots [128 blocks][1 node][16 tokens][64 rows], 8 bytes each
    assert skg.skinny_gemm_workspace_bytes(16, 14336, 7168, c) == 128 * 1 * 16 * 64 * 8
    # 32 rows cannot hold 56
    assert not geom(16, 14336, 7168, mk(backend=skg.SKG_BACKEND_EVEN,
                                        inner=skg.SKG_INNER_MFMA_RING_GA, split_k=2, row_tiles=2,
                                        waves_n=1, waves_k=2, depth=3, rb_per_wg=1))
    # split 4 of 2112 rows: 64 blocks of 33 rows, 3 MFMA waves of 16 rows
    assert geom(16, 7168, 2112, mk(backend=skg.SKG_BACKEND_EVEN, inner=skg.SKG_INNER_MFMA_GA,
                                   split_k=4, row_tiles=1, waves_n=3, waves_k=1, depth=4,
                                   rb_per_wg=1))
    # the split must divide 256 x rb_per_wg
    for S, rpw, ok in ((3, 1, False), (3, 3, True), (5, 1, False), (8, 1, True), (128, 1, False)):
        cfg = mk(backend=skg.SKG_BACKEND_EVEN, inner=skg.SKG_INNER_VALU_GA, split_k=S,
                 row_tiles=4, waves_n=8, waves_k=1, depth=2, rb_per_wg=rpw)
        assert geom(2, 7168, 2048, cfg) == ok, (S, rpw)
    # a K too short for the slices (empty last slice) is rejected
    assert not geom(2, 64, 2048, mk(backend=skg.SKG_BACKEND_EVEN, inner=skg.SKG_INNER_VALU_GA,
                                    split_k=8, row_tiles=4, waves_n=8, waves_k=1, depth=2,
                                    rb_per_wg=1))


def test_lds_ring_sizes():
    """The LDS ring holds depth slots of 4 KB tiles per wave (row_tiles of B,
    plus one of activations for the _GA kind), so it fits where the register
    ring's single transpose tile per wave fits, minus what depth costs."""
    mk = _capi.SkgConfig.make
    # 8 waves x depth 4 x (1 + 1) tiles x 4 KB = 256 KB > 160 KB
    deep = dict(split_k=1, row_tiles=1, waves_n=2, waves_k=4, depth=4)
    assert skg.skinny_gemm_check_config(16, 7168, 256, mk(inner=skg.SKG_INNER_MFMA_GA, **deep))
    assert not skg.skinny_gemm_check_config(16, 7168, 256,
                                            mk(inner=skg.SKG_INNER_MFMA_RING_GA, **deep))
    # 2 waves x depth 4 x 3 tiles x 4 KB = 96 KB
    assert skg.skinny_gemm_check_config(16, 14336, 7168, mk(
        inner=skg.SKG_INNER_MFMA_RING_GA, split_k=1, row_tiles=2, waves_n=1, waves_k=2, depth=4))
    # staged A (1536 x 16 x 2 B = 48 KB) + 4 waves x depth 6 x 4 KB = 144 KB fits; depth 6
    # with 6 waves (192 KB) does not
    assert skg.skinny_gemm_check_config(16, 1536, 24576, mk(
        inner=skg.SKG_INNER_MFMA_RING, split_k=1, row_tiles=1, waves_n=4, waves_k=1, depth=6))
    assert not skg.skinny_gemm_check_config(16, 1536, 24576, mk(
        inner=skg.SKG_INNER_MFMA_RING, split_k=1, row_tiles=1, waves_n=6, waves_k=1, depth=6))


def test_compiled_variant_lists_match_library():
    for inner, allowed in ((skg.SKG_INNER_VALU, _capi.VALU_VARIANTS),
                           (skg.SKG_INNER_VALU_GA, [v for v in _capi.VALU_VARIANTS if 4 * v[1] <= 32]),
                           (skg.SKG_INNER_MFMA, _capi.MFMA_VARIANTS),
                           (skg.SKG_INNER_MFMA_GA, _capi.MFMA_VARIANTS),
                           (skg.SKG_INNER_MFMA_RING, _capi.MFMA_VARIANTS),
                           (skg.SKG_INNER_MFMA_RING_GA, _capi.MFMA_VARIANTS),
                           (skg.SKG_INNER_MFMA_RING_SYNC, _capi.SYNC_VARIANTS),
                           (skg.SKG_INNER_MFMA_RING_SHARED, _capi.SHARED_VARIANTS)):
        for rt in (1, 2, 3, 4, 8):
            for d in range(0, 10):
                cfg = skg.SkgConfig.make(inner=inner, row_tiles=rt, depth=d, waves_k=2)
                ok = skg.skinny_gemm_check_config(4, 1024, 512, cfg)
                assert ok == ((rt, d) in allowed), (inner, rt, d)


def test_barrier_kinds_rules():
    """The barrier kinds take M <= 16 and bf16 weights; the shared
    activation ring needs depth >= 3 and holds one activation tile per depth
    slot and K-wave group beside the waves' weight rings (so a configuration
    whose per-wave rings would overflow the LDS with their own activation
    tiles can fit with the shared one)."""
    mk = skg.SkgConfig.make
    sync = dict(inner=skg.SKG_INNER_MFMA_RING_SYNC, split_k=1, row_tiles=1, waves_n=3,
                waves_k=1, depth=3, rb_per_wg=2)
    shared = dict(sync, inner=skg.SKG_INNER_MFMA_RING_SHARED)
    for kw in (sync, shared):
        assert skg.skinny_gemm_check_config(16, 1536, 24576, mk(**kw))
        assert not skg.skinny_gemm_check_config(17, 1536, 24576, mk(**kw))
        assert not skg.skinny_gemm_f32w_check_config(8, 7168, 256, mk(**kw))
    assert skg.skinny_gemm_check_config(16, 1536, 24576, mk(**dict(sync, depth=2)))
    assert not skg.skinny_gemm_check_config(16, 1536, 24576, mk(**dict(shared, depth=2)))
    # 8 waves x depth 3: with per-wave activation tiles 8 x 3 x 2 x 4 KB = 192 KB;
    # shared, 8 x 3 x 4 KB + 3 x 4 x 4 KB = 144 KB
    big = dict(backend=skg.SKG_BACKEND_SPLITK, split_k=3, row_tiles=1, waves_n=2, waves_k=4,
               depth=3)
    assert not skg.skinny_gemm_check_config(16, 7168, 2112, mk(inner=skg.SKG_INNER_MFMA_RING_SYNC,
                                                               **big))
    assert skg.skinny_gemm_check_config(16, 7168, 2112, mk(inner=skg.SKG_INNER_MFMA_RING_SHARED,
                                                           **big))


def test_workspace_bytes():
    dot = skg.SkgConfig.make(split_k=1, row_tiles=1, waves_k=4)
    assert skg.skinny_gemm_workspace_bytes(4, 7168, 256, dot) == 0
    sk = skg.SkgConfig.make(split_k=4, row_tiles=1, waves_k=4)
    rows = 4
    nrb = 256 // rows
    # one pass: split_k - 1 = 3 tree nodes of one 8-byte slot per output
    assert skg.skinny_gemm_workspace_bytes(4, 7168, 256, sk) == nrb * 3 * 4 * rows * 8
    sk3 = skg.SkgConfig.make(split_k=3, row_tiles=1, waves_k=4)
    assert skg.skinny_gemm_workspace_bytes(4, 7168, 256, sk3) == nrb * 2 * 4 * rows * 8
    # two passes: every slice's fp32 partials
    p2 = skg.SkgConfig.make(backend=skg.SKG_BACKEND_SPLITK_2PASS, split_k=4, row_tiles=1,
                            waves_k=4)
    assert skg.skinny_gemm_workspace_bytes(4, 7168, 256, p2) == nrb * 4 * 4 * rows * 4
    bad = skg.SkgConfig.make(backend=skg.SKG_BACKEND_SPLITK_2PASS, split_k=1, row_tiles=1)
    assert not skg.skinny_gemm_check_config(4, 7168, 256, bad)


def test_warmup_keys_first_seen_order():
    shapes = [(7168, 256), (7168, 384), (2880, 128), (1536, 24576)]
    ms = [1, 2, 3, 4, 8, 16]
    keys = skg.skinny_gemm_warmup_keys(shapes, ms)
    want = []
    for K, N in shapes:
        for M in ms:
            c = skg.skinny_gemm_dispatch(M, K, N)
            if c not in want:
                want.append(c)
    assert keys == want
    assert skg.skinny_gemm_warmup_keys([], ms) == []


# --- argument checks run before any HIP call: fake, never-dereferenced pointers
FAKE = 0x100000  # 16-byte aligned, never touched


def _call(A=FAKE, B=FAKE, C=FAKE, M=4, N=256, K=7168, lda=7168, ldb=7168, ldc=256, odt=0):
    return _capi.lib().skinny_gemm_bf16(A, B, C, M, N, K, lda, ldb, ldc, odt, None)


@pytest.mark.parametrize("kw,code", [
    (dict(M=-1), skg.SKG_ERR_INVALID_ARG),
    (dict(N=-1), skg.SKG_ERR_INVALID_ARG),
    (dict(K=-1), skg.SKG_ERR_INVALID_ARG),
    (dict(M=65), skg.SKG_ERR_UNSUPPORTED),
    (dict(odt=2), skg.SKG_ERR_INVALID_ARG),
    (dict(lda=7160), skg.SKG_ERR_INVALID_ARG),
    (dict(ldb=100), skg.SKG_ERR_INVALID_ARG),
    (dict(ldc=255), skg.SKG_ERR_INVALID_ARG),
    (dict(A=0), skg.SKG_ERR_INVALID_ARG),
    (dict(B=0), skg.SKG_ERR_INVALID_ARG),
    (dict(C=0), skg.SKG_ERR_INVALID_ARG),
    (dict(A=FAKE + 8), skg.SKG_ERR_MISALIGNED),
    (dict(B=FAKE + 2), skg.SKG_ERR_MISALIGNED),
    (dict(lda=7172), skg.SKG_ERR_MISALIGNED),
    (dict(ldb=7176 + 4), skg.SKG_ERR_MISALIGNED),
    (dict(C=FAKE + 2), skg.SKG_ERR_MISALIGNED),
    (dict(C=FAKE + 1, odt=1), skg.SKG_ERR_MISALIGNED),
])
def test_argument_errors(kw, code):
    assert _call(**kw) == code


def test_empty_problems_are_noops():
    # nothing to compute: returns before touching the device or the pointers
    assert _call(M=0) == skg.SKG_OK
    assert _call(N=0) == skg.SKG_OK
    assert _call(M=0, A=0, B=0, C=0) == skg.SKG_OK


def test_with_config_rejects_bad_config():
    bad = skg.SkgConfig.make(row_tiles=3)
    st = _capi.lib().skinny_gemm_bf16_with_config(FAKE, FAKE, FAKE, 4, 256, 7168, 7168, 7168,
                                                  256, 0, None, ctypes.byref(bad))
    assert st == skg.SKG_ERR_INVALID_ARG
    st = _capi.lib().skinny_gemm_bf16_with_config(FAKE, FAKE, FAKE, 4, 256, 7168, 7168, 7168,
                                                  256, 0, None, None)
    assert st == skg.SKG_ERR_INVALID_ARG


def test_warmup_rejects_bad_lists():
    lib = _capi.lib()
    n = ctypes.c_int(0)
    assert lib.skinny_gemm_warmup(None, 1, None, 0, None, ctypes.byref(n)) == skg.SKG_ERR_INVALID_ARG
    assert lib.skinny_gemm_warmup(None, -1, None, 0, None, ctypes.byref(n)) == skg.SKG_ERR_INVALID_ARG


def test_python_dtype_guard():
    torch = pytest.importorskip("torch")
    a = torch.zeros((2, 8), dtype=torch.float32)
    b = torch.zeros((4, 8), dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        skg.skinny_gemm_bf16(a, b)
    with pytest.raises(TypeError):
        skg.skinny_gemm_bf16(b[:2], a)


# --- fp32 weights -------------------------------------------------------------

def _call_f32w(A=FAKE, W=FAKE, C=FAKE, M=4, N=256, K=7168, lda=7168, ldw=7168, ldc=256, odt=0):
    return _capi.lib().skinny_gemm_f32w(A, W, C, M, N, K, lda, ldw, ldc, odt, None)


@pytest.mark.parametrize("kw,code", [
    (dict(M=17), skg.SKG_ERR_UNSUPPORTED),
    (dict(ldw=100), skg.SKG_ERR_INVALID_ARG),
    (dict(W=0), skg.SKG_ERR_INVALID_ARG),
    (dict(W=FAKE + 4), skg.SKG_ERR_MISALIGNED),
    (dict(ldw=7170), skg.SKG_ERR_MISALIGNED),   # rows not 16-byte aligned
    (dict(lda=7172), skg.SKG_ERR_MISALIGNED),
])
def test_f32w_argument_errors(kw, code):
    assert _call_f32w(**kw) == code


def test_f32w_row_stride_multiple_of_4_is_accepted_by_the_checks():
    # ldw = 7172 (a multiple of 4, not of 8) passes the argument checks; with
    # M = 0 nothing is launched
    assert _call_f32w(M=0, ldw=7172) == skg.SKG_OK


def test_f32w_dispatch_is_valu_and_valid():
    for M in range(1, 17):
        for K in (1, 7, 8, 9, 1000, 2880, 7168):
            for N in (1, 3, 256, 384, 2112):
                cfg = skg.skinny_gemm_f32w_dispatch(M, K, N)
                assert cfg.inner in (skg.SKG_INNER_VALU, skg.SKG_INNER_VALU_GA), (M, K, N, cfg)
                assert skg.skinny_gemm_f32w_check_config(M, K, N, cfg), (M, K, N, cfg)
                assert skg.skinny_gemm_f32w_dispatch(M, K, N) == cfg


def test_f32w_rejects_matrix_core_configs():
    mk = _capi.SkgConfig.make
    for inner in (skg.SKG_INNER_MFMA, skg.SKG_INNER_MFMA_GA, skg.SKG_INNER_MFMA_RING,
                  skg.SKG_INNER_MFMA_RING_GA):
        cfg = mk(inner=inner, split_k=2, row_tiles=1, waves_n=1, waves_k=2, depth=2)
        assert skg.skinny_gemm_check_config(16, 7168, 256, cfg)
        assert not skg.skinny_gemm_f32w_check_config(16, 7168, 256, cfg)
    for (rt, d) in _capi.VALU_VARIANTS:
        cfg = mk(inner=skg.SKG_INNER_VALU, row_tiles=rt, depth=d, waves_k=2)
        assert skg.skinny_gemm_f32w_check_config(4, 1024, 512, cfg)


def test_f32w_warmup_keys():
    shapes = [(7168, 256), (7168, 384)]
    ms = [1, 2, 3, 4, 8, 16]
    want = []
    for K, N in shapes:
        for M in ms:
            c = skg.skinny_gemm_f32w_dispatch(M, K, N)
            if c not in want:
                want.append(c)
    assert skg.skinny_gemm_f32w_warmup_keys(shapes, ms) == want


def test_f32w_spilling_variants_are_not_built():
    """Over fp32 weights the (M, rows, depth) combinations whose registers
    would spill are absent (checked per M), while the bf16 kernels exist."""
    mk = _capi.SkgConfig.make
    lds = mk(inner=skg.SKG_INNER_VALU, row_tiles=4, depth=4, waves_k=2)
    assert skg.skinny_gemm_f32w_check_config(8, 1024, 512, lds)
    assert not skg.skinny_gemm_f32w_check_config(9, 1024, 512, lds)
    assert skg.skinny_gemm_check_config(16, 1024, 512, lds)
    ga = mk(inner=skg.SKG_INNER_VALU_GA, row_tiles=2, depth=4, waves_k=2)
    assert skg.skinny_gemm_f32w_check_config(7, 1024, 512, ga)
    assert not skg.skinny_gemm_f32w_check_config(8, 1024, 512, ga)
    assert skg.skinny_gemm_check_config(8, 1024, 512, ga)


def test_bf16_spilling_variants_are_not_built():
    """Over bf16 weights, the activation-ring VALU kernels run up to
    M * depth = 32 tokens x steps, except 4 rows at depth 4, whose ring
    spills at M = 8, and the register-ring MFMA kernel with 2 row tiles at
    depth 4 is not built over a full token tile; their neighbours exist
    (tests/test_code_objects.py checks that no built kernel spills)."""
    mk = _capi.SkgConfig.make
    VG = skg.SKG_INNER_VALU_GA
    for (R, PF), top in {(1, 12): 2, (2, 8): 4, (1, 8): 4, (4, 4): 7, (1, 4): 8,
                         (2, 2): 8}.items():
        cfg = mk(inner=VG, row_tiles=R, depth=PF, waves_k=2)
        assert skg.skinny_gemm_check_config(top, 1024, 512, cfg), (R, PF)
        if top < 8:
            assert not skg.skinny_gemm_check_config(top + 1, 1024, 512, cfg), (R, PF)
        # the LDS-staged kernel of the same shape is built for every M
        assert skg.skinny_gemm_check_config(16, 1024, 512, mk(inner=skg.SKG_INNER_VALU,
                                                              row_tiles=R, depth=PF, waves_k=2))
    ga24 = mk(inner=skg.SKG_INNER_MFMA_GA, row_tiles=2, depth=4, waves_k=1)
    assert skg.skinny_gemm_check_config(8, 1024, 512, ga24)
    assert not skg.skinny_gemm_check_config(9, 1024, 512, ga24)
    assert skg.skinny_gemm_check_config(16, 1024, 512, mk(inner=skg.SKG_INNER_MFMA_RING_GA,
                                                          row_tiles=2, depth=4, waves_k=1))


# --- the middle tier (16 < M <= 64) ---------------------------------------------

def test_mid_tier_rules():
    """Above 16 tokens only the matrix-core kinds run, each token tile of 16
    costing its own activation tile (LDS-staged fragments or a transpose /
    ring tile); combinations that would spill are not built."""
    mk = _capi.SkgConfig.make
    F, GA = skg.SKG_INNER_MFMA, skg.SKG_INNER_MFMA_GA
    RF, RG = skg.SKG_INNER_MFMA_RING, skg.SKG_INNER_MFMA_RING_GA
    for M in (17, 32, 33, 64):
        assert not skg.skinny_gemm_check_config(M, 7168, 2112, mk(
            inner=skg.SKG_INNER_VALU, row_tiles=1, depth=4, waves_n=2, waves_k=2))
        assert skg.skinny_gemm_check_config(M, 7168, 2112, mk(
            inner=RG, row_tiles=1, depth=2, waves_n=2, waves_k=1))
        # staged fragments of a 1024-wide K slice: 32 KB per token tile
        assert skg.skinny_gemm_check_config(M, 7168, 2112, mk(
            inner=F, split_k=7, row_tiles=1, depth=4, waves_n=1, waves_k=2))
    # LDS ring with 4 row tiles spills above one token tile: not built
    ring4 = mk(inner=RG, row_tiles=4, depth=1, waves_n=1, waves_k=1)
    assert skg.skinny_gemm_check_config(16, 7168, 2112, ring4)
    assert not skg.skinny_gemm_check_config(17, 7168, 2112, ring4)
    # 2 row tiles x 3 token tiles is built, x 4 is not
    ring2 = mk(inner=RG, row_tiles=2, depth=2, waves_n=1, waves_k=1)
    assert skg.skinny_gemm_check_config(48, 7168, 2112, ring2)
    assert not skg.skinny_gemm_check_config(49, 7168, 2112, ring2)
    # register ring of activations: 4 x depth x loads + 4 x accumulator tiles <= 176
    assert skg.skinny_gemm_check_config(64, 7168, 2112, mk(inner=GA, row_tiles=2, depth=1,
                                                          waves_n=1, waves_k=1))
    assert not skg.skinny_gemm_check_config(64, 7168, 2112, mk(inner=GA, row_tiles=4, depth=1,
                                                              waves_n=1, waves_k=1))
    # staged activations: K x 16 tokens x 2 B per token tile; 64 x 2880 fits
    # (368 KB does not: K = 7168 needs a split)
    st = mk(inner=F, row_tiles=1, depth=2, waves_n=1, waves_k=1)
    assert skg.skinny_gemm_check_config(64, 1024, 2112, st)
    assert not skg.skinny_gemm_check_config(64, 7168, 2112, st)
    # the split-K workspace holds M rows per block: 3 tree slots (8 bytes) per
    # output in one pass, 4 partials (4 bytes) per output in two passes
    sk = mk(inner=GA, split_k=4, row_tiles=1, depth=2, waves_n=1, waves_k=1)
    nrb = -(-2112 // 16)
    assert skg.skinny_gemm_workspace_bytes(48, 7168, 2112, sk) == nrb * 3 * 48 * 16 * 8
    p2 = mk(backend=skg.SKG_BACKEND_SPLITK_2PASS, inner=GA, split_k=4, row_tiles=1, depth=2,
            waves_n=1, waves_k=1)
    assert skg.skinny_gemm_workspace_bytes(48, 7168, 2112, p2) == nrb * 4 * 48 * 16 * 4


def test_mid_tier_dispatch_and_crossover_defaults():
    for (K, N) in ((7168, 2112), (1536, 24576), (14336, 7168), (100, 7), (2880, 128)):
        for M in (17, 24, 32, 48, 64):
            cfg = skg.skinny_gemm_dispatch(M, K, N)
            assert cfg.inner in (skg.SKG_INNER_MFMA, skg.SKG_INNER_MFMA_GA,
                                 skg.SKG_INNER_MFMA_RING, skg.SKG_INNER_MFMA_RING_GA)
            assert skg.skinny_gemm_check_config(M, K, N, cfg)
    # an unmeasured shape: the skinny tier's own range
    assert skg.skinny_gemm_max_m(1000, 77) == skg.SKG_MAX_M_VALU
    lib = _capi.lib()
    m = ctypes.c_int(0)
    assert lib.skinny_gemm_max_m(7168, 0, ctypes.byref(m)) == skg.SKG_ERR_INVALID_ARG
    assert lib.skinny_gemm_max_m(7168, 256, None) == skg.SKG_ERR_INVALID_ARG
    for (K, N) in ((7168, 2112), (1536, 24576), (14336, 7168)):
        assert 1 <= skg.skinny_gemm_max_m(K, N) <= skg.SKG_MAX_M


def test_binding_shares_torchs_hip_runtime():
    """Loading the library through the binding leaves one HIP runtime in the
    process (torch's), even when nothing imported torch before."""
    import subprocess
    import sys
    code = ("from latency_decode_gemm_amd import _capi; _capi.lib(); import torch; "
            "print(sorted({l.split()[-1] for l in open('/proc/self/maps') if 'amdhip64' in l}))")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                         check=True).stdout.strip().splitlines()[-1]
    import ast
    libs = ast.literal_eval(out)
    assert len(libs) == 1, libs


def test_untuned_m_takes_the_next_tuned_m_of_its_shape():
    """An M the table does not list takes the configuration tuned for the
    smallest listed M above it on the same (K, N), when that can run M."""
    import re
    table = open(os.path.join(ROOT, "latency_decode_gemm_amd", "csrc", "tuned_table.inc")).read()
    rows = [tuple(int(v) for v in m.groups()) for m in
            re.finditer(r"\{(\d+), (\d+), (\d+), \{([-\d]+), ([-\d]+), ([-\d]+), ([-\d]+), "
                        r"([-\d]+), ([-\d]+), ([-\d]+), ([-\d]+)\}\}", table)]
    tuned = {}
    for r in rows:
        tuned.setdefault((r[1], r[2]), {})[r[0]] = _capi.SkgConfig(*r[3:])
    checked = 0
    for (K, N), by_m in tuned.items():
        for M in range(1, 65):
            got = skg.skinny_gemm_dispatch(M, K, N)
            if M in by_m:
                assert got == by_m[M], (M, K, N)
                continue
            above = [m for m in sorted(by_m) if m > M
                     and skg.skinny_gemm_check_config(M, K, N, by_m[m])]
            if above:
                assert got == by_m[above[0]], (M, K, N)
                checked += 1
    assert checked > 50


def test_log_env_prints_the_choice_once_per_shape():
    """SKINNY_GEMM_LOG=1: the entry point reports dispatch's choice once per
    shape (before any device work; on a machine without a GPU the call then
    fails with a status, which is all this checks besides the log)."""
    import subprocess
    import sys
    if os.path.exists("/dev/kfd"):
        pytest.skip("needs a machine without a GPU: the call passes placeholder pointers")
    code = ("from latency_decode_gemm_amd import _capi; lib = _capi.lib(); "
            "[lib.skinny_gemm_bf16(0x100000, 0x100000, 0x100000, 4, 256, 7168, 7168, 7168, 256, 0,"
            " None) for _ in range(3)]")
    env = dict(os.environ, SKINNY_GEMM_LOG="1", HIP_VISIBLE_DEVICES="-1")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                       env=env, timeout=120)
    lines = [ln for ln in r.stderr.splitlines() if ln.startswith("skinny_gemm: bf16 M=4 K=7168")]
    cfg = skg.skinny_gemm_dispatch(4, 7168, 256)
    assert len(lines) == 1, r.stderr
    assert f"backend {cfg.backend} inner {cfg.inner} split_k {cfg.split_k}" in lines[0]


def test_hip_errors_are_recorded_on_the_workspace_path():
    """Without a GPU every HIP call fails. A split-K GEMM call and a warm-up
    both reach the workspace code first; each returns SKG_ERR_HIP, and
    skinny_gemm_last_hip_error() then holds the runtime's code, not 0."""
    import subprocess
    import sys
    if os.path.exists("/dev/kfd"):
        pytest.skip("needs a machine without a GPU: the call passes placeholder pointers")
    assert skg.skinny_gemm_dispatch(16, 7168, 256).split_k > 1
    code = (
        "import ctypes\n"
        "from latency_decode_gemm_amd import _capi\n"
        "lib = _capi.lib()\n"
        "print('start', lib.skinny_gemm_last_hip_error())\n"
        "st = lib.skinny_gemm_bf16(0x100000, 0x100000, 0x100000, 16, 256, 7168, 7168, 7168,"
        " 256, 0, None)\n"
        "print('gemm', st, lib.skinny_gemm_last_hip_error())\n"
        "kn = (ctypes.c_int * 2)(7168, 256)\n"
        "ms = (ctypes.c_int * 1)(16)\n"
        "n = ctypes.c_int(0)\n"
        "st = lib.skinny_gemm_warmup(kn, 1, ms, 1, None, ctypes.byref(n))\n"
        "print('warmup', st, lib.skinny_gemm_last_hip_error())\n")
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                       env=env, timeout=120)
    assert r.returncode == 0, r.stderr
    got = {ln.split()[0]: [int(x) for x in ln.split()[1:]] for ln in r.stdout.splitlines()}
    assert got["start"] == [0]
    for what in ("gemm", "warmup"):
        st, err = got[what]
        assert st == skg.SKG_ERR_HIP, (what, got)
        assert err != 0, (what, got)


def _noalloc(A=FAKE, B=FAKE, C=FAKE, M=4, N=256, K=7168, lda=7168, ldb=7168, ldc=256, odt=0):
    return _capi.lib().skinny_gemm_bf16_noalloc(A, B, C, M, N, K, lda, ldb, ldc, odt, None)


def test_noalloc_checks_arguments_like_the_allocating_entry():
    """The same argument checks as skinny_gemm_bf16, before any HIP call."""
    for kw, code in [(dict(M=-1), skg.SKG_ERR_INVALID_ARG), (dict(M=65), skg.SKG_ERR_UNSUPPORTED),
                     (dict(ldc=255), skg.SKG_ERR_INVALID_ARG), (dict(C=0), skg.SKG_ERR_INVALID_ARG),
                     (dict(A=FAKE + 8), skg.SKG_ERR_MISALIGNED), (dict(odt=2), skg.SKG_ERR_INVALID_ARG),
                     (dict(M=0), skg.SKG_OK), (dict(N=0, A=0, B=0, C=0), skg.SKG_OK)]:
        assert _noalloc(**kw) == code, kw
        assert _call(**kw) == code, kw


def test_noalloc_scratch_covers_the_skinny_tier_and_rejects_larger_workspaces():
    """Every configuration dispatch returns for M <= 16 on the workload shapes
    fits the static scratch (tree slots of a one-pass split within
    SKG_SCRATCH_SLOT_BYTES, partials of a two-pass split within
    SKG_SCRATCH_PARTIAL_BYTES), so the no-allocation entry point does not
    refuse it; a shape whose split-K workspace does not fit (the two-pass split
    of M = 64 at K = 7168, N = 2112) is rejected with SKG_ERR_SCRATCH_TOO_SMALL
    before any GPU work (placeholder pointers)."""
    largest = 0
    for (K, N) in ((7168, 256), (7168, 384), (2880, 128), (7168, 2112), (1536, 24576),
                   (14336, 7168)):
        for M in range(1, 17):
            cfg = skg.skinny_gemm_dispatch(M, K, N)
            need = skg.skinny_gemm_workspace_bytes(M, K, N, cfg)
            limit = (skg.SKG_SCRATCH_PARTIAL_BYTES if cfg.backend == skg.SKG_BACKEND_SPLITK_2PASS
                     else skg.SKG_SCRATCH_SLOT_BYTES)
            assert need <= limit, (M, K, N, cfg, need)
            assert _noalloc(M=M, K=K, N=N, lda=K, ldb=K, ldc=N) != skg.SKG_ERR_SCRATCH_TOO_SMALL
            largest = max(largest, need)
    assert largest > 0  # some dispatched configuration does split K
    M, K, N = 64, 7168, 2112
    cfg = skg.skinny_gemm_dispatch(M, K, N)
    assert cfg.backend == skg.SKG_BACKEND_SPLITK_2PASS, cfg
    assert skg.skinny_gemm_workspace_bytes(M, K, N, cfg) > skg.SKG_SCRATCH_PARTIAL_BYTES
    assert _noalloc(M=M, K=K, N=N, lda=K, ldb=K, ldc=N) == skg.SKG_ERR_SCRATCH_TOO_SMALL
    assert "static scratch" in skg.skinny_gemm_strerror(skg.SKG_ERR_SCRATCH_TOO_SMALL)
