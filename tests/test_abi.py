"""The C ABI without a GPU: libufp4.so loads, exports every function that
include/ufp4.h declares, and rejects bad arguments on the host before
enqueuing anything (so these calls never reach the HIP runtime)."""
import ctypes
import os
import re

import pytest

from uniform_grid_fp4_amd import ufp4 as U

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "ufp4.h")).read()
    return sorted(set(re.findall(r"^\s*(?:ufp4_status|size_t|const char \*)\s*(ufp4_\w+)\(",
                                 src, re.M)))


def test_library_exports_every_declared_symbol():
    decl = declared_functions()
    assert len(decl) == 15, decl
    assert sorted(U.EXPORTS) == decl
    L = U.lib()
    for name in decl:
        assert hasattr(L, name), name


def test_status_strings():
    for code, name in U.STATUS.items():
        assert U.ufp4_status_string(code) == name
    assert U.ufp4_status_string(12345) == "UFP4_ERR_UNKNOWN"


def fake_desc(rows=32, k=32, kpad=32, grid=0, rht=1, mask=0x1234, codes=0x1000, scales=0x2000):
    return U.QTensorDesc(codes, scales, rows, k, kpad, grid, rht, mask, 0)


FAKE = ctypes.c_void_p(0x10000)   # never dereferenced: every call below fails validation


def quant(**kw):
    a = dict(x=FAKE, n_rows=32, n_cols=32, ld=32, axis=0, goff=None, ng=0, rht=1, mask=0x1234,
             grid=0, rnd=0, seed=1, sid=0, out=fake_desc())
    a.update(kw)
    return U.lib().ufp4_rht_quantize(a["x"], a["n_rows"], a["n_cols"], a["ld"], a["axis"],
                                     a["goff"], a["ng"], a["rht"], a["mask"], a["grid"],
                                     a["rnd"], a["seed"], a["sid"], ctypes.byref(a["out"]), None)


@pytest.mark.parametrize("kw,expect", [
    (dict(x=None), -1),
    (dict(out=fake_desc(codes=0)), -1),
    (dict(out=fake_desc(codes=0x1008)), -1),        # codes not 16-byte aligned
    (dict(axis=5), -1), (dict(grid=5), -1), (dict(rnd=2), -1), (dict(rht=3), -1),
    (dict(mask=0x10000), -1),
    (dict(n_rows=0), -2), (dict(n_cols=-1), -2), (dict(ld=16), -2),
    (dict(out=fake_desc(kpad=48)), -2),             # row-wise kpad must be roundup16(n_cols)
    (dict(out=fake_desc(rows=31)), -2),
    (dict(goff=FAKE, ng=2), -1),                    # groups only for ALONG_ROWS
    (dict(axis=1, goff=FAKE, ng=0), -1),
    (dict(axis=1, goff=FAKE, ng=2000), -2),
    (dict(axis=1, goff=FAKE, ng=2, out=fake_desc(kpad=32)), -2),  # needs >= roundup16(32+30)
    (dict(axis=3), -1),
    (dict(axis=2, goff=FAKE, ng=2), -1),            # stacked takes no offsets
    (dict(axis=2, ng=0), -2), (dict(axis=2, ng=3), -2),   # must divide n_rows
    (dict(axis=2, ng=2, out=fake_desc(rows=32, kpad=16)), -2),   # rows must be 2 * 32
    (dict(axis=2, ng=2, out=fake_desc(rows=64, kpad=32)), -2),   # kpad must be 16
])
def test_quantize_rejects(kw, expect):
    assert quant(**kw) == expect


def test_quantize_reserved_field_must_be_zero():
    d = fake_desc()
    d.reserved = 1
    assert quant(out=d) == -1


def gemm(fn, a, b, c=FAKE, ldc=32):
    return fn(ctypes.byref(a), ctypes.byref(b), c, ldc, None)


@pytest.mark.parametrize("name", ["ufp4_gemm_fprop", "ufp4_gemm_dgrad"])
def test_gemm_validation(name):
    fn = getattr(U.lib(), name)
    ok = fake_desc()
    assert gemm(fn, ok, fake_desc(k=16, kpad=16)) == -3        # K mismatch
    assert gemm(fn, ok, fake_desc(grid=1)) == -3               # grid mismatch
    assert gemm(fn, ok, fake_desc(grid=2)) == -3
    assert gemm(fn, fake_desc(grid=3), fake_desc(grid=3)) == -1   # no such grid
    assert gemm(fn, ok, fake_desc(rht=0)) == -3
    assert gemm(fn, ok, fake_desc(mask=0x4321)) == -3          # rotation would not cancel
    assert gemm(fn, ok, fake_desc(kpad=40)) == -2              # kpad % 16
    assert gemm(fn, ok, fake_desc(rows=0)) == -2
    assert gemm(fn, ok, fake_desc(scales=0x2004)) == -1        # misaligned
    assert gemm(fn, ok, ok, c=None) == -1
    assert gemm(fn, ok, fake_desc(rows=64), ldc=32) == -2      # ldc < N


def test_wgrad_and_grouped_validation():
    L = U.lib()
    ok = fake_desc()
    assert L.ufp4_gemm_wgrad(ctypes.byref(ok), ctypes.byref(ok), FAKE, 32, FAKE, 0, None) == -1
    assert L.ufp4_gemm_wgrad(ctypes.byref(ok), ctypes.byref(fake_desc(grid=1)), FAKE, 32,
                             None, 0, None) == -3
    g = L.ufp4_grouped_gemm
    assert g(3, 2, FAKE, ctypes.byref(ok), ctypes.byref(ok), FAKE, 32, None, 0, None) == -1
    assert g(0, 2, None, ctypes.byref(ok), ctypes.byref(ok), FAKE, 32, None, 0, None) == -1
    assert g(0, 0, FAKE, ctypes.byref(ok), ctypes.byref(ok), FAKE, 32, None, 0, None) == -2
    assert g(0, 3, FAKE, ctypes.byref(ok), ctypes.byref(ok), FAKE, 32, None, 0, None) == -2
    assert g(2, 2, FAKE, ctypes.byref(ok), ctypes.byref(fake_desc(k=16, kpad=16)), FAKE, 32,
             None, 0, None) == -3


def test_dequantize_validation():
    L = U.lib()
    ok = fake_desc()
    assert L.ufp4_dequantize(ctypes.byref(ok), 0, None, 32, None) == -1
    assert L.ufp4_dequantize(ctypes.byref(ok), 0, FAKE, 16, None) == -2
    assert L.ufp4_dequantize(ctypes.byref(fake_desc(rht=0)), 1, FAKE, 32, None) == -1
    assert L.ufp4_dequantize(None, 0, FAKE, 32, None) == -1


def dual(**kw):
    a = dict(x=FAKE, n_rows=32, n_cols=48, ld=48, axis=1, goff=None, ng=0, grid=0, rnd=0, seed=1,
             rs=U.QuantSide(1, 0x1234, 0, 0), cs=U.QuantSide(1, 0x4321, 1, 0),
             outr=fake_desc(rows=32, kpad=48), outc=fake_desc(rows=48, kpad=32, codes=0x3000,
                                                              scales=0x4000))
    a.update(kw)
    return U.lib().ufp4_rht_quantize_dual(a["x"], a["n_rows"], a["n_cols"], a["ld"], a["axis"],
                                          a["goff"], a["ng"], a["grid"], a["rnd"], a["seed"],
                                          None if a["rs"] is None else ctypes.byref(a["rs"]),
                                          None if a["cs"] is None else ctypes.byref(a["cs"]),
                                          None if a["outr"] is None else ctypes.byref(a["outr"]),
                                          None if a["outc"] is None else ctypes.byref(a["outc"]),
                                          None)


@pytest.mark.parametrize("kw,expect", [
    (dict(x=None), -1), (dict(rs=None), -1), (dict(cs=None), -1), (dict(outr=None), -1),
    (dict(outc=None), -1),
    (dict(axis=0), -1), (dict(axis=3), -1),            # the second output is column-wise
    (dict(rs=U.QuantSide(1, 0, 0, 7)), -1),           # reserved
    (dict(cs=U.QuantSide(2, 0, 0, 0)), -1),           # rht not 0/1
    (dict(rs=U.QuantSide(1, 0x10000, 0, 0)), -1),     # mask > 16 bits
    (dict(grid=3), -1), (dict(rnd=5), -1),
    (dict(outc=fake_desc(rows=48, kpad=32)), -1),     # shares the row-wise buffers
    (dict(outr=fake_desc(rows=32, kpad=32)), -2),     # row-wise kpad must be 48
    (dict(outc=fake_desc(rows=32, kpad=32, codes=0x3000, scales=0x4000)), -2),  # rows = n_cols
    (dict(axis=1, goff=FAKE, ng=2, outc=fake_desc(rows=48, kpad=32, codes=0x3000,
                                                  scales=0x4000)), -2),   # >= roundup16(62)
    (dict(axis=2, ng=3), -2),                          # stacks must divide n_rows
    (dict(axis=2, goff=FAKE, ng=2), -1),
    (dict(n_rows=0), -2), (dict(ld=40), -2),
])
def test_dual_quantize_rejects(kw, expect):
    assert dual(**kw) == expect


def test_stats_workspace_size_is_a_constant():
    assert U.ufp4_stats_workspace_size() == 1024 * 24 * 8


def qstats(**kw):
    a = dict(x=FAKE, n_rows=32, n_cols=48, ld=48, axis=0, q=fake_desc(rows=32, k=48, kpad=48),
             ws=ctypes.c_void_p(0x20000), nbytes=U.ufp4_stats_workspace_size(),
             out=ctypes.c_void_p(0x30000))
    a.update(kw)
    return U.lib().ufp4_quant_stats(a["x"], a["n_rows"], a["n_cols"], a["ld"], a["axis"],
                                    ctypes.byref(a["q"]), a["ws"], a["nbytes"], a["out"], None)


@pytest.mark.parametrize("kw,expect", [
    (dict(x=None), -1), (dict(ws=None), -1), (dict(out=None), -1),
    (dict(ws=ctypes.c_void_p(0x20004)), -1), (dict(out=ctypes.c_void_p(0x30004)), -1),
    (dict(nbytes=1024), -1),                       # workspace too small
    (dict(axis=2), -1), (dict(axis=7), -1),
    (dict(q=fake_desc(rows=32, k=48, kpad=64)), -2),   # kpad must be roundup16(k)
    (dict(q=fake_desc(rows=31, k=48, kpad=48)), -2),
    (dict(axis=1), -2),                            # transposed: rows = n_cols, k = n_rows
    (dict(ld=40), -2), (dict(n_rows=0), -2),
])
def test_quant_stats_rejects(kw, expect):
    assert qstats(**kw) == expect


def test_output_stats_rejects():
    L = U.lib()
    ws, n, out = ctypes.c_void_p(0x20000), U.ufp4_stats_workspace_size(), ctypes.c_void_p(0x30000)
    f = L.ufp4_output_stats
    assert f(None, 8, FAKE, 8, 4, 8, ws, n, out, None) == -1
    assert f(FAKE, 8, None, 8, 4, 8, ws, n, out, None) == -1
    assert f(FAKE, 8, FAKE, 8, 4, 8, ws, n - 8, out, None) == -1
    assert f(FAKE, 8, FAKE, 8, 4, 8, ws, n, ctypes.c_void_p(0x30002), None) == -1
    assert f(FAKE, 4, FAKE, 8, 4, 8, ws, n, out, None) == -2
    assert f(FAKE, 8, FAKE, 8, 0, 8, ws, n, out, None) == -2


def test_gemm_out_validation():
    L = U.lib()
    ok = fake_desc()
    f = L.ufp4_gemm_out
    assert f(3, ctypes.byref(ok), ctypes.byref(ok), FAKE, 0, 32, None) == -1     # kind
    assert f(0, ctypes.byref(ok), ctypes.byref(ok), FAKE, 2, 32, None) == -1     # dtype
    assert f(0, ctypes.byref(ok), ctypes.byref(ok), None, 1, 32, None) == -1
    assert f(0, ctypes.byref(ok), ctypes.byref(ok), ctypes.c_void_p(0x10001), 1, 32, None) == -1
    assert f(0, ctypes.byref(ok), ctypes.byref(ok), ctypes.c_void_p(0x10002), 0, 32, None) == -1
    assert f(1, ctypes.byref(ok), ctypes.byref(fake_desc(grid=1)), FAKE, 1, 32, None) == -3
    assert f(2, ctypes.byref(ok), ctypes.byref(ok), FAKE, 1, 16, None) == -2     # ldc < N
    g = L.ufp4_grouped_gemm_out
    assert g(0, 2, FAKE, ctypes.byref(ok), ctypes.byref(ok), FAKE, 5, 32, None) == -1
    assert g(0, 2, None, ctypes.byref(ok), ctypes.byref(ok), FAKE, 1, 32, None) == -1
    assert g(0, 0, FAKE, ctypes.byref(ok), ctypes.byref(ok), FAKE, 1, 32, None) == -2
    assert g(1, 2, FAKE, ctypes.byref(ok), ctypes.byref(ok), ctypes.c_void_p(0x10001), 1, 32,
             None) == -1


def test_probe_library_loads_and_rejects_bad_arguments():
    import bench
    L = bench.probe_lib()
    assert L.ufp4_probe_mfma_flops(0) == 2 * 32 * 32 * 16
    assert L.ufp4_probe_mfma_flops(4) == 2 * 32 * 32 * 64
    assert L.ufp4_probe_mfma_flops(6) == 2 * 32 * 32 * 2   # FP32 outer product, two blocks
    assert L.ufp4_probe_mfma_flops(9) == 0
    assert L.ufp4_probe_mfma_tflops(9, 1, 1) == -1.0      # rejected before any HIP call
    assert L.ufp4_probe_mfma_tflops(0, 0, 1) == -1.0
    assert L.ufp4_probe_mix_ms(3, 1, 1) == -1.0
    assert L.ufp4_probe_mix_ms(0, 1, 0) == -1.0
    assert L.ufp4_probe_overlap_ms(3, 1, 1, 1) == -1.0   # unknown matrix-core kind
    assert L.ufp4_probe_overlap_ms(0, 0, 1, 1) == -1.0   # no role
    assert L.ufp4_probe_overlap_ms(0, 4, 1, 1) == -1.0
    assert L.ufp4_probe_overlap_ms(0, 3, 0, 1) == -1.0


def test_size_limits_of_32_bit_offsets():
    # column-wise quantization of rows longer than 2^26 elements, GEMM K beyond 2^24
    assert quant(axis=1, ld=(1 << 26) + 2, out=fake_desc(rows=32, kpad=32)) == -4
    big = fake_desc(k=(1 << 24) + 16, kpad=(1 << 24) + 16)
    assert gemm(U.lib().ufp4_gemm_fprop, big, big) == -4
    L = U.lib()
    assert L.ufp4_gemm_out(0, ctypes.byref(big), ctypes.byref(big), FAKE, 1, 32, None) == -4
    for kind in (0, 1, 2):
        assert L.ufp4_grouped_gemm(kind, 2, FAKE, ctypes.byref(big), ctypes.byref(big), FAKE, 32,
                                   None, 0, None) == -4
        assert L.ufp4_grouped_gemm_out(kind, 2, FAKE, ctypes.byref(big), ctypes.byref(big), FAKE,
                                       0, 32, None) == -4
    # at most 1024 groups
    ok = fake_desc()
    assert L.ufp4_grouped_gemm(0, 1025, FAKE, ctypes.byref(ok), ctypes.byref(ok), FAKE, 32, None,
                               0, None) == -2
    assert L.ufp4_grouped_gemm_out(2, 1025, FAKE, ctypes.byref(ok), ctypes.byref(ok), FAKE, 0, 32,
                                   None) == -2


def test_workspace_size_splits_long_k_of_small_outputs():
    """ufp4_workspace_size: FP32 partial outputs of the K splits of a dense
    WGRAD whose 128x128 output tiles fill fewer than the 512 workgroups the GPU
    runs at once; at most 16 splits of at least 64 blocks each; 0 otherwise."""
    ws = U.ufp4_workspace_size
    # 256 x 256 weight gradient over 149184 tokens (a MoE-124B expert's share):
    # 4 tiles, min(16, 512 // 4, 9324 // 64) = 16 splits
    assert ws(2, 256, 256, 149184, 1) == 16 * 256 * 256 * 4
    # 1024 x 1024 over 8192 tokens: 64 tiles, min(16, 8, 512 // 64) = 8
    assert ws(2, 1024, 1024, 8192, 1) == 8 * 1024 * 1024 * 4
    # the dense 1.5B layer's dW (8192 x 2048 = 1024 tiles) fills the GPU
    assert ws(2, 8192, 2048, 8192, 1) == 0
    # short K: 2048 x 2048 over 1024 tokens (64 blocks) cannot split twice
    assert ws(2, 2048, 2048, 1024, 1) == 0
    # only the dense WGRAD splits; bad shapes need nothing
    assert ws(0, 256, 256, 149184, 1) == 0 and ws(1, 256, 256, 149184, 1) == 0
    assert ws(2, 256, 256, 149184, 4) == 0
    assert ws(2, 0, 256, 4096, 1) == 0 and ws(2, 256, 256, 4008, 1) == 0


def test_wgrad_workspace_arguments():
    L = U.lib()
    a, b = fake_desc(), fake_desc()
    # NULL workspace with a size, a size-0 workspace, a misaligned workspace
    assert L.ufp4_gemm_wgrad(ctypes.byref(a), ctypes.byref(b), FAKE, 32, None, 64, None) == -1
    assert L.ufp4_gemm_wgrad(ctypes.byref(a), ctypes.byref(b), FAKE, 32,
                             ctypes.c_void_p(0x20000), 0, None) == -1
    assert L.ufp4_gemm_wgrad(ctypes.byref(a), ctypes.byref(b), FAKE, 32,
                             ctypes.c_void_p(0x20002), 64, None) == -1
    # operand validation still comes first with a valid workspace
    bad = fake_desc(kpad=48)
    assert L.ufp4_gemm_wgrad(ctypes.byref(a), ctypes.byref(bad), FAKE, 32,
                             ctypes.c_void_p(0x20000), 64, None) == -3


@pytest.mark.parametrize("kw,expect", [
    (dict(x=None), -1), (dict(out=None), -1), (dict(out=ctypes.c_void_p(0x30004)), -1),
    (dict(axis=2), -1), (dict(axis=7), -1),
    (dict(q=fake_desc(rows=32, k=48, kpad=64)), -2),
    (dict(q=fake_desc(rows=31, k=48, kpad=48)), -2),
    (dict(axis=1), -2), (dict(ld=40), -2), (dict(n_rows=0), -2),
])
def test_quant_stats_noalloc_rejects(kw, expect):
    """The no-allocation diagnostics call validates exactly as
    ufp4_quant_stats (it has no workspace to check) before touching the GPU."""
    a = dict(x=FAKE, n_rows=32, n_cols=48, ld=48, axis=0, q=fake_desc(rows=32, k=48, kpad=48),
             out=ctypes.c_void_p(0x30000))
    a.update(kw)
    assert U.lib().ufp4_quant_stats_noalloc(a["x"], a["n_rows"], a["n_cols"], a["ld"], a["axis"],
                                            ctypes.byref(a["q"]), a["out"], None) == expect


def test_grouped_capacity_rows_start_on_128_byte_boundaries():
    """The binding's kpad for a grouped ALONG_ROWS output is at least the
    call's minimum roundup16(rows + 15 * groups) and a multiple of 512, so
    each output row's codes (kpad/2 bytes) and scales (kpad/4 bytes) start on
    a 128-byte boundary; the MoE-124B tokens give 524800, not 524768."""
    for rows, groups in ((524288, 32), (98304, 64), (1, 1), (255, 1), (256, 1), (4096, 1024)):
        kp = U.padded_k_capacity(rows, groups)
        minimum = (rows + 15 * groups + 15) // 16 * 16
        assert kp >= minimum and kp - minimum < 512
        assert kp % 512 == 0 and (kp // 2) % 128 == 0 and (kp // 16 * 4) % 128 == 0
    assert U.padded_k_capacity(524288, 32) == 524800
