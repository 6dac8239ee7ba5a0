"""The C-ABI library on the host: it loads, exports every declared symbol, and its
host-only calls (codebook, sizes, workspace queries, argument validation) behave
as documented.  No kernel is launched here."""
import ctypes as C
import os
import re

import numpy as np
import pytest

from bit_nf4_quantized_11_amd import _lib
from oracle import nf4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "qlora.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(qlora_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported(lib):
    names = _declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
        assert n in _lib.SIGNATURES, n
    assert set(_lib.SIGNATURES) == set(names)


def test_library_codebook_matches_oracle(lib):
    lv = (C.c_float * 16)()
    th = (C.c_float * 15)()
    assert lib.qlora_nf4_codebook(lv, th) == 0
    lv = np.array(lv, dtype=np.float32)
    th = np.array(th, dtype=np.float32)
    assert np.array_equal(lv.view(np.uint32), nf4.nf4_levels().view(np.uint32))
    # thresholds: largest fp32 not above each exact midpoint; encoding with them equals nearest level
    mids = (lv.astype(np.float64)[:-1] + lv.astype(np.float64)[1:]) / 2
    assert np.all(th.astype(np.float64) <= mids)
    assert np.all(np.nextafter(th, np.float32(2)).astype(np.float64) > mids)
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.uniform(-1, 1, 100_000).astype(np.float32), th, np.nextafter(th, np.float32(2)),
                        mids.astype(np.float32)])
    by_thr = (x[:, None] > th[None, :]).sum(axis=1)
    assert np.array_equal(by_thr, nf4.nearest_level(x))


@pytest.mark.parametrize("cb,name", [(0, "nf4"), (1, "fp4"), (2, "int4")])
def test_library_codebook_tables_match_oracle(lib, cb, name):
    """Every table the library offers equals the oracle's bit for bit, and encoding with its
    thresholds equals the oracle's nearest level."""
    lv = (C.c_float * 16)()
    th = (C.c_float * 15)()
    assert lib.qlora_codebook_table(cb, lv, th) == 0
    lv = np.array(lv, dtype=np.float32)
    th = np.array(th, dtype=np.float32)
    ref = nf4.codebook_levels(name)
    assert np.array_equal(lv.view(np.uint32), ref.view(np.uint32))
    mids = (lv.astype(np.float64)[:-1] + lv.astype(np.float64)[1:]) / 2
    assert np.all(th.astype(np.float64) <= mids)
    assert np.all(np.nextafter(th, np.float32(2)).astype(np.float64) > mids)
    rng = np.random.default_rng(cb)
    x = np.concatenate([rng.uniform(-1, 1, 100_000).astype(np.float32), th, np.nextafter(th, np.float32(2))])
    assert np.array_equal((x[:, None] > th[None, :]).sum(axis=1), nf4.nearest_level(x, ref))
    assert lib.qlora_codebook_table(3, lv.ctypes.data_as(C.POINTER(C.c_float)), None) == 4
    assert lib.qlora_codebook_table(-1, None, None) == 4


@pytest.mark.parametrize("block", [0, 32, 64, 128, 256])
@pytest.mark.parametrize("rows,cols,dq", [(4096, 4096, 1), (256, 256, 0), (3, 77, 1), (1, 1, 1), (22016, 8192, 1),
                                          (5, 77, 0)])
def test_sizes_match_oracle(lib, rows, cols, dq, block):
    out = [C.c_size_t() for _ in range(4)]
    assert lib.qlora_nf4_sizes(rows, cols, dq, block, *[C.byref(o) for o in out]) == 0
    ref = nf4.storage_bytes(rows * cols, bool(dq), block or 64)
    assert [o.value for o in out] == [ref["codes"], ref["absmax"], ref["c1"], ref["mu"]]


def test_sizes_reject_bad_arguments(lib):
    z = C.c_size_t()
    assert lib.qlora_nf4_sizes(0, 5, 1, 64, C.byref(z), None, None, None) == 2
    assert lib.qlora_nf4_sizes(5, -1, 1, 64, None, None, None, None) == 2
    assert lib.qlora_nf4_sizes(5, 5, 7, 64, None, None, None, None) == 4
    for b in (16, 48, 512, -64):
        assert lib.qlora_nf4_sizes(5, 5, 1, b, None, None, None, None) == 4


def test_workspace_queries(lib):
    assert lib.qlora_quantize_workspace(4096, 4096, 0, 64) == 0
    assert lib.qlora_quantize_workspace(4096, 4096, 1, 64) >= 4 * 262144
    assert lib.qlora_quantize_workspace(4096, 4096, 1, 32) >= 4 * 2 * 262144
    assert lib.qlora_quantize_workspace(4096, 4096, 1, 48) == 0
    for M in (0, 1, 16, 17, 2048):
        f = lib.qlora_fwd_workspace(M, 4096, 4096, 64)
        b = lib.qlora_bwd_workspace(M, 4096, 4096, 64)
        assert f > 0 and b > 0 and f % 256 == 0 and b % 256 == 0
    assert lib.qlora_fwd_workspace(16, 4096, 4096, 300) == 0
    # queries with an empty dimension answer without dividing by a zero tile count
    for M, din, dout in ((0, 4096, 4096), (128, 4096, 0), (128, 0, 4096), (512, 0, 0), (0, 0, 0)):
        assert lib.qlora_fwd_workspace(M, din, dout, 64) >= 0
        assert lib.qlora_bwd_workspace(M, din, dout, 64) >= 0


def _desc(rows=256, cols=256, dq=1, codes=0x10000, absmax=0x20000, c1=0x30000, mu=0x40000, cb=0, block=0):
    return _lib.qlora_nf4(rows, cols, dq, cb, block, 0, codes, absmax, c1, mu)


def test_validation_errors_return_before_any_launch(lib):
    ok = C.c_void_p(0x100000)
    ws = C.c_void_p(0x200000)
    big = 1 << 40
    d = _desc()
    fwd = lib.qlora_linear_fwd
    # NULL pointers
    assert fwd(None, 16, C.byref(d), ok, ok, 8, 2.0, ok, None, ws, big, None) == 1
    assert fwd(ok, 16, None, ok, ok, 8, 2.0, ok, None, ws, big, None) == 1
    dn = _desc(codes=0)
    assert fwd(ok, 16, C.byref(dn), ok, ok, 8, 2.0, ok, None, ws, big, None) == 1
    dnc = _desc(c1=0)
    assert fwd(ok, 16, C.byref(dnc), ok, ok, 8, 2.0, ok, None, ws, big, None) == 1
    # shapes: in % 64, out % 8, negative M
    assert fwd(ok, 16, C.byref(_desc(cols=100)), ok, ok, 8, 2.0, ok, None, ws, big, None) == 2
    assert fwd(ok, 16, C.byref(_desc(rows=12)), ok, ok, 8, 2.0, ok, None, ws, big, None) == 2
    assert fwd(ok, -1, C.byref(d), ok, ok, 8, 2.0, ok, None, ws, big, None) == 2
    # unsupported rank
    for r in (0, 4, 12, 264):
        assert fwd(ok, 16, C.byref(d), ok, ok, r, 2.0, ok, None, ws, big, None) == 4
    assert fwd(ok, 16, C.byref(_desc(dq=3)), ok, ok, 8, 2.0, ok, None, ws, big, None) == 4
    assert fwd(ok, 16, C.byref(_desc(cb=3)), ok, ok, 8, 2.0, ok, None, ws, big, None) == 4
    assert lib.qlora_quantize_nf4(ok, 256, 256, C.byref(_desc(cb=-1)), ws, big, None) == 4
    # block sizes: unknown sizes are unsupported; a block must not straddle two weight rows
    for b in (16, 96, 512):
        assert fwd(ok, 16, C.byref(_desc(block=b)), ok, ok, 8, 2.0, ok, None, ws, big, None) == 4
        assert lib.qlora_quantize_nf4(ok, 256, 256, C.byref(_desc(block=b)), ws, big, None) == 4
        assert lib.qlora_dequant(C.byref(_desc(block=b)), ok, None) == 4
    assert fwd(ok, 16, C.byref(_desc(cols=320, block=128)), ok, ok, 8, 2.0, ok, None, ws, big, None) == 2
    assert fwd(ok, 16, C.byref(_desc(cols=384, block=256)), ok, ok, 8, 2.0, ok, None, ws, big, None) == 2
    # alignment
    assert fwd(C.c_void_p(0x100002), 16, C.byref(d), ok, ok, 8, 2.0, ok, None, ws, big, None) == 3
    assert fwd(ok, 16, C.byref(_desc(codes=0x10008)), ok, ok, 8, 2.0, ok, None, ws, big, None) == 3
    # workspace
    need = lib.qlora_fwd_workspace(16, 256, 256, 8)
    assert fwd(ok, 16, C.byref(d), ok, ok, 8, 2.0, ok, None, ws, need - 1, None) == 5
    assert fwd(ok, 16, C.byref(d), ok, ok, 8, 2.0, ok, None, None, need, None) == 5

    bwd = lib.qlora_linear_bwd
    assert bwd(None, ok, None, 16, C.byref(d), ok, ok, 8, 2.0, ok, ok, ok, ws, big, None) == 1
    assert bwd(ok, ok, None, 16, C.byref(d), ok, ok, 8, 2.0, ok, None, ok, ws, big, None) == 1
    assert bwd(ok, ok, None, 16, C.byref(d), ok, ok, 8, 2.0, ok, C.c_void_p(0x100001), ok, ws, big, None) == 3
    assert bwd(ok, ok, None, 16, C.byref(d), ok, ok, 8, 2.0, ok, ok, ok, ws, 10, None) == 5

    q = lib.qlora_quantize_nf4
    assert q(None, 256, 256, C.byref(d), ws, big, None) == 1
    assert q(ok, 0, 256, C.byref(d), ws, big, None) == 2
    assert q(ok, 256, 255, C.byref(d), ws, big, None) == 2          # descriptor shape mismatch
    assert q(ok, 256, 256, C.byref(d), ws, 100, None) == 5
    assert q(C.c_void_p(0x100004), 256, 256, C.byref(d), ws, big, None) == 3
    assert lib.qlora_dequant(C.byref(d), None, None) == 1
    assert lib.qlora_dequant(None, ok, None) == 1


def test_merge_validation(lib):
    ok = C.c_void_p(0x100000)
    d = _desc()
    f = lib.qlora_merge_adapter
    assert f(C.byref(d), None, ok, 8, 0.25, ok, None) == 1
    assert f(C.byref(d), ok, ok, 8, 0.25, None, None) == 1
    assert f(None, ok, ok, 8, 0.25, ok, None) == 1
    assert f(C.byref(_desc(cols=100)), ok, ok, 8, 0.25, ok, None) == 2
    assert f(C.byref(d), ok, ok, 12, 0.25, ok, None) == 4
    assert f(C.byref(d), ok, C.c_void_p(0x100008), 8, 0.25, ok, None) == 3


def test_adamw_validation(lib):
    ok = C.c_void_p(0x100000)
    f = lib.qlora_adamw_step
    assert f(None, None, None, None, None, 0, 1, 1e-3, 0.9, 0.999, 1e-8, 0.0, None) == 0   # n = 0: no-op
    assert f(ok, None, ok, ok, ok, -1, 1, 1e-3, 0.9, 0.999, 1e-8, 0.0, None) == 2
    assert f(ok, None, ok, ok, ok, 8, 0, 1e-3, 0.9, 0.999, 1e-8, 0.0, None) == 2
    assert f(ok, None, ok, ok, ok, 8, 1, 1e-3, 1.0, 0.999, 1e-8, 0.0, None) == 4
    assert f(ok, None, ok, ok, ok, 8, 1, 1e-3, 0.9, 0.999, 0.0, 0.0, None) == 4
    assert f(ok, None, None, ok, ok, 8, 1, 1e-3, 0.9, 0.999, 1e-8, 0.0, None) == 1
    assert f(C.c_void_p(0x100004), None, ok, ok, ok, 8, 1, 1e-3, 0.9, 0.999, 1e-8, 0.0, None) == 3
    assert f(ok, C.c_void_p(0x100002), ok, ok, ok, 8, 1, 1e-3, 0.9, 0.999, 1e-8, 0.0, None) == 3


def test_page_validation(lib):
    """Argument checks of the paging calls that need no device: NULL, size, alignment,
    overlap, and the no-op of zero bytes."""
    a, b = C.c_void_p(0x100000), C.c_void_p(0x200000)
    for f in (lib.qlora_state_page_out, lib.qlora_state_page_in):
        assert f(a, b, 0, None) == 0                            # nothing to copy
        assert f(None, b, 64, None) == 1
        assert f(a, None, 64, None) == 1
        assert f(a, b, 6, None) == 2                            # not whole floats
        assert f(C.c_void_p(0x100008), b, 64, None) == 3
        assert f(a, C.c_void_p(0x200004), 64, None) == 3
        assert f(a, C.c_void_p(0x100010), 64, None) == 2        # overlapping ranges


def test_status_strings(lib):
    for s in range(7):
        assert lib.qlora_status_str(s)
    assert b"gfx950" in lib.qlora_version()


def test_version_names_the_sources_it_was_built_from(lib):
    """The loaded library's version string carries the hash of the current sources
    (the loader refuses a library built from other sources)."""
    from bit_nf4_quantized_11_amd import build

    v = lib.qlora_version().decode()
    assert f"src {build.source_hash()})" in v, v
