"""The C ABI on the host: the library loads, exports every function that
include/rfpx.h declares, and rejects bad arguments before launching
anything (these calls never reach the GPU, so they run without one)."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import block_quantized_expert_amd as bqe
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rfpx.h")


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(rfpx_\w+|moe_\w+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bqe.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return bqe.lib()


def test_exports_every_declared_function(lib):
    declared = header_functions()
    assert len(declared) == 27
    assert set(declared) == set(bqe.SYMBOLS)
    for name in declared:
        assert hasattr(lib, name), name


def test_block_and_matrix_bytes(lib):
    assert [lib.rfpx_block_bytes(f) for f in (2, 3, 4)] == [10, 14, 17]
    assert lib.rfpx_block_bytes(5) == 0
    assert lib.rfpx_matrix_bytes(2, 2048, 4096) == 2048 * 128 * 10 == 2621440
    assert lib.rfpx_matrix_bytes(3, 4096, 2048) == 3670016
    assert lib.rfpx_matrix_bytes(4, 2048, 4096) == 4456448
    assert lib.rfpx_matrix_bytes(2, 4, 33) == 0


def _fmts(E, hot=()):
    f = np.empty((E + 1, 3), np.int32)
    f[:, :2], f[:, 2] = 2, 3
    for e in hot:
        f[e] = 4
    f[E] = 4
    return f


def test_image_bytes_equal_canonical_plus_header(lib):
    # decode-size layer: every plane is a multiple of 256 bytes, so the image
    # is the canonical bytes plus the header and the expert table
    E, d, f = 256, 4096, 2048
    fm = _fmts(E)
    n = bqe.moe_image_bytes(d, f, E, fm)
    canonical = 256 * (2 * 2621440 + 3670016) + 3 * 4456448 - 4456448 + 2 * 4456448
    canonical = 256 * 8912896 + 13369344
    assert canonical == 2295070720
    table = (64 + 257 * 64 + 255) // 256 * 256
    assert n == canonical + table
    # hot experts in FP4 (the q=5 mixed layer): 32 * (13369344 - 8912896) more
    n4 = bqe.moe_image_bytes(d, f, E, _fmts(E, hot=range(32)))
    assert n4 - table == 2295070720 + 32 * (13369344 - 8912896) == 2437677056


def test_image_bytes_rejects_bad_tables(lib):
    fm = _fmts(8)
    fm[3, 1] = 7
    assert bqe.moe_image_bytes(256, 128, 8, fm) == 0
    assert bqe.moe_image_bytes(256, 100, 8, _fmts(8)) == 0


class _Dummy:
    """Stand-ins for device tensors: only data_ptr() and numel() are read,
    and every call below fails validation before anything dereferences
    it."""

    def __init__(self, ptr, n=0):
        self._p = ptr
        self._n = n
        self.is_cuda = True

    def data_ptr(self):
        return self._p

    def numel(self):
        return self._n

    def is_contiguous(self):
        return True


def _layer(d=256, f=128, E=8, k=2, fmts=None, image=4096, wr=8192, image_bytes=None):
    """A layer whose image_bytes is, unless given, the layout of its table
    (0 where the table itself is invalid)."""
    fm = _fmts(E) if fmts is None else fmts
    if image_bytes is None:
        image_bytes = bqe.moe_image_bytes(d, f, E, fm) if E >= 1 else 0
    return bqe.MoeLayer(d, f, E, k, _Dummy(wr), _Dummy(image, image_bytes), fm)


def _fwd(lib, L, x=0x10000, xtype=0, q=1, y=0x20000, ws=0x30000, nbytes=1 << 30):
    return lib.moe_layer_forward(L.ref, C.c_void_p(x), xtype, q, C.c_void_p(y),
                                 C.c_void_p(ws), nbytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(d=300), -2), (dict(d=8192), -2), (dict(f=48), -2), (dict(E=0), -2),
    (dict(k=9), -2), (dict(E=4, k=5), -2),
])
def test_forward_rejects_shapes(lib, kw, status):
    E = kw.pop("E", 8)
    fm = _fmts(max(E, 1))[: E + 1] if E > 0 else _fmts(1)[:1]
    L = _layer(E=E, fmts=fm, **kw)
    assert _fwd(lib, L) == status
    assert lib.rfpx_last_error()


def test_forward_rejects_arguments(lib):
    L = _layer()
    assert _fwd(lib, L, q=0) == -2
    assert _fwd(lib, L, q=9) == -2
    assert _fwd(lib, L, xtype=3) == -1
    assert _fwd(lib, L, x=0) == -1
    assert _fwd(lib, L, y=0) == -1
    assert _fwd(lib, L, ws=0) == -1
    assert _fwd(lib, L, ws=0x30010) == -3          # misaligned workspace
    assert _fwd(lib, L, x=0x10004) == -3           # misaligned x
    assert _fwd(lib, _layer(image=4096 + 64)) == -3
    assert _fwd(lib, L, nbytes=16) == -5
    assert b"workspace" in lib.rfpx_last_error()
    fm = _fmts(8)
    fm[2, 1] = 4  # gate FP2, up FP4
    assert _fwd(lib, _layer(fmts=fm)) == -4
    fm = _fmts(8)
    fm[5, 2] = 9
    assert _fwd(lib, _layer(fmts=fm)) == -4


def test_forward_checks_image_bytes(lib):
    """image_bytes must equal the layout of the format table: one byte more
    or less, or the layout of another table, is a format error."""
    n = bqe.moe_image_bytes(256, 128, 8, _fmts(8))
    for bad in (n - 1, n + 1, 0, bqe.moe_image_bytes(256, 128, 8, _fmts(8, hot=[1]))):
        assert _fwd(lib, _layer(image_bytes=bad)) == -4
        assert b"image_bytes" in lib.rfpx_last_error()
        assert _pf(lib, _layer(image_bytes=bad)) == -4
    assert _fwd(lib, _layer(image=0)) == -1


def test_route_topk_does_not_check_the_image(lib):
    """moe_route_topk reads only the router: a null image of size 0 passes
    its host checks; the same layer is rejected by moe_layer_forward."""
    L = _layer(image=0, image_bytes=0)
    ids, w = C.c_void_p(0x40000), C.c_void_p(0x50000)
    st = lib.moe_route_topk(L.ref, C.c_void_p(0x10000), 0, 1, ids, w,
                            C.c_void_p(0x30010), 1 << 30, None)
    assert st == -3  # it gets as far as the workspace alignment
    assert _fwd(lib, L, ws=0x30010) == -1  # image is null


def test_noalloc_rejects_before_any_launch(lib):
    """moe_layer_forward_noalloc makes the checks of moe_layer_forward, and
    refuses a shape whose workspace exceeds the library's scratch, before
    it touches the device."""
    assert lib.moe_noalloc_scratch_bytes() == 8 << 20
    L = _layer()
    x, y = C.c_void_p(0x10000), C.c_void_p(0x20000)
    assert lib.moe_layer_forward_noalloc(L.ref, x, 0, 9, y, None) == -2
    assert lib.moe_layer_forward_noalloc(_layer(image_bytes=3).ref, x, 0, 1, y, None) == -4
    big = _layer(d=4096, f=4096, E=64, k=8, fmts=_fmts(64))
    assert bqe.moe_workspace_bytes(big, 8) > 8 << 20
    assert lib.moe_layer_forward_noalloc(big.ref, x, 1, 8, y, None) == -5
    assert b"scratch" in lib.rfpx_last_error()
    # the spec shapes fit (a q=8 step of the d=4096, E=256, k=6 layer)
    ns = _layer(d=4096, f=2048, E=256, k=6, fmts=_fmts(256))
    assert bqe.moe_workspace_bytes(ns, 8) <= 8 << 20


def test_image_validate_host_checks(lib):
    """moe_image_validate checks its arguments and image_bytes on the host."""
    L = _layer()
    rep = C.c_void_p(0x60000)
    assert lib.moe_image_validate(L.ref, None, None) == -1
    assert lib.moe_image_validate(L.ref, C.c_void_p(0x60002), None) == -3
    assert lib.moe_image_validate(_layer(image_bytes=1).ref, rep, None) == -4
    assert lib.moe_image_validate(_layer(image=4096 + 16).ref, rep, None) == -3
    assert lib.moe_image_validate(_layer(d=300).ref, rep, None) == -2
    assert lib.moe_image_unpack(_layer(image_bytes=5).ref, 0, 0, C.c_void_p(0x70000), None) == -4


def _pf(lib, L, x=0x10000, xtype=1, T=64, y=0x20000, ws=0x30000, nbytes=1 << 32):
    return lib.moe_prefill_forward(L.ref, C.c_void_p(x), xtype, T, C.c_void_p(y),
                                   C.c_void_p(ws), nbytes, None)


def test_prefill_rejects_arguments(lib):
    """Every check of moe_prefill_forward fails before any launch."""
    L = _layer()
    assert _pf(lib, L, T=0) == -2
    assert _pf(lib, L, T=65537) == -2
    assert _pf(lib, L, xtype=3) == -1
    assert _pf(lib, L, x=0) == -1
    assert _pf(lib, L, y=0) == -1
    assert _pf(lib, L, ws=0) == -1
    assert _pf(lib, L, ws=0x30010) == -3           # misaligned workspace
    assert _pf(lib, L, x=0x10008) == -3            # misaligned x
    assert _pf(lib, L, y=0x20004) == -3            # misaligned y
    assert _pf(lib, _layer(image=4096 + 64)) == -3
    need = bqe.moe_workspace_bytes(L, 64, prefill=True)  # sized for fp32 x
    assert need > 0
    assert _pf(lib, L, xtype=0, nbytes=need - 1) == -5
    assert b"workspace" in lib.rfpx_last_error()
    fm = _fmts(8)
    fm[3, 0] = 3  # gate FP3, up FP2
    assert _pf(lib, _layer(fmts=fm)) == -4
    # the prefill workspace grows with T, and fp32 x needs the most
    assert bqe.moe_workspace_bytes(L, 128, prefill=True) > need


def test_workspace_bytes_shapes(lib):
    L = _layer()
    n1 = bqe.moe_workspace_bytes(L, 1)
    n4 = bqe.moe_workspace_bytes(L, 4)
    assert 0 < n1 < n4
    assert bqe.moe_workspace_bytes(L, 9) == 0
    assert bqe.moe_workspace_bytes(_layer(d=4096, f=2048, E=256, k=6,
                                          fmts=_fmts(256)), 5) > 0


def test_codec_rejects_bad_arguments(lib):
    p = C.c_void_p(0x1000)
    assert lib.rfpx_pack(5, p, 4, 64, p, 1 << 20, None) == -4
    assert lib.rfpx_pack(2, p, 4, 33, p, 1 << 20, None) == -2
    assert lib.rfpx_pack(2, p, 4, 64, p, 10, None) == -5
    assert lib.rfpx_pack(2, None, 4, 64, p, 1 << 20, None) == -1
    assert lib.rfpx_pack(2, p, 0, 64, p, 0, None) == 0  # empty matrix: nothing to do
    assert lib.rfpx_unpack(3, None, 4, 64, p, None) == -1
    assert lib.rfpx_pack_codes(4, p, None, 4, 64, p, 1 << 20, None) == -1
    assert lib.rfpx_pack_weighted(2, p, None, 4, 64, p, 1 << 20, None) == -1
    assert lib.rfpx_pack_weighted(7, p, p, 4, 64, p, 1 << 20, None) == -4
    assert lib.rfpx_pack_weighted(3, p, p, 4, 40, p, 1 << 20, None) == -2
    assert lib.rfpx_pack_weighted(4, p, p, 4, 64, p, 16, None) == -5


def test_dense_host_checks(lib):
    """Shapes, formats and arguments of the dense projection entry points,
    all checked before any launch."""
    assert lib.rfpx_dense_image_bytes(4, 64, 4096) == 64 * 128 * 16 + 64 * 128 * 1
    assert lib.rfpx_dense_image_bytes(2, 128, 256) == 128 * 8 * 8 + 128 * 8 * 2
    assert lib.rfpx_dense_image_bytes(3, 64, 96) == (64 * 3 * 12 + 255) // 256 * 256 + 64 * 3 * 2
    assert lib.rfpx_dense_image_bytes(4, 100, 256) == 0     # rows not a multiple of 64
    assert lib.rfpx_dense_image_bytes(2, 64, 96) == 0       # FP2 needs cols % 64
    assert lib.rfpx_dense_image_bytes(5, 64, 256) == 0
    assert lib.rfpx_dense_workspace_bytes(4, 4096, 4096, 9) == 0
    assert lib.rfpx_dense_workspace_bytes(4, 4096, 4096, 5) > 0
    p = C.c_void_p(0x1000)
    fwd = lambda **k: lib.rfpx_dense_forward(  # noqa: E731
        k.get("fmt", 4), k.get("img", p), k.get("rows", 64), k.get("cols", 256),
        k.get("x", p), k.get("xt", 1), k.get("q", 1), k.get("y", p), k.get("ws", p),
        k.get("nbytes", 1 << 30), None)
    assert fwd(q=0) == -2 and fwd(q=9) == -2 and fwd(rows=65) == -2
    assert fwd(fmt=7) == -4 and fwd(xt=2) == -1 and fwd(x=None) == -1
    assert fwd(img=C.c_void_p(0x1010)) == -3 and fwd(x=C.c_void_p(0x1008)) == -3
    # a tile split over several workgroups keeps partial sums in the workspace
    assert lib.rfpx_dense_workspace_bytes(4, 64, 4096, 1) > 256
    assert fwd(cols=4096, nbytes=256) == -5
    assert lib.rfpx_dense_image_build(4, p, 64, 256, p, 16, None) == -5
    assert lib.rfpx_dense_image_build(4, None, 64, 256, p, 1 << 20, None) == -1


def test_stream_read_host_checks(lib):
    p = C.c_void_p(0x1000)
    assert lib.rfpx_stream_read_sink_words() == 2048
    assert lib.rfpx_stream_read(None, 64, p, None) == -1
    assert lib.rfpx_stream_read(p, 0, p, None) == -3
    assert lib.rfpx_stream_read(p, 40, p, None) == -3
    assert lib.rfpx_stream_read(C.c_void_p(0x1008), 64, p, None) == -3
    assert lib.rfpx_stream_read(p, 64, C.c_void_p(0x2002), None) == -3


def test_status_strings(lib):
    assert lib.rfpx_status_str(0) == b"ok"
    assert lib.rfpx_status_str(-5).startswith(b"workspace")
    assert lib.rfpx_status_str(42) == b"unknown status"


def test_generator_layer_shapes_match_library(lib):
    lay = synth.gen_layer(synth.WORKLOADS[synth.TINY], 0, threads=2)
    for e in range(lay.E + 1):
        for m in range(3):
            rows, cols = lay.matrix_shape(m)
            assert lay.mat(e, m).size == lib.rfpx_matrix_bytes(int(lay.fmts[e][m]), rows, cols)
