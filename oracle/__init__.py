"""TEST INFRASTRUCTURE ONLY: ctypes access to the plain-C CPU oracle.

The oracle (oracle.c) is an independent double-precision reference for one
routed-MoE layer over ROCmFP2/FP3/FP4 experts.  It shares no code with the GPU
library.  Only the tests, the package smoke check and the benchmark's CPU
baseline may import this module; the library never does.

``build()`` compiles oracle.c with gcc into oracle/liboracle.so.  The ctypes
calls release the GIL, so independent oracle calls may run on several Python
threads at once.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
import threading

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

FP2, FP3, FP4 = 2, 3, 4
_lock = threading.Lock()
_lib = None


def build() -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared",
           "-o", LIB + ".tmp", SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if (not os.path.exists(LIB)
                or os.path.getmtime(LIB) < os.path.getmtime(SRC)):
            build()
        lib = C.CDLL(LIB)
        P = C.c_void_p
        i, d = C.c_int, C.c_double
        sig = {
            "orc_block_bytes": (i, [i]),
            "orc_half_to_double": (d, [C.c_uint16]),
            "orc_bf16_to_double": (d, [C.c_uint16]),
            "orc_double_to_half_rne": (C.c_uint16, [d]),
            "orc_block_codes": (None, [i, P, P, P]),
            "orc_decode_block": (None, [i, P, P]),
            "orc_unpack": (None, [i, P, i, i, P]),
            "orc_pack_codes": (None, [i, P, P, i, i, P]),
            "orc_pack": (None, [i, P, i, i, P]),
            "orc_router_scores": (None, [P, i, i, P, i, P]),
            "orc_topk": (None, [P, i, i, P]),
            "orc_gating": (None, [P, P, i, d, P]),
            "orc_expert_forward": (None, [P, i, P, i, P, i, i, i, P, P]),
            "orc_layer_forward": (None, [i, i, i, i, d, P, P, P, P, i, i, P, P, P]),
            "orc_pack_weighted": (None, [i, P, P, i, i, P]),
            "orc_dense_forward": (None, [i, P, i, i, P, i, i, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
        return lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(C.c_void_p)


def block_bytes(fmt: int) -> int:
    return _load().orc_block_bytes(fmt)


def half_to_double(bits: int) -> float:
    return _load().orc_half_to_double(bits)


def bf16_to_double(bits: int) -> float:
    return _load().orc_bf16_to_double(bits)


def double_to_half_rne(v: float) -> int:
    return _load().orc_double_to_half_rne(v)


def block_codes(fmt: int, blk) -> tuple:
    b = np.ascontiguousarray(np.frombuffer(bytes(blk), np.uint8))
    codes = np.zeros(32, np.int32)
    s = np.zeros(1, np.float64)
    _load().orc_block_codes(fmt, _p(b), _p(codes), _p(s))
    return codes, float(s[0])


def decode_block(fmt: int, blk) -> np.ndarray:
    b = np.ascontiguousarray(np.frombuffer(bytes(blk), np.uint8))
    w = np.zeros(32, np.float64)
    _load().orc_decode_block(fmt, _p(b), _p(w))
    return w


def unpack(fmt: int, data: np.ndarray, rows: int, cols: int) -> np.ndarray:
    data = np.ascontiguousarray(data, np.uint8)
    assert data.size == rows * (cols // 32) * block_bytes(fmt)
    w = np.empty((rows, cols), np.float64)
    _load().orc_unpack(fmt, _p(data), rows, cols, _p(w))
    return w


def pack(fmt: int, w: np.ndarray) -> np.ndarray:
    w = np.ascontiguousarray(w, np.float32)
    rows, cols = w.shape
    out = np.empty(rows * (cols // 32) * block_bytes(fmt), np.uint8)
    _load().orc_pack(fmt, _p(w), rows, cols, _p(out))
    return out


def pack_weighted(fmt: int, w: np.ndarray, imp: np.ndarray) -> np.ndarray:
    """Importance-weighted quantizer: imp[cols] >= 0 per input column."""
    w = np.ascontiguousarray(w, np.float32)
    rows, cols = w.shape
    imp = np.ascontiguousarray(imp, np.float32)
    assert imp.shape == (cols,)
    out = np.empty(rows * (cols // 32) * block_bytes(fmt), np.uint8)
    _load().orc_pack_weighted(fmt, _p(w), _p(imp), rows, cols, _p(out))
    return out


def dense_forward(fmt: int, data: np.ndarray, rows: int, cols: int, x: np.ndarray,
                  xtype: str) -> np.ndarray:
    """y[q][rows] fp32 = W x_c for each column of x ([q][cols] fp32, or
    uint16 bf16 bits with xtype "bf16")."""
    data = np.ascontiguousarray(data, np.uint8)
    assert data.size == rows * (cols // 32) * block_bytes(fmt)
    xt = 1 if xtype == "bf16" else 0
    x = np.ascontiguousarray(x, np.uint16 if xt else np.float32).reshape(-1, cols)
    q = x.shape[0]
    y = np.empty((q, rows), np.float32)
    _load().orc_dense_forward(fmt, _p(data), rows, cols, _p(x), xt, q, _p(y))
    return y


def pack_codes(fmt: int, codes: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    rows, cols = codes.shape
    sb = np.ascontiguousarray(scale_bits, np.uint16)
    assert sb.size == rows * (cols // 32)
    out = np.empty(rows * (cols // 32) * block_bytes(fmt), np.uint8)
    _load().orc_pack_codes(fmt, _p(codes), _p(sb), rows, cols, _p(out))
    return out


def router_scores(x: np.ndarray, wr: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(np.atleast_2d(x), np.float64)
    wr = np.ascontiguousarray(wr, np.float32)
    q, d = x.shape
    E = wr.shape[0]
    s = np.empty((q, E), np.float64)
    _load().orc_router_scores(_p(x), q, d, _p(wr), E, _p(s))
    return s


def topk(s: np.ndarray, k: int) -> np.ndarray:
    s = np.ascontiguousarray(s, np.float64)
    ids = np.empty(k, np.int32)
    _load().orc_topk(_p(s), s.size, k, _p(ids))
    return ids


def gating(s: np.ndarray, ids: np.ndarray, routed_scale: float = 1.0) -> np.ndarray:
    s = np.ascontiguousarray(s, np.float64)
    ids = np.ascontiguousarray(ids, np.int32)
    w = np.empty(ids.size, np.float64)
    _load().orc_gating(_p(s), _p(ids), ids.size, routed_scale, _p(w))
    return w


def expert_forward(gate, up, down, fmts, d: int, f: int, x: np.ndarray) -> np.ndarray:
    g, u, dn = (np.ascontiguousarray(a, np.uint8) for a in (gate, up, down))
    x = np.ascontiguousarray(x, np.float64)
    o = np.empty(d, np.float64)
    _load().orc_expert_forward(_p(g), int(fmts[0]), _p(u), int(fmts[1]), _p(dn),
                               int(fmts[2]), d, f, _p(x), _p(o))
    return o


def layer_forward(d: int, f: int, E: int, k: int, wr: np.ndarray, mats, fmts,
                  x: np.ndarray, xtype: str, routed_scale: float = 1.0):
    """y[q][d] fp32, ids[q][k], w[q][k] for q columns.

    mats: (E+1)*3 uint8 arrays (gate, up, down per expert; the last expert is
    the shared one); fmts: matching formats; x: float32 [q][d] (xtype "f32")
    or uint16 bf16 bits (xtype "bf16")."""
    lib = _load()
    wr = np.ascontiguousarray(wr, np.float32)
    arrs = [np.ascontiguousarray(m, np.uint8) for m in mats]
    assert len(arrs) == 3 * (E + 1)
    ptrs = (C.c_void_p * len(arrs))(*[a.ctypes.data for a in arrs])
    fm = np.ascontiguousarray(np.asarray(fmts).reshape(-1), np.int32)
    xt = 1 if xtype == "bf16" else 0
    x = np.ascontiguousarray(x, np.uint16 if xt else np.float32)
    x = x.reshape(-1, d)
    q = x.shape[0]
    y = np.empty((q, d), np.float32)
    ids = np.empty((q, k), np.int32)
    w = np.empty((q, k), np.float64)
    lib.orc_layer_forward(d, f, E, k, routed_scale, _p(wr), ptrs, _p(fm), _p(x),
                          xt, q, _p(y), _p(ids), _p(w))
    return y, ids, w


def layer_forward_synth(lay, cols_x: np.ndarray, xtype: str):
    """Convenience: run the oracle on a synth.Layer."""
    mats = [lay.mat(e, m) for e in range(lay.E + 1) for m in range(3)]
    return layer_forward(lay.d, lay.f, lay.E, lay.k, lay.wr, mats, lay.fmts,
                         cols_x, xtype, lay.routed_scale)
