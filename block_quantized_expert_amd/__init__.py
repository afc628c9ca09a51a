"""Python binding of librfpx (include/rfpx.h): argument marshalling only.

Every computation runs in the HIP kernels of librfpx.so; PyTorch supplies
device memory and the current stream.  The functions carry the C names and
raise ``RfpxError`` on any non-zero status.  If the library is not built, or
was linked against a different HIP runtime than the one torch loaded, import
of the library fails loudly -- there is no fallback.

Format and layer definitions are in include/rfpx.h; they follow page
"DeepSeek V4 Flash 在 128GB 锐龙 AI MAX+ 上跑到 32 tok/s" (taozi.news),
section "ROCmFPX：把 284B 权重压进 128 GB", and page "Lucebox专攻DeepSeek V4…"
(m.mzlw.cn), section "MoE 专家并行".
"""
from __future__ import annotations

import ctypes as C
import os
import threading
from typing import Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "librfpx.so")

RFPX_FP2, RFPX_FP3, RFPX_FP4 = 2, 3, 4
RFPX_X_F32, RFPX_X_BF16 = 0, 1
Q_MAX, K_MAX, E_MAX = 8, 8, 1024
BLOCK_BYTES = {RFPX_FP2: 10, RFPX_FP3: 14, RFPX_FP4: 17}

# every symbol include/rfpx.h declares
SYMBOLS = (
    "rfpx_block_bytes", "rfpx_matrix_bytes", "rfpx_pack", "rfpx_pack_weighted",
    "rfpx_pack_codes",
    "rfpx_unpack", "moe_image_bytes", "moe_image_build", "moe_image_validate",
    "moe_image_unpack",
    "moe_workspace_bytes", "moe_route_topk", "moe_layer_forward",
    "moe_layer_forward_timed", "moe_layer_forward_noalloc", "moe_noalloc_scratch_bytes",
    "moe_prefill_forward", "moe_prefill_forward_timed",
    "rfpx_dense_image_bytes", "rfpx_dense_image_build", "rfpx_dense_image_unpack",
    "rfpx_dense_workspace_bytes", "rfpx_dense_forward",
    "rfpx_stream_read", "rfpx_stream_read_sink_words",
    "rfpx_status_str", "rfpx_last_error",
)


class RfpxError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: status {status}: {msg}")
        self.status = status


class MoeLayerC(C.Structure):
    _fields_ = [("d", C.c_int), ("f", C.c_int), ("n_experts", C.c_int),
                ("top_k", C.c_int), ("routed_scale", C.c_float),
                ("router_w", C.c_void_p), ("image", C.c_void_p),
                ("fmts", C.POINTER(C.c_int)), ("image_bytes", C.c_size_t)]


_lock = threading.Lock()
_lib = None


def lib():
    """Load librfpx.so once (after torch, so that both share one HIP
    runtime)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        import torch  # noqa: F401  -- torch's HIP runtime must be loaded first
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run __graft_entry__.build() "
                "(hipcc --offload-arch=gfx950)")
        l = C.CDLL(LIB_PATH)
        hips = set()
        with open("/proc/self/maps") as fh:
            for line in fh:
                if "libamdhip64" in line:
                    hips.add(line.split()[-1])
        if len(hips) > 1:
            raise RuntimeError(f"two HIP runtimes in one process: {sorted(hips)}")
        P, I, S = C.c_void_p, C.c_int, C.c_size_t
        LP = C.POINTER(MoeLayerC)
        sig = {
            "rfpx_block_bytes": (S, [I]),
            "rfpx_matrix_bytes": (S, [I, I, I]),
            "rfpx_pack": (I, [I, P, I, I, P, S, P]),
            "rfpx_pack_weighted": (I, [I, P, P, I, I, P, S, P]),
            "rfpx_pack_codes": (I, [I, P, P, I, I, P, S, P]),
            "rfpx_unpack": (I, [I, P, I, I, P, P]),
            "moe_image_bytes": (S, [I, I, I, P]),
            "moe_image_build": (I, [I, I, I, P, P, P, S, P]),
            "moe_image_validate": (I, [LP, P, P]),
            "moe_image_unpack": (I, [LP, I, I, P, P]),
            "moe_workspace_bytes": (S, [LP, I, I]),
            "moe_route_topk": (I, [LP, P, I, I, P, P, P, S, P]),
            "moe_layer_forward": (I, [LP, P, I, I, P, P, S, P]),
            "moe_layer_forward_timed": (I, [LP, P, I, I, P, P, S, P, P]),
            "moe_layer_forward_noalloc": (I, [LP, P, I, I, P, P]),
            "moe_noalloc_scratch_bytes": (S, []),
            "moe_prefill_forward": (I, [LP, P, I, I, P, P, S, P]),
            "moe_prefill_forward_timed": (I, [LP, P, I, I, P, P, S, P, P]),
            "rfpx_dense_image_bytes": (S, [I, I, I]),
            "rfpx_dense_image_build": (I, [I, P, I, I, P, S, P]),
            "rfpx_dense_image_unpack": (I, [I, P, I, I, P, P]),
            "rfpx_dense_workspace_bytes": (S, [I, I, I, I]),
            "rfpx_dense_forward": (I, [I, P, I, I, P, I, I, P, P, S, P]),
            "rfpx_stream_read": (I, [P, S, P, P]),
            "rfpx_stream_read_sink_words": (S, []),
            "rfpx_status_str": (C.c_char_p, [I]),
            "rfpx_last_error": (C.c_char_p, []),
        }
        for name, (res, args) in sig.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
        return l


def _check(fn: str, st: int) -> None:
    if st != 0:
        l = lib()
        raise RfpxError(fn, st, (l.rfpx_last_error() or b"").decode())


def _stream(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _ptr(t) -> C.c_void_p:
    return C.c_void_p(t.data_ptr())


def _need_cuda(*ts):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensor must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensor must be contiguous")


# ------------------------------------------------------------------- codec

def rfpx_block_bytes(fmt: int) -> int:
    return lib().rfpx_block_bytes(fmt)


def rfpx_matrix_bytes(fmt: int, rows: int, cols: int) -> int:
    return lib().rfpx_matrix_bytes(fmt, rows, cols)


def rfpx_pack(fmt: int, w, out=None, stream=None):
    """Quantize w (cuda fp32 [rows][cols]) into canonical blocks (uint8)."""
    import torch
    _need_cuda(w)
    rows, cols = w.shape
    n = rfpx_matrix_bytes(fmt, rows, cols)
    if out is None:
        out = torch.empty(n, dtype=torch.uint8, device=w.device)
    _check("rfpx_pack", lib().rfpx_pack(fmt, _ptr(w), rows, cols, _ptr(out),
                                        out.numel(), _stream(stream)))
    return out


def rfpx_pack_weighted(fmt: int, w, imp, out=None, stream=None):
    """Importance-weighted quantizer: w cuda fp32 [rows][cols], imp cuda
    fp32 [cols] (>= 0)."""
    import torch
    _need_cuda(w, imp)
    rows, cols = w.shape
    if imp.numel() != cols:
        raise ValueError("imp must hold one importance per column")
    n = rfpx_matrix_bytes(fmt, rows, cols)
    if out is None:
        out = torch.empty(n, dtype=torch.uint8, device=w.device)
    _check("rfpx_pack_weighted", lib().rfpx_pack_weighted(
        fmt, _ptr(w), _ptr(imp), rows, cols, _ptr(out), out.numel(), _stream(stream)))
    return out


def rfpx_pack_codes(fmt: int, codes, scale_bits, out=None, stream=None):
    """codes: cuda uint8 [rows][cols]; scale_bits: cuda int16/uint16 bits
    [rows][cols/32]."""
    import torch
    _need_cuda(codes, scale_bits)
    rows, cols = codes.shape
    n = rfpx_matrix_bytes(fmt, rows, cols)
    if out is None:
        out = torch.empty(n, dtype=torch.uint8, device=codes.device)
    _check("rfpx_pack_codes", lib().rfpx_pack_codes(
        fmt, _ptr(codes), _ptr(scale_bits), rows, cols, _ptr(out), out.numel(),
        _stream(stream)))
    return out


def rfpx_unpack(fmt: int, data, rows: int, cols: int, out=None, stream=None):
    import torch
    _need_cuda(data)
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.float32, device=data.device)
    _check("rfpx_unpack", lib().rfpx_unpack(fmt, _ptr(data), rows, cols, _ptr(out),
                                            _stream(stream)))
    return out


# ------------------------------------------------------------------- image

def _fmts_array(fmts) -> C.Array:
    flat = [int(v) for row in fmts for v in (row if hasattr(row, "__len__") else [row])]
    return (C.c_int * len(flat))(*flat)


def moe_image_bytes(d: int, f: int, n_experts: int, fmts) -> int:
    return lib().moe_image_bytes(d, f, n_experts, C.cast(_fmts_array(fmts), C.c_void_p))


def moe_image_build(d: int, f: int, n_experts: int, fmts,
                    canonical: Sequence, out=None, stream=None):
    """canonical: (E+1)*3 cuda uint8 tensors (gate, up, down per expert, the
    shared expert last).  Returns the image (cuda uint8, 256-B aligned)."""
    import torch
    fa = _fmts_array(fmts)
    n = lib().moe_image_bytes(d, f, n_experts, C.cast(fa, C.c_void_p))
    if n == 0:
        raise RfpxError("moe_image_bytes", -2, "unsupported shape or format table")
    for t in canonical:
        _need_cuda(t)
    ptrs = (C.c_void_p * len(canonical))(*[t.data_ptr() for t in canonical])
    if out is None:
        out = torch.empty(n, dtype=torch.uint8, device=canonical[0].device)
    _check("moe_image_build", lib().moe_image_build(
        d, f, n_experts, C.cast(fa, C.c_void_p), C.cast(ptrs, C.c_void_p), _ptr(out),
        out.numel(), _stream(stream)))
    return out


class MoeLayer:
    """A layer descriptor (moe_layer) plus references that keep its device
    buffers and format table alive.  image_bytes defaults to the size of
    the image tensor."""

    def __init__(self, d: int, f: int, n_experts: int, top_k: int, router_w,
                 image, fmts, routed_scale: float = 1.0,
                 image_bytes: Optional[int] = None):
        _need_cuda(router_w, image)
        self._fmts = _fmts_array(fmts)
        self._router_w = router_w
        self._image = image
        if image_bytes is None:
            image_bytes = image.numel()
        self.c = MoeLayerC(d, f, n_experts, top_k, routed_scale,
                           router_w.data_ptr(), image.data_ptr(),
                           C.cast(self._fmts, C.POINTER(C.c_int)), image_bytes)
        self.d, self.f, self.n_experts, self.top_k = d, f, n_experts, top_k

    @property
    def ref(self):
        return C.byref(self.c)


def moe_image_validate(layer: MoeLayer, report=None, stream=None):
    """Enqueue the device check of the layer's image; returns the report
    tensor (cuda int32 [4], read as uint32: header faults, mismatching table
    entries, blocks with a non-finite scale, 0), valid once the stream
    passes."""
    import torch
    if report is None:
        report = torch.empty(4, dtype=torch.int32, device=layer._image.device)
    _need_cuda(report)
    _check("moe_image_validate", lib().moe_image_validate(layer.ref, _ptr(report),
                                                          _stream(stream)))
    return report


def check_image(layer: MoeLayer, stream=None) -> None:
    """moe_image_validate, waited for: raises RfpxError if the image fails."""
    import torch
    rep = moe_image_validate(layer, stream=stream)
    (stream or torch.cuda.current_stream()).synchronize()
    r = [int(v) & 0xFFFFFFFF for v in rep.cpu().tolist()]
    if any(r):
        raise RfpxError("moe_image_validate", -4,
                        f"header faults 0x{r[0]:x}, {r[1]} table entries differ from the "
                        f"format table, {r[2]} blocks with a non-finite scale")


def moe_image_unpack(layer: MoeLayer, expert: int, matrix: int, out=None,
                     stream=None):
    import torch
    rows, cols = (layer.f, layer.d) if matrix < 2 else (layer.d, layer.f)
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.float32, device=layer._image.device)
    _check("moe_image_unpack", lib().moe_image_unpack(layer.ref, expert, matrix,
                                                      _ptr(out), _stream(stream)))
    return out


# ---------------------------------------------------------------- forward

def moe_workspace_bytes(layer: MoeLayer, q_or_T: int, prefill: bool = False) -> int:
    return lib().moe_workspace_bytes(layer.ref, q_or_T, 1 if prefill else 0)


def workspace(layer: MoeLayer, q_or_T: int, prefill: bool = False):
    """A workspace of the right size (uninitialized: the library needs no
    particular contents)."""
    import torch
    n = moe_workspace_bytes(layer, q_or_T, prefill)
    if n == 0:
        raise RfpxError("moe_workspace_bytes", -2, "unsupported shape")
    return torch.empty(n, dtype=torch.uint8, device=layer._image.device)


def _xtype(x) -> int:
    import torch
    if x.dtype == torch.bfloat16:
        return RFPX_X_BF16
    if x.dtype == torch.float32:
        return RFPX_X_F32
    raise ValueError("x must be bfloat16 or float32")


def moe_route_topk(layer: MoeLayer, x, ids=None, w=None, ws=None, stream=None):
    import torch
    _need_cuda(x)
    q = x.shape[0]
    if ids is None:
        ids = torch.empty((q, layer.top_k), dtype=torch.int32, device=x.device)
    if w is None:
        w = torch.empty((q, layer.top_k), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = workspace(layer, q)
    _check("moe_route_topk", lib().moe_route_topk(
        layer.ref, _ptr(x), _xtype(x), q, _ptr(ids), _ptr(w), _ptr(ws), ws.numel(),
        _stream(stream)))
    return ids, w


def moe_layer_forward(layer: MoeLayer, x, y=None, ws=None, stream=None):
    import torch
    _need_cuda(x)
    q = x.shape[0]
    if y is None:
        y = torch.empty((q, layer.d), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = workspace(layer, q)
    _check("moe_layer_forward", lib().moe_layer_forward(
        layer.ref, _ptr(x), _xtype(x), q, _ptr(y), _ptr(ws), ws.numel(),
        _stream(stream)))
    return y


def moe_layer_forward_timed(layer: MoeLayer, x, y, ws, events, stream=None):
    """events: a ctypes array of 6 hipEvent_t handles (created by the
    caller on this device), stamped with the start and end of the routing
    kernels, the gate/up kernel and the down kernel."""
    _need_cuda(x)
    if events is not None and len(events) != 6:
        raise ValueError("moe_layer_forward_timed takes 6 events")
    _check("moe_layer_forward_timed", lib().moe_layer_forward_timed(
        layer.ref, _ptr(x), _xtype(x), x.shape[0], _ptr(y), _ptr(ws), ws.numel(),
        _stream(stream), C.cast(events, C.c_void_p) if events is not None else None))
    return y


def moe_layer_forward_noalloc(layer: MoeLayer, x, y, stream=None):
    """moe_layer_forward on the library's own device scratch: y (cuda fp32
    [q][d]) is given by the caller, nothing is allocated."""
    _need_cuda(x, y)
    _check("moe_layer_forward_noalloc", lib().moe_layer_forward_noalloc(
        layer.ref, _ptr(x), _xtype(x), x.shape[0], _ptr(y), _stream(stream)))
    return y


def moe_prefill_forward(layer: MoeLayer, x, y=None, ws=None, stream=None):
    import torch
    _need_cuda(x)
    T = x.shape[0]
    if y is None:
        y = torch.empty((T, layer.d), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = workspace(layer, T, prefill=True)
    _check("moe_prefill_forward", lib().moe_prefill_forward(
        layer.ref, _ptr(x), _xtype(x), T, _ptr(y), _ptr(ws), ws.numel(),
        _stream(stream)))
    return y


def moe_prefill_forward_timed(layer: MoeLayer, x, y, ws, events, stream=None):
    """events: a ctypes array of 6 hipEvent_t handles (created by the
    caller on this device), stamped with the start of the router scores, the
    end of the expert grouping, the start and end of the grouped gate/up
    product, the start of the grouped down product and the end of the
    combine."""
    _need_cuda(x)
    if events is not None and len(events) != 6:
        raise ValueError("moe_prefill_forward_timed takes 6 events")
    _check("moe_prefill_forward_timed", lib().moe_prefill_forward_timed(
        layer.ref, _ptr(x), _xtype(x), x.shape[0], _ptr(y), _ptr(ws), ws.numel(),
        _stream(stream), C.cast(events, C.c_void_p) if events is not None else None))
    return y


# ------------------------------------------------------ dense projections

class DenseMatrix:
    """A dense block-quantized matrix in its device image (rows x cols,
    format fmt), built from canonical blocks by rfpx_dense_image_build."""

    def __init__(self, fmt: int, rows: int, cols: int, canonical, stream=None):
        import torch
        _need_cuda(canonical)
        n = lib().rfpx_dense_image_bytes(fmt, rows, cols)
        if n == 0:
            raise RfpxError("rfpx_dense_image_bytes", -2, f"unsupported {rows} x {cols}")
        self.image = torch.empty(n, dtype=torch.uint8, device=canonical.device)
        _check("rfpx_dense_image_build", lib().rfpx_dense_image_build(
            fmt, _ptr(canonical), rows, cols, _ptr(self.image), n, _stream(stream)))
        self.fmt, self.rows, self.cols = fmt, rows, cols

    def unpack(self, out=None, stream=None):
        import torch
        if out is None:
            out = torch.empty((self.rows, self.cols), dtype=torch.float32,
                              device=self.image.device)
        _check("rfpx_dense_image_unpack", lib().rfpx_dense_image_unpack(
            self.fmt, _ptr(self.image), self.rows, self.cols, _ptr(out), _stream(stream)))
        return out

    def workspace(self, q: int):
        import torch
        n = lib().rfpx_dense_workspace_bytes(self.fmt, self.rows, self.cols, q)
        if n == 0:
            raise RfpxError("rfpx_dense_workspace_bytes", -2, "unsupported shape")
        return torch.empty(n, dtype=torch.uint8, device=self.image.device)


def rfpx_dense_forward(m: DenseMatrix, x, y=None, ws=None, stream=None):
    """y[q][rows] = W x_c for the q columns of x (cuda bf16 or fp32
    [q][cols])."""
    import torch
    _need_cuda(x)
    q = x.shape[0]
    if y is None:
        y = torch.empty((q, m.rows), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = m.workspace(q)
    _check("rfpx_dense_forward", lib().rfpx_dense_forward(
        m.fmt, _ptr(m.image), m.rows, m.cols, _ptr(x), _xtype(x), q, _ptr(y), _ptr(ws),
        ws.numel(), _stream(stream)))
    return y


# ------------------------------------------------------------ measurement

def rfpx_stream_read(buf, sink=None, stream=None):
    """A plain streaming read of the cuda tensor buf (its bytes); returns the
    sink tensor (int32 [rfpx_stream_read_sink_words()]), whose words XOR to
    the XOR of buf's 32-bit words (words past the workgroup count are left
    as they were: pass a zeroed sink to check)."""
    import torch
    _need_cuda(buf)
    n = lib().rfpx_stream_read_sink_words()
    if sink is None:
        sink = torch.zeros(n, dtype=torch.int32, device=buf.device)
    _check("rfpx_stream_read", lib().rfpx_stream_read(
        _ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), _stream(stream)))
    return sink


# ----------------------------------------------------------- convenience

def upload_layer(lay, device="cuda", stream=None, validate: bool = True) -> MoeLayer:
    """Build the device image of a synthetic layer (an object with d, f, E,
    k, wr, fmts, blob, offsets, mat(e, m)): one host-to-device copy of all
    canonical bytes, then moe_image_build on the GPU, then (by default)
    moe_image_validate, raising if the image fails it."""
    import numpy as np
    import torch
    blob = torch.from_numpy(np.ascontiguousarray(lay.blob)).to(device)
    canon = []
    for e in range(lay.E + 1):
        for m in range(3):
            i = 3 * e + m
            n = lay.mat(e, m).size
            canon.append(blob[int(lay.offsets[i]):int(lay.offsets[i]) + n])
    image = moe_image_build(lay.d, lay.f, lay.E, lay.fmts, canon, stream=stream)
    wr = torch.from_numpy(np.ascontiguousarray(lay.wr)).to(device)
    L = MoeLayer(lay.d, lay.f, lay.E, lay.k, wr, image, lay.fmts,
                 getattr(lay, "routed_scale", 1.0))
    if validate:
        check_image(L)  # waits for the stream, so the canonical bytes may go
    else:
        torch.cuda.current_stream().synchronize()
    del blob, canon
    return L
