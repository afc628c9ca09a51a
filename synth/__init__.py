"""Seeded synthetic inputs for one routed-MoE layer over block-quantized experts.

This module serves both the GPU library and the CPU oracle, and holds none of
the layer's arithmetic: no block decode, no expert product, no top-k, no
softmax, no combine.  It draws

* canonical ROCmFP2 / FP3 / FP4 blocks: every code bit pattern is uniform
  (uniform codes are uniform bytes), scales are |N(0, 0.05)| (+ a floor where
  the workload asks for one) rounded to fp16, or, for FP4, the nearest E8M0
  power of two;
* router weights N(0, 0.02) in fp32 and activations N(0, 1) stored as bf16
  (or fp32 for the tiny workload);
* for the speculative-verify and prefill workloads, each column's six experts
  from a Zipf(1.1) law over the 256 experts, in draw order, and then moves the
  activation (a least-squares step through the router's row space) so that the
  router, run on the stored activation, ranks exactly those experts first.

Columns are redrawn until the six (or two) chosen scores and the next one are
separated by at least ``GAP`` after the activation is rounded to its stored
type, so that no fp32 summation order can change the selection.  The check
uses numpy float64 products; the expected routing in the tests comes from the
oracle, not from here.

Workloads (d = model width, f = expert width, E routed experts, k chosen):

=====  =================================================================
1      d=256 f=128 E=8 k=2 + shared; 4 columns run as q=1; x fp32;
       gate/up FP2, down FP3, shared FP4; scales |N(0,.05)|+1e-3
2      d=4096 f=2048 E=256 k=6 + shared; q=1; x bf16; natural routing
3      as 2, q=4, Zipf(1.1) routing per column
4      as 2, q=5, Zipf(1.1); the 32 hottest experts (by Zipf rank) FP4
       for gate, up and down; 43 layers with their own seeds
5      as 2, a 2048-token prefill chunk, Zipf(1.1) per token
=====  =================================================================
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os
from typing import List, Optional

import numpy as np

FP2, FP3, FP4 = 2, 3, 4
BLOCK_BYTES = {FP2: 10, FP3: 14, FP4: 17}
GAP = 1e-3  # minimum score gap between consecutive ranks 1..k+1
ZIPF_S = 1.1

# stream ids for the seed sequences
_S_ROUTER, _S_MATRIX, _S_PERM, _S_X, _S_ZIPF = 0, 1, 2, 3, 4


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    d: int
    f: int
    E: int
    k: int
    q: int                 # verify columns per call (prefill: tokens per call)
    xtype: str             # "f32" or "bf16"
    routing: str           # "natural" or "zipf"
    scale_sigma: float = 0.05
    scale_floor: float = 0.0
    hot_fp4: int = 0       # experts of Zipf rank < hot_fp4 stored as FP4
    layers: int = 1
    prefill: bool = False
    master: int = 0


TINY = "tiny-d256-e8-top2"
DECODE_Q1 = "decode-q1-d4096-e256-top6"
VERIFY_Q4 = "verify-q4-zipf"
VERIFY_Q5 = "verify-q5-zipf-hot32fp4-43layers"
PREFILL = "prefill-t2048-zipf"

WORKLOADS = {
    TINY: Config(TINY, 256, 128, 8, 2, 1, "f32", "natural", scale_floor=1e-3, master=1),
    DECODE_Q1: Config(DECODE_Q1, 4096, 2048, 256, 6, 1, "bf16", "natural", master=2),
    VERIFY_Q4: Config(VERIFY_Q4, 4096, 2048, 256, 6, 4, "bf16", "zipf", master=3),
    VERIFY_Q5: Config(VERIFY_Q5, 4096, 2048, 256, 6, 5, "bf16", "zipf", hot_fp4=32,
                      layers=43, master=4),
    PREFILL: Config(PREFILL, 4096, 2048, 256, 6, 2048, "bf16", "zipf", prefill=True,
                    master=5),
}


# Layer instances a timed run rotates over (so that no weight is re-read
# from the 256 MB last-level cache within a rotation; each layer image is
# about 2.3 GB), and activation batches drawn per instance (variant 0..3).
# The benchmark times these instances and the parity tests check every one.
ROTATION = {DECODE_Q1: 8, VERIFY_Q4: 8, VERIFY_Q5: 43, PREFILL: 2}
ACTIVATION_BATCHES = 4


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


# ----------------------------------------------------------------- blocks

def matrix_bytes(fmt: int, rows: int, cols: int) -> int:
    return rows * (cols // 32) * BLOCK_BYTES[fmt]


def fill_matrix(out: np.ndarray, rng: np.random.Generator, fmt: int, rows: int,
                cols: int, sigma: float, floor: float) -> None:
    """Write rows*cols/32 canonical blocks into the uint8 view ``out``."""
    nb = rows * (cols // 32)
    bb = BLOCK_BYTES[fmt]
    blocks = out.reshape(nb, bb)
    blocks[:] = rng.integers(0, 256, size=(nb, bb), dtype=np.uint8)
    s = np.abs(rng.standard_normal(nb)) * sigma + floor
    if fmt == FP4:
        with np.errstate(divide="ignore"):
            e = np.clip(127 + np.rint(np.log2(s)), 1, 254)
        blocks[:, 16] = e.astype(np.uint8)
    else:
        h = s.astype(np.float16)  # round to nearest even
        blocks[:, bb - 2:] = h.view(np.uint8).reshape(nb, 2)


def random_matrix(seed: int, fmt: int, rows: int, cols: int,
                  sigma: float = 0.05, floor: float = 0.0) -> np.ndarray:
    out = np.empty(matrix_bytes(fmt, rows, cols), np.uint8)
    fill_matrix(out, _rng(seed, fmt, rows, cols), fmt, rows, cols, sigma, floor)
    return out


# ------------------------------------------------------------------ layer

@dataclasses.dataclass
class Layer:
    d: int
    f: int
    E: int
    k: int
    wr: np.ndarray          # [E][d] float32
    fmts: np.ndarray        # [(E+1)][3] int32; row E is the shared expert
    blob: np.ndarray        # every matrix's canonical bytes, back to back
    offsets: np.ndarray     # [(E+1)*3] int64 byte offsets into blob
    perm: np.ndarray        # Zipf rank -> expert id
    routed_scale: float = 1.0

    def mat(self, e: int, m: int) -> np.ndarray:
        i = 3 * e + m
        fmt = int(self.fmts[e][m])
        rows, cols = (self.f, self.d) if m < 2 else (self.d, self.f)
        n = matrix_bytes(fmt, rows, cols)
        return self.blob[self.offsets[i]:self.offsets[i] + n]

    def matrix_shape(self, m: int):
        return (self.f, self.d) if m < 2 else (self.d, self.f)


def expert_formats(E: int, perm: np.ndarray, hot_fp4: int) -> np.ndarray:
    """Routed gate/up FP2 and down FP3; the hottest ``hot_fp4`` experts and
    the shared expert FP4 for all three matrices."""
    fmts = np.empty((E + 1, 3), np.int32)
    fmts[:, 0:2] = FP2
    fmts[:, 2] = FP3
    for r in range(min(hot_fp4, E)):
        fmts[perm[r], :] = FP4
    fmts[E, :] = FP4
    return fmts


def gen_router(cfg: Config, layer: int = 0, *, d: Optional[int] = None,
               E: Optional[int] = None, master: Optional[int] = None):
    """Router weights [E][d] fp32 ~ N(0, 0.02) and the Zipf rank -> expert
    permutation of one layer."""
    d = cfg.d if d is None else d
    E = cfg.E if E is None else E
    master = cfg.master if master is None else master
    wr = (_rng(master, layer, _S_ROUTER).standard_normal((E, d)) * 0.02
          ).astype(np.float32)
    perm = _rng(master, layer, _S_PERM).permutation(E).astype(np.int64)
    return wr, perm


def gen_layer(cfg: Config, layer: int = 0, *, d: Optional[int] = None,
              f: Optional[int] = None, E: Optional[int] = None,
              k: Optional[int] = None, master: Optional[int] = None,
              threads: Optional[int] = None) -> Layer:
    d = cfg.d if d is None else d
    f = cfg.f if f is None else f
    E = cfg.E if E is None else E
    k = cfg.k if k is None else k
    master = cfg.master if master is None else master
    wr, perm = gen_router(cfg, layer, d=d, E=E, master=master)
    fmts = expert_formats(E, perm, cfg.hot_fp4)
    sizes = []
    for e in range(E + 1):
        for m in range(3):
            rows, cols = (f, d) if m < 2 else (d, f)
            sizes.append(matrix_bytes(int(fmts[e][m]), rows, cols))
    offsets = np.zeros(len(sizes), np.int64)
    offsets[1:] = np.cumsum(sizes)[:-1]
    blob = np.empty(int(sum(sizes)), np.uint8)

    def job(i: int) -> None:
        e, m = divmod(i, 3)
        rows, cols = (f, d) if m < 2 else (d, f)
        fill_matrix(blob[offsets[i]:offsets[i] + sizes[i]],
                    _rng(master, layer, _S_MATRIX, e, m), int(fmts[e][m]),
                    rows, cols, cfg.scale_sigma, cfg.scale_floor)

    n = len(sizes)
    with _cf.ThreadPoolExecutor(threads or _threads()) as ex:
        list(ex.map(job, range(n)))
    return Layer(d, f, E, k, wr, fmts, blob, offsets, perm)


# ------------------------------------------------------------ activations

def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float -> bf16 bit patterns (via fp32, round to nearest even)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def zipf_draws(rng: np.random.Generator, E: int, k: int, n: int,
               perm: np.ndarray, s: float = ZIPF_S) -> np.ndarray:
    """n sets of k experts drawn without replacement from p_r ~ r^-s over
    ranks r = 1..E, each draw in proportion to the remaining mass; rank r is
    expert perm[r-1].  Returned in draw order."""
    p = np.arange(1, E + 1, dtype=np.float64) ** (-s)
    out = np.empty((n, k), np.int64)
    for c in range(n):
        alive = np.ones(E, bool)
        for j in range(k):
            w = np.where(alive, p, 0.0)
            cdf = np.cumsum(w)
            r = int(np.searchsorted(cdf, rng.random() * cdf[-1], side="right"))
            r = min(r, E - 1)
            while not alive[r]:  # guard against a zero-width step at the top
                r -= 1
            alive[r] = False
            out[c, j] = perm[r]
    return out


@dataclasses.dataclass
class Columns:
    x: np.ndarray             # [n][d] uint16 bf16 bits, or float32
    xtype: str
    drawn: Optional[np.ndarray]  # [n][k] prescribed experts in rank order
    redraws: int

    def x_f64(self) -> np.ndarray:
        if self.xtype == "bf16":
            return bf16_bits_to_f64(self.x)
        return self.x.astype(np.float64)


def _store(x: np.ndarray, xtype: str):
    if xtype == "bf16":
        bits = to_bf16_bits(x)
        return bits, bf16_bits_to_f64(bits)
    x32 = x.astype(np.float32)
    return x32, x32.astype(np.float64)


def gen_columns(cfg: Config, lay, n: int, variant: int = 0,
                layer: int = 0, master: Optional[int] = None) -> Columns:
    """n activation columns for ``lay`` (a Layer, or a (wr, perm, k) tuple);
    Zipf-steered when cfg.routing says so.  Failing columns are redrawn from
    the same continuing stream until every column passes."""
    master = cfg.master if master is None else master
    if isinstance(lay, Layer):
        wr, perm, k = lay.wr, lay.perm, lay.k
    else:
        wr, perm, k = lay
    E, d = wr.shape
    W = wr.astype(np.float64)
    rng_x = _rng(master, layer, _S_X, variant)
    drawn = None
    if cfg.routing == "zipf":
        drawn = zipf_draws(_rng(master, layer, _S_ZIPF, variant), E, k, n,
                           perm)
        G = W @ W.T
        Ginv = np.linalg.inv(G)
    xs = np.empty((n, d), np.uint16 if cfg.xtype == "bf16" else np.float32)
    todo = np.arange(n)
    redraws = -n
    while todo.size:
        redraws += todo.size
        x0 = rng_x.standard_normal((todo.size, d))
        x = x0
        if drawn is not None:
            s0 = x0 @ W.T
            ds = np.zeros_like(s0)
            for i, c in enumerate(todo):
                row = s0[i]
                top = np.argsort(-row, kind="stable")[:k]
                target = row.copy()
                for j in range(k):
                    holder = int(np.flatnonzero(target == row[top[j]])[0])
                    e = int(drawn[c, j])
                    target[holder], target[e] = target[e], target[holder]
                ds[i] = target - row
            x = x0 + (ds @ Ginv) @ W
        stored, xv = _store(x, cfg.xtype)
        s = xv @ W.T
        ok = np.ones(todo.size, bool)
        for i, c in enumerate(todo):
            order = np.argsort(-s[i], kind="stable")[:k + 1]
            gaps = s[i][order[:-1]] - s[i][order[1:]]
            good = bool(np.all(gaps >= GAP))
            if drawn is not None:
                good = good and bool(np.array_equal(order[:k], drawn[c]))
            ok[i] = good
        xs[todo[ok]] = stored[ok]
        todo = todo[~ok]
    return Columns(xs, cfg.xtype, drawn, max(redraws, 0))
