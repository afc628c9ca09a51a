"""Pins for the CPU oracle: it is checked against things other than itself.

* the pages' block sizes and bits per weight (page 'DeepSeek V4 Flash 在
  128GB 锐龙 AI MAX+ 上跑到 32 tok/s', section 'ROCmFPX：把 284B 权重压进
  128 GB');
* hand-worked blocks in tests/golden/blocks.json;
* numpy's IEEE half conversions as the textbook routine for fp16;
* brute force on tiny inputs: an independent big-integer bit reader, dense
  numpy products, exhaustive ranking and exhaustive code search;
* closed forms for structured layers, and invariants (column independence,
  relabelling, linearity, the shared-expert-only special case).
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "blocks.json")
OFFSET = {2: 1.5, 3: 3.5, 4: 7.5}
NBITS = {2: 2, 3: 3, 4: 4}


# ------------------------------------------------------ independent readers

def bigint_codes(fmt, blk: bytes):
    """Codes and scale of one block through Python big integers, a reader
    that has nothing in common with the oracle's bit-at-a-time loop."""
    nb = NBITS[fmt]
    v = int.from_bytes(blk[: 4 * nb], "little")
    codes = [(v >> (nb * j)) & ((1 << nb) - 1) for j in range(32)]
    if fmt == 4:
        scale = 2.0 ** (blk[16] - 127)
    else:
        scale = float(np.frombuffer(blk[4 * nb:4 * nb + 2], "<f2")[0])
    return codes, scale


def dense(fmt, data: np.ndarray, rows, cols):
    bb = synth.BLOCK_BYTES[fmt]
    out = np.empty((rows, cols))
    raw = data.tobytes()
    for r in range(rows):
        for b in range(cols // 32):
            i = (r * (cols // 32) + b) * bb
            codes, s = bigint_codes(fmt, raw[i:i + bb])
            out[r, 32 * b:32 * b + 32] = (np.array(codes) - OFFSET[fmt]) * s
    return out


def silu(g):
    return g / (1.0 + np.exp(-g))


# ------------------------------------------------------------ page numbers

def test_block_bytes_match_pages():
    # 10 bytes per 32 weights is 2.50 bit/weight; FP3 3.50; FP4 4.25
    assert [oracle.block_bytes(f) for f in (2, 3, 4)] == [10, 14, 17]
    assert [8 * oracle.block_bytes(f) / 32 for f in (2, 3, 4)] == [2.5, 3.5, 4.25]
    assert oracle.block_bytes(5) == 0


# --------------------------------------------------------- worked examples

def _cases():
    with open(GOLDEN) as fh:
        return json.load(fh)["cases"]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"])
def test_golden_block(case):
    blk = bytes.fromhex(case["hex"])
    assert len(blk) == oracle.block_bytes(case["fmt"])
    codes, s = oracle.block_codes(case["fmt"], blk)
    assert list(codes) == case["codes"]
    assert s == case["scale"]
    w = oracle.decode_block(case["fmt"], blk)
    assert list(w) == case["values"]
    # the oracle's packer reproduces the hand-made bytes from codes + scale
    cb = np.array(case["codes"], np.uint8).reshape(1, 32)
    sb = np.array([blk[16] if case["fmt"] == 4 else blk[-2] | blk[-1] << 8],
                  np.uint16)
    assert oracle.pack_codes(case["fmt"], cb, sb).tobytes() == blk


# -------------------------------------------------------------- half / bf16

def test_half_to_double_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.half_to_double(int(b)) for b in bits])
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite], ref[finite])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[np.isinf(ref)], ref[np.isinf(ref)])


def test_double_to_half_matches_numpy_rne():
    rng = np.random.default_rng(7)
    v = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 6, 20000),
        # exact ties: halfway between adjacent halves, normal and subnormal
        (np.arange(1, 2000, dtype=np.float64) + 0.5) * 2.0 ** -24,
        (np.arange(2048, 4096, dtype=np.float64) + 0.5) * 2.0 ** -10,
        [65504.0, 65519.99, 65520.0, 1e9, 0.0, -0.0, 2.0 ** -25, 2.0 ** -26],
    ])
    with np.errstate(over="ignore"):
        ref = v.astype(np.float16).view(np.uint16)
    got = np.array([oracle.double_to_half_rne(float(x)) for x in v], np.uint16)
    assert np.array_equal(got, ref)


def test_bf16_reader():
    rng = np.random.default_rng(3)
    f = rng.standard_normal(1000).astype(np.float32)
    bits = (f.view(np.uint32) >> 16).astype(np.uint16)
    ref = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    got = np.array([oracle.bf16_to_double(int(b)) for b in bits])
    assert np.array_equal(got, ref)


# ------------------------------------------------------------ block decode

@pytest.mark.parametrize("fmt", [2, 3, 4])
def test_unpack_matches_bigint_reader(fmt):
    data = synth.random_matrix(11 + fmt, fmt, 6, 128)
    w = oracle.unpack(fmt, data, 6, 128)
    assert np.array_equal(w, dense(fmt, data, 6, 128))
    # every dequantized weight is exact in fp32 (at most 15 significant bits)
    assert np.array_equal(w.astype(np.float32).astype(np.float64), w)


@pytest.mark.parametrize("fmt", [2, 3, 4])
def test_pack_codes_roundtrip_random(fmt):
    rng = np.random.default_rng(fmt)
    codes = rng.integers(0, 2 ** NBITS[fmt], size=(3, 96)).astype(np.uint8)
    if fmt == 4:
        sb = rng.integers(0, 255, size=9).astype(np.uint16)
    else:
        sb = rng.integers(0, 0x7C00, size=9).astype(np.uint16)
    data = oracle.pack_codes(fmt, codes, sb)
    bb = synth.BLOCK_BYTES[fmt]
    raw = data.tobytes()
    for i in range(9):
        c, s = bigint_codes(fmt, raw[i * bb:(i + 1) * bb])
        assert c == list(codes.reshape(9, 32)[i])
        if fmt == 4:
            assert s == 2.0 ** (int(sb[i]) - 127)
        else:
            assert s == float(np.uint16(sb[i]).view(np.float16))


# ------------------------------------------------------------------ packing

def _brute_codes(fmt, w, s):
    """Exhaustive nearest code for each weight (ties to the even code)."""
    vals = (np.arange(2 ** NBITS[fmt]) - OFFSET[fmt]) * s
    out = []
    for x in w:
        err = np.abs(vals - float(x))
        best = np.flatnonzero(err == err.min())
        out.append(int(best[0]) if len(best) == 1 else int(best[best % 2 == 0][0]))
    return out


@pytest.mark.parametrize("fmt", [2, 3, 4])
def test_pack_scale_and_codes_brute_force(fmt):
    rng = np.random.default_rng(100 + fmt)
    w = (rng.standard_normal((4, 256)) * rng.choice([1e-3, 0.05, 3.0, 700.0],
                                                     (4, 1))).astype(np.float32)
    data = oracle.pack(fmt, w)
    bb = synth.BLOCK_BYTES[fmt]
    raw = data.tobytes()
    for i in range(w.size // 32):
        blk = w.reshape(-1, 32)[i].astype(np.float64)
        codes, s = bigint_codes(fmt, raw[i * bb:(i + 1) * bb])
        a = np.abs(blk).max()
        if fmt == 4:
            # smallest power of two with 7.5 * 2^k >= a
            k = math.ceil(math.log2(a / 7.5))
            if 7.5 * 2.0 ** (k - 1) >= a:
                k -= 1
            assert s == 2.0 ** k
        else:
            # s is the fp16 nearest to a / offset: no neighbour is closer
            target = a / OFFSET[fmt]
            h = np.float16(s).view(np.uint16)
            for nb_ in (h - 1, h + 1):
                other = float(np.uint16(nb_).view(np.float16))
                assert abs(s - target) <= abs(other - target)
        assert codes == _brute_codes(fmt, blk, s)
        # every reconstructed weight is within half a step
        rec = (np.array(codes) - OFFSET[fmt]) * s
        assert np.all(np.abs(rec - blk) <= s / 2 + 1e-300)


@pytest.mark.parametrize("fmt", [2, 3, 4])
def test_pack_of_unpack_is_identity_with_extreme_code(fmt):
    rng = np.random.default_rng(fmt + 40)
    codes = rng.integers(0, 2 ** NBITS[fmt], size=(8, 64)).astype(np.uint8)
    codes[:, ::32] = np.where(np.arange(8)[:, None] % 2 == 0, 0,
                              2 ** NBITS[fmt] - 1)
    if fmt == 4:
        sb = rng.integers(100, 150, size=16).astype(np.uint16)
    else:
        sb = np.abs(rng.standard_normal(16) * 0.05).astype(np.float16).view(np.uint16)
        sb = sb | np.uint16(0x0400)  # keep them normal and nonzero
    data = oracle.pack_codes(fmt, codes, sb)
    w = oracle.unpack(fmt, data, 8, 64).astype(np.float32)
    assert np.array_equal(oracle.pack(fmt, w), data)


def test_pack_zero_and_vanishing_blocks():
    z = np.zeros((1, 32), np.float32)
    for fmt in (2, 3, 4):
        assert not oracle.pack(fmt, z).any()
    tiny = np.full((1, 32), 1e-9, np.float32)  # a/1.5 rounds to fp16 zero
    assert not oracle.pack(2, tiny).any()
    huge = np.full((1, 32), 3e5, np.float32)  # a/1.5 overflows fp16
    data = oracle.pack(2, huge)
    assert int(data[8]) | int(data[9]) << 8 == 0x7BFF
    assert np.all(oracle.unpack(2, data, 1, 32) == 1.5 * 65504.0)


# ------------------------------------------------------------------ routing

def test_router_scores_match_numpy():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((3, 64))
    wr = rng.standard_normal((10, 64)).astype(np.float32)
    s = oracle.router_scores(x, wr)
    assert np.allclose(s, x @ wr.astype(np.float64).T, rtol=1e-13, atol=1e-13)


def test_topk_hand_example():
    s = np.array([0.1, 0.9, -0.3, 0.9, 0.5, 0.0, 2.0, -1.0])
    # ranks: 6 (2.0), then the tie 1/3 (0.9, lower index first), then 4
    assert list(oracle.topk(s, 4)) == [6, 1, 3, 4]


def test_topk_brute_force():
    rng = np.random.default_rng(9)
    for trial in range(200):
        E = int(rng.integers(2, 40))
        k = int(rng.integers(1, E + 1))
        s = np.round(rng.standard_normal(E), 1)  # many ties on purpose
        # rank of e = number of experts that come before it
        rank = [sum(1 for o in range(E) if s[o] > s[e] or (s[o] == s[e] and o < e))
                for e in range(E)]
        want = [rank.index(r) for r in range(k)]
        assert list(oracle.topk(s, k)) == want


def test_gating_closed_forms():
    s = np.array([0.3, 1.7, -0.2, 1.1])
    ids = oracle.topk(s, 2)
    w = oracle.gating(s, ids)
    assert list(ids) == [1, 3]
    assert w[0] == pytest.approx(1.0 / (1.0 + math.exp(1.1 - 1.7)), rel=1e-15)
    assert w[1] == pytest.approx(1.0 / (1.0 + math.exp(1.7 - 1.1)), rel=1e-15)
    assert oracle.gating(s, ids[:1], 2.5)[0] == 2.5
    w3 = oracle.gating(s, oracle.topk(s, 4), 1.0)
    assert w3.sum() == pytest.approx(1.0, abs=1e-15)
    assert np.all(np.diff(w3) <= 0)


# ------------------------------------------------------------------- expert

def _expert_brute(mats, fmts, d, f, x):
    G = dense(fmts[0], mats[0], f, d)
    U = dense(fmts[1], mats[1], f, d)
    D = dense(fmts[2], mats[2], d, f)
    return D @ (silu(G @ x) * (U @ x))


@pytest.mark.parametrize("fmts", [(2, 2, 3), (4, 4, 4), (3, 2, 4)])
def test_expert_forward_brute_force(fmts):
    d, f = 96, 64  # d != f catches a transposed operand
    mats = [synth.random_matrix(20 + m, fmts[m], *((f, d) if m < 2 else (d, f)))
            for m in range(3)]
    x = np.random.default_rng(1).standard_normal(d)
    o = oracle.expert_forward(*mats, fmts, d, f, x)
    ref = _expert_brute(mats, fmts, d, f, x)
    assert np.allclose(o, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def _const_block(fmt, code, scale_bits):
    codes = np.full((1, 32), code, np.uint8)
    return oracle.pack_codes(fmt, codes, np.array([scale_bits], np.uint16))


def _const_matrix(fmt, code, scale_bits, rows, cols):
    blk = _const_block(fmt, code, scale_bits)
    return np.tile(blk, rows * cols // 32)


def test_layer_closed_form():
    """d = f = 64, E = 3, k = 2, every matrix a constant block and x all ones:
    g = 64 * (cg - og) * sg, u likewise, h = silu(g) u, o = 64 * (cd - od) *
    sd * h; y = w0 o_a + w1 o_b + o_shared, w from a two-way softmax."""
    d = f = 64
    E, k = 3, 2
    x = np.ones((1, d), np.float32)
    wr = np.zeros((E, d), np.float32)
    wr[0, :] = 0.01   # score 0.64
    wr[1, :] = -0.02  # score -1.28 (not selected)
    wr[2, :] = 0.015  # score 0.96 (rank 0)
    # (code, fp16 scale bits) per expert/matrix; shared FP4 with E8M0
    spec = {
        0: [(2, 3, 0x3800), (2, 2, 0x3C00), (3, 7, 0x2E66)],
        1: [(2, 0, 0x3C00), (2, 0, 0x3C00), (3, 0, 0x3C00)],
        2: [(2, 0, 0x3400), (2, 3, 0x3A00), (3, 1, 0x3000)],
        3: [(4, 9, 124), (4, 12, 123), (4, 3, 122)],
    }
    mats, fmts = [], []
    val = {}
    for e in range(E + 1):
        vals = []
        for m, (fmt, code, sbits) in enumerate(spec[e]):
            rows, cols = (f, d) if m < 2 else (d, f)
            mats.append(_const_matrix(fmt, code, sbits, rows, cols))
            fmts.append(fmt)
            s = 2.0 ** (sbits - 127) if fmt == 4 else float(
                np.uint16(sbits).view(np.float16))
            vals.append((code - OFFSET[fmt]) * s)
        g = d * vals[0]
        u = d * vals[1]
        h = g / (1 + math.exp(-g)) * u
        val[e] = f * vals[2] * h
    y, ids, w = oracle.layer_forward(d, f, E, k, wr, mats, fmts, x, "f32")
    assert list(ids[0]) == [2, 0]
    s2, s0 = 64 * float(np.float32(0.015)), 64 * float(np.float32(0.01))
    w2 = 1.0 / (1.0 + math.exp(s0 - s2))
    want = w2 * val[2] + (1 - w2) * val[0] + val[3]
    assert w[0, 0] == pytest.approx(w2, rel=1e-14)
    assert np.all(y[0] == np.float32(want))


def _tiny_layer(seed=0, d=96, f=64, E=6, k=2, fp4_expert=None):
    cfg = synth.Config("t", d, f, E, k, 1, "f32", "natural",
                       scale_floor=1e-3, master=seed,
                       hot_fp4=0 if fp4_expert is None else 1)
    return synth.gen_layer(cfg, 0, threads=2), cfg


def test_layer_brute_force_tiny():
    lay, cfg = _tiny_layer(seed=31, fp4_expert=True)
    cols = synth.gen_columns(cfg, lay, 3)
    y, ids, w = oracle.layer_forward_synth(lay, cols.x, "f32")
    X = cols.x_f64()
    for c in range(3):
        s = lay.wr.astype(np.float64) @ X[c]
        order = np.argsort(-s, kind="stable")[:lay.k]
        assert list(ids[c]) == list(order)
        ww = np.exp(s[order] - s[order[0]])
        ww /= ww.sum()
        acc = np.zeros(lay.d)
        for j, e in enumerate(order):
            acc += ww[j] * _expert_brute([lay.mat(e, m) for m in range(3)],
                                         lay.fmts[e], lay.d, lay.f, X[c])
        acc += _expert_brute([lay.mat(lay.E, m) for m in range(3)],
                             lay.fmts[lay.E], lay.d, lay.f, X[c])
        # both sides are double; only the final fp32 rounding may differ
        assert np.max(np.abs(y[c] - acc)) <= 2 * np.spacing(
            np.float32(np.abs(acc).max()))


# --------------------------------------------------------------- invariants

def test_column_independence():
    lay, cfg = _tiny_layer(seed=32)
    cols = synth.gen_columns(cfg, lay, 4)
    y4, _, _ = oracle.layer_forward_synth(lay, cols.x, "f32")
    for c in range(4):
        y1, _, _ = oracle.layer_forward_synth(lay, cols.x[c:c + 1], "f32")
        assert np.array_equal(y1[0], y4[c])


def test_relabelling_invariance():
    lay, cfg = _tiny_layer(seed=33)
    cols = synth.gen_columns(cfg, lay, 2)
    y, ids, _ = oracle.layer_forward_synth(lay, cols.x, "f32")
    perm = np.random.default_rng(0).permutation(lay.E)  # new id of old e
    wr2 = np.empty_like(lay.wr)
    wr2[perm] = lay.wr
    mats, fmts = [None] * (3 * (lay.E + 1)), [0] * (3 * (lay.E + 1))
    for e in range(lay.E + 1):
        ne = perm[e] if e < lay.E else lay.E
        for m in range(3):
            mats[3 * ne + m] = lay.mat(e, m)
            fmts[3 * ne + m] = int(lay.fmts[e][m])
    y2, ids2, _ = oracle.layer_forward(lay.d, lay.f, lay.E, lay.k, wr2, mats,
                                       fmts, cols.x, "f32")
    assert np.array_equal(ids2, perm[ids])
    assert np.array_equal(y, y2)


def _scale_down_scales(mat, fmt, factor_bits):
    """Copy of a canonical matrix with every fp16 scale multiplied by 2 (add
    one to the exponent field) -- exact for normal scales."""
    bb = synth.BLOCK_BYTES[fmt]
    m = mat.copy().reshape(-1, bb)
    sc = m[:, bb - 2:].copy().view(np.uint16).reshape(-1)
    assert np.all((sc & 0x7C00) != 0) and np.all((sc & 0x7C00) < 0x7800)
    sc = sc + np.uint16(factor_bits)
    m[:, bb - 2:] = sc.view(np.uint8).reshape(-1, 2)
    return m.reshape(-1)


def test_linearity_in_down_scales():
    lay, cfg = _tiny_layer(seed=34)
    cols = synth.gen_columns(cfg, lay, 1)
    y, ids, w = oracle.layer_forward_synth(lay, cols.x, "f32")
    e = int(ids[0][1])
    mats = [lay.mat(a, m) for a in range(lay.E + 1) for m in range(3)]
    mats[3 * e + 2] = _scale_down_scales(lay.mat(e, 2), lay.fmts[e][2], 0x0400)
    y2, _, _ = oracle.layer_forward(lay.d, lay.f, lay.E, lay.k, lay.wr, mats,
                                    lay.fmts, cols.x, "f32")
    x = cols.x_f64()[0]
    o_e = oracle.expert_forward(*[lay.mat(e, m) for m in range(3)], lay.fmts[e],
                                lay.d, lay.f, x)
    diff = y2[0].astype(np.float64) - y[0].astype(np.float64)
    tol = 4 * np.spacing(np.abs(y[0]).max()) + 4 * np.spacing(np.abs(y2[0]).max())
    assert np.max(np.abs(diff - w[0][1] * o_e)) <= tol


def test_shared_expert_only_when_routed_down_scales_vanish():
    lay, cfg = _tiny_layer(seed=35)
    cols = synth.gen_columns(cfg, lay, 2)
    mats = [lay.mat(a, m) for a in range(lay.E + 1) for m in range(3)]
    for e in range(lay.E):
        bb = synth.BLOCK_BYTES[int(lay.fmts[e][2])]
        m = mats[3 * e + 2].copy().reshape(-1, bb)
        m[:, bb - 2:] = 0
        mats[3 * e + 2] = m.reshape(-1)
    y, _, _ = oracle.layer_forward(lay.d, lay.f, lay.E, lay.k, lay.wr, mats,
                                   lay.fmts, cols.x, "f32")
    for c in range(2):
        o_s = oracle.expert_forward(*[lay.mat(lay.E, m) for m in range(3)],
                                    lay.fmts[lay.E], lay.d, lay.f,
                                    cols.x_f64()[c])
        assert np.array_equal(y[c], o_s.astype(np.float32))


def test_bf16_activations_are_read_exactly():
    lay, cfg = _tiny_layer(seed=36)
    rng = np.random.default_rng(2)
    xf = rng.standard_normal((2, lay.d)).astype(np.float32)
    bits = synth.to_bf16_bits(xf)
    exact = synth.bf16_bits_to_f64(bits).astype(np.float32)
    yb, _, _ = oracle.layer_forward_synth(lay, bits, "bf16")
    yf, _, _ = oracle.layer_forward_synth(lay, exact, "f32")
    assert np.array_equal(yb, yf)


# ------------------------------------------- importance-weighted quantizer

def _fp16_rne(v: float) -> float:
    """numpy's double -> half conversion (round to nearest even), with the
    quantizer's overflow clamp to 65504."""
    h = float(np.float64(v).astype(np.float16))
    return 65504.0 if math.isinf(h) else h


def _weighted_candidates(fmt, a):
    """The candidate scales of the importance-weighted quantizer, in order,
    written out from its definition: t = 1, 1 + 1/16, 1 - 1/16, ..., for
    FP2/FP3; e0, e0 - 1, e0 + 1 for FP4."""
    out = []
    if fmt == 4:
        k = math.ceil(math.log2(a / 7.5))
        if 7.5 * 2.0 ** (k - 1) >= a:
            k -= 1
        for e in (127 + k, 126 + k, 128 + k):
            e = min(max(e, 1), 254)
            if 2.0 ** (e - 127) not in out:
                out.append(2.0 ** (e - 127))
        return out
    for i in range(17):
        k = (i + 1) // 2 * (1 if i % 2 else -1)
        s = _fp16_rne(a / (OFFSET[fmt] * (1 + k / 16)))
        if s != 0.0 and s not in out:
            out.append(s)
    return out


def _weighted_error(fmt, w, imp, codes, s):
    err = 0.0
    for j in range(32):
        d = float(w[j]) - (codes[j] - OFFSET[fmt]) * s
        err += float(imp[j]) * (d * d)
    return err


@pytest.mark.parametrize("fmt", [2, 3, 4])
def test_weighted_pack_brute_force(fmt):
    """Every block: the stored scale is the first candidate of least
    importance-weighted error, the codes the exhaustive nearest codes of
    that scale (errors summed in plain Python floats, in column order)."""
    rng = np.random.default_rng(500 + fmt)
    rows, cols = 6, 256
    w = (rng.standard_normal((rows, cols)) * rng.choice([1e-3, 0.05, 2.0], (rows, 1))
         ).astype(np.float32)
    w[:, 5::37] *= 6.0                                     # outliers to clip or not
    imp = rng.choice([0.0, 0.1, 1.0, 30.0], size=cols).astype(np.float32)
    data = oracle.pack_weighted(fmt, w, imp)
    bb = synth.BLOCK_BYTES[fmt]
    raw = data.tobytes()
    changed = 0
    for r in range(rows):
        for b in range(cols // 32):
            blk = w[r, 32 * b:32 * b + 32].astype(np.float64)
            im = imp[32 * b:32 * b + 32]
            best = None
            for s in _weighted_candidates(fmt, float(np.abs(blk).max())):
                codes = _brute_codes(fmt, blk, s)
                e = _weighted_error(fmt, blk, im, codes, s)
                if best is None or e < best[0]:
                    best = (e, s, codes)
            i = r * (cols // 32) + b
            codes, s = bigint_codes(fmt, raw[i * bb:(i + 1) * bb])
            assert s == best[1] and codes == best[2], (r, b)
            changed += s != _weighted_candidates(fmt, float(np.abs(blk).max()))[0]
    assert changed > 0  # the search does move scales away from absmax


@pytest.mark.parametrize("fmt", [2, 3, 4])
def test_weighted_pack_not_worse_than_absmax(fmt):
    """The absmax scale is a candidate, so no block's weighted error exceeds
    the absmax quantizer's; with all importances 0 every error ties and the
    first candidate, absmax, is kept: the bytes equal rfpx_pack's."""
    rng = np.random.default_rng(600 + fmt)
    w = (rng.standard_normal((16, 128)) * 0.05).astype(np.float32)
    imp = (rng.standard_normal(128) ** 2).astype(np.float32)
    wa = oracle.unpack(fmt, oracle.pack(fmt, w), 16, 128)
    ww = oracle.unpack(fmt, oracle.pack_weighted(fmt, w, imp), 16, 128)
    ea = ((wa - w) ** 2 * imp).reshape(16, 4, 32).sum(-1)
    ew = ((ww - w) ** 2 * imp).reshape(16, 4, 32).sum(-1)
    assert np.all(ew <= ea * (1 + 1e-12))
    assert ew.sum() < ea.sum()
    assert np.array_equal(oracle.pack_weighted(fmt, w, np.zeros(128, np.float32)),
                          oracle.pack(fmt, w))


def test_weighted_pack_invariances():
    """Scaling every importance by a power of two leaves the choice alone;
    a zero block stays all-zero bytes."""
    rng = np.random.default_rng(7)
    w = (rng.standard_normal((8, 96)) * 0.1).astype(np.float32)
    w[3, :32] = 0.0
    imp = rng.random(96).astype(np.float32)
    for fmt in (2, 3, 4):
        a = oracle.pack_weighted(fmt, w, imp)
        assert np.array_equal(a, oracle.pack_weighted(fmt, w, imp * 8.0))
        bb = synth.BLOCK_BYTES[fmt]
        assert not a[9 * bb:10 * bb].any()  # row 3, block 0


# ------------------------------------------------------- dense projection

@pytest.mark.parametrize("fmt,xtype", [(4, "bf16"), (2, "f32"), (3, "bf16")])
def test_dense_forward_brute_force(fmt, xtype):
    """y[c] = W x_c against numpy's product with the big-integer reader's
    dense matrix, for q = 5 columns."""
    rng = np.random.default_rng(700 + fmt)
    rows, cols, q = 48, 160, 5
    data = synth.random_matrix(800 + fmt, fmt, rows, cols, 0.05, 1e-3)
    xf = rng.standard_normal((q, cols))
    x = synth.to_bf16_bits(xf) if xtype == "bf16" else xf.astype(np.float32)
    xd = synth.bf16_bits_to_f64(x) if xtype == "bf16" else x.astype(np.float64)
    y = oracle.dense_forward(fmt, data, rows, cols, x, xtype)
    want = xd @ dense(fmt, data, rows, cols).T
    assert y.shape == (q, rows)
    assert np.allclose(y, want, rtol=1e-6, atol=1e-6 * np.abs(want).max())


def test_dense_forward_columns_are_independent():
    rng = np.random.default_rng(9)
    data = synth.random_matrix(901, 4, 64, 256)
    x = rng.standard_normal((4, 256)).astype(np.float32)
    y = oracle.dense_forward(4, data, 64, 256, x, "f32")
    for c in range(4):
        assert np.array_equal(y[c:c + 1], oracle.dense_forward(4, data, 64, 256, x[c:c + 1], "f32"))
