"""GPU codec parity: rfpx_pack / rfpx_pack_codes / rfpx_unpack and the device
image against the CPU oracle, bit-exact."""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bqe():
    import block_quantized_expert_amd as m
    m.lib()
    return m


def _weights(seed, rows, cols):
    rng = np.random.default_rng(seed)
    mag = rng.choice([1e-6, 1e-3, 0.05, 1.0, 300.0, 7e4], size=(rows, cols // 32, 1))
    w = (rng.standard_normal((rows, cols // 32, 32)) * mag).reshape(rows, cols)
    w = w.astype(np.float32)
    w[0, :32] = 0.0                      # all-zero block
    w[0, 32:64] = 1e-9                   # scale rounds to fp16 zero
    w[1, :32] = 4e5                      # scale overflows fp16
    w[1, 32:64] = -3.5 * 0.25            # exactly representable extremes
    w[1, 64:96] = np.linspace(-1, 1, 32)  # ties at half steps
    w[2, :32] = 2e-38                    # FP4 exponent clamps at 1
    return w


@pytest.mark.parametrize("fmt", [2, 3, 4])
def test_pack_bit_exact(bqe, fmt):
    import torch
    w = _weights(fmt, 64, 512)
    got = bqe.rfpx_pack(fmt, torch.from_numpy(w).cuda()).cpu().numpy()
    assert np.array_equal(got, oracle.pack(fmt, w))


@pytest.mark.parametrize("fmt", [2, 3, 4])
def test_pack_full_matrix_bit_exact(bqe, fmt):
    import torch
    rows, cols = (2048, 4096) if fmt != 3 else (4096, 2048)
    w = (np.random.default_rng(fmt + 10).standard_normal((rows, cols)) * 0.05).astype(np.float32)
    got = bqe.rfpx_pack(fmt, torch.from_numpy(w).cuda()).cpu().numpy()
    assert np.array_equal(got, oracle.pack(fmt, w))


@pytest.mark.parametrize("fmt", [2, 3, 4])
def test_pack_codes_bit_exact(bqe, fmt):
    import torch
    rng = np.random.default_rng(fmt + 20)
    rows, cols = 33, 256  # ragged row count
    codes = rng.integers(0, 256, size=(rows, cols)).astype(np.uint8)  # high bits ignored
    sb = rng.integers(0, 65536, size=(rows, cols // 32)).astype(np.uint16)
    got = bqe.rfpx_pack_codes(
        fmt, torch.from_numpy(codes).cuda(),
        torch.from_numpy(sb.view(np.int16)).cuda()).cpu().numpy()
    want = oracle.pack_codes(fmt, codes & ((1 << fmt) - 1),
                             sb & (0xFF if fmt == 4 else 0xFFFF))
    assert np.array_equal(got, want)


@pytest.mark.parametrize("fmt", [2, 3, 4])
def test_unpack_exact(bqe, fmt):
    import torch
    data = synth.random_matrix(30 + fmt, fmt, 96, 512)
    got = bqe.rfpx_unpack(fmt, torch.from_numpy(data).cuda(), 96, 512).cpu().numpy()
    want = oracle.unpack(fmt, data, 96, 512).astype(np.float32)
    assert np.array_equal(got, want)


def test_empty_matrix(bqe):
    import torch
    out = bqe.rfpx_pack(2, torch.zeros((0, 64), device="cuda"))
    assert out.numel() == 0


@pytest.fixture(scope="module")
def tiny(bqe):
    lay = synth.gen_layer(synth.WORKLOADS[synth.TINY], 0, threads=4)
    return lay, bqe.upload_layer(lay)


def test_image_roundtrip_tiny_every_matrix(bqe, tiny):
    lay, L = tiny
    for e in range(lay.E + 1):
        for m in range(3):
            rows, cols = lay.matrix_shape(m)
            got = bqe.moe_image_unpack(L, e, m).cpu().numpy()
            want = oracle.unpack(int(lay.fmts[e][m]), lay.mat(e, m), rows, cols)
            assert np.array_equal(got, want.astype(np.float32)), (e, m)


def test_image_roundtrip_decode_size_sample(bqe):
    import torch
    lay = synth.gen_layer(synth.WORKLOADS[synth.VERIFY_Q5], 3)  # mixed FP2/FP3/FP4 layer
    L = bqe.upload_layer(lay)
    hot = int(lay.perm[0])
    for e in (0, hot, 131, lay.E - 1, lay.E):
        for m in range(3):
            rows, cols = lay.matrix_shape(m)
            got = bqe.moe_image_unpack(L, e, m).cpu().numpy()
            want = oracle.unpack(int(lay.fmts[e][m]), lay.mat(e, m), rows, cols)
            assert np.array_equal(got, want.astype(np.float32)), (e, m)
    del L
    torch.cuda.empty_cache()


# ------------------------------------------------------- image validation

def _table(img, E):
    """Header and expert table of an image (host copy): the planes of
    every (expert, matrix) as read by the layer kernels."""
    raw = img[64:64 + 64 * (E + 1)].view(np.uint64).reshape(E + 1, 8)
    codes, scales = raw[:, 0:3], raw[:, 3:6]
    fmts = img[64:64 + 64 * (E + 1)].view(np.int32).reshape(E + 1, 16)[:, 12:15]
    return codes, scales, fmts


def _report(bqe, L):
    import torch
    rep = bqe.moe_image_validate(L)
    torch.cuda.synchronize()
    return [int(v) & 0xFFFFFFFF for v in rep.cpu().tolist()]


def test_image_validate_clean(bqe, tiny):
    """An image built from valid blocks passes every check."""
    lay, L = tiny
    assert _report(bqe, L) == [0, 0, 0, 0]


def test_image_validate_reports_each_fault(bqe, tiny):
    """Each kind of damage is reported on its own: header magic, version,
    shape, byte count; a table entry's format and plane offset; fp16 Inf
    and NaN scales (FP2, FP3 blocks) and E8M0 = 255 (FP4)."""
    import torch
    lay, L0 = tiny
    img = L0._image.cpu().numpy().copy()
    E = lay.E
    codes, scales, fmts = _table(img, E)
    assert np.array_equal(fmts, lay.fmts)

    def check(mutate, want):
        bad = img.copy()
        mutate(bad)
        t = torch.from_numpy(bad).cuda()
        L = bqe.MoeLayer(lay.d, lay.f, lay.E, lay.k, L0._router_w, t, lay.fmts)
        assert _report(bqe, L) == want

    def put(buf, off, arr):
        b = np.asarray(arr).reshape(1).view(np.uint8)
        buf[off:off + b.size] = b

    check(lambda b: put(b, 0, np.uint32(0x12345678)), [1, 0, 0, 0])
    check(lambda b: put(b, 4, np.uint32(7)), [2, 0, 0, 0])
    check(lambda b: put(b, 8, np.int32(lay.d * 2)), [4, 0, 0, 0])
    check(lambda b: put(b, 24, np.uint64(img.size + 256)), [8, 0, 0, 0])
    # expert 3, down matrix: format field, then codes offset
    check(lambda b: put(b, 64 + 3 * 64 + 48 + 8, np.int32(4)), [0, 1, 0, 0])
    check(lambda b: put(b, 64 + 3 * 64 + 16, np.uint64(int(codes[3, 2]) + 256)), [0, 1, 0, 0])
    # scales: one FP2 gate block Inf, one FP3 down block NaN, one -Inf,
    # one FP4 (shared expert) block E8M0 = 255; a large finite fp16 is fine
    assert lay.fmts[0][0] == 2 and lay.fmts[1][2] == 3 and lay.fmts[E][0] == 4

    def scales_bad(b):
        put(b, int(scales[0, 0]) + 2 * 5, np.uint16(0x7C00))
        put(b, int(scales[1, 2]) + 2 * 17, np.uint16(0x7E01))
        put(b, int(scales[2, 1]) + 2 * 3, np.uint16(0xFC00))
        put(b, int(scales[E, 0]) + 9, np.uint8(0xFF))
        put(b, int(scales[4, 0]), np.uint16(0x7BFF))
    check(scales_bad, [0, 0, 4, 0])


# ------------------------------------------- importance-weighted quantizer

@pytest.mark.parametrize("fmt", [2, 3, 4])
def test_pack_weighted_bit_exact(bqe, fmt):
    """rfpx_pack_weighted against the oracle's quantizer, byte for byte, on
    blocks with outliers, zero and vanishing blocks and importances that are
    zero, tiny, equal or spread over many orders of magnitude."""
    import torch
    rng = np.random.default_rng(50 + fmt)
    rows, cols = 96, 512
    w = _weights(fmt + 60, rows, cols)
    w[3:, 7::41] *= 9.0
    imp = (rng.lognormal(0.0, 2.0, size=cols)).astype(np.float32)
    imp[::13] = 0.0
    imp[5] = 1e-30
    got = bqe.rfpx_pack_weighted(fmt, torch.from_numpy(w).cuda(),
                                 torch.from_numpy(imp).cuda()).cpu().numpy()
    want = oracle.pack_weighted(fmt, w, imp)
    assert np.array_equal(got, want)
    # the search moved some scales away from the absmax choice
    assert not np.array_equal(want, oracle.pack(fmt, w))


def test_pack_weighted_full_matrix_bit_exact(bqe):
    """A 2048 x 4096 FP2 matrix (a gate matrix of the decode layer) with
    synthetic importances: the mean square of 64 N(0,1) activations per
    column, scaled per column by a lognormal factor."""
    import torch
    rng = np.random.default_rng(77)
    rows, cols = 2048, 4096
    w = (rng.standard_normal((rows, cols)) * 0.05).astype(np.float32)
    acts = rng.standard_normal((64, cols)) * rng.lognormal(0.0, 1.0, size=cols)
    imp = (acts ** 2).mean(0).astype(np.float32)
    got = bqe.rfpx_pack_weighted(2, torch.from_numpy(w).cuda(),
                                 torch.from_numpy(imp).cuda()).cpu().numpy()
    assert np.array_equal(got, oracle.pack_weighted(2, w, imp))


# ------------------------------------------------------- plain read

@pytest.mark.parametrize("nbytes", [16, 4096 + 48, 26476544])
def test_stream_read_reads_every_word(bqe, nbytes):
    """rfpx_stream_read touches every 32-bit word once: the XOR of its sink
    words is the XOR of the buffer's words (numpy), also for sizes that are
    not a whole number of batches."""
    import torch
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 256, size=nbytes, dtype=np.uint8)
    buf = torch.from_numpy(host).cuda()
    sink = bqe.rfpx_stream_read(buf)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host.view(np.uint32))
