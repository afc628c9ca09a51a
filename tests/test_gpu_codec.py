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
