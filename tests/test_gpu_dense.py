"""GPU parity of the dense q-column product (rfpx_dense_forward) against the
CPU oracle: max |y_gpu - y_oracle| <= 2e-3 * RMS(y_oracle) over each call's
q * rows outputs; the dense image bit-exact against the oracle's unpack;
columns independent and results identical from run to run, bit for bit."""
import concurrent.futures as cf

import numpy as np
import pytest

import oracle
import synth
from gpu_common import assert_close, to_device_x

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bqe():
    import block_quantized_expert_amd as m
    m.lib()
    return m


def _matrix(bqe, fmt, rows, cols, seed):
    import torch
    data = synth.random_matrix(seed, fmt, rows, cols, 0.05, 1e-3)
    return data, bqe.DenseMatrix(fmt, rows, cols, torch.from_numpy(data).cuda())


def _x(q, cols, xtype, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((q, cols))
    return synth.to_bf16_bits(x) if xtype == "bf16" else x.astype(np.float32)


def _oracle(fmt, data, rows, cols, x, xtype, threads=8):
    """The oracle, one column per thread."""
    with cf.ThreadPoolExecutor(threads) as ex:
        parts = list(ex.map(lambda c: oracle.dense_forward(fmt, data, rows, cols, x[c:c + 1],
                                                           xtype), range(x.shape[0])))
    return np.concatenate(parts)


def _run(bqe, m, x_np):
    import torch
    y = bqe.rfpx_dense_forward(m, to_device_x(x_np))
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("fmt", [2, 3, 4])
def test_dense_image_roundtrip(bqe, fmt):
    rows, cols = 192, 256
    data, m = _matrix(bqe, fmt, rows, cols, 10 + fmt)
    got = m.unpack().cpu().numpy()
    assert np.array_equal(got, oracle.unpack(fmt, data, rows, cols).astype(np.float32))


@pytest.mark.parametrize("fmt,rows,cols", [
    (4, 64, 256),      # one tile, one chunk per wave, no split
    (4, 64, 4096),     # one tile split over two workgroups (partial sums)
    (2, 128, 128),     # FP2 chunks of two blocks, fewer waves than eight
    (3, 320, 96),      # FP3, three chunks per row: four waves... of one
    (4, 192, 1024),
    (2, 256, 2048),
    (3, 128, 4096),
])
def test_dense_small_shapes_every_q(bqe, fmt, rows, cols):
    """q = 1..8 columns, bf16 and fp32 activations, against the oracle."""
    data, m = _matrix(bqe, fmt, rows, cols, rows + cols + fmt)
    for xtype in ("bf16", "f32"):
        for q in range(1, 9):
            x = _x(q, cols, xtype, 100 * q + fmt)
            y_ref = _oracle(fmt, data, rows, cols, x, xtype)
            assert_close(_run(bqe, m, x), y_ref, what=f"{xtype} q={q}")


@pytest.mark.parametrize("fmt", [4, 2])
def test_dense_projection_size(bqe, fmt):
    """A 16384 x 4096 projection (the benchmark's shape) at q = 1, 4, 5:
    every output against the oracle."""
    import torch
    rows, cols = 16384, 4096
    data, m = _matrix(bqe, fmt, rows, cols, 7000 + fmt)
    for q in (1, 4, 5):
        x = _x(q, cols, "bf16", 90 + q)
        y_ref = _oracle(fmt, data, rows, cols, x, "bf16")
        assert_close(_run(bqe, m, x), y_ref, what=f"q={q}")
    del m
    torch.cuda.empty_cache()


def test_dense_columns_independent_and_deterministic(bqe):
    """Column c of a q = 8 call equals the q = 1 call on column c, bit for
    bit (each lane sums its row in the same order at every q); two calls
    give the same bits."""
    rows, cols = 4096, 4096
    data, m = _matrix(bqe, 4, rows, cols, 4242)
    x = _x(8, cols, "bf16", 5)
    y8 = _run(bqe, m, x)
    assert np.array_equal(y8, _run(bqe, m, x))
    for c in (0, 3, 7):
        assert np.array_equal(y8[c:c + 1], _run(bqe, m, x[c:c + 1]))
