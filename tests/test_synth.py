"""The seeded generators: determinism, byte counts, and that the routing they
prescribe is what the oracle's own router computes from the stored inputs,
with the score gaps the tests rely on."""
import numpy as np
import pytest

import oracle
import synth


def test_same_seed_same_bytes():
    a = synth.random_matrix(5, synth.FP3, 64, 256)
    b = synth.random_matrix(5, synth.FP3, 64, 256)
    c = synth.random_matrix(6, synth.FP3, 64, 256)
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    assert a.size == 64 * 8 * 14


def test_tiny_layer_sizes_and_formats():
    cfg = synth.WORKLOADS[synth.TINY]
    lay = synth.gen_layer(cfg, 0, threads=2)
    assert lay.fmts.shape == (9, 3)
    assert list(lay.fmts[0]) == [2, 2, 3] and list(lay.fmts[8]) == [4, 4, 4]
    # 8 routed experts (FP2, FP2, FP3) + shared FP4, d=256, f=128
    per_routed = 2 * 128 * 8 * 10 + 256 * 4 * 14
    per_fp4 = 2 * 128 * 8 * 17 + 256 * 4 * 17
    assert lay.blob.size == 8 * per_routed + per_fp4 == 330752
    lay2 = synth.gen_layer(cfg, 0, threads=3)
    assert np.array_equal(lay.blob, lay2.blob)


def test_scale_distribution_tiny():
    cfg = synth.WORKLOADS[synth.TINY]
    lay = synth.gen_layer(cfg, 0, threads=2)
    g = lay.mat(0, 0).reshape(-1, 10)
    s = g[:, 8:].copy().view(np.float16).astype(np.float64).reshape(-1)
    assert np.all(s >= 1e-3 - 1e-6)
    assert abs(np.mean(s) - (0.05 * np.sqrt(2 / np.pi) + 1e-3)) < 2e-3


def test_hot_experts_fp4():
    cfg = synth.WORKLOADS[synth.VERIFY_Q5]
    wr, perm = synth.gen_router(cfg, 7)
    fm = synth.expert_formats(cfg.E, perm, cfg.hot_fp4)
    assert set(np.flatnonzero(fm[:256, 0] == 4)) == set(perm[:32].tolist())
    assert np.all(fm[256] == 4)


def _check_columns(cfg, wr, perm, cols, k):
    X = cols.x_f64()
    for c in range(X.shape[0]):
        s = oracle.router_scores(X[c], wr)[0]
        ids = oracle.topk(s, k + 1)
        gaps = s[ids[:-1]] - s[ids[1:]]
        assert np.all(gaps >= synth.GAP), gaps
        if cols.drawn is not None:
            assert list(ids[:k]) == list(cols.drawn[c])


def test_natural_routing_gap_guard_tiny():
    cfg = synth.WORKLOADS[synth.TINY]
    wr, perm = synth.gen_router(cfg, 0)
    cols = synth.gen_columns(cfg, (wr, perm, cfg.k), 16)
    assert cols.x.dtype == np.float32
    _check_columns(cfg, wr, perm, cols, cfg.k)


def test_natural_routing_gap_guard_decode():
    cfg = synth.WORKLOADS[synth.DECODE_Q1]
    wr, perm = synth.gen_router(cfg, 0)
    cols = synth.gen_columns(cfg, (wr, perm, cfg.k), 8)
    assert cols.x.dtype == np.uint16
    _check_columns(cfg, wr, perm, cols, cfg.k)


@pytest.mark.parametrize("name", [synth.VERIFY_Q4, synth.VERIFY_Q5])
def test_zipf_routing_is_realized_by_the_oracle(name):
    cfg = synth.WORKLOADS[name]
    wr, perm = synth.gen_router(cfg, 1)
    cols = synth.gen_columns(cfg, (wr, perm, cfg.k), cfg.q, layer=1)
    _check_columns(cfg, wr, perm, cols, cfg.k)
    # activations keep a unit-normal look after steering
    X = cols.x_f64()
    assert 0.8 < X.std() < 1.3


def test_zipf_draw_law():
    rng = np.random.default_rng(0)
    perm = np.arange(256)
    draws = synth.zipf_draws(rng, 256, 6, 3000, perm)
    assert all(len(set(r)) == 6 for r in draws)
    # first draw follows p_r ~ r^-1.1: rank 1 has probability 0.2065
    p1 = np.mean(draws[:, 0] == 0)
    assert abs(p1 - 0.2065) < 0.025
    # expected distinct experts over 4 columns is about 18.4
    u = np.mean([len(set(draws[i:i + 4].reshape(-1))) for i in range(0, 3000, 4)])
    assert 17.5 < u < 19.3


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.00390625, 1.005859375, -2.5e-3, 3.3e38], np.float32)
    b = synth.to_bf16_bits(x)
    back = synth.bf16_bits_to_f64(b)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: goes to the even 1.0
    assert back[0] == 1.0 and back[1] == 1.0
    assert back[2] == 1.0078125
    assert np.all(np.abs(back - x) <= np.abs(x) * 2.0 ** -8)
