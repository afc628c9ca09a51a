"""GPU routing parity: expert ids bit-exact against the oracle's sorted
top-k (score descending, ties to the lower index); gating weights within
1e-6 relative (fp32 exp on the GPU, double in the oracle)."""
import numpy as np
import pytest

import oracle
import synth
from gpu_common import to_device_x

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bqe():
    import block_quantized_expert_amd as m
    m.lib()
    return m


def _router_layer(bqe, wr, k, f=128, fmts=None):
    """Layer descriptor for routing only: moe_route_topk reads the router
    and nothing of the image (its header says so; the image pointer is not
    passed to any of its kernels), so a small aligned buffer stands in."""
    import torch
    E, d = wr.shape
    fm = synth.expert_formats(E, np.arange(E), 0) if fmts is None else fmts
    image = torch.zeros(256, dtype=torch.uint8, device="cuda")
    return bqe.MoeLayer(d, f, E, k, torch.from_numpy(wr).cuda(), image, fm)


def _check(bqe, L, wr, k, x_np, xtype):
    x = to_device_x(x_np)
    ids, w = bqe.moe_route_topk(L, x)
    ids, w = ids.cpu().numpy(), w.cpu().numpy()
    X = synth.bf16_bits_to_f64(x_np) if xtype == "bf16" else x_np.astype(np.float64)
    s = oracle.router_scores(X, wr)
    for c in range(X.shape[0]):
        want = oracle.topk(s[c], k)
        assert list(ids[c]) == list(want), (c, ids[c], want)
        gw = oracle.gating(s[c], want)
        assert np.allclose(w[c], gw, rtol=1e-6, atol=1e-7)
    return ids


@pytest.mark.parametrize("name", [synth.TINY, synth.DECODE_Q1, synth.VERIFY_Q4, synth.VERIFY_Q5])
def test_route_workloads(bqe, name):
    cfg = synth.WORKLOADS[name]
    wr, perm = synth.gen_router(cfg, 0)
    L = _router_layer(bqe, wr, cfg.k, f=cfg.f)
    q = 4 if name == synth.TINY else cfg.q
    for variant in range(3):
        cols = synth.gen_columns(cfg, (wr, perm, cfg.k), q, variant=variant)
        ids = _check(bqe, L, wr, cfg.k, cols.x, cfg.xtype)
        if cols.drawn is not None:
            assert np.array_equal(ids, cols.drawn)


def test_route_prefill_tokens_in_chunks(bqe):
    cfg = synth.WORKLOADS[synth.PREFILL]
    wr, perm = synth.gen_router(cfg, 0)
    L = _router_layer(bqe, wr, cfg.k, f=cfg.f)
    cols = synth.gen_columns(cfg, (wr, perm, cfg.k), 256)
    for c0 in range(0, 256, 8):
        ids = _check(bqe, L, wr, cfg.k, cols.x[c0:c0 + 8], "bf16")
        assert np.array_equal(ids, cols.drawn[c0:c0 + 8])


def test_route_ties_go_to_lower_index(bqe):
    rng = np.random.default_rng(1)
    wr = (rng.standard_normal((64, 256)) * 0.02).astype(np.float32)
    wr[40] = wr[7]     # equal scores for experts 7 and 40
    wr[41] = wr[7]
    # make 7/40/41 the top scores: push x along their (shared) router row
    x = (rng.standard_normal((3, 256)) + 40.0 * wr[7][None, :]).astype(np.float32)
    L = _router_layer(bqe, wr, 4)
    xt = to_device_x(x)
    ids, _ = bqe.moe_route_topk(L, xt)
    ids = ids.cpu().numpy()
    for c in range(3):
        assert list(ids[c][:3]) == [7, 40, 41]
        s = oracle.router_scores(x[c].astype(np.float64), wr)[0]
        assert list(oracle.topk(s, 3)) == [7, 40, 41]


@pytest.mark.parametrize("E,k,q", [(1, 1, 1), (100, 8, 8), (1024, 8, 3), (256, 6, 8)])
def test_route_edge_sizes(bqe, E, k, q):
    rng = np.random.default_rng(E + k + q)
    wr = (rng.standard_normal((E, 512)) * 0.02).astype(np.float32)
    cfg = synth.Config("t", 512, 128, E, k, q, "f32", "natural", master=E)
    cols = synth.gen_columns(cfg, (wr, np.arange(E), k), q)
    L = _router_layer(bqe, wr, k)
    _check(bqe, L, wr, k, cols.x, "f32")
