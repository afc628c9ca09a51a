"""GPU parity of the prefill path (moe_prefill_forward) against the CPU oracle.

The oracle treats every token as one column of the decode definition; the
prefill path groups tokens by expert and runs the products on the matrix
cores, so only the order of fp32 sums differs.  Tolerance as for decode:
max |y_gpu - y_oracle| <= 2e-3 * RMS(y_oracle) over the compared tokens.
Every test compares every token: small layers (ragged token counts,
several chunks per expert, every format in every matrix position) and the
largest chunk the entry point takes; the 2048-token Zipf workload is checked
on every token in test_gpu_workloads.py.
"""
import concurrent.futures as cf

import numpy as np
import pytest

import oracle
import synth
from gpu_common import HipEvents, assert_close, check_stamps, to_device_x

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bqe():
    import block_quantized_expert_amd as m
    m.lib()
    return m


def _prefill(bqe, L, x_np):
    import torch
    y = bqe.moe_prefill_forward(L, to_device_x(x_np))
    torch.cuda.synchronize()
    return y.cpu().numpy()


def _oracle_rows(lay, x, xtype, rows=None, threads=8):
    """Oracle outputs of the given token rows (all rows by default)."""
    rows = range(x.shape[0]) if rows is None else rows
    rows = list(rows)
    chunks = [rows[i::threads] for i in range(threads)]

    def run(ch):
        if not ch:
            return {}
        y, _, _ = oracle.layer_forward_synth(lay, x[ch], xtype)
        return dict(zip(ch, y))

    out = {}
    with cf.ThreadPoolExecutor(threads) as ex:
        for part in ex.map(run, chunks):
            out.update(part)
    return np.stack([out[r] for r in rows])


def _mixed_layer(d, f, E, k, seed):
    """A layer whose format table cycles every format through every matrix."""
    cfg = synth.Config("t", d, f, E, k, 1, "f32", "natural", scale_floor=1e-3,
                       master=200 + seed)
    lay = synth.gen_layer(cfg, 0, threads=4)
    rng = np.random.default_rng(seed)
    fm = lay.fmts.copy()
    for e in range(E + 1):
        g = [2, 3, 4][(e + seed) % 3]
        fm[e] = [g, g, [2, 3, 4][(e + 2 * seed) % 3]]
    mats = []
    for e in range(E + 1):
        for m in range(3):
            rows, cols = (f, d) if m < 2 else (d, f)
            mats.append(synth.random_matrix(int(rng.integers(1 << 30)), int(fm[e][m]),
                                            rows, cols, 0.05, 1e-3))
    lay.fmts = fm
    lay.offsets = np.concatenate([[0], np.cumsum([m.size for m in mats])[:-1]]).astype(np.int64)
    lay.blob = np.concatenate(mats)
    return cfg, lay


def test_prefill_tiny_every_token(bqe):
    cfg = synth.WORKLOADS[synth.TINY]
    lay = synth.gen_layer(cfg, 0, threads=4)
    L = bqe.upload_layer(lay)
    for xt, T in (("f32", 64), ("bf16", 37)):
        c = synth.Config(**{**cfg.__dict__, "xtype": xt})
        x = synth.gen_columns(c, lay, T, variant=5).x
        assert_close(_prefill(bqe, L, x), _oracle_rows(lay, x, xt), what=f"{xt} T={T}")


@pytest.mark.parametrize("d,f,E,k,T,seed", [(512, 256, 16, 4, 150, 1), (256, 1024, 12, 3, 61, 2),
                                             (1024, 64, 32, 8, 200, 3)])
def test_prefill_mixed_formats(bqe, d, f, E, k, T, seed):
    """Every format in every position; T large enough that the busiest
    experts need several 128-row chunks, and ragged chunks everywhere."""
    cfg, lay = _mixed_layer(d, f, E, k, seed)
    L = bqe.upload_layer(lay)
    for xt in ("bf16", "f32"):
        c = synth.Config(**{**cfg.__dict__, "xtype": xt})
        x = synth.gen_columns(c, lay, T, variant=7).x
        assert_close(_prefill(bqe, L, x), _oracle_rows(lay, x, xt), what=f"{xt} T={T}")


def test_prefill_single_token_and_one_expert(bqe):
    # T = 1; and E = k = 1 (every token picks the only routed expert)
    cfg = synth.Config("t", 256, 128, 1, 1, 1, "bf16", "natural", scale_floor=1e-3, master=300)
    lay = synth.gen_layer(cfg, 0, threads=4)
    L = bqe.upload_layer(lay)
    for T in (1, 5, 130):
        x = synth.gen_columns(cfg, lay, T, variant=T).x
        assert_close(_prefill(bqe, L, x), _oracle_rows(lay, x, "bf16"), what=f"T={T}")


def test_prefill_deterministic(bqe):
    cfg, lay = _mixed_layer(512, 256, 16, 4, 5)
    L = bqe.upload_layer(lay)
    c = synth.Config(**{**cfg.__dict__, "xtype": "bf16"})
    x = synth.gen_columns(c, lay, 170, variant=9).x
    assert np.array_equal(_prefill(bqe, L, x), _prefill(bqe, L, x))


def test_prefill_timed_entry_point(bqe):
    """moe_prefill_forward_timed gives moe_prefill_forward's output bit for
    bit and stamps the stages' starts and ends in launch order."""
    import torch
    cfg, lay = _mixed_layer(512, 256, 16, 4, 6)
    L = bqe.upload_layer(lay)
    c = synth.Config(**{**cfg.__dict__, "xtype": "bf16"})
    x = to_device_x(synth.gen_columns(c, lay, 150, variant=11).x)
    ws = bqe.workspace(L, 150, prefill=True)
    y0 = bqe.moe_prefill_forward(L, x, ws=ws)
    y1 = torch.full_like(y0, float("nan"))
    he = HipEvents()
    ev = he.create(6)
    bqe.moe_prefill_forward_timed(L, x, y1, ws, ev)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
    check_stamps(he, ev)
    he.destroy(ev)


def test_prefill_max_tokens(bqe):
    """The largest chunk the entry point accepts (T = 65536) on the tiny
    layer: the busiest experts get over a thousand 64-row tasks.  Every
    token against the oracle, 16 against the decode path."""
    import torch
    cfg = synth.Config(**{**synth.WORKLOADS[synth.TINY].__dict__, "xtype": "bf16"})
    lay = synth.gen_layer(cfg, 0, threads=4)
    L = bqe.upload_layer(lay)
    T = 65536
    cols = synth.gen_columns(cfg, lay, T, variant=13)
    y = _prefill(bqe, L, cols.x)
    assert y.shape == (T, cfg.d) and np.all(np.isfinite(y))
    rng = np.random.default_rng(13)
    assert_close(y, _oracle_rows(lay, cols.x, "bf16", threads=16), what="every token")
    xd = to_device_x(cols.x)
    for t in rng.choice(T, 16, replace=False).tolist():
        yd = bqe.moe_layer_forward(L, xd[t:t + 1])
        torch.cuda.synchronize()
        assert_close(y[t:t + 1], yd.cpu().numpy(), tol=1e-4, what=f"decode vs prefill token {t}")
    del L, xd
    torch.cuda.empty_cache()
