"""moe_layer_forward_noalloc (the library's own device scratch, no
allocation) against moe_layer_forward (a caller workspace) on the same
inputs, through the C ABI: two calls in a row, the second with a smaller
input (fewer columns, then a smaller layer), each bit for bit equal to the
workspace entry point (the same kernels on the same data) and within
2e-3 * RMS of the oracle."""
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


def _pair(bqe, L, x_np):
    """y of moe_layer_forward_noalloc and of moe_layer_forward on x."""
    import torch
    x = to_device_x(x_np)
    q = x.shape[0]
    y_na = torch.full((q, L.d), float("nan"), dtype=torch.float32, device="cuda")
    bqe.moe_layer_forward_noalloc(L, x, y_na)
    y_ws = bqe.moe_layer_forward(L, x)
    torch.cuda.synchronize()
    return y_na.cpu().numpy(), y_ws.cpu().numpy()


def test_noalloc_matches_workspace_entry_point(bqe):
    import torch
    assert bqe.lib().moe_noalloc_scratch_bytes() == 8 << 20
    # first call: the q=5 verify layer (d=4096, 256 experts, hot experts FP4)
    cfg = synth.WORKLOADS[synth.VERIFY_Q5]
    lay = synth.gen_layer(cfg, 7)
    L = bqe.upload_layer(lay)
    assert bqe.moe_workspace_bytes(L, 5) <= 8 << 20
    cols = synth.gen_columns(cfg, lay, 5, layer=7)
    y_na, y_ws = _pair(bqe, L, cols.x)
    assert np.array_equal(y_na, y_ws)
    refs = [oracle.layer_forward_synth(lay, cols.x[c:c + 1], "bf16")[0] for c in range(5)]
    assert_close(y_na, np.concatenate(refs), what="q=5, first call")
    # second call, smaller: two of the columns on the same layer
    y_na, y_ws = _pair(bqe, L, cols.x[1:3])
    assert np.array_equal(y_na, y_ws)
    assert_close(y_na, np.concatenate(refs[1:3]), what="q=2, second call")
    del L
    torch.cuda.empty_cache()
    # third call, smaller still: the tiny layer, one fp32 column
    tcfg = synth.WORKLOADS[synth.TINY]
    tlay = synth.gen_layer(tcfg, 0, threads=4)
    TL = bqe.upload_layer(tlay)
    tcols = synth.gen_columns(tcfg, tlay, 1, variant=21)
    y_na, y_ws = _pair(bqe, TL, tcols.x)
    assert np.array_equal(y_na, y_ws)
    assert_close(y_na, oracle.layer_forward_synth(tlay, tcols.x, "f32")[0], what="tiny q=1")


def test_noalloc_rejects_shapes_beyond_the_scratch(bqe):
    """The largest decode shape needs more than the scratch: refused before
    any launch, with the workspace entry point named in the message."""
    import torch
    cfg = synth.Config("big", 4096, 4096, 64, 8, 8, "bf16", "natural", scale_floor=1e-3,
                       master=901)
    wr = torch.zeros((64, 4096), dtype=torch.float32, device="cuda")
    fm = synth.expert_formats(64, np.arange(64), 0)
    n = bqe.moe_image_bytes(4096, 4096, 64, fm)
    img = torch.empty(256, dtype=torch.uint8, device="cuda")
    L = bqe.MoeLayer(4096, 4096, 64, 8, wr, img, fm, image_bytes=n)
    assert bqe.moe_workspace_bytes(L, 8) > 8 << 20
    x = torch.zeros((8, 4096), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((8, 4096), dtype=torch.float32, device="cuda")
    with pytest.raises(bqe.RfpxError) as ei:
        bqe.moe_layer_forward_noalloc(L, x, y)
    assert ei.value.status == -5 and "moe_layer_forward with a workspace" in str(ei.value)
    del cfg
