"""moe_forward_static, the entry point for callers that cannot allocate:
through the C ABI, its outputs equal moe_forward's (one stream, its own
workspace) bit for bit, on two calls in a row with the second smaller, for
the one-token decode launches, the small-batch path and the large path; a
call needing more scratch than the fixed maximum is refused."""
import numpy as np
import pytest
import torch

import routed_expert_ffn_router_amd as moe
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()
    return torch.device("cuda:0")


def _run_both(dl, x, dev):
    T = x.shape[0]
    f = moe.Forward(dl, T, dev, side_stream=False)
    f(x)
    out = torch.full((T, dl.H), float("nan"), dtype=torch.float32, device=dev)
    idx = torch.full((T, dl.k), -1, dtype=torch.int32, device=dev)
    w = torch.full((T, dl.k), float("nan"), dtype=torch.float32, device=dev)
    moe.forward_static(dl, x, out, idx, w)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int32), f.out.view(torch.int32))
    assert torch.equal(idx, f.idx) and torch.equal(w.view(torch.int32), f.w.view(torch.int32))


@pytest.mark.parametrize("first,second", [(200, 16), (16, 1), (4, 1)])
def test_forward_static_equals_forward(dev, first, second):
    layer = synth.gen_layer(synth.Q2, 0)
    dl = moe.DeviceLayer.upload(layer, device=dev)
    for T, seed in ((first, 1), (second, 2)):
        x = torch.from_numpy(synth.gen_x(4096, T, seed=seed).view(np.int16)).to(dev)
        _run_both(dl, x, dev)


def test_forward_static_tiny_and_limit(dev):
    tiny = moe.DeviceLayer.upload(synth.gen_layer(synth.TINY, 0), device=dev)
    for T in (13, 4):
        x = torch.from_numpy(synth.gen_x(256, T, seed=T).view(np.int16)).to(dev)
        _run_both(tiny, x, dev)
    layer = moe.DeviceLayer.upload(synth.gen_layer(synth.Q2, 0), device=dev)
    T = 512  # 113 MB of workspace: above the 64 MiB scratch
    assert layer.forward_workspace(T) > 64 << 20
    x = torch.zeros((T, 4096), dtype=torch.int16, device=dev)
    out = torch.empty((T, 4096), dtype=torch.float32, device=dev)
    idx = torch.empty((T, 8), dtype=torch.int32, device=dev)
    w = torch.empty((T, 8), dtype=torch.float32, device=dev)
    with pytest.raises(moe.MoeError) as e:
        moe.forward_static(layer, x, out, idx, w)
    assert e.value.code == moe.ENOSPC
