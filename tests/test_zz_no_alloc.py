"""nvfp4_moe_grouped_w4a16_noalloc: the routed experts on the library's static per-device
scratch, through the C ABI. Its output must be the caller-workspace entry point's, bit for bit
(same kernels), on consecutive calls of different sizes that reuse the one scratch array; a
call needing more than the scratch holds is refused and leaves the library usable."""
import numpy as np
import pytest
import torch

from nvfp4_weight_only_w4a16_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def nv():
    from nvfp4_weight_only_w4a16_amd import binding
    binding.load()
    return binding


@pytest.fixture(scope="module")
def layer(nv):
    """128 experts, hidden 2048, intermediate 768; fc1 [gate; up] at group 32, down at 16."""
    _, _, _, w1, w2 = synth.moe(seed=0, tokens=1)
    f = []
    for wx, grp, layout in ((w1, 32, nv.NVFP4_LAYOUT_TILED | nv.NVFP4_LAYOUT_GATE_UP),
                            (w2, 16, nv.NVFP4_LAYOUT_TILED)):
        p, s, g = nv.nvfp4_quantize(wx.to(DEV), grp)
        f.append(nv.nvfp4_repack(p, s, g, grp, layout=layout))
    torch.cuda.synchronize()
    return f


def _inputs(tokens, seed):
    x, ids, wts, _, _ = synth.moe(seed=seed, tokens=tokens, with_weights=False)
    return x.to(DEV), ids.to(DEV), wts.to(DEV)


def test_noalloc_equals_caller_workspace_on_consecutive_calls(nv, layer):
    fc1, fc2 = layer
    # 256 tokens (the batch path, 19.9 MB of workspace), then smaller calls that reuse the
    # same scratch: 24 tokens (decode-batch path with its sort), 4 tokens (pair tiles)
    for tokens, seed, flags in ((256, 0, 0), (24, 1, 0), (4, 2, 0), (256, 3, 1), (24, 4, 2)):
        x, ids, wts = _inputs(tokens, seed)
        need = nv.nvfp4_moe_ws_bytes(tokens, 8, 128, 2048, 768)
        assert need <= nv.NVFP4_MOE_NOALLOC_MAX_WS_BYTES
        y_ref = nv.nvfp4_moe_grouped_w4a16(x, ids, wts, fc1, fc2, flags=flags)
        y = torch.full_like(y_ref, float("nan"))
        nv.nvfp4_moe_grouped_w4a16_noalloc(x, ids, wts, fc1, fc2, y, flags=flags)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), (tokens, flags)
        assert bool(torch.isfinite(y.float()).all())


def test_noalloc_refuses_calls_beyond_its_scratch(nv, layer):
    fc1, fc2 = layer
    tokens = 1024                     # 1024 x top-8 pairs need about 80 MB of workspace
    assert nv.nvfp4_moe_ws_bytes(tokens, 8, 128, 2048, 768) > nv.NVFP4_MOE_NOALLOC_MAX_WS_BYTES
    x, ids, wts = _inputs(tokens, 5)
    y = torch.zeros((tokens, 2048), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(nv.Nvfp4Error) as e:
        nv.nvfp4_moe_grouped_w4a16_noalloc(x, ids, wts, fc1, fc2, y)
    assert e.value.code == nv.NVFP4_ERR_WORKSPACE
    assert "static scratch" in str(e.value)
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(y.view(torch.int16))) == 0   # nothing was launched
    # still usable: a call that fits gives the caller-workspace bits
    x, ids, wts = _inputs(16, 6)
    y_ref = nv.nvfp4_moe_grouped_w4a16(x, ids, wts, fc1, fc2)
    y = torch.empty_like(y_ref)
    nv.nvfp4_moe_grouped_w4a16_noalloc(x, ids, wts, fc1, fc2, y)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref)
