"""beam_moe_forward_noalloc (the library's static device scratch instead of a workspace)
against beam_moe_forward on the same arguments, through the C ABI: two calls in a row, the
second with fewer tokens and without the sublayer, so the second call runs on the scratch
the first one left behind.  The kernels are the same, so the results are bit-identical.
Shapes beyond the scratch limit are refused before any launch."""
import math

import numpy as np
import pytest

import oracle
from synth.configs import Config, make_inputs

from moe_cases import dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_moe_layer_04_amd  # noqa: F401


def _cfg(T, sublayer):
    return Config("noalloc_t%d" % T, T=T, H=512, E=64, I=256, n_group=8, topk_group=4, top_k=8, rho=2.5,
                  dtype="bf16", wr_std=math.sqrt(1.0 / 512), w_std=0.05, wd_std=0.05, bias="uniform:0.05",
                  sublayer=sublayer, seed_base=31000 + T, weight_seed=31000)


def _both(cfg, inp):
    """(out, idx, w, moe_y) of beam_moe_forward and of beam_moe_forward_noalloc."""
    import torch
    import sparse_moe_layer_04_amd as bm
    shape = bm.make_shape(cfg.T, cfg.H, cfg.E, cfg.I, cfg.n_group, cfg.topk_group, cfg.top_k, cfg.rho, "bf16")
    x, wr, b = dev(inp.x), dev(inp.w_router), dev(inp.bias)
    wg, wu, wd = dev(inp.w_gate), dev(inp.w_up), dev(inp.w_down)
    sub = None
    if cfg.sublayer:
        g1, g2 = dev(inp.pre_gain), dev(inp.post_gain)
        sub = bm.sublayer(g1, g2, cfg.eps, cfg.residual_k)
    res = []
    for noalloc in (False, True):
        out = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device="cuda")
        idx = torch.empty((cfg.T, cfg.top_k), dtype=torch.int32, device="cuda")
        w = torch.empty((cfg.T, cfg.top_k), dtype=torch.float32, device="cuda")
        moe_y = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device="cuda") if cfg.sublayer else None
        if noalloc:
            bm.forward_noalloc(shape, x, wr, b, wg, wu, wd, out, sublayer=sub, topk_idx=idx, topk_w=w, moe_y=moe_y)
        else:
            op = bm.OP_FORWARD_SUBLAYER if cfg.sublayer else bm.OP_FORWARD
            ws = torch.empty(bm.workspace_size(shape, op), dtype=torch.uint8, device="cuda")
            bm.forward(shape, x, wr, b, wg, wu, wd, out, ws, sublayer=sub, topk_idx=idx, topk_w=w, moe_y=moe_y)
        torch.cuda.synchronize()
        res.append((out, idx, w, moe_y))
    return res


def test_noalloc_equals_forward_on_two_calls_the_second_smaller():
    import torch
    for T, sublayer in ((300, True), (40, False)):
        cfg = _cfg(T, sublayer)
        inp = make_inputs(cfg)
        (o1, i1, w1, y1), (o2, i2, w2, y2) = _both(cfg, inp)
        assert torch.equal(i1, i2) and torch.equal(w1, w2)
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
        if sublayer:
            assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
        # and the routing is the oracle's (the inputs are not checked for near-ties here:
        # compare where the oracle's margins are clear)
        u = oracle.rmsnorm_pinned(inp.x, inp.pre_gain, cfg.eps) if sublayer else inp.x
        r = oracle.route(u, inp.w_router, inp.bias, cfg.n_group, cfg.topk_group, cfg.top_k, cfg.rho)
        clear = r.margin.min(axis=1) >= 1e-6
        got = np.sort(i2.cpu().numpy(), axis=1)
        assert (got[clear] == np.sort(r.idx, axis=1)[clear]).all()
        print("noalloc T=%d sublayer=%s: bit-identical to beam_moe_forward" % (T, sublayer))


def test_noalloc_refuses_shapes_beyond_its_scratch_before_launch():
    import torch
    import sparse_moe_layer_04_amd as bm
    T = 1024   # the Beam layer at 1024 tokens needs ~152 MiB of workspace
    shape = bm.make_shape(T, 5120, 256, 2560, 8, 4, 8, 2.5, "bf16")
    assert bm.workspace_size(shape, bm.OP_FORWARD) > bm.NOALLOC_SCRATCH_BYTES
    t = torch.zeros(16, dtype=torch.bfloat16, device="cuda")   # never read: refused first
    with pytest.raises(bm.BeamError) as ei:
        bm.forward_noalloc(shape, t, t, t, t, t, t, t)
    assert ei.value.status == bm.BEAM_ERR_WORKSPACE
