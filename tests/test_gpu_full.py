"""GPU parity at the full Beam shapes (H=5120, E=256, I=2560; 20 GB of bf16 expert weights),
in the launch configuration the benchmark times, at two serving shapes between decode and
prefill (256 and 1024 tokens: 8 and 32 routed rows per expert, on either side of the kernel
switch), and for decode and prefill with the weights in 8-bit (E4M3) and 4-bit (MXFP4: E2M1)
storage with E8M0 scales per 32 weights.

Routing is compared bit-exact (as sets) on ALL tokens; outputs are compared on a seeded
sample of 256 tokens plus, for every non-empty expert, the tokens of its first and last
rows (the rows of every expert's final partial tile), within 1e-2 * max|ref|."""
import time

import numpy as np
import pytest

import oracle
import synth
from synth.configs import CONFIGS, expert_weights, fp8_weights, make_inputs, mxfp4_weights

from moe_cases import as_f64, assert_routing_equal, dev, host, rel_err, shape_of

pytestmark = [pytest.mark.gpu, pytest.mark.full]


@pytest.fixture(scope="module")
def weights():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_moe_layer_04_amd  # noqa: F401
    cfg = CONFIGS["prefill_t8192"]
    t0 = time.time()
    hw = expert_weights(cfg)
    t1 = time.time()
    dw = tuple(dev(a) for a in hw)
    torch.cuda.synchronize()
    print("\nweights: generated in %.1fs, uploaded in %.1fs" % (t1 - t0, time.time() - t1), flush=True)
    yield hw, dw
    del dw
    torch.cuda.empty_cache()


@pytest.fixture(scope="module")
def weights_mxfp4(weights):
    """The same weights in 4-bit storage (E2M1 codes two per byte + E8M0 block scales)."""
    import torch
    hw, _ = weights
    t0 = time.time()
    hq, scales = mxfp4_weights(hw)
    dq = tuple(dev(a) for a in hq)
    ds = tuple(dev(a) for a in scales)
    torch.cuda.synchronize()
    print("\nmxfp4 weights: quantized and uploaded in %.1fs" % (time.time() - t0), flush=True)
    yield hq, scales, dq, ds
    del dq, ds
    torch.cuda.empty_cache()


@pytest.fixture(scope="module")
def weights_fp8(weights):
    """The same weights in 8-bit storage (E4M3 codes + E8M0 block scales)."""
    import torch
    hw, _ = weights
    t0 = time.time()
    hq, scales = fp8_weights(hw)
    dq = tuple(dev(a) for a in hq)
    ds = tuple(dev(a) for a in scales)
    torch.cuda.synchronize()
    print("\nfp8 weights: quantized and uploaded in %.1fs" % (time.time() - t0), flush=True)
    yield hq, scales, dq, ds
    del dq, ds
    torch.cuda.empty_cache()


def _sample(cfg, idx, extra_cap=512):
    T = cfg.T
    if T <= 512:
        return np.arange(T)
    base = synth.subset(cfg.seed_base + 777, 99, T, 256)
    off, srt, _ = oracle.permutation(idx, cfg.E)
    ends = []
    for e in range(cfg.E):
        if off[e + 1] > off[e]:
            ends += [srt[off[e]] // cfg.top_k, srt[off[e + 1] - 1] // cfg.top_k]
    ends = np.unique(np.array(ends, dtype=np.int64))
    if ends.size > extra_cap:
        ends = ends[synth.subset(cfg.seed_base + 778, 99, ends.size, extra_cap)]
    return np.union1d(base, ends)


@pytest.mark.parametrize("name", ["decode_t64", "serve_t256", "serve_t1024", "skew_t6000", "prefill_t8192",
                                  "sublayer_t32768", "decode_t64_fp8", "prefill_t8192_fp8", "decode_t64_mxfp4",
                                  "prefill_t8192_mxfp4", "serve_t512_fp8", "serve_t512_mxfp4"])
def test_full_shape_layer(name, request):
    import torch
    import sparse_moe_layer_04_amd as bm
    cfg = CONFIGS[name]
    if cfg.weights != "bf16":
        hw, w_scales, dw, d_scales = request.getfixturevalue("weights_" + cfg.weights)
    else:
        hw, dw = request.getfixturevalue("weights")
        w_scales = d_scales = None
    inp = make_inputs(cfg, weights=hw, w_scales=w_scales)
    print("\n[%s] x-seed %d" % (name, inp.x_seed), flush=True)
    t0 = time.time()
    u = oracle.rmsnorm_pinned(inp.x, inp.pre_gain, cfg.eps) if cfg.sublayer else inp.x
    r = oracle.route(u, inp.w_router, inp.bias, cfg.n_group, cfg.topk_group, cfg.top_k, cfg.rho)
    assert r.min_margin() >= 1e-6 and r.agree.min() == 1
    print("[%s] oracle routing of %d tokens: %.1fs, min margin %.2e" % (name, cfg.T, time.time() - t0,
                                                                       r.min_margin()), flush=True)

    shape = shape_of(cfg)
    op = bm.OP_FORWARD_SUBLAYER if cfg.sublayer else bm.OP_FORWARD
    ws = torch.empty(bm.workspace_size(shape, op), dtype=torch.uint8, device="cuda")
    x = dev(inp.x)
    out = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device="cuda")
    idx = torch.empty((cfg.T, cfg.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((cfg.T, cfg.top_k), dtype=torch.float32, device="cuda")
    moe_y = torch.empty_like(out) if cfg.sublayer else None
    sub = None
    if cfg.sublayer:
        g1, g2 = dev(inp.pre_gain), dev(inp.post_gain)
        sub = bm.sublayer(g1, g2, cfg.eps, cfg.residual_k)
    bm.forward(shape, x, dw[0], dev(inp.bias), dw[1], dw[2], dw[3], out, ws, sublayer=sub, topk_idx=idx, topk_w=w,
               moe_y=moe_y, w_scales=d_scales, w_format=cfg.code_format or "e4m3")
    torch.cuda.synchronize()
    g_idx, g_w = host(idx), host(w)
    assert_routing_equal(g_idx, g_w, r.idx, r.w, cfg.rho)
    counts = np.bincount(r.idx.reshape(-1), minlength=cfg.E)
    print("[%s] routing bit-exact on all %d tokens; experts touched %d, max load %d, empty %d" % (
        name, cfg.T, (counts > 0).sum(), counts.max(), (counts == 0).sum()), flush=True)

    tok = _sample(cfg, r.idx)
    t0 = time.time()
    y = oracle.experts(u, inp.w_gate, inp.w_up, inp.w_down, r.idx, r.w, tok, w_scales=inp.w_scales)
    ref = oracle.post_residual(y, np.ascontiguousarray(inp.x[tok]), inp.post_gain, cfg.eps, cfg.residual_k) \
        if cfg.sublayer else y
    print("[%s] oracle experts on %d tokens: %.1fs" % (name, tok.size, time.time() - t0), flush=True)
    got = as_f64(host(out)[tok])
    err = rel_err(got, ref)
    print("[%s] max|out - ref| / max|ref| = %.3e" % (name, err), flush=True)
    assert err <= 1e-2
    if cfg.sublayer:
        erry = rel_err(as_f64(host(moe_y)[tok]), y)
        print("[%s] moe_y rel err %.3e" % (name, erry), flush=True)
        assert erry <= 1e-2
