"""Shared helpers of the GPU parity tests: device upload, one library call per stage, and
the comparison rules against the CPU oracle."""
from __future__ import annotations

import math

import numpy as np

import oracle
import synth
from synth.configs import CONFIGS, Config, make_inputs


def torch_mod():
    import torch
    return torch


def dev(a: np.ndarray):
    torch = torch_mod()
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t) -> np.ndarray:
    torch = torch_mod()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def as_f64(a: np.ndarray) -> np.ndarray:
    return synth.bf16_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)


def shape_of(cfg: Config, T=None):
    import sparse_moe_layer_04_amd as bm
    return bm.make_shape(cfg.T if T is None else T, cfg.H, cfg.E, cfg.I, cfg.n_group, cfg.topk_group, cfg.top_k,
                         cfg.rho, cfg.dtype)


class DeviceInputs:
    def __init__(self, inp):
        self.inp = inp
        self.x = dev(inp.x)
        self.wr = dev(inp.w_router)
        self.bias = dev(inp.bias)
        self.wg = dev(inp.w_gate)
        self.wu = dev(inp.w_up)
        self.wd = dev(inp.w_down)
        self.g1 = dev(inp.pre_gain) if inp.pre_gain is not None else None
        self.g2 = dev(inp.post_gain) if inp.post_gain is not None else None
        self.w_scales = tuple(dev(a) for a in inp.w_scales) if inp.w_scales is not None else None


def run_forward(cfg: Config, d: DeviceInputs, timer=None):
    """One beam_moe_forward call; returns numpy out, idx, w, moe_y (moe_y only with sublayer)."""
    import sparse_moe_layer_04_amd as bm
    torch = torch_mod()
    shape = shape_of(cfg)
    op = bm.OP_FORWARD_SUBLAYER if cfg.sublayer else bm.OP_FORWARD
    ws = torch.empty(max(bm.workspace_size(shape, op), 1), dtype=torch.uint8, device="cuda")
    act_dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    out = torch.empty((cfg.T, cfg.H), dtype=act_dt, device="cuda")
    idx = torch.empty((cfg.T, cfg.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((cfg.T, cfg.top_k), dtype=torch.float32, device="cuda")
    moe_y = torch.empty((cfg.T, cfg.H), dtype=act_dt, device="cuda") if cfg.sublayer else None
    sub = bm.sublayer(d.g1, d.g2, cfg.eps, cfg.residual_k) if cfg.sublayer else None
    bm.forward(shape, d.x, d.wr, d.bias, d.wg, d.wu, d.wd, out, ws, sublayer=sub, topk_idx=idx, topk_w=w,
               moe_y=moe_y, stage_events=timer.events if timer else None, w_scales=d.w_scales,
               w_format=cfg.code_format or "e4m3")
    torch.cuda.synchronize()
    return dict(out=host(out), idx=host(idx), w=host(w), moe_y=host(moe_y) if moe_y is not None else None)


def tie_free_inputs(cfg: Config, max_tries=40, margin=1e-6):
    """Inputs of cfg for the first seed offset whose routing has no near-tie (checked by the oracle)."""
    for j in range(max_tries):
        inp = make_inputs(cfg, j=j)
        u = oracle.rmsnorm_pinned(inp.x, inp.pre_gain, cfg.eps) if cfg.sublayer else inp.x
        r = oracle.route(u, inp.w_router, inp.bias, cfg.n_group, cfg.topk_group, cfg.top_k, cfg.rho)
        if r.min_margin() >= margin and r.agree.min() == 1:
            return inp
    raise RuntimeError("no tie-free seed for %s" % cfg.name)


def assert_routing_equal(gpu_idx, gpu_w, ref_idx, ref_w, rho):
    """Chosen sets bit-exact per token; weights matched per expert id (fp32 vs fp64)."""
    gi = np.sort(gpu_idx, axis=1)
    ri = np.sort(ref_idx, axis=1)
    bad = np.nonzero((gi != ri).any(axis=1))[0]
    assert bad.size == 0, "routing differs on %d tokens, first %s: gpu %s ref %s" % (
        bad.size, bad[:5], gpu_idx[bad[0]], ref_idx[bad[0]])
    go = np.argsort(gpu_idx, axis=1)
    ro = np.argsort(ref_idx, axis=1)
    gw = np.take_along_axis(gpu_w.astype(np.float64), go, axis=1)
    rw = np.take_along_axis(ref_w, ro, axis=1)
    err = np.abs(gw - rw).max() if gw.size else 0.0
    assert err <= 4e-6 * rho, "routing weight error %g" % err
    return err


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max|got - ref| / max|ref|."""
    scale = np.abs(ref).max()
    return float(np.abs(got - ref).max() / (scale if scale > 0 else 1.0))


# small bf16 shapes that the oracle finishes in seconds; each spans several tiles and a ragged tail
def mid_config(name, T, **kw) -> Config:
    base = dict(H=512, E=64, I=256, n_group=8, topk_group=4, top_k=8, rho=2.5, dtype="bf16",
                wr_std=math.sqrt(1.0 / 512), w_std=0.05, wd_std=0.05, bias="uniform:0.05", seed_base=10000,
                weight_seed=None)
    base.update(kw)
    return Config(name, T=T, **base)


MID_CASES = {
    "mid_prefill_t1000": mid_config("mid_prefill_t1000", 1000),          # ~125 rows per expert
    "mid_ragged_t300": mid_config("mid_ragged_t300", 300, seed_base=11000),  # ~37 rows per expert
    "mid_decode_t24": mid_config("mid_decode_t24", 24, seed_base=12000),   # ~3 rows per expert
    "mid_t1": mid_config("mid_t1", 1, seed_base=13000),
    "mid_skew_t700": mid_config("mid_skew_t700", 700, bias="zipf:0.6", seed_base=14000),
    "mid_sublayer_t333": mid_config("mid_sublayer_t333", 333, bias="zero", sublayer=True, seed_base=15000),
    "mid_dense_t2503": mid_config("mid_dense_t2503", 2503, seed_base=17000),  # ~313 rows per expert: 320-row tiles
    # (20 row blocks) and split ones;
    # T >= 1024 and not a multiple of 4: the selection's last 4-token work-group is partial
    # the largest routing shape the ABI takes: E = 1024 experts in 64 groups, top-32
    "mid_maxshape_t200": mid_config("mid_maxshape_t200", 200, H=256, E=1024, I=128, n_group=64, topk_group=8,
                                    top_k=32, wr_std=math.sqrt(1.0 / 256), seed_base=18000),
    # 10 rows per expert: just above the kernel switch, the line kernel's smallest tiles
    "mid_serve_t80": mid_config("mid_serve_t80", 80, seed_base=19000),
    # 6 rows per expert on average but skewed: the decode kernel with tiles of up to T rows
    "mid_skew_decode_t48": mid_config("mid_skew_decode_t48", 48, bias="zipf:0.6", seed_base=20000),
    # 8-bit expert weights (E4M3 + E8M0 block scales): the line kernel, the decode kernel's
    # 64-k stream (gate/up, K = 512) and 32-k steps (down, K = 256), and its large-tile loop
    "mid_fp8_prefill_t1000": mid_config("mid_fp8_prefill_t1000", 1000, weights="fp8", seed_base=21000),
    # expert counts that are not a multiple of 8, with more than one chunk of pairs: the work
    # list dealt to the 8 XCD runs ends in a partial round (60 experts: 7 full rounds, the
    # last dealt backwards; 20 experts: 2 full rounds, the last dealt forwards); 27-60 rows
    # per expert on the line kernel, and 47 rows per expert with 8-bit weights
    "mid_e60_t400": mid_config("mid_e60_t400", 400, E=60, n_group=4, topk_group=2, top_k=4, seed_base=53000),
    "mid_e20_t300": mid_config("mid_e20_t300", 300, E=20, n_group=4, topk_group=2, top_k=4, seed_base=54000),
    "mid_fp8_e60_t700": mid_config("mid_fp8_e60_t700", 700, E=60, n_group=4, topk_group=2, top_k=4,
                                   weights="fp8", seed_base=55000),
    # ~313 rows per expert with 8-bit weights: the line kernel's 320-row tiles (20 row blocks)
    # and experts above 320 rows split in two
    "mid_fp8_dense_t2503": mid_config("mid_fp8_dense_t2503", 2503, weights="fp8", seed_base=52000),
    "mid_fp8_decode_t24": mid_config("mid_fp8_decode_t24", 24, weights="fp8", seed_base=22000),
    # one token with quantized weights: eight tiles of one row (the small-tile decode kernel for
    # gate/up at K = 512, 32-k steps for down at K = 256)
    "mid_fp8_t1": mid_config("mid_fp8_t1", 1, weights="fp8", seed_base=50000),
    "mid_mxfp4_t1": mid_config("mid_mxfp4_t1", 1, weights="mxfp4", seed_base=51000),
    "mid_fp8_skew_decode_t48": mid_config("mid_fp8_skew_decode_t48", 48, bias="zipf:0.6", weights="fp8",
                                          seed_base=23000),
    "mid_fp8_sublayer_t333": mid_config("mid_fp8_sublayer_t333", 333, sublayer=True, residual_k=40,
                                        weights="fp8", seed_base=24000),
    # K = 2560 and 1536 (5 and 3 activation chunks of 512): the decode kernel's streaming
    # loop over several chunks, and with 8-bit weights its scale groups of four chunks
    # (the second group partial)
    "mid_decode_h2560_t12": mid_config("mid_decode_h2560_t12", 12, H=2560, I=1536, E=16, n_group=4, topk_group=2,
                                       top_k=4, wr_std=math.sqrt(1.0 / 2560), seed_base=25000),
    "mid_fp8_decode_h2560_t12": mid_config("mid_fp8_decode_h2560_t12", 12, H=2560, I=1536, E=16, n_group=4,
                                           topk_group=2, top_k=4, weights="fp8", wr_std=math.sqrt(1.0 / 2560),
                                           seed_base=26000),
    # 4-bit expert weights (MXFP4: E2M1 codes two per byte + E8M0 block scales): the line
    # kernel's 8-byte loads, the decode kernel's 256-k stream steps (gate/up, one chunk at
    # K = 512, five at K = 2560), its 32-k steps (down, K = 256) and its large-tile loop
    "mid_mxfp4_prefill_t1000": mid_config("mid_mxfp4_prefill_t1000", 1000, weights="mxfp4", seed_base=27000),
    "mid_mxfp4_decode_t24": mid_config("mid_mxfp4_decode_t24", 24, weights="mxfp4", seed_base=28000),
    "mid_mxfp4_skew_decode_t48": mid_config("mid_mxfp4_skew_decode_t48", 48, bias="zipf:0.6", weights="mxfp4",
                                            seed_base=29000),
    "mid_mxfp4_sublayer_t333": mid_config("mid_mxfp4_sublayer_t333", 333, sublayer=True, residual_k=40,
                                          weights="mxfp4", seed_base=30000),
    "mid_mxfp4_decode_h2560_t12": mid_config("mid_mxfp4_decode_h2560_t12", 12, H=2560, I=1536, E=16, n_group=4,
                                             topk_group=2, top_k=4, weights="mxfp4", wr_std=math.sqrt(1.0 / 2560),
                                             seed_base=31000),
    # 17-32 rows in some experts: the streaming loop's 32-row tiles (256-column activation
    # chunks; with quantized weights, chunks of 8 scale bytes per row), at K = 512 / 256 and,
    # with several chunks, at K = 2560 / 1536
    "mid_mxfp4_skew_decode_t32": mid_config("mid_mxfp4_skew_decode_t32", 32, bias="zipf:0.6", weights="mxfp4",
                                            seed_base=32000),
    "mid_fp8_skew_h2560_t28": mid_config("mid_fp8_skew_h2560_t28", 28, H=2560, I=1536, E=16, n_group=4,
                                         topk_group=2, top_k=4, bias="zipf:0.6", weights="fp8",
                                         wr_std=math.sqrt(1.0 / 2560), seed_base=34000),
    "mid_mxfp4_skew_h2560_t28": mid_config("mid_mxfp4_skew_h2560_t28", 28, H=2560, I=1536, E=16, n_group=4,
                                           topk_group=2, top_k=4, bias="zipf:0.6", weights="mxfp4",
                                           wr_std=math.sqrt(1.0 / 2560), seed_base=34000),
    # 8-bit and 4-bit weights at 20 rows per expert: below the quantized formats' kernel
    # switch (24), so the decode kernel with tiles of every size
    "mid_fp8_serve_t160": mid_config("mid_fp8_serve_t160", 160, weights="fp8", seed_base=35000),
    "mid_mxfp4_serve_t160": mid_config("mid_mxfp4_serve_t160", 160, weights="mxfp4", seed_base=36000),
    # 8-bit weights at 32 rows per expert (below their switch at 40): the stream's 64-row
    # tiles (128-column chunks, 4 scale bytes per row and chunk)
    "mid_fp8_serve_t256": mid_config("mid_fp8_serve_t256", 256, weights="fp8", seed_base=37000),
    # ... and 4-bit weights there (below their switch at 44): the 64-row tiles' half-line steps
    "mid_mxfp4_serve_t256": mid_config("mid_mxfp4_serve_t256", 256, weights="mxfp4", seed_base=39000),
    # 256 experts at 6 rows per expert, skewed: tiles of up to 200 rows on the decode kernel
    # (its 32-k loop for tiles above 64 rows, the stream below), in all three formats
    "mid_skew_e256_t200": mid_config("mid_skew_e256_t200", 200, E=256, bias="zipf:0.6", seed_base=38000),
    "mid_fp8_skew_e256_t200": mid_config("mid_fp8_skew_e256_t200", 200, E=256, bias="zipf:0.6", weights="fp8",
                                         seed_base=38000),
    "mid_mxfp4_skew_e256_t200": mid_config("mid_mxfp4_skew_e256_t200", 200, E=256, bias="zipf:0.6",
                                           weights="mxfp4", seed_base=38000),
    "mid_h1024_t257": mid_config("mid_h1024_t257", 257, H=1024, I=384, E=32, n_group=4, topk_group=2, top_k=6,
                                 wr_std=math.sqrt(1.0 / 1024), seed_base=16000),
    # many decode work items (1400-1500 gate/up and 700-750 down: ~93 touched experts of
    # 128, 16 and 8 column blocks), more than two work-groups per CU hold at once; the mild
    # skew puts tiles of 1, 2 and up to 4 row blocks (and in the bf16 case one larger tile)
    # among them; K = 1024 gives the 16-row stream two activation chunks; all three formats
    "mid_items_e128_t96": mid_config("mid_items_e128_t96", 96, H=1024, I=1024, E=128, bias="zipf:0.12",
                                     wr_std=math.sqrt(1.0 / 1024), seed_base=42000),
    "mid_fp8_items_e128_t96": mid_config("mid_fp8_items_e128_t96", 96, H=1024, I=1024, E=128, bias="zipf:0.12",
                                         weights="fp8", wr_std=math.sqrt(1.0 / 1024), seed_base=43000),
    "mid_mxfp4_items_e128_t96": mid_config("mid_mxfp4_items_e128_t96", 96, H=1024, I=1024, E=128, bias="zipf:0.12",
                                           weights="mxfp4", wr_std=math.sqrt(1.0 / 1024), seed_base=44000),
    # at most 64 tokens with weight rows of at most 1280 bytes (8-bit and 4-bit at K = 1024):
    # the decode kernel's small-tile variant (three work-groups per CU) for gate/up and down,
    # the skew giving tiles of 1, 2 and up to 4 row blocks
    "mid_fp8_skew_h1024_t64": mid_config("mid_fp8_skew_h1024_t64", 64, H=1024, I=1024, E=32, n_group=4,
                                         topk_group=2, bias="zipf:0.6", weights="fp8",
                                         wr_std=math.sqrt(1.0 / 1024), seed_base=48000),
    "mid_mxfp4_skew_h1024_t64": mid_config("mid_mxfp4_skew_h1024_t64", 64, H=1024, I=1024, E=32, n_group=4,
                                           topk_group=2, bias="zipf:0.6", weights="mxfp4",
                                           wr_std=math.sqrt(1.0 / 1024), seed_base=49000),
    # the line kernel at K = 2560 (gate/up) and 1536 (down): 50 rows per expert, above every
    # format's switch (bf16 8, 8-bit 40, 4-bit 44), 12 and 10 column blocks, 40 and 24 steps
    "mid_line_h2560_t200": mid_config("mid_line_h2560_t200", 200, H=2560, I=1536, E=16, n_group=4, topk_group=2,
                                      top_k=4, wr_std=math.sqrt(1.0 / 2560), seed_base=45000),
    "mid_fp8_line_h2560_t200": mid_config("mid_fp8_line_h2560_t200", 200, H=2560, I=1536, E=16, n_group=4,
                                          topk_group=2, top_k=4, weights="fp8", wr_std=math.sqrt(1.0 / 2560),
                                          seed_base=46000),
    "mid_mxfp4_line_h2560_t200": mid_config("mid_mxfp4_line_h2560_t200", 200, H=2560, I=1536, E=16, n_group=4,
                                            topk_group=2, top_k=4, weights="mxfp4", wr_std=math.sqrt(1.0 / 2560),
                                            seed_base=47000),
}


def full_configs():
    return [CONFIGS[n] for n in ("decode_t64", "prefill_t8192", "skew_t6000", "sublayer_t32768")]
