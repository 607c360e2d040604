"""The five Beam MoE workloads and their seeded input recipes.

Shapes and routing constants come from the Beam pages: hidden 5120, 256 experts in 8
groups of 32 with the best 4 groups kept, top-8, routed scaling 2.5, SwiGLU experts of
intermediate size 2560 (Glonce, "Reflection releases Beam, a 501B open MoE model with
1M context", architecture paragraphs; transformers "Beam" model doc, Overview, "Sparse
MoE").  Value distributions are the synthetic workload recipes (no trained weights exist
here).  Normal "N(0, 1/H)" means variance 1/H; "N(0, 0.02)" means standard deviation
0.02.

Seeds: config 0 uses seed 0 throughout.  Configs 1-4 share one weight set (seed 1000:
router W and the expert weights); each draws its activations and per-config tensors from
seed ``1000*c + j``, where ``j`` is the first index whose inputs have no routing near-tie
(every fp64 margin >= 1e-6); the chosen ``j`` values are stored in
``tests/golden/seeds.json`` by ``tests/golden/make_seeds.py``.
"""
from __future__ import annotations

import dataclasses
import json
import math
import os
from typing import Optional

import numpy as np

# tensor ids inside a seed's stream family
TID_X, TID_WR, TID_BIAS, TID_WG, TID_WU, TID_WD, TID_G1, TID_G2, TID_RANK = range(1, 10)
WEIGHT_SEED = 1000

_SEEDS_JSON = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "tests", "golden",
                           "seeds.json")


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    T: int
    H: int
    E: int
    I: int
    n_group: int
    topk_group: int
    top_k: int
    rho: float = 2.5
    dtype: str = "bf16"          # activations and expert weights: "bf16" or "f32"
    x_std: float = 1.0
    wr_std: Optional[float] = None   # default sqrt(1/H)
    bias: str = "zero"           # "zero" | "uniform:<a>" (U(-a, a)) | "zipf:<c>" (-c*ln(rank))
    w_std: Optional[float] = None    # gate/up std; default sqrt(1/H)
    wd_std: Optional[float] = None   # down std; default sqrt(1/I)
    sublayer: bool = False       # pre-RMSNorm + post-RMSNorm + depth-scaled residual
    residual_k: int = 40
    eps: float = 1e-6
    gain_std: float = 0.02
    seed_base: int = 0           # x-seed = seed_base + j
    weight_seed: Optional[int] = None  # None: same seed as x (config 0)
    weights: str = "bf16"        # expert weight storage: "bf16", "fp8" (E4M3 codes + E8M0 block
                                 # scales from the bf16 draw, see synth.quantize_e4m3) or "mxfp4"
                                 # (E2M1 codes two per byte + E8M0 block scales, synth.quantize_e2m1)

    @property
    def P(self) -> int:
        return self.T * self.top_k

    @property
    def code_format(self) -> Optional[str]:
        """The weight code format of a quantized config ("e4m3", "e2m1"), else None."""
        return {"fp8": "e4m3", "mxfp4": "e2m1"}.get(self.weights)

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


_BEAM = dict(H=5120, E=256, I=2560, n_group=8, topk_group=4, top_k=8, rho=2.5, dtype="bf16",
             wr_std=math.sqrt(1.0 / 5120), w_std=0.02, wd_std=0.02, weight_seed=WEIGHT_SEED)

CONFIGS = {
    "tiny_f32": Config("tiny_f32", T=32, H=64, E=16, I=32, n_group=4, topk_group=2, top_k=4, dtype="f32",
                       bias="uniform:0.1", seed_base=0, weight_seed=None),
    "decode_t64": Config("decode_t64", T=64, bias="uniform:0.05", seed_base=1000, **_BEAM),
    "prefill_t8192": Config("prefill_t8192", T=8192, bias="zero", seed_base=2000, **_BEAM),
    "skew_t6000": Config("skew_t6000", T=6000, bias="zipf:0.6", seed_base=3000, **_BEAM),
    "sublayer_t32768": Config("sublayer_t32768", T=32768, bias="zero", sublayer=True, residual_k=40,
                              seed_base=4000, **_BEAM),
    # serving shapes between decode and prefill (the decode inputs at more tokens): 8 and 32
    # routed rows per expert on average
    "serve_t256": Config("serve_t256", T=256, bias="uniform:0.05", seed_base=5000, **_BEAM),
    "serve_t1024": Config("serve_t1024", T=1024, bias="uniform:0.05", seed_base=6000, **_BEAM),
    # the decode and prefill workloads with 8-bit expert weights (E4M3 codes + E8M0 scales per
    # 32 elements, quantized from the same bf16 draw)
    "decode_t64_fp8": Config("decode_t64_fp8", T=64, bias="uniform:0.05", seed_base=1000, weights="fp8", **_BEAM),
    "prefill_t8192_fp8": Config("prefill_t8192_fp8", T=8192, bias="zero", seed_base=2000, weights="fp8", **_BEAM),
    # ... and with 4-bit expert weights (MXFP4: E2M1 codes + E8M0 scales per 32 elements)
    "decode_t64_mxfp4": Config("decode_t64_mxfp4", T=64, bias="uniform:0.05", seed_base=1000, weights="mxfp4",
                               **_BEAM),
    "prefill_t8192_mxfp4": Config("prefill_t8192_mxfp4", T=8192, bias="zero", seed_base=2000, weights="mxfp4",
                                  **_BEAM),
    # serving shape with quantized weights: 16 rows per expert, below their kernel switch
    "serve_t512_fp8": Config("serve_t512_fp8", T=512, bias="uniform:0.05", seed_base=7000, weights="fp8", **_BEAM),
    "serve_t512_mxfp4": Config("serve_t512_mxfp4", T=512, bias="uniform:0.05", seed_base=7000, weights="mxfp4",
                               **_BEAM),
}
CONFIG_ORDER = ["tiny_f32", "decode_t64", "prefill_t8192", "skew_t6000", "sublayer_t32768", "serve_t256",
                "serve_t1024", "decode_t64_fp8", "prefill_t8192_fp8", "decode_t64_mxfp4", "prefill_t8192_mxfp4",
                "serve_t512_fp8", "serve_t512_mxfp4"]


def seed_index(name: str) -> int:
    """The near-tie-free seed offset j recorded for a named config (0 if not recorded)."""
    try:
        with open(_SEEDS_JSON) as f:
            return int(json.load(f)["seed_index"].get(name, 0))
    except (OSError, KeyError, ValueError):
        return 0


@dataclasses.dataclass
class MoEInputs:
    cfg: Config
    x_seed: int
    x: np.ndarray            # [T,H] uint16 (bf16) or float32
    w_router: np.ndarray     # [E,H] float32
    bias: np.ndarray         # [E] float32
    w_gate: np.ndarray       # [E,I,H]
    w_up: np.ndarray         # [E,I,H]
    w_down: np.ndarray       # [E,H,I]
    pre_gain: Optional[np.ndarray] = None   # [H] float32
    post_gain: Optional[np.ndarray] = None  # [H] float32
    w_scales: Optional[tuple] = None        # fp8 / mxfp4 weights: E8M0 scales of (w_gate, w_up, w_down)


def _act(cfg: Config, seed: int, tid: int, shape, std: float, mean: float = 0.0):
    from . import normal_bf16, normal_f32
    if cfg.dtype == "bf16":
        return normal_bf16(seed, tid, shape, mean, std)
    return normal_f32(seed, tid, shape, mean, std)


def fp8_weights(weights):
    """(w_router, w_gate, w_up, w_down) with bf16 experts -> the same tuple with E4M3 expert
    codes, and the (s_gate, s_up, s_down) E8M0 block scales."""
    from . import quantize_e4m3
    wr, wg, wu, wd = weights
    (cg, sg), (cu, su), (cd, sd) = quantize_e4m3(wg), quantize_e4m3(wu), quantize_e4m3(wd)
    return (wr, cg, cu, cd), (sg, su, sd)


def mxfp4_weights(weights):
    """(w_router, w_gate, w_up, w_down) with bf16 experts -> the same tuple with packed E2M1
    expert codes (last dimension halved), and the (s_gate, s_up, s_down) E8M0 block scales."""
    from . import quantize_e2m1
    wr, wg, wu, wd = weights
    (cg, sg), (cu, su), (cd, sd) = quantize_e2m1(wg), quantize_e2m1(wu), quantize_e2m1(wd)
    return (wr, cg, cu, cd), (sg, su, sd)


def quantized_weights(cfg: Config, weights):
    """The expert weights of a config in its storage format: (weights, scales or None)."""
    if cfg.weights == "fp8":
        return fp8_weights(weights)
    if cfg.weights == "mxfp4":
        return mxfp4_weights(weights)
    return weights, None


def expert_weights(cfg: Config, seed: Optional[int] = None):
    """(w_router, w_gate, w_up, w_down) of a config; w_router is always float32."""
    from . import normal_f32
    s = cfg.weight_seed if seed is None else seed
    wr_std = cfg.wr_std if cfg.wr_std is not None else math.sqrt(1.0 / cfg.H)
    w_std = cfg.w_std if cfg.w_std is not None else math.sqrt(1.0 / cfg.H)
    wd_std = cfg.wd_std if cfg.wd_std is not None else math.sqrt(1.0 / cfg.I)
    wr = normal_f32(s, TID_WR, (cfg.E, cfg.H), 0.0, wr_std)
    wg = _act(cfg, s, TID_WG, (cfg.E, cfg.I, cfg.H), w_std)
    wu = _act(cfg, s, TID_WU, (cfg.E, cfg.I, cfg.H), w_std)
    wd = _act(cfg, s, TID_WD, (cfg.E, cfg.H, cfg.I), wd_std)
    return wr, wg, wu, wd


def make_bias(cfg: Config, seed: int) -> np.ndarray:
    from . import permutation, uniform_f32
    kind = cfg.bias
    if kind == "zero":
        return np.zeros(cfg.E, dtype=np.float32)
    if kind.startswith("uniform:"):
        a = float(kind.split(":")[1])
        return uniform_f32(seed, TID_BIAS, (cfg.E,), -a, a)
    if kind.startswith("zipf:"):
        c = float(kind.split(":")[1])
        rank = permutation(seed, TID_RANK, cfg.E) + 1          # a seeded permutation of 1..E
        return np.array([c * math.log(1.0 / r) for r in rank], dtype=np.float32)
    raise ValueError(kind)


def make_inputs(cfg: Config, j: Optional[int] = None, weights=None, w_scales=None) -> MoEInputs:
    """All inputs of a config.  ``weights`` may pass a pre-generated (wr, wg, wu, wd) tuple
    (for an fp8 or mxfp4 config: the codes, with their ``w_scales``)."""
    from . import normal_f32
    if j is None:
        j = seed_index(cfg.name)
    xs = cfg.seed_base + j
    if weights is None:
        weights = expert_weights(cfg, seed=(xs if cfg.weight_seed is None else cfg.weight_seed))
        if cfg.weights != "bf16":
            weights, w_scales = quantized_weights(cfg, weights)
    wr, wg, wu, wd = weights
    x = _act(cfg, xs, TID_X, (cfg.T, cfg.H), cfg.x_std)
    bias = make_bias(cfg, xs)
    g1 = g2 = None
    if cfg.sublayer:
        g1 = normal_f32(xs, TID_G1, (cfg.H,), 1.0, cfg.gain_std)
        g2 = normal_f32(xs, TID_G2, (cfg.H,), 1.0, cfg.gain_std)
    return MoEInputs(cfg, xs, x, wr, bias, wg, wu, wd, g1, g2, w_scales)
