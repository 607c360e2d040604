"""Choose, for every workload, the first seed offset j whose inputs have no routing near-tie.

Rule: for config c try x-seed ``seed_base + j`` for j = 0, 1, ...; accept the first j for
which, on every token, the fp64 gap between the last kept and the first dropped group
score and the gap between the k-th and (k+1)-th biased expert score are both >= 1e-6, and
deciding on fp64 or on fp32 values gives the same routing.  Config 0 ("tiny_f32") is fixed
to seed 0 by its recipe; it is checked, not searched.

Calls only ``oracle`` and ``synth``.  Writes ``tests/golden/seeds.json``.
Run: ``python tests/golden/make_seeds.py``.
"""
import json
import math
import os
import sys
import time

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))

import oracle  # noqa: E402
import synth  # noqa: E402
from synth.configs import CONFIG_ORDER, CONFIGS, TID_WR, expert_weights, make_inputs  # noqa: E402

MARGIN = 1e-6
OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "seeds.json")


def check(cfg, j, wr):
    inp = make_inputs(cfg, j=j, weights=(wr, None, None, None))
    u = oracle.rmsnorm_pinned(inp.x, inp.pre_gain, cfg.eps) if cfg.sublayer else inp.x
    r = oracle.route(u, inp.w_router, inp.bias, cfg.n_group, cfg.topk_group, cfg.top_k, cfg.rho)
    return r.min_margin(), int(r.agree.min())


def main():
    res = {"rule": "first j with every fp64 routing margin >= %g and fp32/fp64 decisions equal" % MARGIN,
           "seed_index": {}, "min_margin": {}, "tries": {}}
    for name in CONFIG_ORDER:
        cfg = CONFIGS[name]
        t0 = time.time()
        wr = None
        j = 0
        while True:
            if cfg.weight_seed is None:          # config 0: every tensor from the one seed
                wr = expert_weights(cfg, seed=cfg.seed_base + j)[0]
            elif wr is None:                     # shared weight set: only the router matrix matters
                wr = synth.normal_f32(cfg.weight_seed, TID_WR, (cfg.E, cfg.H), 0.0,
                                      cfg.wr_std or math.sqrt(1.0 / cfg.H))
            m, agree = check(cfg, j, wr)
            print("%-16s j=%d min_margin=%.3e agree=%d (%.1fs)" % (name, j, m, agree, time.time() - t0), flush=True)
            if m >= MARGIN and agree:
                break
            if cfg.weight_seed is None:
                raise SystemExit("seed 0 of %s has a near-tie; its recipe fixes seed 0" % name)
            j += 1
        res["seed_index"][name] = j
        res["min_margin"][name] = m
        res["tries"][name] = j + 1
    with open(OUT, "w") as f:
        json.dump(res, f, indent=1)
        f.write("\n")
    print("wrote", OUT)


if __name__ == "__main__":
    main()
