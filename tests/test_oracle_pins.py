"""Pins of the CPU oracle against what the Beam pages and mathematics fix (no GPU).

Each test ties one oracle function to something other than itself:
  * hand-worked routing fixtures (tests/golden/route_*.json): sigmoid scoring,
    top-2 group score, contiguous groups, exclusion (not zeroing) of dropped
    groups, bias used for selection only, normalisation and the 2.5 scale;
  * brute-force enumeration of every (group subset, expert subset) at the tiny shape;
  * routing invariants on every token of the tiny and decode workloads;
  * closed forms of the SwiGLU expert (rank-one weights), identical experts
    (out = 2.5 * expert(u)), top-1 routing and dense routing;
  * RMSNorm: a hand-worked value, scale and gain laws, unit RMS, sign pattern;
  * the depth-scaled residual: the page's "sum divided by sqrt(k)" statement,
    the W_d = 0 and k = 1 cases;
  * the parameter counts the pages print (three H x I matrices per expert);
  * 8-bit expert weights: the E4M3 values the OCP FP8 format fixes (largest 448,
    smallest normal 2^-6, subnormals m * 2^-9, NaN code), exact round trips of
    representable blocks through the input quantizer, and the fp8 layer equal to the
    layer on the decoded weights.
Sources: Glonce "Reflection releases Beam, a 501B open MoE model with 1M context"
(architecture paragraphs); transformers "Beam" model doc (Overview bullets "Sparse MoE"
and "Sandwich norms with depth-scaled residuals", FP32 numerics paragraph).
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth
from synth.configs import CONFIGS, make_inputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _sig(x):
    return 1.0 / (1.0 + np.exp(-x))


# ----------------------------------------------------------------------------- routing

def _one_token_router(logit_col, H=4):
    """u = e_0 (exact in bf16 and fp32) and W_r[:,0] = logits: the logits are exactly W_r[:,0]."""
    E = len(logit_col)
    wr = np.zeros((E, H), np.float32)
    wr[:, 0] = logit_col
    u = np.zeros((1, H), np.float32)
    u[0, 0] = 1.0
    return u, wr


def test_route_known_scores_fixture():
    fx = _golden("route_known_scores.json")
    n = np.array(fx["score_numerators"], dtype=np.float64)
    u, wr = _one_token_router(np.log(n / (32.0 - n)).astype(np.float32))
    for act in (u, synth.f32_to_bf16(u)):
        r = oracle.route(act, wr, np.zeros(fx["E"], np.float32), fx["n_group"], fx["topk_group"], fx["top_k"],
                         fx["rho"])
        assert r.idx[0].tolist() == fx["expected_idx"]
        np.testing.assert_allclose(r.w[0], fx["expected_w"], rtol=2e-7)
        assert abs(r.w[0].sum() - fx["rho"]) < 1e-12
        # distance to the nearest tie: the scores are n/32 up to the fp32 rounding of the logits
        np.testing.assert_allclose(r.margin[0], fx["expected_margin"], rtol=0, atol=1e-6)
        assert r.agree[0] == 1


def _margins_by_definition(sb, n_group, topk_group, top_k):
    """fp64 distance to the nearest tie, from the biased scores sb [T,E]: the last kept group
    score minus the first dropped one, and the top_k-th biased score among the experts of the
    kept groups minus the next one (inf where nothing is dropped)."""
    T, E = sb.shape
    gsz = E // n_group
    out = np.full((T, 2), np.inf)
    for t in range(T):
        top2 = np.sort(sb[t].reshape(n_group, gsz), axis=1)[:, ::-1][:, :2].sum(1)
        order = np.argsort(-top2, kind="stable")
        if topk_group < n_group:
            out[t, 0] = top2[order[topk_group - 1]] - top2[order[topk_group]]
        cand = np.sort(np.concatenate([sb[t, g * gsz:(g + 1) * gsz] for g in order[:topk_group]]))[::-1]
        if cand.size > top_k:
            out[t, 1] = cand[top_k - 1] - cand[top_k]
    return out


@pytest.mark.parametrize("name,j", [("tiny_f32", 0), ("tiny_f32", 1), ("tiny_f32", 2), ("decode_t64", 0)])
def test_route_margins_match_their_definition(name, j):
    # the margins decide which seeds count as tie-free for every parity test: recompute them
    # from the oracle's fp64 logits with numpy sorts and compare
    cfg = CONFIGS[name]
    if cfg.H > 1024:   # the Beam router shape at a few tokens (routing does not read the experts)
        cfg = cfg.replace(T=8, I=16)
    inp = make_inputs(cfg, j=j)
    r = oracle.route(inp.x, inp.w_router, inp.bias, cfg.n_group, cfg.topk_group, cfg.top_k, cfg.rho,
                     want_logits=True)
    sb = _sig(r.logits) + inp.bias.astype(np.float64)[None, :]
    np.testing.assert_allclose(r.margin, _margins_by_definition(sb, cfg.n_group, cfg.topk_group, cfg.top_k),
                               rtol=0, atol=1e-12)
    assert (r.margin > 0).all()


def test_route_bias_dominated_fixture_and_masking():
    fx = _golden("route_bias_dominated.json")
    E = fx["E"]
    cfg = CONFIGS["tiny_f32"]
    inp = make_inputs(cfg, j=0)
    bias = np.array(fx["bias"], np.float32)
    for shift in (0.0, -100.0, 37.0):
        r = oracle.route(inp.x, inp.w_router, bias + np.float32(shift), fx["n_group"], fx["topk_group"],
                         fx["top_k"], fx["rho"], want_logits=True)
        assert (r.idx == np.array(fx["expected_idx"], np.int32)[None, :]).all(), shift
        # weights come from the unbiased sigmoid scores of the chosen experts
        s = _sig(r.logits)
        sel = np.take_along_axis(s, r.idx.astype(np.int64), axis=1)
        np.testing.assert_allclose(r.w, fx["rho"] * sel / sel.sum(1, keepdims=True), rtol=1e-12)
    assert E == cfg.E


def test_route_exact_ties_go_to_lower_index():
    # all logits equal: every score ties; the kept groups are the first ones, experts the lowest ids
    u, wr = _one_token_router(np.zeros(16, np.float32))
    r = oracle.route(u, wr, np.zeros(16, np.float32), 4, 2, 4, 2.5)
    assert r.idx[0].tolist() == [0, 1, 2, 3]
    np.testing.assert_allclose(r.w[0], [0.625] * 4, rtol=0, atol=0)


def _brute_force(sb, n_group, topk_group, top_k):
    """Lexicographic optimum over every group subset and every expert subset in it:
    maximise the summed group scores, then the summed biased scores."""
    E = sb.size
    gs = E // n_group
    gscore = [np.sort(sb[g * gs:(g + 1) * gs])[::-1][:2].sum() for g in range(n_group)]
    best = None
    for groups in itertools.combinations(range(n_group), topk_group):
        cand = [e for g in groups for e in range(g * gs, (g + 1) * gs)]
        for chosen in itertools.combinations(cand, top_k):
            key = (sum(gscore[g] for g in groups), sum(sb[e] for e in chosen))
            if best is None or key > best[0]:
                best = (key, set(groups), set(chosen))
    return best[1], best[2]


@pytest.mark.parametrize("seed_j", [0, 1, 2])
def test_route_brute_force_tiny(seed_j):
    cfg = CONFIGS["tiny_f32"]
    inp = make_inputs(cfg, j=seed_j)
    r = oracle.route(inp.x, inp.w_router, inp.bias, cfg.n_group, cfg.topk_group, cfg.top_k, cfg.rho,
                     want_logits=True)
    assert r.min_margin() > 1e-9
    sb = _sig(r.logits) + inp.bias.astype(np.float64)[None, :]
    gsz = cfg.E // cfg.n_group
    for t in range(cfg.T):
        groups, chosen = _brute_force(sb[t], cfg.n_group, cfg.topk_group, cfg.top_k)
        assert set(r.idx[t].tolist()) == chosen
        assert {e // gsz for e in chosen} <= groups


def _check_invariants(cfg, r, bias):
    T, K = r.idx.shape
    gsz = cfg.E // cfg.n_group
    s = _sig(r.logits)
    for t in range(T):
        ids = r.idx[t].astype(np.int64)
        assert len(set(ids.tolist())) == K
        assert ids.min() >= 0 and ids.max() < cfg.E
        assert len({int(e) // gsz for e in ids}) <= cfg.topk_group
        # pre-scale weights sum to 1; weights proportional to unbiased scores
        assert abs(r.w[t].sum() / cfg.rho - 1.0) < 1e-12
        np.testing.assert_allclose(r.w[t] / s[t, ids], cfg.rho / s[t, ids].sum(), rtol=1e-12)
        # no unchosen expert of a group that holds a chosen one has a larger biased score
        sb = s[t] + bias
        groups = {int(e) // gsz for e in ids}
        rest = [e for g in groups for e in range(g * gsz, (g + 1) * gsz) if e not in set(ids.tolist())]
        if rest:
            assert sb[rest].max() < sb[ids].min()
        # decision order is descending biased score
        assert (np.diff(sb[ids]) <= 0).all()


def test_route_invariants_tiny_and_decode():
    for name in ("tiny_f32", "decode_t64"):
        cfg = CONFIGS[name]
        wr = synth.normal_f32(cfg.weight_seed if cfg.weight_seed is not None else cfg.seed_base, 2, (cfg.E, cfg.H), 0.0,
                              cfg.wr_std or math.sqrt(1.0 / cfg.H))
        inp = make_inputs(cfg, weights=(wr, None, None, None))
        r = oracle.route(inp.x, inp.w_router, inp.bias, cfg.n_group, cfg.topk_group, cfg.top_k, cfg.rho,
                         want_logits=True)
        assert r.min_margin() >= 1e-6 and r.agree.min() == 1
        _check_invariants(cfg, r, inp.bias.astype(np.float64))


def test_route_logits_are_the_matrix_product():
    # basis-vector tokens read one column of W_r each (exact in fp64)
    cfg = CONFIGS["tiny_f32"]
    inp = make_inputs(cfg, j=0)
    u = np.eye(cfg.H, dtype=np.float32)[:8] * np.float32(2.0)
    r = oracle.route(u, inp.w_router, inp.bias, cfg.n_group, cfg.topk_group, cfg.top_k, want_logits=True)
    np.testing.assert_array_equal(r.logits, 2.0 * inp.w_router[:, :8].T.astype(np.float64))


def test_route_bias_shift_invariance_decode():
    cfg = CONFIGS["decode_t64"]
    wr = synth.normal_f32(cfg.weight_seed, 2, (cfg.E, cfg.H), 0.0, cfg.wr_std)
    inp = make_inputs(cfg, weights=(wr, None, None, None))
    a = oracle.route(inp.x, wr, inp.bias, cfg.n_group, cfg.topk_group, cfg.top_k)
    b = oracle.route(inp.x, wr, inp.bias + np.float32(0.25), cfg.n_group, cfg.topk_group, cfg.top_k)
    assert np.array_equal(np.sort(a.idx, 1), np.sort(b.idx, 1))
    np.testing.assert_allclose(a.w, b.w, rtol=1e-12)


def test_route_dense_special_case():
    # one group, keep it, choose every expert: weights are rho * s / sum(s) over all experts
    cfg = CONFIGS["tiny_f32"]
    inp = make_inputs(cfg, j=0)
    r = oracle.route(inp.x, inp.w_router, inp.bias, 1, 1, cfg.E, cfg.rho, want_logits=True)
    s = _sig(r.logits)
    dense = cfg.rho * s / s.sum(1, keepdims=True)
    got = np.zeros_like(dense)
    np.put_along_axis(got, r.idx.astype(np.int64), r.w, axis=1)
    np.testing.assert_allclose(got, dense, rtol=1e-12)


def test_route_rejects_bad_shapes():
    u = np.zeros((1, 4), np.float32)
    wr = np.zeros((16, 4), np.float32)
    b = np.zeros(16, np.float32)
    for ng, tg, k in ((5, 2, 4), (4, 5, 4), (4, 2, 9), (4, 0, 1)):
        with pytest.raises(ValueError):
            oracle.route(u, wr, b, ng, tg, k)


# ----------------------------------------------------------------------------- experts

def _rank_one_expert(H, I, seed):
    rng = np.random.default_rng(seed)
    p, r, s = rng.normal(size=I), rng.normal(size=I), rng.normal(size=I)
    q, q2, v = rng.normal(size=H), rng.normal(size=H), rng.normal(size=H)
    wg = np.outer(p, q).astype(np.float32)
    wu = np.outer(r, q2).astype(np.float32)
    wd = np.outer(v, s).astype(np.float32)
    return wg, wu, wd


def _rank_one_value(wg, wu, wd, u):
    """Closed form of W_d (silu(W_g u) * (W_u u)) for rank-one W = a b^T, from the factors."""
    # recover factors exactly as stored: a_i b_h with the first nonzero row/column
    p, q = wg[:, 0].astype(np.float64), wg[0, :].astype(np.float64) / wg[0, 0]
    r, q2 = wu[:, 0].astype(np.float64), wu[0, :].astype(np.float64) / wu[0, 0]
    v, s = wd[:, 0].astype(np.float64), wd[0, :].astype(np.float64) / wd[0, 0]
    alpha, beta = float(q @ u), float(q2 @ u)
    a = p * alpha
    c = r * beta
    return v * float(np.sum(s * (a / (1.0 + np.exp(-a))) * c))


def test_experts_rank_one_closed_form_identical_experts():
    H, I, E = 12, 5, 4
    wg1, wu1, wd1 = _rank_one_expert(H, I, 7)
    wg, wu, wd = (np.repeat(a[None], E, 0).copy() for a in (wg1, wu1, wd1))
    rng = np.random.default_rng(3)
    u = rng.normal(size=(6, H)).astype(np.float32)
    br = rng.normal(size=(E, H)).astype(np.float32)
    r = oracle.route(u, br, np.zeros(E, np.float32), 2, 1, 2, 2.5)
    y = oracle.experts(u, wg, wu, wd, r.idx, r.w)
    for t in range(u.shape[0]):
        ref = 2.5 * _rank_one_value(wg1, wu1, wd1, u[t].astype(np.float64))
        np.testing.assert_allclose(y[t], ref, rtol=1e-5, atol=1e-9 * np.abs(ref).max())


def test_experts_gate_and_up_are_not_interchangeable():
    H, I = 12, 5
    wg, wu, wd = _rank_one_expert(H, I, 11)
    u = np.random.default_rng(5).normal(size=(1, H)).astype(np.float32)
    one = np.zeros((1, 1), np.int32)
    w1 = np.ones((1, 1))
    y = oracle.experts(u, wg[None], wu[None], wd[None], one, w1)
    y_swapped = oracle.experts(u, wu[None], wg[None], wd[None], one, w1)
    ref = _rank_one_value(wg, wu, wd, u[0].astype(np.float64))
    np.testing.assert_allclose(y[0], ref, rtol=1e-5)
    assert np.abs(y_swapped[0] - ref).max() > 1e-3 * np.abs(ref).max()


def test_experts_per_expert_scale_and_top1():
    # experts differ by a scalar on W_d: y = sum_j w_j c_{e_j} FFN(u); top-1 gives rho * c_e * FFN(u)
    H, I, E = 16, 8, 8
    wg1, wu1, wd1 = _rank_one_expert(H, I, 21)
    c = np.arange(1, E + 1, dtype=np.float32) * np.float32(0.5)
    wg = np.repeat(wg1[None], E, 0).copy()
    wu = np.repeat(wu1[None], E, 0).copy()
    wd = (np.repeat(wd1[None], E, 0) * c[:, None, None]).astype(np.float32)
    rng = np.random.default_rng(9)
    u = rng.normal(size=(5, H)).astype(np.float32)
    wr = rng.normal(size=(E, H)).astype(np.float32)
    for ng, tg, k in ((2, 1, 3), (E, 1, 1), (4, 2, 4)):
        r = oracle.route(u, wr, np.zeros(E, np.float32), ng, tg, k, 2.5)
        y = oracle.experts(u, wg, wu, wd, r.idx, r.w)
        for t in range(u.shape[0]):
            f = _rank_one_value(wg1, wu1, wd1, u[t].astype(np.float64))
            scale = float(np.sum(r.w[t] * c[r.idx[t]].astype(np.float64)))
            np.testing.assert_allclose(y[t], scale * f, rtol=1e-5, atol=1e-9 * np.abs(f).max())
        if k == 1:
            assert np.allclose(r.w, 2.5)


def test_experts_sparse_equals_dense_mask_tiny():
    # gathering the chosen experts equals evaluating every expert and masking with the weights
    cfg = CONFIGS["tiny_f32"]
    inp = make_inputs(cfg, j=0)
    r = oracle.route(inp.x, inp.w_router, inp.bias, cfg.n_group, cfg.topk_group, cfg.top_k, cfg.rho)
    y = oracle.experts(inp.x, inp.w_gate, inp.w_up, inp.w_down, r.idx, r.w)
    dense = np.zeros_like(y)
    ones = np.ones((cfg.T, 1))
    for e in range(cfg.E):
        ye = oracle.experts(inp.x, inp.w_gate, inp.w_up, inp.w_down, np.full((cfg.T, 1), e, np.int32), ones)
        mask = (r.idx == e)
        we = (r.w * mask).sum(1)
        dense += we[:, None] * ye
    np.testing.assert_allclose(y, dense, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------- RMSNorm

def test_rmsnorm_hand_worked_value():
    fx = _golden("rmsnorm_value.json")
    x = synth.f32_to_bf16(np.full((1, fx["H"]), fx["x"], np.float32))
    u = oracle.rmsnorm_pinned(x, np.full(fx["H"], fx["gain"], np.float32), fx["eps"])
    assert (u == fx["expected_bits"]).all()
    assert synth.bf16_to_f32(u)[0, 0] == fx["expected_value"]


def test_rmsnorm_laws():
    rng = np.random.default_rng(0)
    T, H = 16, 256
    xf = rng.normal(loc=3.0, size=(T, H)).astype(np.float32)
    x = synth.f32_to_bf16(xf)
    g1 = np.ones(H, np.float32)
    u = synth.bf16_to_f32(oracle.rmsnorm_pinned(x, g1, 1e-6)).astype(np.float64)
    # unit RMS with unit gain (bf16 rounding only)
    np.testing.assert_allclose(np.sqrt((u ** 2).mean(1)), 1.0, atol=3e-3)
    # sign pattern of the input is kept (no mean subtraction)
    assert (np.sign(u) == np.sign(synth.bf16_to_f32(x))).all()
    # scale invariance is exact with eps = 0 (power-of-two scale commutes with rounding)
    x2 = synth.f32_to_bf16(synth.bf16_to_f32(x) * np.float32(2.0))
    a = oracle.rmsnorm_pinned(x, g1, 0.0)
    b = oracle.rmsnorm_pinned(x2, g1, 0.0)
    assert np.array_equal(a, b)
    # gain enters as a plain multiplier: gain 2 doubles every value exactly
    c = oracle.rmsnorm_pinned(x, np.full(H, 2.0, np.float32), 0.0)
    assert np.array_equal(synth.bf16_to_f32(c), 2.0 * synth.bf16_to_f32(a))
    # a zero row stays zero
    z = oracle.rmsnorm_pinned(np.zeros((1, H), np.uint16), g1, 1e-6)
    assert not z.any()


# ----------------------------------------------------------------------------- residual

def test_residual_sum_over_sqrt_k():
    # Beam counts the embedding as contribution 1; after k contributions the stream is their sum / sqrt(k).
    rng = np.random.default_rng(1)
    H = 64
    n = _golden("beam_facts.json")["residual_additions"]["value"] + 1
    contrib = [rng.normal(size=H)]
    for _ in range(1, n):
        contrib.append(np.where(rng.random(H) < 0.5, -1.0, 1.0))  # RMS exactly 1: the post-norm is the identity
    x = contrib[0].astype(np.float32)[None]
    g = np.ones(H, np.float32)
    for k in range(2, n + 1):
        x = oracle.post_residual(contrib[k - 1][None], x, g, 0.0, k).astype(np.float32)
    np.testing.assert_allclose(x[0], np.sum(contrib, axis=0) / math.sqrt(n), rtol=0, atol=2e-5)


def test_residual_special_cases():
    rng = np.random.default_rng(2)
    H = 32
    x = rng.normal(size=(3, H)).astype(np.float32)
    g = (1.0 + 0.02 * rng.normal(size=H)).astype(np.float32)
    zero = np.zeros((3, H))
    out = oracle.post_residual(zero, x, g, 1e-6, 40)
    np.testing.assert_allclose(out, math.sqrt(39.0 / 40.0) * x.astype(np.float64), rtol=1e-15)
    y = rng.normal(size=(3, H)) * 5.0
    out1 = oracle.post_residual(y, x, g, 1e-6, 1)
    rms = np.sqrt((y ** 2).mean(1, keepdims=True) + 1e-6)
    np.testing.assert_allclose(out1, g.astype(np.float64) * y / rms, rtol=1e-12)


# ----------------------------------------------------------------------------- permutation

def test_permutation_is_the_stable_counting_sort():
    rng = np.random.default_rng(4)
    for T, K, E in ((1, 1, 1), (7, 3, 5), (50, 8, 16), (300, 8, 64)):
        idx = rng.integers(0, E, size=(T, K)).astype(np.int32)
        off, srt, pos = oracle.permutation(idx, E)
        flat = idx.reshape(-1)
        # textbook identities: exclusive scan of the histogram; stable argsort; inverse map
        np.testing.assert_array_equal(off, np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
        np.testing.assert_array_equal(srt, np.argsort(flat, kind="stable"))
        assert sorted(srt.tolist()) == list(range(T * K))
        np.testing.assert_array_equal(srt[pos], np.arange(T * K))
        for e in range(E):
            seg = srt[off[e]:off[e + 1]]
            assert (flat[seg] == e).all() and (np.diff(seg) > 0).all()


def test_permutation_brute_force_tiny():
    # every assignment of 4 pairs to 3 experts
    for code in range(3 ** 4):
        idx = np.array([(code // 3 ** i) % 3 for i in range(4)], np.int32).reshape(2, 2)
        off, srt, pos = oracle.permutation(idx, 3)
        expect = [p for e in range(3) for p in range(4) if idx.reshape(-1)[p] == e]
        assert srt.tolist() == expect


# ----------------------------------------------------------------------------- page figures

def test_expert_structure_matches_printed_parameter_counts():
    fx = _golden("beam_facts.json")
    H, I, E = fx["hidden"]["value"], fx["intermediate"]["value"], fx["experts"]["value"]
    per_expert = 3 * H * I  # gate, up and down matrices of a SwiGLU expert
    assert abs(per_expert - fx["expert_params_approx"]["value"]) < fx["expert_params_approx"]["tol"]
    experts_total = fx["moe_layers"]["value"] * E * per_expert
    share = experts_total / fx["total_params"]["value"]
    assert abs(share - fx["expert_param_share"]["value"]) < fx["expert_param_share"]["tol"]
    active = fx["moe_layers"]["value"] * fx["top_k"]["value"] * per_expert + fx["replicated_params"]["value"]
    assert abs(active - fx["active_params"]["value"]) < 0.1e9
    assert fx["groups"]["value"] * fx["group_size"]["value"] == E
    assert fx["dense_layers"]["value"] + fx["moe_layers"]["value"] == fx["layers"]["value"]
    assert 2 * fx["layers"]["value"] == fx["residual_additions"]["value"]
    cfg = CONFIGS["prefill_t8192"]
    assert (cfg.H, cfg.I, cfg.E, cfg.n_group, cfg.topk_group, cfg.top_k, cfg.rho) == (
        H, I, E, fx["groups"]["value"], fx["kept_groups"]["value"], fx["top_k"]["value"],
        fx["routed_scaling"]["value"])


def test_recorded_seeds_are_tie_free():
    seeds = _golden("seeds.json")
    for name in ("tiny_f32", "decode_t64"):
        assert seeds["min_margin"][name] >= 1e-6
    cfg = CONFIGS["decode_t64"]
    wr = synth.normal_f32(cfg.weight_seed, 2, (cfg.E, cfg.H), 0.0, cfg.wr_std)
    inp = make_inputs(cfg, weights=(wr, None, None, None))
    r = oracle.route(inp.x, wr, inp.bias, cfg.n_group, cfg.topk_group, cfg.top_k)
    assert abs(r.min_margin() - seeds["min_margin"]["decode_t64"]) < 1e-15


# ---- 8-bit (OCP FP8 E4M3 + E8M0 block scale) expert weights ----------------------

def test_e4m3_values_fixed_by_the_format():
    # OCP 8-bit floating point specification, E4M3: bias 7, largest finite 448 (S.1111.110),
    # smallest normal 2^-6, largest subnormal 0.875 * 2^-6, smallest subnormal 2^-9,
    # S.1111.111 is NaN, no infinities.
    fixed = {0x00: 0.0, 0x38: 1.0, 0x40: 2.0, 0x30: 0.5, 0x3C: 1.5, 0x7E: 448.0, 0x08: 2.0 ** -6,
             0x07: 0.875 * 2.0 ** -6, 0x01: 2.0 ** -9, 0x04: 2.0 ** -7, 0xB8: -1.0, 0xFE: -448.0, 0x0F: 1.875 * 2.0 ** -6}
    for code, v in fixed.items():
        assert oracle.e4m3_value(code) == v, hex(code)
    assert math.isnan(oracle.e4m3_value(0x7F)) and math.isnan(oracle.e4m3_value(0xFF))
    assert math.copysign(1.0, oracle.e4m3_value(0x80)) < 0 and oracle.e4m3_value(0x80) == 0.0
    pos = [oracle.e4m3_value(c) for c in range(0x7F)]
    assert all(b > a for a, b in zip(pos, pos[1:]))                         # 127 increasing values
    assert all(oracle.e4m3_value(0x80 | c) == -pos[c] for c in range(1, 0x7F))
    # the normal binade [2^e, 2^(e+1)) holds 8 equally spaced values
    for e in range(-6, 9):
        vals = [v for v in pos if 2.0 ** e <= v < 2.0 ** (e + 1)]
        assert len(vals) == (7 if e == 8 else 8) and vals[0] == 2.0 ** e
        assert np.allclose(np.diff(vals), 2.0 ** (e - 3))


def _representable_blocks(rows, cols, seed):
    """bf16 weights whose every 32-element block is exactly E4M3 values times 2^(s-127),
    with one element at 448 * 2^(s-127), so the block scale is s; returns (bf16, codes, s)."""
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 0x7F, size=(rows, cols), dtype=np.uint8) | (rng.integers(0, 2, size=(rows, cols),
                                                                                   dtype=np.uint8) << 7)
    codes[codes == 0x80] = 0x00                                  # the quantizer writes +0 for zero
    codes[:, ::32] = 0x7E | (codes[:, ::32] & 0x80)               # the block maximum
    s = rng.integers(100, 130, size=(rows, cols // 32), dtype=np.uint8)
    vals = np.array([oracle.e4m3_value(c) for c in range(256)])
    w = vals[codes] * np.ldexp(1.0, s.astype(np.int64) - 127).repeat(32, axis=1)
    return synth.f32_to_bf16(w.astype(np.float32)), codes, s


def test_quantizer_round_trips_representable_blocks():
    w, codes, s = _representable_blocks(6, 128, 21)
    assert (synth.bf16_to_f32(w).astype(np.float64) ==
            np.array([oracle.e4m3_value(c) for c in range(256)])[codes] *
            np.ldexp(1.0, s.astype(np.int64) - 127).repeat(32, axis=1)).all()   # bf16 holds them exactly
    c2, s2 = synth.quantize_e4m3(w)
    assert (c2 == codes).all() and (s2 == s).all()


def test_fp8_layer_equals_the_layer_on_the_decoded_weights():
    # the fp8 path of the oracle against its bf16 path on weights that are exactly the
    # decoded fp8 values (representable blocks: the two paths see identical numbers)
    H, I, E, T = 64, 32, 4, 5
    wg, cg, sg = _representable_blocks(E * I, H, 31)
    wu, cu, su = _representable_blocks(E * I, H, 32)
    wd, cd, sd = _representable_blocks(E * H, I, 33)
    rng = np.random.default_rng(8)
    u = synth.f32_to_bf16(rng.normal(size=(T, H)).astype(np.float32))
    idx = rng.integers(0, E, size=(T, 2)).astype(np.int32)
    wts = rng.uniform(0.1, 1.0, size=(T, 2))
    y_bf16 = oracle.experts(u, wg.reshape(E, I, H), wu.reshape(E, I, H), wd.reshape(E, H, I), idx, wts)
    y_fp8 = oracle.experts(u, cg.reshape(E, I, H), cu.reshape(E, I, H), cd.reshape(E, H, I), idx, wts,
                           w_scales=(sg.reshape(E, I, H // 32), su.reshape(E, I, H // 32), sd.reshape(E, H, I // 32)))
    assert (y_bf16 == y_fp8).all()
    # and a swapped scale tensor is seen
    y_bad = oracle.experts(u, cg.reshape(E, I, H), cu.reshape(E, I, H), cd.reshape(E, H, I), idx, wts,
                           w_scales=(su.reshape(E, I, H // 32), sg.reshape(E, I, H // 32), sd.reshape(E, H, I // 32)))
    assert not np.allclose(y_bad, y_fp8)


def test_e8m0_values_fixed_by_the_format():
    # OCP microscaling specification, E8M0 scale: an 8-bit exponent with bias 127 and no
    # sign or mantissa; 0x00 is 2^-127 (there is no zero), 0xFF is NaN (no infinity)
    assert oracle.e8m0_value(127) == 1.0
    assert oracle.e8m0_value(128) == 2.0 and oracle.e8m0_value(126) == 0.5
    assert oracle.e8m0_value(0) == math.ldexp(1.0, -127)
    assert oracle.e8m0_value(254) == math.ldexp(1.0, 127)
    assert math.isnan(oracle.e8m0_value(255))
    for s in range(255):
        assert oracle.e8m0_value(s) == math.ldexp(1.0, s - 127)


def test_e8m0_edge_bytes_reach_the_expert_path():
    # a block scaled by byte 0 gives its codes times 2^-127; a NaN scale makes the output NaN
    H, I, E, T = 64, 32, 2, 3
    rng = np.random.default_rng(5)
    codes = np.full((E, I, H), 0x40, np.uint8)          # E4M3 2.0
    cd = np.full((E, H, I), 0x38, np.uint8)             # E4M3 1.0
    sg = np.full((E, I, H // 32), 127, np.uint8)
    sd = np.full((E, H, I // 32), 127, np.uint8)
    u = synth.f32_to_bf16(rng.normal(size=(T, H)).astype(np.float32))
    idx = np.zeros((T, 1), np.int32)
    wts = np.ones((T, 1))
    y = oracle.experts(u, codes, codes, cd, idx, wts, w_scales=(sg, sg, sd))
    su = sg.copy()
    su[0, :, 0] = 0                                     # up rows: first block scaled by 2^-127
    ub = synth.bf16_to_f32(u).astype(np.float64)
    a = 2.0 * ub.sum(1)                                 # gate rows: 2 * sum(u)
    c = 2.0 * ub[:, 32:].sum(1) + 2.0 * math.ldexp(1.0, -127) * ub[:, :32].sum(1)
    h = a / (1.0 + np.exp(-a)) * c
    y0 = oracle.experts(u, codes, codes, cd, idx, wts, w_scales=(sg, su, sd))
    np.testing.assert_allclose(y0, np.repeat((I * h)[:, None], H, 1), rtol=1e-12)
    assert not np.allclose(y0, y)
    sn = sd.copy()
    sn[0, 5, 0] = 255                                   # one NaN scale in output row 5 of expert 0
    yn = oracle.experts(u, codes, codes, cd, idx, wts, w_scales=(sg, sg, sn))
    assert np.isnan(yn[:, 5]).all() and np.isfinite(np.delete(yn, 5, axis=1)).all()


def test_e2m1_values_fixed_by_the_format():
    # OCP microscaling specification, FP4 E2M1: bias 1, magnitudes 0, 0.5 (the one
    # subnormal), 1, 1.5, 2, 3, 4, 6 (the largest); bit 3 is the sign; no infinities or NaN
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for c in range(8):
        assert oracle.e2m1_value(c) == mags[c]
        assert oracle.e2m1_value(8 | c) == -mags[c]
    assert math.copysign(1.0, oracle.e2m1_value(8)) < 0


def _representable_blocks_e2m1(rows, cols, seed):
    """bf16 weights whose every 32-element block is exactly E2M1 values times 2^(s-127),
    with one element at 6 * 2^(s-127), so the block scale is s; returns (bf16, packed, s)."""
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 16, size=(rows, cols), dtype=np.uint8)
    codes[codes == 8] = 0                                       # the quantizer writes +0 for zero
    codes[:, ::32] = 7 | (codes[:, ::32] & 8)                   # the block maximum
    s = rng.integers(100, 130, size=(rows, cols // 32), dtype=np.uint8)
    vals = np.array([oracle.e2m1_value(c) for c in range(16)])
    w = vals[codes] * np.ldexp(1.0, s.astype(np.int64) - 127).repeat(32, axis=1)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)   # even element in the low nibble
    return synth.f32_to_bf16(w.astype(np.float32)), packed, s


def test_e2m1_quantizer_round_trips_representable_blocks():
    w, packed, s = _representable_blocks_e2m1(6, 128, 41)
    c2, s2 = synth.quantize_e2m1(w)
    assert c2.shape == (6, 64) and (c2 == packed).all() and (s2 == s).all()


def test_mxfp4_layer_equals_the_layer_on_the_decoded_weights():
    H, I, E, T = 64, 32, 4, 5
    wg, cg, sg = _representable_blocks_e2m1(E * I, H, 51)
    wu, cu, su = _representable_blocks_e2m1(E * I, H, 52)
    wd, cd, sd = _representable_blocks_e2m1(E * H, I, 53)
    rng = np.random.default_rng(9)
    u = synth.f32_to_bf16(rng.normal(size=(T, H)).astype(np.float32))
    idx = rng.integers(0, E, size=(T, 2)).astype(np.int32)
    wts = rng.uniform(0.1, 1.0, size=(T, 2))
    scales = (sg.reshape(E, I, H // 32), su.reshape(E, I, H // 32), sd.reshape(E, H, I // 32))
    y_bf16 = oracle.experts(u, wg.reshape(E, I, H), wu.reshape(E, I, H), wd.reshape(E, H, I), idx, wts)
    y_fp4 = oracle.experts(u, cg.reshape(E, I, H // 2), cu.reshape(E, I, H // 2), cd.reshape(E, H, I // 2), idx,
                           wts, w_scales=scales)
    assert (y_bf16 == y_fp4).all()
    # the nibble order is seen: codes with their two nibbles swapped give another layer
    sw = lambda c: ((c >> 4) | (c << 4)).astype(np.uint8)
    y_bad = oracle.experts(u, sw(cg).reshape(E, I, H // 2), sw(cu).reshape(E, I, H // 2),
                           sw(cd).reshape(E, H, I // 2), idx, wts, w_scales=scales)
    assert not np.allclose(y_bad, y_fp4)


def test_e2m1_quantizer_error_bound_on_gaussian_weights():
    # nearest-value rounding: |w - q| <= half the E2M1 spacing around w/2^(s-127) times the
    # scale (spacing 0.5 below 2, 1 in [2, 4), 2 in [4, 6]); |w| <= 6 * 2^(s-127)
    w = synth.normal_bf16(7, 4, (16, 256), 0.0, 0.02)
    packed, s = synth.quantize_e2m1(w)
    codes = np.empty((16, 256), dtype=np.uint8)
    codes[:, 0::2], codes[:, 1::2] = packed & 15, packed >> 4
    vals = np.array([oracle.e2m1_value(c) for c in range(16)])
    scale = np.ldexp(1.0, s.astype(np.int64) - 127).repeat(32, axis=1)
    q = vals[codes] * scale
    wf = synth.bf16_to_f32(w).astype(np.float64)
    x = np.abs(wf) / scale
    assert (x <= 6.0).all()
    spacing = np.where(x < 2.0, 0.5, np.where(x < 4.0, 1.0, 2.0)) * scale
    assert (np.abs(wf - q) <= 0.5 * spacing * (1 + 1e-12)).all()
    # the block maximum lands in the top binade [3, 6] (the scale is the smallest that fits)
    assert (x.reshape(16, 8, 32).max(axis=2) > 3.0).all()


def test_quantizer_error_bound_on_gaussian_weights():
    # nearest-value rounding: |w - q| <= half the E4M3 spacing at q's binade times the scale
    w = synth.normal_bf16(7, 3, (16, 256), 0.0, 0.02)
    codes, s = synth.quantize_e4m3(w)
    vals = np.array([oracle.e4m3_value(c) for c in range(256)])
    q = vals[codes] * np.ldexp(1.0, s.astype(np.int64) - 127).repeat(32, axis=1)
    wf = synth.bf16_to_f32(w).astype(np.float64)
    blk_max = np.abs(wf).reshape(16, 8, 32).max(axis=2).repeat(32, axis=1)
    assert (np.abs(q).reshape(16, 8, 32).max(axis=2) <= 448 * np.ldexp(1.0, s.astype(np.int64) - 127)).all()
    assert (blk_max <= 448 * np.ldexp(1.0, s.astype(np.int64) - 127).repeat(32, axis=1)).all()
    spacing = np.maximum(np.ldexp(1.0, np.floor(np.log2(np.maximum(np.abs(wf), 1e-30))).astype(np.int64) - 3),
                         np.ldexp(1.0, s.astype(np.int64) - 127 - 9).repeat(32, axis=1))
    assert (np.abs(wf - q) <= 0.5 * spacing * (1 + 1e-12)).all()
