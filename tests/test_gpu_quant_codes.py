"""GPU parity of the 8-bit and 4-bit expert weights code by code.

The storage formats are OCP FP8 E4M3 and FP4 E2M1 codes with one E8M0 scale byte per 32
elements of a row (the OCP microscaling layout; the Beam pages quote FP8 and ~4.5-bit
checkpoints without a scale scheme -- Glonce, "Reflection releases Beam...", "Hardware" and
"Running it" paragraphs).  The layer must equal the oracle, which decodes each code by the
format's definition, for:

* every non-NaN code: each gate/up/down row holds one magnitude class (an E4M3 exponent
  field, subnormals included; for E2M1 all sixteen codes), every sign and mantissa in every
  32-element block, with row scales that give every class the same weight in the result, so
  a class decoded wrongly moves the output by far more than the tolerance;
* scale bytes across the E8M0 range: gate/up column blocks scaled by 2^(s-127) for
  s = 0, 1, 126, 127, 128, 200, 253, 254 (with codes whose decoded values stay normal bf16),
  with the token activations of each block scaled by about 2^(127-s) so every block
  contributes O(1), and the router reading only the moderate blocks;
* the NaN scale byte 255: the tokens routed to that expert, and only they, come out NaN.

Both expert kernels are exercised (few rows per expert: the decode kernel's stream; 50 rows
per expert: the line kernel).  Bar: routing bit-exact, outputs within 1e-2 * max|ref|."""
import numpy as np
import pytest

import oracle
import synth

from moe_cases import as_f64, assert_routing_equal, dev, host, rel_err

pytestmark = pytest.mark.gpu

H, I, E, NG, KG, TOPK = 256, 128, 16, 4, 2, 4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_moe_layer_04_amd  # noqa: F401


def _e4m3_vals():
    return np.array([oracle.e4m3_value(c) for c in range(256)])


def _e2m1_vals():
    return np.array([oracle.e2m1_value(c) for c in range(16)])


def _e4m3_rows(n_rows, K, row0):
    """E4M3 codes [n_rows, K]: row r holds exponent field (row0 + r) % 16 only, element k the
    sign (k // 8) % 2 and mantissa k % 8 (the NaN code S.1111.111 replaced by S.1111.110)."""
    r = (row0 + np.arange(n_rows))[:, None] % 16
    k = np.arange(K)[None, :]
    codes = (((k // 8) % 2) << 7) | (r << 3) | (k % 8)
    nan = (codes & 0x7F) == 0x7F
    codes[nan] -= 1
    return codes.astype(np.uint8)


def _row_scales(codes_vals, n_blocks, rng, target_log2=-3):
    """E8M0 bytes [n_rows, n_blocks] that bring each row's largest decoded magnitude near
    2^target_log2, varied by +-2 per block."""
    amax = np.abs(codes_vals).max(axis=1)
    base = 127 + target_log2 - np.floor(np.log2(amax)).astype(np.int64)
    s = base[:, None] + rng.integers(-2, 3, size=(codes_vals.shape[0], n_blocks))
    assert s.min() >= 1 and s.max() <= 254
    return s.astype(np.uint8)


def _pack_e2m1(codes):
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def _codes_case(fmt, seed):
    """(w_codes (gate, up, down), scales (gate, up, down)) covering every non-NaN code."""
    rng = np.random.default_rng(seed)
    out_codes, out_scales = [], []
    for n_rows, K, row0 in ((E * I, H, 0), (E * I, H, 5), (E * H, I, 11)):
        if fmt == "e4m3":
            codes = _e4m3_rows(n_rows, K, row0)
            vals = _e4m3_vals()[codes]
            packed = codes
        else:   # every E2M1 code in every 16 elements, rotated per row
            k = np.arange(K)[None, :]
            codes = ((k + (row0 + np.arange(n_rows))[:, None]) % 16).astype(np.uint8)
            vals = _e2m1_vals()[codes]
            packed = _pack_e2m1(codes)
        s = _row_scales(vals, K // 32, rng)
        out_codes.append(packed)
        out_scales.append(s)
    shp = ((E, I, -1), (E, I, -1), (E, H, -1))
    return tuple(c.reshape(sh) for c, sh in zip(out_codes, shp)), tuple(s.reshape(sh) for s, sh in zip(out_scales, shp))


# gate/up column blocks: scale byte and activation exponent (products ~ code * 2^(s-127+c))
SCALE_BYTES = (0, 1, 126, 127, 128, 200, 253, 254)
ACT_EXP = tuple(max(-120, min(124, 127 - s)) for s in SCALE_BYTES)
ROUTER_BLOCKS = (2, 3, 4)   # the blocks with activations near 1


def _scale_case(fmt, seed):
    """Gate/up rows whose 32-element block b has scale byte SCALE_BYTES[b]; the codes keep
    the decoded values normal bf16: magnitudes in [2, 4) (E2M1: 2 and 3) in blocks with
    s <= 128, in [1, 2) (E2M1: 1 and 1.5) above; down rows as in the code case."""
    rng = np.random.default_rng(seed)
    sc = np.array(SCALE_BYTES, np.uint8)
    low = np.repeat(sc <= 128, 32)[None, :]             # per column: the block's scale is small
    wcodes, wscales = [], []
    for _ in range(2):
        sign = rng.integers(0, 2, size=(E * I, H))
        if fmt == "e4m3":
            field = np.where(low, 8, 7)                 # exponent field: [2, 4) or [1, 2)
            codes = ((sign << 7) | (field << 3) | rng.integers(0, 8, size=(E * I, H))).astype(np.uint8)
            packed = codes
        else:   # E2M1 codes 4, 5 (2, 3) or 2, 3 (1, 1.5), with the sign bit 3
            mag = np.where(low, 4, 2) + rng.integers(0, 2, size=(E * I, H))
            codes = (mag | (sign << 3)).astype(np.uint8)
            packed = _pack_e2m1(codes)
        wcodes.append(packed.reshape(E, I, -1))
        wscales.append(np.tile(sc, (E * I, 1)).reshape(E, I, H // 32))
    (cd,), (sd,) = [c[2:] for c in _codes_case(fmt, seed + 1)]
    return (wcodes[0], wcodes[1], cd), (wscales[0], wscales[1], sd)


def _inputs(T, seed, act_exp=None):
    """bf16 activations (block b scaled by 2^act_exp[b]), fp32 router, bias; the router reads
    only ROUTER_BLOCKS when act_exp is given; the first seed offset without a routing near-tie."""
    for j in range(40):
        rng = np.random.default_rng([seed, j])
        x = rng.standard_normal((T, H)).astype(np.float32)
        wr = (rng.standard_normal((E, H)) / np.sqrt(H)).astype(np.float32)
        if act_exp is not None:
            x *= np.repeat(np.ldexp(1.0, np.array(act_exp)), 32)[None, :].astype(np.float32)
            keep = np.zeros(H // 32, bool)
            keep[list(ROUTER_BLOCKS)] = True
            wr *= np.repeat(keep, 32)[None, :] * np.float32(np.sqrt(H / 96.0))
        xb = synth.f32_to_bf16(x)
        bias = rng.uniform(-0.05, 0.05, E).astype(np.float32)
        r = oracle.route(xb, wr, bias, NG, KG, TOPK, 2.5)
        if r.min_margin() >= 1e-6 and r.agree.min() == 1:
            return xb, wr, bias, r
    raise RuntimeError("no tie-free inputs")


def _run(fmt, T, codes, scales, xb, wr, bias, ref_route):
    import torch
    import sparse_moe_layer_04_amd as bm
    shape = bm.make_shape(T, H, E, I, NG, KG, TOPK, 2.5, "bf16")
    ws = torch.empty(bm.workspace_size(shape, bm.OP_FORWARD), dtype=torch.uint8, device="cuda")
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    idx = torch.empty((T, TOPK), dtype=torch.int32, device="cuda")
    w = torch.empty((T, TOPK), dtype=torch.float32, device="cuda")
    dc = tuple(dev(np.ascontiguousarray(c)) for c in codes)
    ds = tuple(dev(np.ascontiguousarray(s)) for s in scales)
    bm.forward(shape, dev(xb), dev(wr), dev(bias), dc[0], dc[1], dc[2], out, ws, topk_idx=idx, topk_w=w,
               w_scales=ds, w_format=fmt)
    torch.cuda.synchronize()
    assert_routing_equal(host(idx), host(w), ref_route.idx, ref_route.w, 2.5)
    y = oracle.experts(xb, codes[0], codes[1], codes[2], ref_route.idx, ref_route.w, w_scales=scales)
    assert np.isfinite(y).all()
    return rel_err(as_f64(host(out)), y)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
@pytest.mark.parametrize("T", [24, 200])
def test_every_code_decodes_exactly(fmt, T):
    codes, scales = _codes_case(fmt, 100 + T)
    xb, wr, bias, r = _inputs(T, 200 + T)
    err = _run(fmt, T, codes, scales, xb, wr, bias, r)
    print("%s T=%d every code: rel err %.3e" % (fmt, T, err))
    assert err <= 1e-2


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
@pytest.mark.parametrize("T", [24, 200])
def test_scale_bytes_across_the_range(fmt, T):
    codes, scales = _scale_case(fmt, 300 + T)
    xb, wr, bias, r = _inputs(T, 400 + T, act_exp=ACT_EXP)
    err = _run(fmt, T, codes, scales, xb, wr, bias, r)
    print("%s T=%d scale bytes %s: rel err %.3e" % (fmt, T, SCALE_BYTES, err))
    assert err <= 1e-2


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_nan_scale_reaches_exactly_the_tokens_of_its_expert(fmt):
    T = 64
    codes, scales = _codes_case(fmt, 500)
    xb, wr, bias, r = _inputs(T, 600)
    e = int(np.bincount(r.idx.reshape(-1), minlength=E).argmax())
    sg = scales[0].copy()
    sg[e, 3, 1] = 255                                   # one gate block of expert e
    scales = (sg, scales[1], scales[2])
    import torch
    import sparse_moe_layer_04_amd as bm
    shape = bm.make_shape(T, H, E, I, NG, KG, TOPK, 2.5, "bf16")
    ws = torch.empty(bm.workspace_size(shape, bm.OP_FORWARD), dtype=torch.uint8, device="cuda")
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    dc = tuple(dev(np.ascontiguousarray(c)) for c in codes)
    ds = tuple(dev(np.ascontiguousarray(s)) for s in scales)
    bm.forward(shape, dev(xb), dev(wr), dev(bias), dc[0], dc[1], dc[2], out, ws, w_scales=ds, w_format=fmt)
    torch.cuda.synchronize()
    got = as_f64(host(out))
    y = oracle.experts(xb, codes[0], codes[1], codes[2], r.idx, r.w, w_scales=scales)
    hit = (r.idx == e).any(axis=1)
    assert hit.sum() > 0 and (~hit).sum() > 0
    assert np.isnan(y[hit]).all() and np.isfinite(y[~hit]).all()
    assert np.isnan(got[hit]).all() and np.isfinite(got[~hit]).all()
    err = rel_err(got[~hit], y[~hit])
    print("%s NaN scale: %d tokens NaN, the rest rel err %.3e" % (fmt, hit.sum(), err))
    assert err <= 1e-2


def test_code_cases_cover_every_code_and_the_class_weights_are_even():
    # host-side check of the construction above (runs with the GPU tests)
    codes, scales = _codes_case("e4m3", 1)
    seen = set(np.unique(np.concatenate([c.reshape(-1) for c in codes])).tolist())
    assert seen == set(range(256)) - {0x7F, 0xFF}
    v = _e4m3_vals()[codes[0].reshape(E * I, H)] * np.ldexp(1.0, scales[0].reshape(E * I, -1).astype(int) - 127
                                                            ).repeat(32, axis=1)
    amax = np.abs(v).max(axis=1)
    assert amax.max() / amax.min() < 2 ** 6
    codes4, _ = _codes_case("e2m1", 1)
    lo = codes4[0] & 15
    hi = codes4[0] >> 4
    assert set(np.unique(np.concatenate([lo.reshape(-1), hi.reshape(-1)])).tolist()) == set(range(16))
