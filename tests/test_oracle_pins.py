"""Pins of the CPU oracle against things other than itself.

Each test names the oracle function it pins and the independent source of
truth: a library routine (torch casts, numpy/torch fp64 matmuls, Python's
stable sort), a brute-force search, exact rational arithmetic, or the hand
cases under tests/golden/ (exact by construction).
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from workloads import WORKLOADS, make_inputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ------------------------------------------------------------------ bf16 RNE

def test_bf16_rne_exhaustive_vs_torch_cast():
    """orc_bf16_bits over all 2^32 fp32 bit patterns vs torch's CPU cast."""
    step = 1 << 26
    for start in range(0, 1 << 32, step):
        bits = np.arange(start, start + step, dtype=np.uint64).astype(np.uint32)
        v = bits.view(np.float32)
        ours = oracle.bf16_bits(v)
        ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        nan = np.isnan(v)
        assert np.array_equal(ours[~nan], ref[~nan]), f"mismatch in chunk at {start:#x}"
        # NaN stays NaN (payload is not part of the contract)
        assert np.all((ours[nan] & 0x7F80) == 0x7F80) and np.all((ours[nan] & 0x7F) != 0)


# ------------------------------------------------------------------ E4M3 / E8M0

def _e4m3_table():
    """All finite E4M3FN values from torch's float8 dtype (a library decode)."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    vals = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return vals


def test_e4m3_decode_vs_torch():
    vals = _e4m3_table()
    for c in range(256):
        ours = oracle.e4m3_decode(c)
        if np.isnan(vals[c]):
            assert np.isnan(ours)
        else:
            assert ours == vals[c], c


def test_e4m3_encode_vs_brute_force_nearest():
    """Nearest finite E4M3FN value, ties to the even code, by exhaustive search."""
    vals = _e4m3_table()
    finite = [c for c in range(256) if not np.isnan(vals[c])]
    rng = np.random.default_rng(5)
    # every midpoint between neighbours, every exact value, and random values
    pos = sorted(set(vals[c] for c in finite if vals[c] >= 0))
    mids = [(a + b) / 2 for a, b in zip(pos[:-1], pos[1:])]
    samples = list(pos) + mids + list(rng.uniform(0, 448, 3000)) + \
        list(2.0 ** rng.uniform(-12, 8.8, 3000))
    samples = [s for s in samples if s <= 448]
    for s in samples:
        for v in (s, -s):
            ours = oracle.e4m3_encode(v)
            d = [abs(vals[c] - v) for c in finite]
            best = min(d)
            cands = [c for c, dd in zip(finite, d) if dd == best]
            if len(cands) > 1:
                cands = [c for c in cands if (c & 1) == 0] or cands
                # +0/-0 both sit at distance |v|: keep the sign of v
                if best == abs(v):
                    cands = [c for c in cands if (c & 0x80) == (0x80 if v < 0 or
                                                                 (v == 0 and np.signbit(v)) else 0)]
            assert ours in cands, (v, ours, cands)


def test_e4m3_encode_vs_torch_cast():
    rng = np.random.default_rng(6)
    v = np.concatenate([rng.uniform(-448, 448, 20000), 2.0 ** rng.uniform(-12, 8.8, 20000)])
    v = v.astype(np.float32).astype(np.float64)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = np.array([oracle.e4m3_encode(x) for x in v], dtype=np.uint8)
    assert np.array_equal(ours, ref)


def _e8m0_linear(amax):
    if amax == 0:
        return -127
    for e in range(-127, 128):
        if Fraction(amax) <= 448 * Fraction(2) ** e:
            return e
    return 127


def test_e8m0_vs_linear_search():
    rng = np.random.default_rng(7)
    vals = [0.0, 448.0, 449.0, 2.0, 1.75, 1.7500001, 3.5, 3.4999998, 1e-45, 1e-38, 3.4e38]
    vals += [float(np.float32(448.0 * 2.0 ** e)) for e in range(-126, 119)]
    vals += [float(np.nextafter(np.float32(448.0 * 2.0 ** e), np.float32(np.inf)))
             for e in range(-120, 119)]
    vals += list((2.0 ** rng.uniform(-140, 127, 2000)).astype(np.float32).astype(float))
    for a in vals:
        a32 = float(np.float32(a))
        assert oracle.e8m0_exponent(a32) == _e8m0_linear(a32), a32


def test_mx_blocks_golden():
    """Hand cases of the block quantizer (tests/golden/mx_blocks.json)."""
    with open(os.path.join(GOLDEN, "mx_blocks.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        blk = np.array(c["block"], dtype=np.float32)[None, :]
        codes, scales = oracle.mx_quantize(blk)
        assert int(scales[0, 0]) == c["scale_exp"] + 127, c["name"]
        deq = oracle.mx_dequantize(codes, scales)[0]
        assert np.array_equal(deq, np.array(c["values"])), c["name"]


def test_mx_quantize_vs_torch():
    """Codes = torch E4M3 cast of v / 2^e with e from the linear search."""
    rng = np.random.default_rng(8)
    v = (rng.standard_normal((64, 256)) * 2.0 ** rng.integers(-20, 20, (64, 1))).astype(np.float32)
    v[3, :32] = 0
    codes, scales = oracle.mx_quantize(v)
    for r in range(v.shape[0]):
        for b in range(v.shape[1] // 32):
            blk = v[r, b * 32:(b + 1) * 32]
            e = _e8m0_linear(float(np.max(np.abs(blk))))
            assert scales[r, b] == e + 127
            ref = torch.from_numpy(blk.astype(np.float64) * 2.0 ** -e).to(
                torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert np.array_equal(codes[r, b * 32:(b + 1) * 32], ref)


# ------------------------------------------------------------------ MXFP4 primitives

E2M1_MAGNITUDES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]   # codes 0..7 (OCP MX FP4)


def _e2m1_by_intervals(v):
    """Nearest E2M1 code with ties to the even code, written as the intervals
    between neighbouring magnitudes (an independent formulation of the rule)."""
    a = abs(v)
    if a <= 0.25: c = 0
    elif a < 0.75: c = 1
    elif a <= 1.25: c = 2
    elif a < 1.75: c = 3
    elif a <= 2.5: c = 4
    elif a < 3.5: c = 5
    elif a <= 5.0: c = 6
    else: c = 7
    return c | (8 if np.signbit(v) else 0)


def test_e2m1_decode_table():
    for c in range(16):
        mag = E2M1_MAGNITUDES[c & 7]
        want = -mag if c & 8 else mag
        got = oracle.e2m1_decode(c)
        assert got == want and np.signbit(got) == bool(c & 8), c


def test_e2m1_encode_vs_intervals():
    rng = np.random.default_rng(23)
    vals = [i / 64 for i in range(-384, 385)] + [-0.0, 0.0]
    vals += list(rng.uniform(-6, 6, 4000))
    vals += [m + d for m in (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0) for d in (-1e-9, 1e-9)]
    for v in vals:
        assert oracle.e2m1_encode(v) == _e2m1_by_intervals(v), v


def _e8m0_fp4_linear(amax):
    if amax == 0:
        return -127
    for e in range(-127, 128):
        if Fraction(amax) <= 6 * Fraction(2) ** e:
            return e
    return 127


def test_e8m0_fp4_vs_linear_search():
    rng = np.random.default_rng(24)
    vals = [0.0, 6.0, 6.000001, 3.0, 2.9999998, 1.5, 1.0, 1e-45, 1e-38, 3.4e38]
    vals += [float(np.float32(6.0 * 2.0 ** e)) for e in range(-126, 126)]
    vals += [float(np.nextafter(np.float32(6.0 * 2.0 ** e), np.float32(np.inf)))
             for e in range(-120, 125)]
    vals += list((2.0 ** rng.uniform(-140, 127, 2000)).astype(np.float32).astype(float))
    for a in vals:
        a32 = float(np.float32(a))
        assert oracle.e8m0_exponent_fp4(a32) == _e8m0_fp4_linear(a32), a32


def test_mx4_blocks_golden():
    """Hand cases of the MXFP4 block quantizer (tests/golden/mx4_blocks.json)."""
    with open(os.path.join(GOLDEN, "mx4_blocks.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        blk = np.array(c["block"], dtype=np.float32)[None, :]
        codes, scales = oracle.mx4_quantize(blk)
        assert int(scales[0, 0]) == c["scale_exp"] + 127, c["name"]
        deq = oracle.mx4_dequantize(codes, scales)[0]
        assert np.array_equal(deq, np.array(c["values"])), c["name"]


def test_mx4_quantize_vs_rules():
    """Scales from the linear search, codes from the interval rule."""
    rng = np.random.default_rng(25)
    v = (rng.standard_normal((32, 128)) * 2.0 ** rng.integers(-20, 20, (32, 1))).astype(np.float32)
    v[5, 32:64] = 0
    codes, scales = oracle.mx4_quantize(v)
    for r in range(v.shape[0]):
        for b in range(v.shape[1] // 32):
            blk = v[r, b * 32:(b + 1) * 32]
            e = _e8m0_fp4_linear(float(np.max(np.abs(blk))))
            assert scales[r, b] == e + 127
            want = [_e2m1_by_intervals(float(x) * 2.0 ** -e) for x in blk]
            assert list(codes[r, b * 32:(b + 1) * 32]) == want


# ------------------------------------------------------------------ router

def test_route_vs_sort_and_numpy_softmax():
    rng = np.random.default_rng(9)
    T, E, k = 300, 40, 6
    lg = rng.standard_normal((T, E)).astype(np.float32)
    lg[5, 3] = lg[5, 17] = lg[5].max() + 1       # tie at the top: lower id first
    lg[7, :] = 0.0                                # all tied: ids 0..k-1
    ids, probs, err = oracle.route(lg, T, k)
    assert err == 0
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(lg[t, e]), e))[:k]
        assert list(ids[t]) == sorted(order), t
        z = np.exp(lg[t].astype(np.float64) - lg[t].max())
        p = z / z.sum()
        q = p[sorted(order)] / p[sorted(order)].sum()
        np.testing.assert_allclose(probs[t], q, rtol=2e-7, atol=0)
    assert list(ids[7]) == list(range(k))


def test_route_live_bounds():
    lg = np.random.default_rng(1).standard_normal((8, 8)).astype(np.float32)
    ids, probs, err = oracle.route(lg, 3, 2)
    assert err == 0 and np.all(ids[3:] == -1) and np.all(np.isnan(probs[3:]))
    ids, probs, err = oracle.route(lg, 9, 2)
    assert err == oracle.ERR_LIVE_HIGH and np.all(ids >= 0)
    ids, probs, err = oracle.route(lg, -1, 2)
    assert err == oracle.ERR_LIVE_NEG and np.all(ids == -1)


# ------------------------------------------------------------------ permutation

def _prepare_reference(ids, probs, live, E):
    """Python's stable sorted() over the token-major route list."""
    T, k = ids.shape
    T = max(0, min(live, T))
    routes = []
    sorted_ids = np.zeros((T, k), np.int64)
    for t in range(T):
        pairs = sorted(((int(ids[t, j]), j) for j in range(k)), key=lambda q: q[0])
        for j, (e, _) in enumerate(pairs):
            sorted_ids[t, j] = e
            routes.append((e, t * k + j))
    # a route is dropped if its id is out of range or repeats the id of the
    # route before it in canonical order (the same expert listed twice)
    valid = [(e, r) for e, r in routes
             if 0 <= e < E and not (r % k > 0 and sorted_ids.reshape(-1)[r - 1] == e)]
    perm = [r for e, r in sorted(valid, key=lambda q: q[0])]
    counts = np.bincount([e for e, _ in valid], minlength=E)
    dst = -np.ones(T * k, np.int64)
    for pos, r in enumerate(perm):
        dst[r] = pos
    return sorted_ids, counts, np.array(perm, np.int64), dst.reshape(T, k)


@pytest.mark.parametrize("T,E,k,live", [(64, 8, 2, 64), (200, 16, 5, 137), (33, 128, 8, 33),
                                        (16, 4, 4, 16), (10, 8, 1, 0)])
def test_prepare_vs_python_sorted(T, E, k, live):
    rng = np.random.default_rng(T + E + k)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    probs = rng.random((T, k)).astype(np.float32)
    got = oracle.prepare(ids, probs, live, E)
    s_ids, counts, perm, dst = _prepare_reference(ids, probs, live, E)
    assert got["err"] == 0
    assert np.array_equal(got["sorted_ids"], s_ids)
    assert np.array_equal(got["counts"], counts)
    assert np.array_equal(got["offsets"], np.concatenate([[0], np.cumsum(counts)]))
    assert np.array_equal(got["perm_src"], perm)
    assert np.array_equal(got["dst"], dst)
    # probabilities travel with their ids
    for t in range(got["T"]):
        pairs = {int(ids[t, j]): probs[t, j] for j in range(k)}
        assert all(got["sorted_probs"][t, j] == pairs[int(s_ids[t, j])] for j in range(k))


def test_prepare_contract_violations():
    ids = np.array([[0, 9], [1, 1], [2, 0]], np.int32)
    probs = np.ones((3, 2), np.float32)
    got = oracle.prepare(ids, probs, 3, 4)
    assert got["err"] == oracle.ERR_BAD_ID | oracle.ERR_DUP_ID
    s_ids, counts, perm, dst = _prepare_reference(ids, probs, 3, 4)
    assert np.array_equal(got["dst"], dst) and np.array_equal(got["perm_src"], perm)


# ------------------------------------------------------------------ finalize

def _fma_f32_exact(a, b, c):
    """Correctly rounded fp32 fma from exact rationals (ties to even)."""
    exact = Fraction(float(a)) * Fraction(float(b)) + Fraction(float(c))
    if exact == 0:
        return np.float32(0.0)
    guess = np.float32(float(exact))
    cands = {guess, np.nextafter(guess, np.float32(np.inf)), np.nextafter(guess, np.float32(-np.inf))}
    best = min(cands, key=lambda v: (abs(Fraction(float(v)) - exact),
                                     int(np.array(v).view(np.uint32)) & 1))
    return np.float32(best)


def test_finalize_vs_exact_fma_chain():
    rng = np.random.default_rng(10)
    T, k, H = 40, 4, 8
    R = T * k
    O = (rng.standard_normal((R, H)) * 2.0 ** rng.integers(-30, 30, (R, 1))).astype(np.float32)
    p = rng.random((T, k)).astype(np.float32)
    dst = rng.permutation(R).astype(np.int32).reshape(T, k)
    dst[3, 1] = -1                                       # a dropped route adds nothing
    out = oracle.finalize(O, dst, p, H)
    for t in range(T):
        for m in range(H):
            acc = np.float32(0.0)
            for j in range(k):
                if dst[t, j] >= 0:
                    acc = _fma_f32_exact(p[t, j], O[dst[t, j], m], acc)
            assert out[t, m].view(np.uint32) == np.float32(acc).view(np.uint32), (t, m)


# ------------------------------------------------------------------ combine variants

def _load_combine_cases():
    with open(os.path.join(GOLDEN, "combine_cases.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("c", _load_combine_cases(), ids=lambda c: c["name"])
def test_combine_golden(c):
    """Hand cases of the bf16 combine and the row mode (tests/golden/combine_cases.json)."""
    O = np.array(c["O"], np.float32)
    dst = np.array(c["dst"], np.int32)
    p = np.array(c["probs"], np.float32)
    if c["mode"] == "bf16":
        got = oracle.finalize_bf16(O, dst, p, c["H"])
        assert np.array_equal(got, np.array(c["expected_bf16"], np.uint16)), got
    else:
        got = oracle.finalize_rows(O, dst, c["H"])
        assert np.array_equal(got.view(np.uint32), np.array(c["expected_rows_bits"], np.uint32)), got


def _random_combine_inputs(seed):
    rng = np.random.default_rng(seed)
    T, k, H = 30, 5, 12
    R = T * k
    O = (rng.standard_normal((R, H)) * 2.0 ** rng.integers(-20, 20, (R, 1))).astype(np.float32)
    O[rng.random((R, H)) < 0.05] = -0.0
    p = rng.random((T, k)).astype(np.float32)
    dst = rng.permutation(R).astype(np.int32).reshape(T, k)
    dst[2, 3] = -1
    dst[7, 0] = -1
    return O, dst, p, H


def test_finalize_bf16_is_torch_cast_of_fp32_chain():
    """The bf16 combine rounds the (separately pinned) fp32 chain; torch's cast is an
    independent round-to-nearest-even."""
    O, dst, p, H = _random_combine_inputs(21)
    f32 = oracle.finalize(O, dst, p, H)
    ref = torch.from_numpy(f32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.finalize_bf16(O, dst, p, H), ref)


def test_finalize_rows_closed_form():
    """Row mode: the routed row plus +0 (numpy's IEEE add), zeros for a dropped route,
    probabilities ignored."""
    O, dst, p, H = _random_combine_inputs(22)
    ref = np.where((dst >= 0)[:, :, None], O[np.maximum(dst, 0)] + np.float32(0.0), np.float32(0.0))
    got = oracle.finalize_rows(O, dst, H)
    assert np.array_equal(got.view(np.uint32), ref.astype(np.float32).view(np.uint32))
    assert not np.any(got.view(np.uint32) == 0x80000000), "a -0 survived"


@pytest.mark.parametrize("precision", ["bf16", "mxfp8"])
def test_forward_rows_are_top1_tokens_with_probability_one(precision):
    """Row mode by its definition: every route of the k-model equals the forward of a
    top-1 model on that route's token alone, with probability 1."""
    w = WORKLOADS["tiny"]
    inp = make_inputs(w, seed=13, outliers=(precision == "mxfp8"))
    ids, probs, _ = oracle.route(inp["logits"], w.T, w.k)
    m = oracle.Model(w.E, w.H, w.F, w.k, inp["w1_bits"], inp["w2_bits"], precision)
    rows, err, _ = m.forward(inp["x_bits"], ids[:, ::-1].copy(), None, w.T, combine="rows")
    assert err == 0 and rows.shape == (w.T_cap, w.k, w.H)
    m1 = oracle.Model(w.E, w.H, w.F, 1, inp["w1_bits"], inp["w2_bits"], precision)
    sid = np.sort(ids[: w.T], axis=1)                      # canonical order of the routes
    x1 = np.repeat(inp["x_bits"][: w.T], w.k, axis=0)
    one, err1, _ = m1.forward(x1, sid.reshape(-1, 1).copy(), np.ones((w.T * w.k, 1), np.float32),
                              w.T * w.k)
    assert err1 == 0
    assert np.array_equal(rows[: w.T].reshape(-1, w.H).view(np.uint32), one.view(np.uint32))
    assert np.all(np.isnan(rows[w.T:])), "rows of tokens past live were written"


@pytest.mark.parametrize("precision", ["bf16", "mxfp8"])
def test_forward_bf16_combine_is_rounded_fp32_combine(precision):
    w = WORKLOADS["tiny"].with_tokens(40, 64)
    inp = make_inputs(w, seed=11, outliers=(precision == "mxfp8"))
    ids, probs, _ = oracle.route(inp["logits"], w.T, w.k)
    m = oracle.Model(w.E, w.H, w.F, w.k, inp["w1_bits"], inp["w2_bits"], precision)
    f32, _, _ = m.forward(inp["x_bits"], ids, probs, w.T)
    b16, err, _ = m.forward(inp["x_bits"], ids, probs, w.T, combine="bf16")
    assert err == 0
    ref = torch.from_numpy(f32[: w.T]).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b16[: w.T], ref)
    assert np.all(b16[w.T:] == 0xFFFF), "rows of tokens past live were written"


# ------------------------------------------------------------------ hand cases

def _load_hand_cases():
    with open(os.path.join(GOLDEN, "hand_cases.json")) as f:
        return json.load(f)["cases"]


def _bits(vals):
    a = np.array(vals, dtype=np.float32)
    b = a.view(np.uint32)
    finite = ~np.isnan(a)
    assert np.all((b[finite] & 0xFFFF) == 0), "hand-case values must be exact bf16"
    out = (b >> 16).astype(np.uint16)
    out[~finite] = 0x7FC0
    return out


def hand_case_arrays(c):
    """Numpy inputs of a hand case; NaN patterns past the live count."""
    x = _bits(c["x"])
    ids = np.array([[0x7FC00000 if v is None else v for v in r] for r in c["ids"]],
                   dtype=np.int64).astype(np.int32)
    pr = np.array([[np.nan if v is None else v for v in r] for r in c["probs"]], np.float32)
    w1 = _bits(c["w1"])
    w2 = _bits(c["w2"])
    return x, ids, pr, w1, w2


@pytest.mark.parametrize("precision", ["mxfp8", "mxfp4"])
@pytest.mark.parametrize("c", _load_hand_cases(), ids=lambda c: c["name"])
def test_oracle_hand_cases_block_scaled(c, precision):
    """The hand cases' operands (one-hot x, gate 32, small integers, powers of two)
    are exact in E4M3 and in E2M1 with their block scales, so the MXFP8 and MXFP4
    paths must reproduce the exact outputs too."""
    x, ids, pr, w1, w2 = hand_case_arrays(c)
    m = oracle.Model(c["E"], c["H"], c["F"], c["k"], w1, w2, precision)
    out, err, _ = m.forward(x, ids, pr, c["live"])
    assert err == 0
    for t, row in enumerate(c["expected"]):
        if row is None:
            assert np.all(np.isnan(out[t]))
        else:
            assert np.array_equal(out[t], np.array(row, np.float32)), t


@pytest.mark.parametrize("c", _load_hand_cases(), ids=lambda c: c["name"])
def test_oracle_hand_cases(c):
    x, ids, pr, w1, w2 = hand_case_arrays(c)
    m = oracle.Model(c["E"], c["H"], c["F"], c["k"], w1, w2, c["precision"])
    out, err, _ = m.forward(x, ids, pr, c["live"])
    assert err == 0
    for t, row in enumerate(c["expected"]):
        if row is None:
            assert np.all(np.isnan(out[t])), f"row {t} past live was written"
        else:
            assert np.array_equal(out[t], np.array(row, np.float32)), t
    if c["name"].startswith("HC4"):
        # a different order breaks the pin: +1 last gives 1, not 0
        O = np.array([[2.0 ** 24], [-(2.0 ** 24)], [1.0]], np.float32)
        assert oracle.finalize(O, np.array([[0, 1, 2]], np.int32),
                               np.ones((1, 3), np.float32), 1)[0, 0] == 1.0


def test_hand_case_hc3_bitwise_hc2():
    cases = {c["name"]: c for c in _load_hand_cases()}
    outs = []
    for name in ("HC2_top2_quarters", "HC3_listed_order_irrelevant"):
        x, ids, pr, w1, w2 = hand_case_arrays(cases[name])
        c = cases[name]
        outs.append(oracle.Model(c["E"], c["H"], c["F"], c["k"], w1, w2).forward(x, ids, pr, 2)[0])
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))


# ------------------------------------------------------------------ expert MLP

def _operand_values(precision, xv, w1v, w2v, w):
    """Operand values of x and the weights for a precision: bf16 values as they
    are; MXFP8 activations for "mxfp8" and "mxfp4"; weights MXFP8 ("mxfp8") or
    MXFP4 ("mxfp4"), each quantized per 32-block along K (the quantizers are
    pinned on their own above)."""
    if precision == "bf16":
        return xv, w1v, w2v
    xv = oracle.mx_dequantize(*oracle.mx_quantize(xv.astype(np.float32)))
    q, dq = ((oracle.mx_quantize, oracle.mx_dequantize) if precision == "mxfp8"
             else (oracle.mx4_quantize, oracle.mx4_dequantize))
    w1v = dq(*q(w1v.reshape(-1, w.H).astype(np.float32))).reshape(w1v.shape)
    w2v = dq(*q(w2v.reshape(-1, w.F).astype(np.float32))).reshape(w2v.shape)
    return xv, w1v, w2v


def _dense_mlp_fp64(x_vals, w1_vals, w2_vals, F, mx_h=False):
    """torch fp64 reference of one expert: g, u rounded to fp32, SwiGLU in fp64
    rounded to fp32, FC2 operand rounded to bf16 (torch cast) or MXFP8, FC2 in
    fp64 rounded to fp32."""
    x = torch.from_numpy(x_vals)
    w1 = torch.from_numpy(w1_vals)
    w2 = torch.from_numpy(w2_vals)
    g = (x @ w1[:F].T).float().double()
    u = (x @ w1[F:].T).float().double()
    a = (g / (1.0 + torch.exp(-g)) * u).float()
    if not mx_h:
        h = a.to(torch.bfloat16).double()
    else:
        codes, scales = oracle.mx_quantize(a.numpy())
        h = torch.from_numpy(oracle.mx_dequantize(codes, scales))
    return (h @ w2.T).float()


@pytest.mark.parametrize("precision", ["bf16", "mxfp8", "mxfp4"])
def test_expert_mlp_top1_vs_dense_torch(precision):
    """Top-1 routing with p = 1 reduces the layer to dense per-expert MLPs."""
    w = WORKLOADS["tiny"]
    inp = make_inputs(w, seed=12)
    rng = np.random.default_rng(3)
    ids = rng.integers(0, w.E, (w.T, 1)).astype(np.int32)
    probs = np.ones((w.T, 1), np.float32)
    m = oracle.Model(w.E, w.H, w.F, 1, inp["w1_bits"], inp["w2_bits"], precision)
    out, err, _ = m.forward(inp["x_bits"], ids, probs, w.T)
    assert err == 0
    xv = oracle.bf16_value(inp["x_bits"]).astype(np.float64)
    w1v = oracle.bf16_value(inp["w1_bits"]).astype(np.float64)
    w2v = oracle.bf16_value(inp["w2_bits"]).astype(np.float64)
    xv, w1v, w2v = _operand_values(precision, xv, w1v, w2v, w)
    for e in range(w.E):
        rows = np.nonzero(ids[:, 0] == e)[0]
        if len(rows) == 0:
            continue
        ref = _dense_mlp_fp64(xv[rows], w1v[e], w2v[e], w.F, precision != "bf16").numpy()
        got = out[rows]
        # independent fp64 summation orders: agree to fp32 rounding, except where a
        # rounding decision on the FC2 operand flips (rare, one operand step)
        err_rel = np.abs(got - ref) / (np.abs(ref).max() + 1e-30)
        assert np.quantile(err_rel, 0.99) < 1e-6 and err_rel.max() < 5e-3, (e, err_rel.max())


def test_gate_up_roles_and_expert_index_matter():
    """Swapping gate/up, or routing to a neighbouring expert, changes the output
    well beyond tolerance (guards against transposed or shifted operands)."""
    w = WORKLOADS["tiny"]
    inp = make_inputs(w, seed=13)
    ids, probs, _ = oracle.route(inp["logits"], w.T, w.k)
    m = oracle.Model(w.E, w.H, w.F, w.k, inp["w1_bits"], inp["w2_bits"])
    out, _, _ = m.forward(inp["x_bits"], ids, probs, w.T)
    w1s = inp["w1_bits"].copy()
    w1s[:, : w.F], w1s[:, w.F:] = inp["w1_bits"][:, w.F:], inp["w1_bits"][:, : w.F]
    out_sw, _, _ = oracle.Model(w.E, w.H, w.F, w.k, w1s, inp["w2_bits"]).forward(
        inp["x_bits"], ids, probs, w.T)
    out_sh, _, _ = m.forward(inp["x_bits"], (ids + 1) % w.E, probs, w.T)
    scale = np.linalg.norm(out)
    assert np.linalg.norm(out_sw - out) > 0.1 * scale
    assert np.linalg.norm(out_sh - out) > 0.1 * scale


@pytest.mark.parametrize("precision", ["bf16", "mxfp8", "mxfp4"])
def test_forward_vs_numpy_fp64_formulation(precision):
    """Whole layer vs an independent dense fp64 formulation (k = 2, real probs)."""
    w = WORKLOADS["tiny"]
    inp = make_inputs(w, seed=11)
    ids, probs, err = oracle.route(inp["logits"], w.T, w.k)
    assert err == 0
    m = oracle.Model(w.E, w.H, w.F, w.k, inp["w1_bits"], inp["w2_bits"], precision)
    out, err, _ = m.forward(inp["x_bits"], ids, probs, w.T)
    xv = oracle.bf16_value(inp["x_bits"]).astype(np.float64)
    w1v = oracle.bf16_value(inp["w1_bits"]).astype(np.float64)
    w2v = oracle.bf16_value(inp["w2_bits"]).astype(np.float64)
    xv, w1v, w2v = _operand_values(precision, xv, w1v, w2v, w)
    ref = np.zeros((w.T, w.H))
    for t in range(w.T):
        for j in range(w.k):
            e = ids[t, j]
            o = _dense_mlp_fp64(xv[t:t + 1], w1v[e], w2v[e], w.F, precision != "bf16")
            ref[t] += float(probs[t, j]) * o.numpy()[0].astype(np.float64)
    rel = np.linalg.norm(out - ref) / np.linalg.norm(ref)
    assert rel < 1e-5, rel


@pytest.mark.parametrize("name,precision", [("tiny", "bf16"), ("tiny", "mxfp8"), ("tiny", "mxfp4")])
def test_forward_bitwise_equals_naive_per_token_loop(name, precision):
    """Permutation bookkeeping: permuted forward == per-token loop, bitwise."""
    w = WORKLOADS[name]
    inp = make_inputs(w, seed=12, outliers=(precision == "mxfp8"))
    ids, probs, _ = oracle.route(inp["logits"], w.T, w.k)
    ids = ids[:, ::-1].copy()          # listed in descending order: canonical sort must undo
    probs = probs[:, ::-1].copy()
    m = oracle.Model(w.E, w.H, w.F, w.k, inp["w1_bits"], inp["w2_bits"], precision)
    out, _, _ = m.forward(inp["x_bits"], ids, probs, w.T)
    naive = m.forward_tokens(inp["x_bits"], ids, probs, np.arange(w.T))
    assert np.array_equal(out.view(np.uint32), naive.view(np.uint32))


def test_forward_live_prefix_and_capacity():
    """Rows past live are neither read (NaN there changes nothing) nor written."""
    w = WORKLOADS["tiny"].with_tokens(40, 64)
    inp = make_inputs(w, seed=11)
    ids, probs, _ = oracle.route(inp["logits"], w.T, w.k)
    m = oracle.Model(w.E, w.H, w.F, w.k, inp["w1_bits"], inp["w2_bits"])
    out, err, _ = m.forward(inp["x_bits"], ids, probs, w.T)
    assert err == 0 and np.all(np.isnan(out[w.T:])) and not np.any(np.isnan(out[: w.T]))
    # the first 40 tokens alone give the same bits (batch invariance of the definition)
    out2, _, _ = m.forward(inp["x_bits"][:20].copy(), ids[:20].copy(), probs[:20].copy(), 20)
    assert np.array_equal(out2.view(np.uint32), out[:20].view(np.uint32))


# ------------------------------------------------------------------ packer

def _interleave(w, F):
    """Packed FC1 row 64b+i = gate row 32b+i (i<32) or up row F+32b+i-32."""
    E, N2, H = w.shape
    rows = [32 * b + i if i < 32 else F + 32 * b + i - 32 for b in range(F // 32) for i in range(64)]
    return w[:, rows]


def _unswizzle_bf16(buf, E, N, K):
    """Inverse of the bf16 tiled layout by array reshapes, one 512-row group
    at a time: per expert, groups of w = min(32, N/16 - 32 g) column blocks,
    each group [K/32][w] blocks of [4 (k%32 / 8)][16 (n%16)][8 (k%8)]."""
    nt, KS = N // 16, K // 32
    per_e = buf.reshape(E, nt * KS * 512)
    out = np.empty((E, N, K), dtype=buf.dtype)
    for g in range((nt + 31) // 32):
        w = min(32, nt - 32 * g)
        t = per_e[:, g * 32 * KS * 512:(g * 32 + w) * KS * 512].reshape(E, KS, w, 4, 16, 8)
        out[:, g * 512:g * 512 + 16 * w] = t.transpose(0, 2, 4, 1, 3, 5).reshape(E, 16 * w, K)
    return out


def _unswizzle_mx(codes, scales, E, N, K):
    KS = (K + 127) // 128
    KQ = (KS + 3) // 4
    c = codes.reshape(E, N // 16, KS, 2, 4, 16, 16)            # e n16 step half kg r16 byte
    c = c.transpose(0, 1, 5, 2, 3, 4, 6).reshape(E, N, KS * 128)
    sc = scales.reshape(E, N // 16, KQ, 4, 16, 4)               # e n16 group kg r16 step%4
    sc = sc.transpose(0, 1, 4, 2, 5, 3).reshape(E, N, KQ * 16)
    return c, sc


def _unswizzle_mx4(codes, scales, E, N, K):
    """Inverse of the MXFP4 layout by reshapes, one 512-row group at a time:
    per expert, groups of w = min(32, N/16 - 32 g) column blocks, each group
    [KS][w] code blocks of [4 (k%128 / 32)][16 (n%16)][16 bytes] (two codes per
    byte, low nibble first) and [KQ][w] scale groups of [4 (b%4)][16 (n%16)][4
    (step%4)]."""
    KS = (K + 127) // 128
    KQ = (KS + 3) // 4
    nt = N // 16
    cb = codes.reshape(E, nt * KS * 1024)
    sb = scales.reshape(E, nt * KQ * 256)
    c = np.empty((E, N, KS * 128), dtype=np.uint8)
    sc = np.empty((E, N, KQ * 16), dtype=np.uint8)
    for g in range((nt + 31) // 32):
        w = min(32, nt - 32 * g)
        b = cb[:, g * 32 * KS * 1024:(g * 32 + w) * KS * 1024].reshape(E, KS, w, 4, 16, 16)
        nib = np.stack([b & 15, b >> 4], axis=-1)               # e step c16 kg r16 byte nibble
        c[:, g * 512:g * 512 + 16 * w] = nib.transpose(0, 2, 4, 1, 3, 5, 6).reshape(E, 16 * w, KS * 128)
        q = sb[:, g * 32 * KQ * 256:(g * 32 + w) * KQ * 256].reshape(E, KQ, w, 4, 16, 4)
        sc[:, g * 512:g * 512 + 16 * w] = q.transpose(0, 2, 4, 1, 5, 3).reshape(E, 16 * w, KQ * 16)
    return c, sc


@pytest.mark.parametrize("H,F", [(64, 96), (96, 320)])
def test_pack_bf16_layout_definition(H, F):
    """Unswizzled by reshapes, the packed buffer is the interleaved weight
    (F = 320: FC1 has 40 column blocks, one full 512-row group and one of 8)."""
    E = 2
    rng = np.random.default_rng(4)
    w1 = rng.integers(0, 65535, (E, 2 * F, H)).astype(np.uint16)
    w2 = rng.integers(0, 65535, (E, H, F)).astype(np.uint16)
    buf = oracle.pack(E, H, F, w1, w2, "bf16").view(np.uint16)
    p1 = _unswizzle_bf16(buf[: E * 2 * F * H], E, 2 * F, H)
    p2 = _unswizzle_bf16(buf[E * 2 * F * H:], E, H, F)
    assert np.array_equal(p1, _interleave(w1, F))
    assert np.array_equal(p2, w2)
    # spot checks of the block order and the lane order, written out by hand
    KS, nt = H // 32, 2 * F // 16
    # element (e=1, n=17, k=45): column block 1 of group 0, K step 1
    w0 = min(32, nt)
    idx = (1 * nt * KS + 1 * w0 + 1) * 512 + (13 // 8) * 128 + 1 * 8 + 45 % 8
    assert buf[idx] == _interleave(w1, F)[1, 17, 45]
    if nt > 32:
        # element (e=0, n=16*33+5, k=33): column block 33 = block 1 of group 1
        # (width nt - 32), K step 1, one block past the group's first
        idx = (32 * KS + 1 * (nt - 32) + 1) * 512 + (1 // 8) * 128 + 5 * 8 + 33 % 8
        assert buf[idx] == _interleave(w1, F)[0, 16 * 33 + 5, 33]


@pytest.mark.parametrize("H,F", [(64, 96), (160, 96)])
def test_pack_mxfp8_layout_definition(H, F):
    """Codes and scales, unswizzled, are the per-row quantization of the
    interleaved bf16 weight; padding past K is code 0 and scale 127."""
    E = 2
    rng = np.random.default_rng(4)
    w1 = oracle.bf16_bits(rng.standard_normal((E, 2 * F, H)).astype(np.float32))
    w2 = oracle.bf16_bits(rng.standard_normal((E, H, F)).astype(np.float32))
    buf = oracle.pack(E, H, F, w1, w2, "mxfp8")
    off = oracle.pack_mx_offsets(E, H, F)
    assert len(buf) == off[4] == oracle.pack_bytes(E, H, F, "mxfp8")
    for (codes_at, scales_at, w, N, K, fc1) in ((0, 2, w1, 2 * F, H, True),
                                                (1, 3, w2, H, F, False)):
        KS = (K + 127) // 128
        KQ = (KS + 3) // 4
        nc = E * (N // 16) * KS * 2048
        ns = E * (N // 16) * KQ * 256
        c, sc = _unswizzle_mx(buf[off[codes_at]:off[codes_at] + nc],
                              buf[off[scales_at]:off[scales_at] + ns], E, N, K)
        logical = _interleave(w, F) if fc1 else w
        qc, qs = oracle.mx_quantize(oracle.bf16_value(logical).reshape(-1, K))
        assert np.array_equal(c[:, :, :K].reshape(-1, K), qc)
        assert np.array_equal(sc[:, :, :K // 32].reshape(-1, K // 32), qs)
        assert np.all(c[:, :, K:] == 0) and np.all(sc[:, :, K // 32:] == 127)


@pytest.mark.parametrize("H,F", [(256, 128), (96, 160), (640, 320)])
def test_pack_mxfp4_layout_definition(H, F):
    """MXFP4 codes and scales, unswizzled, are the per-row E2M1 quantization of
    the interleaved bf16 weight; padding past K is code 0 and scale 127
    (H = 640, F = 320: both sections have 40 column blocks, one full 512-row
    group and one of 8, and FC1 five K steps, so two scale groups)."""
    E = 2
    rng = np.random.default_rng(5)
    w1 = oracle.bf16_bits(rng.standard_normal((E, 2 * F, H)).astype(np.float32))
    w2 = oracle.bf16_bits(rng.standard_normal((E, H, F)).astype(np.float32))
    buf = oracle.pack(E, H, F, w1, w2, "mxfp4")
    off = oracle.pack_mx_offsets(E, H, F, "mxfp4")
    assert len(buf) == off[4] == oracle.pack_bytes(E, H, F, "mxfp4")
    for (codes_at, scales_at, w, N, K, fc1) in ((0, 2, w1, 2 * F, H, True),
                                                (1, 3, w2, H, F, False)):
        KS = (K + 127) // 128
        KQ = (KS + 3) // 4
        nc = E * (N // 16) * KS * 1024
        ns = E * (N // 16) * KQ * 256
        c, sc = _unswizzle_mx4(buf[off[codes_at]:off[codes_at] + nc],
                               buf[off[scales_at]:off[scales_at] + ns], E, N, K)
        logical = _interleave(w, F) if fc1 else w
        qc, qs = oracle.mx4_quantize(oracle.bf16_value(logical).reshape(-1, K))
        assert np.array_equal(c[:, :, :K].reshape(-1, K), qc)
        assert np.array_equal(sc[:, :, :K // 32].reshape(-1, K // 32), qs)
        assert np.all(c[:, :, K:] == 0) and np.all(sc[:, :, K // 32:] == 127)
        # spot checks of the group order, written out by hand: row n = 16 c + 5
        # of the last column block, K step t = KS - 1, lane group kg = 1
        nt = N // 16
        cl = nt - 1
        g, w = cl // 32, min(32, nt - 32 * (cl // 32))
        t, kg, n = KS - 1, 1, 16 * cl + 5
        k = 128 * t + 32 * kg + 6                               # byte 3, low nibble
        if k < K:
            blk = 1 * nt * KS + g * 32 * KS + t * w + cl % 32   # expert 1
            byte = buf[off[codes_at] + blk * 1024 + (kg * 16 + 5) * 16 + 3]
            assert (byte & 15) == qc.reshape(E, N, K)[1, n, k]
            b = k // 32                                         # its scale
            grp = 1 * nt * KQ + g * 32 * KQ + (b // 16) * w + cl % 32
            assert buf[off[scales_at] + grp * 256 + ((b % 4) * 16 + 5) * 4 + (b // 4) % 4] == \
                qs.reshape(E, N, K // 32)[1, n, b]


# ------------------------------------------------------------------ apply_topk_in_fc1

def _load_fc1_topk_cases():
    with open(os.path.join(GOLDEN, "fc1_topk_cases.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("precision", ["bf16", "mxfp8", "mxfp4"])
@pytest.mark.parametrize("c", _load_fc1_topk_cases(), ids=lambda c: c["name"])
def test_fc1_topk_hand_cases(c, precision):
    """The probability applied inside FC1 (before the FC2-input rounding), the
    weighted rows summed: exact hand cases (tests/golden/make_fc1_topk_cases.py)."""
    x, ids, pr, w1, w2 = hand_case_arrays(c)
    m = oracle.Model(c["E"], c["H"], c["F"], c["k"], w1, w2, precision)
    out, err, _ = m.forward(x, ids, pr, c["live"], topk_in_fc1=True)
    assert err == 0
    assert np.array_equal(out, np.array(c["expected"][precision], np.float32))
    naive = m.forward_tokens(x, ids, pr, np.arange(c["live"]), topk_in_fc1=True)
    assert np.array_equal(naive, out[: c["live"]])
    if "default_combine_bf16" in c and precision == "bf16":
        # the default combine (probability after FC2) differs: the case pins the
        # rounding point, not just the value
        ref, _, _ = m.forward(x, ids, pr, c["live"])
        assert np.array_equal(ref, np.array(c["default_combine_bf16"], np.float32))
        assert not np.array_equal(ref, out)


def _random_case(precision, seed, probs_kind):
    w = WORKLOADS["tiny"]
    inp = make_inputs(w, seed=seed, outliers=precision != "bf16")
    ids, probs, _ = oracle.route(inp["logits"], w.T, w.k)
    rng = np.random.default_rng(seed)
    if probs_kind == "pow2":
        probs = (2.0 ** -rng.integers(0, 4, probs.shape)).astype(np.float32)
    elif probs_kind == "ones":
        probs = np.ones_like(probs)
    m = oracle.Model(w.E, w.H, w.F, w.k, inp["w1_bits"], inp["w2_bits"], precision)
    return w, inp, ids, probs, m


@pytest.mark.parametrize("precision", ["bf16", "mxfp8", "mxfp4"])
@pytest.mark.parametrize("probs_kind", ["ones", "pow2"])
def test_fc1_topk_equals_default_for_exact_scalings(precision, probs_kind):
    """Scaling by p = 1, or by a power of two, commutes with every rounding step
    (bf16 RNE, the MX block scale shifts by the same exponent, fp32 products and
    the fp32 chain), so the two placements of the probability agree bit for bit:
    out = sum_j O'_j with O'_j = p_j O_j exactly, and fma(p_j, O_j, acc) =
    acc + p_j O_j."""
    w, inp, ids, probs, m = _random_case(precision, 11, probs_kind)
    a, _, _ = m.forward(inp["x_bits"], ids, probs, w.T)
    b, _, _ = m.forward(inp["x_bits"], ids, probs, w.T, topk_in_fc1=True)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("precision", ["bf16", "mxfp8", "mxfp4"])
def test_fc1_topk_vs_dense_fp64_formulation(precision):
    """Whole layer with the probability inside FC1 vs an independent dense fp64
    formulation: the SwiGLU row scaled by p in fp32, rounded to the FC2 operand
    (torch's bf16 cast, or MX quantization), FC2 in fp64, rows summed."""
    w, inp, ids, probs, m = _random_case(precision, 12, "router")
    out, err, _ = m.forward(inp["x_bits"], ids, probs, w.T, topk_in_fc1=True)
    assert err == 0
    xv = oracle.bf16_value(inp["x_bits"]).astype(np.float64)
    w1v = oracle.bf16_value(inp["w1_bits"]).astype(np.float64)
    w2v = oracle.bf16_value(inp["w2_bits"]).astype(np.float64)
    xv, w1v, w2v = _operand_values(precision, xv, w1v, w2v, w)
    ref = np.zeros((w.T, w.H))
    for t in range(w.T):
        for j in range(w.k):
            e = ids[t, j]
            x = torch.from_numpy(xv[t:t + 1])
            w1 = torch.from_numpy(w1v[e])
            g = (x @ w1[: w.F].T).float().double()
            u = (x @ w1[w.F:].T).float().double()
            a = (g / (1.0 + torch.exp(-g)) * u).float() * float(probs[t, j])
            if precision == "bf16":
                h = a.float().to(torch.bfloat16).double()
            else:
                h = torch.from_numpy(oracle.mx_dequantize(*oracle.mx_quantize(a.float().numpy())))
            ref[t] += (h @ torch.from_numpy(w2v[e]).T).float().numpy()[0]
    rel = np.linalg.norm(out - ref) / np.linalg.norm(ref)
    assert rel < 1e-5, rel
    # and it is a different computation from the default placement
    dflt, _, _ = m.forward(inp["x_bits"], ids, probs, w.T)
    assert not np.array_equal(dflt, out)


def test_finalize_sum_is_fma_chain_with_unit_probabilities():
    """The weighted-row finalize is the fp32 FMA chain with p = 1 (fma(1, o, acc)
    = acc + o exactly), including dropped routes; its bf16 variant is torch's
    bf16 cast of the fp32 result."""
    rng = np.random.default_rng(7)
    T, k, H = 9, 5, 64
    O = (rng.standard_normal((T * k, H)) * 10.0 ** rng.integers(-3, 4, (T * k, 1))).astype(np.float32)
    dst = rng.permutation(T * k).astype(np.int32).reshape(T, k)
    dst[2, 1] = -1
    dst[5, 0] = -1
    s = oracle.finalize_sum(O, dst, H)
    f = oracle.finalize(O, dst, np.ones((T, k), np.float32), H)
    assert np.array_equal(s.view(np.uint32), f.view(np.uint32))
    b = oracle.finalize_sum(O, dst, H, to_bf16=True)
    assert np.array_equal(b, torch.from_numpy(s).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
