"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Bit-exact: the kernel-weight bytes, routing ids, the permutation indices, the
MXFP8 codes/scales and the finalize.  Floating point: outputs within relative
L2 <= 5e-3 and max |err| <= 2e-2 * max|ref| of the oracle, on the same seeded
inputs.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from workloads import WORKLOADS, Workload
from gpu_common import (Case, assert_close, live_tensor, sentinel_out, to_dev_bits,
                        SENTINEL_BITS)

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import swiglu_expert_mlp_amd  # noqa: F401  (raises if the library is missing)


def _moe():
    from swiglu_expert_mlp_amd import MoE
    return MoE


# Small workloads the oracle finishes in seconds, spanning several tiles and a
# ragged tail, with the shapes (H, F, E, k, precision) of each benchmark workload.
SMALL = {
    "tiny": WORKLOADS["tiny"],
    "decode_T64": WORKLOADS["decode"].with_tokens(64),
    "logprob_T128": WORKLOADS["logprob"].with_tokens(128),
    "mxfp8_T96": WORKLOADS["mxfp8_16k"].with_tokens(96),
    "bounded_T40_cap512": WORKLOADS["bounded_decode"].with_tokens(40, 512),
    "odd_bf16": Workload("odd_bf16", 77, 80, 96, 160, 5, 3, "bf16"),
    "odd_mxfp8": Workload("odd_mxfp8", 77, 80, 96, 160, 5, 3, "mxfp8"),
    # experts past 128 rows (LDS-staged GEMM): ragged 256-row tiles, partial
    # 256-column tiles, an odd number of 32-wide K steps in both GEMMs
    "odd_bf16_big": Workload("odd_bf16_big", 700, 720, 96, 160, 5, 3, "bf16"),
    # and an even number of K steps in both GEMMs
    "mid_bf16_big": Workload("mid_bf16_big", 600, 600, 256, 192, 4, 2, "bf16"),
    # bf16 experts of 95..121 rows: two 64-row tiles each, the first with four
    # 16-row groups, the second ragged (2..4 groups); FC1 N = 320 and FC2 N = 96
    # leave the 512-column tiles partial and FC2's last 64-column block half full
    "rows128_bf16": Workload("rows128_bf16", 220, 224, 96, 160, 4, 2, "bf16"),
    # one expert of 129 rows (a ragged 256-row tile) beside 64-row tiles in the
    # same launches
    "mixed129_bf16": Workload("mixed129_bf16", 180, 192, 96, 160, 3, 2, "bf16"),
    # token capacities above 1024, where the 256-row tiles run on the 8-wave
    # 256 x 256 kernel when K is a multiple of its 64-wide stage (below 1024,
    # or with other K, the 64-row kernel takes them as four 64-row tiles):
    # K = 96 / 160 (the 64-row kernel takes everything at this capacity too)
    "odd_bf16_big_cap": Workload("odd_bf16_big_cap", 700, 1100, 96, 160, 5, 3, "bf16"),
    "mixed129_bf16_cap": Workload("mixed129_bf16_cap", 180, 1040, 96, 160, 3, 2, "bf16"),
    # the 256 x 256 kernel: 4 stages and a partial 256-column tile (FC1 N =
    # 384), 3 stages (odd: the repeated last stage) in FC2
    "mid_bf16_big_cap": Workload("mid_bf16_big_cap", 600, 1200, 256, 192, 4, 2, "bf16"),
    # 3 and 5 stages, FC1 N = 640 (two and a half column tiles), FC2 N = 192
    # (the last quarter of the tile's columns stored by no wave), second row
    # tiles of 150..190 rows (the lower waves partly past the rows)
    "odd64_bf16_big_cap": Workload("odd64_bf16_big_cap", 700, 1100, 192, 320, 5, 3, "bf16"),
    # second row tiles of under 128 rows (the lower waves wholly past them and
    # idle), 2 stages in FC1, FC2 N = 128
    "idle_bf16_big_cap": Workload("idle_bf16_big_cap", 700, 1100, 128, 192, 4, 2, "bf16"),
    # an expert of 129 rows beside two of 64-row tiles, both kernels in one stage
    "mixed129_64_cap": Workload("mixed129_64_cap", 182, 1040, 128, 192, 3, 2, "bf16"),
    # MXFP8 experts past 128 rows with K a multiple of 128 (LDS-staged kernel):
    # ragged 256-row tiles, a partial 256-column tile, 2 and 3 K steps
    "mx_big": Workload("mx_big", 600, 600, 256, 384, 4, 2, "mxfp8"),
    # MXFP4 weights: the 64-row LDS-staged kernel (K a multiple of 128; in mx4_big
    # it also takes the larger experts as 64-row tiles, with partial 512-column
    # tiles, 2 and 3 K steps), and the streaming tiles in odd_mxfp4 (K = 96)
    "decode_mx4_T64": WORKLOADS["decode_mxfp4"].with_tokens(64),
    "mx4_T96": WORKLOADS["mxfp4_16k"].with_tokens(96),
    "odd_mxfp4": Workload("odd_mxfp4", 77, 80, 96, 160, 5, 3, "mxfp4"),
    "mx4_big": Workload("mx4_big", 600, 600, 256, 384, 4, 2, "mxfp4"),
    # MXFP4 with one K step in both GEMMs (K = 128): only the prologue's and
    # the tail's steps of the 64-row kernel, 256-column tiles
    "mx4_k128": Workload("mx4_k128", 70, 72, 128, 128, 6, 2, "mxfp4"),
    # MXFP4 with H = 160: FC1 (K = 160) on the streaming tiles, FC2 (K = 256) on
    # the 64-row LDS kernel with N = 160, its last 64-column block half full
    "mx4_h160": Workload("mx4_h160", 60, 64, 160, 256, 4, 2, "mxfp4"),
}

_cases = {}


def get_case(name, seed=11):
    key = (name, seed)
    if key not in _cases:
        _cases[key] = Case(SMALL[name], seed=seed, outliers=SMALL[name].precision != "bf16")
    return _cases[key]


def run_gpu(case, T_cap=None, live=None, moe=None):
    w = case.w
    MoE = _moe()
    if moe is None:
        moe = MoE(w.E, w.H, w.F, w.k, w.precision)
        w1, w2 = case.weights_dev()
        moe.load_weights(w1, w2)
    x, ids, probs = case.dev()
    ws = moe.new_workspace(w.T_cap)
    out = sentinel_out(w.T_cap, w.H)
    moe.forward(x, ids, probs, live_tensor(w.T if live is None else live), out=out, ws=ws)
    torch.cuda.synchronize()
    return moe, ws, out.cpu().numpy()


# ------------------------------------------------------------------ hand cases

def _hand_cases():
    with open(os.path.join(GOLDEN, "hand_cases.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("precision", ["bf16", "mxfp8", "mxfp4"])
@pytest.mark.parametrize("c", _hand_cases(), ids=lambda c: c["name"])
def test_hand_cases_exact(c, precision):
    from test_oracle_pins import hand_case_arrays
    x, ids, pr, w1, w2 = hand_case_arrays(c)
    MoE = _moe()
    moe = MoE(c["E"], c["H"], c["F"], c["k"], precision)
    moe.load_weights(to_dev_bits(w1), to_dev_bits(w2))
    out = sentinel_out(c["T_cap"], c["H"])
    ws = moe.new_workspace(c["T_cap"])
    moe.forward(to_dev_bits(x), torch.from_numpy(ids).cuda(), torch.from_numpy(pr).cuda(),
                live_tensor(c["live"]), out=out, ws=ws)
    got = out.cpu().numpy()
    # the hand-case operands (one-hot x, small integers, powers of two, 32) are
    # exact in E4M3 and E2M1 with their block scales too, so every precision is exact
    for t, row in enumerate(c["expected"]):
        if row is None:
            assert np.all(got[t].view(np.uint32) == SENTINEL_BITS), f"row {t} past live written"
        else:
            assert np.array_equal(got[t], np.array(row, np.float32)), (t, got[t][:8], row[:8])
    assert moe.check(ws) == 0


# ------------------------------------------------------------------ packer

@pytest.mark.parametrize("precision", ["bf16", "mxfp8", "mxfp4"])
@pytest.mark.parametrize("name", ["tiny", "odd_bf16", "bounded_T40_cap512"])
def test_pack_bytes_bitwise(name, precision):
    c = get_case(name)
    w = c.w
    moe = _moe()(w.E, w.H, w.F, w.k, precision)
    w1, w2 = c.weights_dev()
    kbuf = moe.load_weights(w1, w2)
    torch.cuda.synchronize()
    ref = oracle.pack(w.E, w.H, w.F, c.inp["w1_bits"], c.inp["w2_bits"], precision)
    got = kbuf.cpu().numpy()
    assert got.shape == ref.shape
    # every defined section bit for bit, its K padding included (the bytes that
    # round a section up to 256 are unspecified)
    n1, n2 = w.E * 2 * w.F * w.H, w.E * w.H * w.F
    if precision == "bf16":
        sections = [(0, 2 * (n1 + n2))]
    else:
        off = oracle.pack_mx_offsets(w.E, w.H, w.F, precision)
        KS = lambda K: (K + 127) // 128
        blk = 2048 if precision == "mxfp8" else 1024
        sizes = [w.E * (2 * w.F // 16) * KS(w.H) * blk, w.E * (w.H // 16) * KS(w.F) * blk,
                 w.E * (2 * w.F // 16) * ((KS(w.H) + 3) // 4) * 256,
                 w.E * (w.H // 16) * ((KS(w.F) + 3) // 4) * 256]
        sections = [(off[i], off[i] + sizes[i]) for i in range(4)]
    for a, b in sections:
        assert np.array_equal(got[a:b], ref[a:b]), (a, b)


# ------------------------------------------------------------------ router

@pytest.mark.parametrize("name", ["tiny", "decode_T64", "logprob_T128", "bounded_T40_cap512",
                                  "odd_bf16"])
def test_route_ids_bitwise_probs_close(name):
    c = get_case(name)
    w = c.w
    moe = _moe()(w.E, w.H, w.F, w.k, "bf16")
    logits = torch.from_numpy(c.inp["logits"]).cuda()
    ids = torch.full((w.T_cap, w.k), -5, dtype=torch.int32, device="cuda")
    probs = torch.full((w.T_cap, w.k), -5.0, dtype=torch.float32, device="cuda")
    ws = moe.new_workspace(w.T_cap)
    moe.route(logits, live_tensor(w.T), ids=ids, probs=probs, ws=ws)
    gi, gp = ids.cpu().numpy(), probs.cpu().numpy()
    ri, rp, _ = oracle.route(c.inp["logits"], w.T, w.k)
    assert np.array_equal(gi[: w.T], ri[: w.T])
    np.testing.assert_allclose(gp[: w.T], rp[: w.T], rtol=2e-6, atol=1e-7)
    assert np.all(gi[w.T:] == -5) and np.all(gp[w.T:] == -5.0), "rows past live were written"
    assert moe.check(ws) == 0


def test_route_ties_go_to_lower_id():
    E, k, T = 64, 4, 8
    lg = np.zeros((T, E), np.float32)
    lg[1, [5, 9, 40, 41, 63]] = 3.0
    lg[2, :] = np.float32(-1.0)
    lg[3, ::7] = 2.0
    moe = _moe()(E, 32, 32, k, "bf16")
    ids, probs = moe.route(torch.from_numpy(lg).cuda(), live_tensor(T))
    ri, rp, _ = oracle.route(lg, T, k)
    assert np.array_equal(ids.cpu().numpy(), ri)
    np.testing.assert_allclose(probs.cpu().numpy(), rp, rtol=2e-6)


@pytest.mark.parametrize("E,k", [(40, 5), (200, 16), (1024, 16)])
def test_route_edge_values_and_threshold_ties(E, k):
    """Logits drawn from a handful of values (many ties at the k-th place),
    with -0 and +0, subnormals of both signs and -inf among them; E not a
    multiple of the wave width except for 1024.  Ids must match the oracle's
    sort on (-logit, id) bit for bit (-0 and +0 compare equal there too)."""
    T = 96
    rng = np.random.default_rng(E + k)
    # three larger logits per row, the rest from small sets, so that the k-th
    # place falls among the zeros (even rows) or the positive subnormals (odd)
    lo_a = np.array([0.0, -0.0, -1e-40, -2.0, -np.inf], np.float32)
    lo_b = np.array([1e-40, 1e-40, 0.0, -0.0, -1e-40, -np.inf], np.float32)
    lg = np.where((np.arange(T) % 2 == 0)[:, None], rng.choice(lo_a, size=(T, E)),
                  rng.choice(lo_b, size=(T, E))).astype(np.float32)
    for t in range(T):
        a, b = rng.choice(E, size=2, replace=False)
        lg[t, a], lg[t, b] = 7.0, 3.25
    lg[:, E // 2] = np.float32(0.5)            # every row has a finite largest logit
    moe = _moe()(E, 32, 32, k, "bf16")
    ids, probs = moe.route(torch.from_numpy(lg).cuda(), live_tensor(T))
    ri, rp, _ = oracle.route(lg, T, k)
    assert np.array_equal(ids.cpu().numpy(), ri)
    np.testing.assert_allclose(probs.cpu().numpy(), rp, rtol=2e-6, atol=1e-30)


# ------------------------------------------------------------------ permutation

@pytest.mark.parametrize("name", ["tiny", "decode_T64", "logprob_T128", "bounded_T40_cap512",
                                  "odd_bf16"])
def test_indices_bitwise(name):
    c = get_case(name)
    w = c.w
    moe, ws, _ = run_gpu(c)
    got = moe.get_indices(ws, w.T_cap)
    ref = oracle.prepare(c.ids, c.probs, w.T, w.E)
    assert got["T"] == ref["T"] == w.T
    assert np.array_equal(got["counts"], ref["counts"])
    assert np.array_equal(got["offsets"], ref["offsets"])
    assert np.array_equal(got["perm_src"], ref["perm_src"])
    assert np.array_equal(got["dst"], ref["dst"])


def test_indices_many_chunks_and_skew():
    """More than one 256-token chunk, one hot expert and empty experts."""
    w = Workload("skew", 700, 700, 64, 64, 16, 4, "bf16")
    rng = np.random.default_rng(2)
    ids = np.stack([rng.permutation(16)[:4] for _ in range(w.T)]).astype(np.int32)
    ids[::3, 0] = 7          # expert 7 is hot
    for t in range(0, w.T, 3):
        row = ids[t]
        if len(set(row.tolist())) < 4:
            ids[t] = [7, 8, 9, 10]
    ids[ids == 3] = 4        # expert 3 is empty
    for t in range(w.T):
        if len(set(ids[t].tolist())) < 4:
            ids[t] = [7, 8, 9, 10]
    probs = rng.random((w.T, 4)).astype(np.float32)
    moe = _moe()(16, 64, 64, 4, "bf16")
    moe.load_weights(torch.zeros((16, 128, 64), dtype=torch.bfloat16, device="cuda"),
                     torch.zeros((16, 64, 64), dtype=torch.bfloat16, device="cuda"))
    ws = moe.new_workspace(w.T_cap)
    moe.forward(torch.zeros((w.T, 64), dtype=torch.bfloat16, device="cuda"),
                torch.from_numpy(ids).cuda(), torch.from_numpy(probs).cuda(), live_tensor(w.T),
                ws=ws)
    got = moe.get_indices(ws, w.T_cap)
    ref = oracle.prepare(ids, probs, w.T, 16)
    for key in ("counts", "offsets", "perm_src", "dst"):
        assert np.array_equal(got[key], ref[key]), key
    assert got["counts"][3] == 0


# ------------------------------------------------------------------ finalize

@pytest.mark.parametrize("name", ["tiny", "decode_T64", "bounded_T40_cap512"])
def test_finalize_bitwise_on_gpu_rows(name):
    """The GPU finalize equals the oracle's fp32 FMA chain applied to the GPU's
    own FC2 rows, bit for bit."""
    c = get_case(name)
    w = c.w
    moe, ws, out = run_gpu(c)
    idx = moe.get_indices(ws, w.T_cap)
    rows = moe.get_rows(ws, w.T_cap, idx["n_rows"], idx["T"])
    ref = oracle.finalize(rows["fc2_rows"], idx["dst"], rows["sorted_probs"], w.H)
    assert np.array_equal(out[: w.T].view(np.uint32), ref.view(np.uint32))
    assert np.all(out[w.T:].view(np.uint32) == SENTINEL_BITS)


# ------------------------------------------------------------------ forward

@pytest.mark.parametrize("name", list(SMALL))
def test_forward_parity_small(name):
    c = get_case(name)
    w = c.w
    moe, ws, out = run_gpu(c)
    ref, err, extras = c.oracle_model().forward(c.inp["x_bits"], c.ids, c.probs, w.T,
                                                want_rows=True)
    assert err == 0 and moe.check(ws) == 0
    assert_close(out[: w.T], ref[: w.T], name)
    assert np.all(out[w.T:].view(np.uint32) == SENTINEL_BITS), "rows past live were written"
    # intermediate rows: FC2 operand and FC2 output in grouped order
    idx = moe.get_indices(ws, w.T_cap)
    rows = moe.get_rows(ws, w.T_cap, idx["n_rows"], idx["T"])
    n = idx["n_rows"]
    assert_close(rows["fc2_rows"], extras["O"][:n], name + " fc2 rows")
    if w.precision == "bf16":
        h = oracle.bf16_value(rows["fc1_out"])
    else:
        h = oracle.mx_dequantize(rows["fc1_codes"], rows["fc1_scales"])
    assert_close(h, extras["H"][:n], name + " swiglu rows")
