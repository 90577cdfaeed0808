"""K2, the MXFP8 activation quantization, bit for bit against the oracle.

cudnn-frontend PR #448 (MoeEp, MXFP8 = E4M3 data with one E8M0 scale per 32
elements) and the MXFP8 workload's scale rule (the power-of-two ceiling of a
block's max magnitude / 448): the E4M3 codes and E8M0 scale bytes the GPU
writes for the live tokens' x rows must equal oracle.mx_quantize of the same
bf16 values, byte for byte.  The special blocks cover what end-to-end
tolerance parity cannot see: an all-zero block, exact E4M3 ties (17, 19, 21
with amax 448: spacing 2 in [16, 32), ties to the even code), a block whose
max sits just past the scale boundary (450 > 448: scale 2^1), bf16 subnormals, blocks
whose scale clamps at 2^-127, negative zero, and the 30x outlier tokens.
"""
import numpy as np
import pytest
import torch

import oracle
from workloads import WORKLOADS, Workload
from gpu_common import Case, live_tensor, sentinel_out, to_dev_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import swiglu_expert_mlp_amd  # noqa: F401


def _bf16_bits(vals) -> np.ndarray:
    """float values -> bf16 bit patterns (the values below are all exact in bf16)."""
    v = np.asarray(vals, dtype=np.float32)
    b = (v.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal((b.astype(np.uint32) << 16).view(np.float32), v), "not exact in bf16"
    return b


def _special_rows(H: int) -> np.ndarray:
    """Rows of H bf16 values made of hand-picked 32-blocks."""
    assert H % 32 == 0
    blocks = []
    blocks.append(np.zeros(32, np.uint16))                                     # all zero -> scale byte 0
    b = np.zeros(32, np.float32); b[:4] = [448.0, 17.0, 19.0, 21.0]; b[4:8] = [-17, -19, -21, -23]
    blocks.append(_bf16_bits(b))                                               # ties at scale 2^0
    b = np.zeros(32, np.float32); b[0] = 450.0; b[1] = 226.0; b[2] = -450.0
    blocks.append(_bf16_bits(b))                                               # scale 2^1: 225 -> 224, 113 -> 112
    b = np.linspace(-2.0, 2.0, 32).astype(np.float32)
    blocks.append(_bf16_bits(np.round(b * 16) / 16))                           # amax 2 -> scale 2^-7
    sub = np.array([1, 2, 3, 0x7F, 0x40, 0x8001, 0x807F, 0] * 4, np.uint16)   # bf16 subnormals
    blocks.append(sub)
    tiny = np.full(32, 0x0080, np.uint16); tiny[::3] = 0x8100                  # 2^-126 .. 2^-125: scale clamps
    blocks.append(tiny)
    negz = np.full(32, 0x8000, np.uint16); negz[5] = 0x3F80                    # -0 beside 1.0
    blocks.append(negz)
    big = _bf16_bits(np.array([2.0 ** 100, -(2.0 ** 99), 3.0 * 2.0 ** 90] + [1.0] * 29, np.float32))
    blocks.append(big)                                                         # large exponents
    rows = []
    nb = H // 32
    for r in range(max(1, (len(blocks) + nb - 1) // nb) + 1):
        row = [blocks[(r * nb + j) % len(blocks)] for j in range(nb)]
        rows.append(np.concatenate(row))
    return np.stack(rows)


def _gpu_quant(w, x_bits, ids, probs, T):
    """Run the forward and return the GPU's activation codes and scales."""
    from swiglu_expert_mlp_amd import MoE
    m = MoE(w.E, w.H, w.F, w.k, w.precision)
    g = torch.Generator(device="cuda").manual_seed(5)
    w1 = (torch.randn((w.E, 2 * w.F, w.H), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    w2 = (torch.randn((w.E, w.H, w.F), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    m.load_weights(w1, w2)
    ws = m.new_workspace(x_bits.shape[0])
    out = sentinel_out(x_bits.shape[0], w.H)
    m.forward(to_dev_bits(x_bits), torch.from_numpy(ids).cuda(), torch.from_numpy(probs).cuda(),
              live_tensor(T), out=out, ws=ws)
    torch.cuda.synchronize()
    idx = m.get_indices(ws, x_bits.shape[0])
    rows = m.get_rows(ws, x_bits.shape[0], idx["n_rows"], idx["T"])
    assert idx["T"] == T
    return rows["x_codes"], rows["x_scales"]


def _check(x_bits, T, codes, scales):
    ref_c, ref_s = oracle.mx_quantize(oracle.bf16_value(x_bits[:T]))
    assert codes.shape == ref_c.shape and scales.shape == ref_s.shape
    bad_s = np.argwhere(scales != ref_s)
    assert bad_s.size == 0, f"{len(bad_s)} scale bytes differ, first at {bad_s[0]}"
    bad_c = np.argwhere(codes != ref_c)
    assert bad_c.size == 0, f"{len(bad_c)} codes differ, first at {bad_c[0]}"


@pytest.mark.parametrize("precision", ["mxfp8", "mxfp4"])
@pytest.mark.parametrize("H", [96, 2048])
def test_special_blocks_bitwise(precision, H):
    rows = _special_rows(H)
    T = rows.shape[0]
    w = Workload("quant_special", T, T + 3, H, 128, 4, 2, precision)
    x = np.full((T + 3, H), 0x7FC0, np.uint16)          # bf16 NaN past live: never read
    x[:T] = rows
    ids = np.tile(np.array([[0, 1]], np.int32), (T + 3, 1))
    probs = np.full((T + 3, 2), 0.5, np.float32)
    print(f"[quant_x] special blocks {precision} H={H} T={T}", flush=True)
    codes, scales = _gpu_quant(w, x, ids, probs, T)
    _check(x, T, codes, scales)
    # the hand values themselves: the tie block at scale 2^0 and the 449 block
    nb = H // 32
    flat_c = codes.reshape(-1, 32)
    flat_s = scales.reshape(-1)
    assert flat_s[0] == 0 and np.all(flat_c[0] == 0)
    assert flat_s[1] == 127
    dec = [oracle.e4m3_decode(c) for c in flat_c[1][:8]]
    assert dec == [448.0, 16.0, 20.0, 20.0, -16.0, -20.0, -20.0, -24.0]
    assert flat_s[2] == 128
    assert [oracle.e4m3_decode(c) for c in flat_c[2][:3]] == [224.0, 112.0, -224.0]
    assert nb >= 3


@pytest.mark.parametrize("name", ["mxfp8_T96", "odd_mxfp8", "mxfp8_16k"])
def test_activation_codes_bitwise(name):
    w = {"mxfp8_T96": WORKLOADS["mxfp8_16k"].with_tokens(96),
         "odd_mxfp8": Workload("odd_mxfp8", 77, 80, 96, 160, 5, 3, "mxfp8"),
         "mxfp8_16k": WORKLOADS["mxfp8_16k"]}[name]
    print(f"[quant_x] {name}: T={w.T} H={w.H}", flush=True)
    c = Case(w, seed=11, outliers=True, weights=False)
    codes, scales = _gpu_quant(w, c.inp["x_bits"], c.ids, c.probs, w.T)
    _check(c.inp["x_bits"], w.T, codes, scales)
