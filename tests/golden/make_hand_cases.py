"""Write hand_cases.json: tiny routed-MoE cases whose outputs are exact by construction.

The source pages print no worked numeric example of the MoE forward, so these
cases are built so that the expected output follows in closed form from the
method's definition, independent of exp() accuracy and of any implementation:

* Every gate entry is 32 and every x row is one-hot, so the gate pre-activation
  is g = 32 and silu(g) = g / (1 + exp(-g)) = 32 exactly in fp32 (exp(-32) is
  far below half an ulp of 1).  The SwiGLU output is then 32 * u with u an
  integer, exact in bf16.
* Up and down weights are small integers (or powers of two), so both GEMMs
  are exact sums of integers and the fp32 outputs are exact.
* Routing probabilities are 1, 1/4 or 3/4, so the fp32 finalize is exact
  except where a case is built to exercise its rounding (HC4).

Run ``python tests/golden/make_hand_cases.py`` to regenerate.  It uses only
integer/float arithmetic written here: no oracle call, no GPU code.

Sources for the rules the cases exercise (web pages):
  Megatron-LM PR #7830 (flashinfer_mega backend), "1. Mega backend for
    generation": routes summed in canonical (ascending expert id) order; SwiGLU
    experts with gate and up stacked in one weight.
  Megatron-LM PR #7798 (moe_training_matches_inference), "What is changed":
    finalize = fp32 fused multiply-adds of probability and row, from zero.
  Megatron-LM PR #8367 (bound the MoE expert kernels by token count),
    "Problem": work bounded by a device-side live token count; fp32 output.
"""
import json
import os

H = F = 32
GATE = 32.0


def up_weight(e, n, h):
    return float(((3 * e + n + 2 * h) % 5) - 2)        # in {-2..2}


def down_weight(e, m, n):
    return float(((e + m + 3 * n) % 3) - 1)            # in {-1, 0, 1}


def expert_weights(E):
    w1 = [[[GATE] * H for _ in range(F)] + [[up_weight(e, n, h) for h in range(H)]
                                             for n in range(F)] for e in range(E)]
    w2 = [[[down_weight(e, m, n) for n in range(F)] for m in range(H)] for e in range(E)]
    return w1, w2


def expert_out(w1, w2, e, hot):
    """FC2 output row of expert e for the one-hot x at position `hot`."""
    u = [w1[e][F + n][hot] for n in range(F)]
    hvec = [GATE * un for un in u]                      # silu(32) * u = 32 u
    return [sum(hvec[n] * w2[e][m][n] for n in range(F)) for m in range(H)]


def onehot(h):
    return [1.0 if i == h else 0.0 for i in range(H)]


def case(name, cite, derivation, E, k, T_cap, live, x, ids, probs, w1, w2, expected,
         precision="bf16"):
    return dict(name=name, cite=cite, derivation=derivation, E=E, H=H, F=F, k=k,
                T_cap=T_cap, live=live, precision=precision, x=x, ids=ids, probs=probs,
                w1=w1, w2=w2, expected=expected)


def main():
    cases = []
    FIN = "Megatron-LM PR #7798, 'What is changed' (fp32 FMA of probability and row, from zero)"
    ORD = "Megatron-LM PR #7830, '1. Mega backend for generation' (canonical expert-id order)"
    LIVE = "Megatron-LM PR #8367, 'Problem' (work bounded by the device-side live count)"

    # HC1: k = 1, each token to its own expert, p = 1 -> integer outputs.
    w1, w2 = expert_weights(2)
    exp = [expert_out(w1, w2, 0, 0), expert_out(w1, w2, 1, 1)]
    cases.append(case("HC1_top1_integer", FIN,
                      "out[t] = W2_e (32 * u_e(x_t)) with e = t; every term an exact integer",
                      2, 1, 2, 2, [onehot(0), onehot(1)], [[0], [1]], [[1.0], [1.0]],
                      w1, w2, exp))

    # HC2: k = 2, probabilities 1/4 and 3/4 -> exact quarter-integers.
    exp = []
    for t in range(2):
        o0, o1 = expert_out(w1, w2, 0, t), expert_out(w1, w2, 1, t)
        exp.append([0.25 * a + 0.75 * b for a, b in zip(o0, o1)])
    cases.append(case("HC2_top2_quarters", FIN,
                      "out[t] = fma(3/4, O_1, fma(1/4, O_0, 0)); quarter-integers, exact",
                      2, 2, 2, 2, [onehot(0), onehot(1)], [[0, 1], [0, 1]],
                      [[0.25, 0.75], [0.25, 0.75]], w1, w2, exp))

    # HC3: HC2 with each token's routes listed in descending id order.
    cases.append(case("HC3_listed_order_irrelevant", ORD,
                      "same routes as HC2 listed as (1, 0); canonical sort makes it bitwise HC2",
                      2, 2, 2, 2, [onehot(0), onehot(1)], [[1, 0], [1, 0]],
                      [[0.75, 0.25], [0.75, 0.25]], w1, w2, exp))

    # HC4: three routes contributing +2^24, +1, -2^24 (ascending id).  In ascending
    # id order the fp32 chain gives 2^24 (2^24 + 1 rounds to even), then 0.  Any
    # order that adds +1 last gives 1.
    E4 = 3
    w1 = [[[GATE] * H for _ in range(F)] + [[1.0 if (n == 0 and h == 0) else 0.0
                                              for h in range(H)] for n in range(F)]
          for _ in range(E4)]
    col = [2.0 ** 19, 2.0 ** -5, -(2.0 ** 19)]      # times h[0] = 32 -> 2^24, 1, -2^24
    w2 = [[[col[e] if n == 0 else 0.0 for n in range(F)] for m in range(H)] for e in range(E4)]
    cases.append(case("HC4_order_pins_rounding", FIN + "; " + ORD,
                      "contributions +2^24 (id 0), +1 (id 1), -2^24 (id 2); ascending-id fp32 "
                      "FMA chain from +0 gives 0 (any other order that adds +1 last gives 1)",
                      E4, 3, 1, 1, [onehot(0)], [[2, 0, 1]], [[1.0, 1.0, 1.0]], w1, w2,
                      [[0.0] * H]))

    # HC6: capacity 8, live 3; rows 3..7 hold NaN x and NaN-pattern ids/probs and
    # must be neither read nor written (expected None = left untouched).
    w1, w2 = expert_weights(2)
    x = [onehot(t % H) for t in range(3)] + [[float("nan")] * H for _ in range(5)]
    ids = [[t % 2] for t in range(3)] + [[None]] * 5
    probs = [[1.0]] * 3 + [[None]] * 5
    exp = [expert_out(w1, w2, t % 2, t % H) for t in range(3)] + [None] * 5
    cases.append(case("HC6_live_prefix_only", LIVE,
                      "rows < live as HC1; rows >= live untouched (None); NaN inputs past live "
                      "must not be read", 2, 1, 8, 3, x, ids, probs, w1, w2, exp))

    # HC7: every route to expert 2 of 4; the other experts are empty.
    E7 = 4
    w1, w2 = expert_weights(E7)
    exp = [expert_out(w1, w2, 2, t) for t in range(8)]
    cases.append(case("HC7_one_expert_takes_all", FIN,
                      "all 8 tokens route to expert 2 with p = 1; experts 0, 1, 3 receive no rows",
                      E7, 1, 8, 8, [onehot(t) for t in range(8)], [[2]] * 8, [[1.0]] * 8,
                      w1, w2, exp))

    # HC8: live = 0 -> nothing is written.
    w1, w2 = expert_weights(2)
    cases.append(case("HC8_live_zero", LIVE, "live count 0: every output row untouched",
                      2, 1, 4, 0, [onehot(t) for t in range(4)], [[0]] * 4, [[1.0]] * 4,
                      w1, w2, [None] * 4))

    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hand_cases.json")
    with open(path, "w") as f:
        json.dump(dict(
            about="Routed SwiGLU MoE hand cases, exact by construction; see make_hand_cases.py",
            cases=cases), f, separators=(",", ":"), allow_nan=True)
    print(f"wrote {len(cases)} cases to {path}")

    # HC5: the MXFP8 block-quantization cases (fp32 block -> E8M0 scale byte, E4M3 codes).
    mx = [
        dict(name="amax2", cite="MXFP8: one E8M0 scale per 32 elements, scale = power-of-two "
             "ceiling of amax/448", block=[1.0, 2.0] + [0.0] * 30,
             scale_exp=-7, values=[1.0, 2.0] + [0.0] * 30,
             derivation="448 * 2^-8 = 1.75 < 2 <= 448 * 2^-7 = 3.5; 1 and 2 are exact"),
        dict(name="amax448", cite="as above", block=[448.0, -448.0] + [1.0] * 30,
             scale_exp=0, values=[448.0, -448.0] + [1.0] * 30,
             derivation="448 <= 448 * 2^0 and > 448 * 2^-1"),
        dict(name="amax449", cite="as above", block=[449.0] + [0.0] * 31,
             scale_exp=1, values=[448.0] + [0.0] * 31,
             derivation="449 > 448, so e = 1; 449 / 2 = 224.5 lies between E4M3 neighbours "
                        "224 and 240 (spacing 16 in [128, 256)) and rounds to 224; 224 * 2 = 448"),
        dict(name="amax0", cite="as above", block=[0.0] * 32, scale_exp=-127,
             values=[0.0] * 32, derivation="an all-zero block takes the smallest scale, byte 0"),
        dict(name="tie_to_even", cite="as above",
             block=[448.0, 17.0, 19.0, 21.0, 0.5 * 2.0 ** -9, 1.5 * 2.0 ** -9] + [0.0] * 26,
             scale_exp=0, values=[448.0, 16.0, 20.0, 20.0, 0.0, 2.0 * 2.0 ** -9] + [0.0] * 26,
             derivation="spacing 2 in [16, 32): 17 -> 16, 19 -> 20, 21 -> 20 (ties to the "
                        "even code); subnormal spacing 2^-9: 0.5 ulp -> 0, 1.5 ulp -> 2 ulp"),
    ]
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "mx_blocks.json")
    with open(path, "w") as f:
        json.dump(dict(about="MXFP8 block quantization hand cases; see make_hand_cases.py",
                       cases=mx), f, indent=1)
    print(f"wrote {len(mx)} MXFP8 cases to {path}")


if __name__ == "__main__":
    main()
