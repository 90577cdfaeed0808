"""Write fc1_topk_cases.json: hand cases of the apply_topk_in_fc1 option.

cudnn-frontend PR #448 gives MoeEp an ``apply_topk_in_fc1`` constructor flag
(default on) without spelling out its arithmetic.  The reading taken here:
a route's probability multiplies its SwiGLU row in fp32 inside the FC1
epilogue, before the FC2-input rounding (bf16 nearest even, or the MXFP8
requantization per 32-block), and the finalize then adds the (already
weighted) FC2 rows as an fp32 chain from +0 in canonical order.

Two cases, exact by construction (no oracle call, no GPU code; values and
derivations are written out below):

* FC1TK_rounding_point: one token, one route with p = 3/4, a one-hot x whose
  gate pre-activation is 32 (silu(32) = 32 in fp32) and whose up value is
  u = 2^-5 + 2^-12, so the SwiGLU value is h = 1 + 2^-7 exactly.  With the
  probability applied inside FC1, p * h = 0.755859375 is rounded to bf16
  before FC2: 0.755859375 = 1.51171875 * 2^-1 lies exactly halfway between
  the bf16 neighbours 1.5078125 * 2^-1 and 1.515625 * 2^-1 and goes to the even
  mantissa, 0.7578125.  With the probability applied after FC2 (the default
  combine) the result would be 0.75 * 1.0078125 = 0.755859375, so the case
  pins where the multiply happens.  Every W2 entry of column 0 is 1 (others
  0), so each output equals that operand value.
  MXFP8: x and the gate weights are exact in E4M3; the up weight u =
  1.0078125 * 2^-5 takes scale 2^-13 and becomes 258 -> 256 (E4M3 spacing 32
  in [256, 512)), i.e. u = 2^-5; then h = 1, p * h = 0.75, exact in E4M3 with
  scale 2^-9 (384); output 0.75.  MXFP4 weights: u's block scale is 2^-7
  (6 * 2^-8 < u <= 6 * 2^-7), u / 2^-7 = 4.03 -> E2M1 4, u = 2^-5 again; h = 1,
  output 0.75.
* FC1TK_quarters: the two-expert, top-2 case with p = (1/4, 3/4) and small
  integer weights: every intermediate is exact in every precision, so the
  result equals the default combine's exact quarter-integers.

Run ``python tests/golden/make_fc1_topk_cases.py`` to regenerate.
"""
import json
import os

H = F = 32
GATE = 32.0


def up_weight(e, n, h):
    return float(((3 * e + n + 2 * h) % 5) - 2)        # in {-2..2}


def down_weight(e, m, n):
    return float(((e + m + 3 * n) % 3) - 1)            # in {-1, 0, 1}


def onehot(h):
    return [1.0 if i == h else 0.0 for i in range(H)]


def main():
    cases = []
    cite = ("cudnn-frontend PR #448, MoeEp constructor (apply_topk_in_fc1); "
            "Megatron-LM PR #7798, 'Background' (FC2-input conversion in the FC1 epilogue)")

    # rounding point
    u0 = 2.0 ** -5 + 2.0 ** -12
    w1 = [[[GATE] * H for _ in range(F)] +
          [[u0 if (n == 0 and h == 0) else 0.0 for h in range(H)] for n in range(F)]]
    w2 = [[[1.0 if n == 0 else 0.0 for n in range(F)] for m in range(H)]]
    hval = GATE * u0                                   # 1 + 2^-7
    assert hval == 1.0 + 2.0 ** -7
    ph = 0.75 * hval                                   # 0.755859375, exact in binary64
    assert ph == 0.755859375
    bf16_val = 0.7578125                               # the even bf16 neighbour (see above)
    cases.append(dict(
        name="FC1TK_rounding_point", cite=cite,
        derivation="h = 32 * (2^-5 + 2^-12) = 1 + 2^-7; p * h = 0.755859375 is a bf16 tie "
                   "between 0.75390625 and 0.7578125 and goes to the even mantissa; MXFP8 "
                   "and MXFP4 weights quantize u to 2^-5, so h = 1 and the result is 0.75",
        E=1, H=H, F=F, k=1, T_cap=1, live=1, x=[onehot(0)], ids=[[0]], probs=[[0.75]],
        w1=w1, w2=w2,
        expected={"bf16": [[bf16_val] * H], "mxfp8": [[0.75] * H], "mxfp4": [[0.75] * H]},
        default_combine_bf16=[[0.75 * hval] * H]))

    # quarters: exact everywhere, equals the default combine
    E = 2
    w1 = [[[GATE] * H for _ in range(F)] + [[up_weight(e, n, h) for h in range(H)]
                                             for n in range(F)] for e in range(E)]
    w2 = [[[down_weight(e, m, n) for n in range(F)] for m in range(H)] for e in range(E)]

    def weighted_row(e, hot, p):
        hvec = [p * GATE * w1[e][F + n][hot] for n in range(F)]   # 8 u or 24 u: exact
        return [sum(hvec[n] * w2[e][m][n] for n in range(F)) for m in range(H)]

    exp = []
    for t in range(2):
        r0, r1 = weighted_row(0, t, 0.25), weighted_row(1, t, 0.75)
        exp.append([a + b for a, b in zip(r0, r1)])
    cases.append(dict(
        name="FC1TK_quarters", cite=cite,
        derivation="p * 32 * u in {8 u, 24 u} with u in -2..2 is exact in bf16, E4M3 and at "
                   "E2M1-exact weights; FC2 sums of integers are exact; out = O'_0 + O'_1",
        E=E, H=H, F=F, k=2, T_cap=2, live=2, x=[onehot(0), onehot(1)], ids=[[0, 1], [1, 0]],
        probs=[[0.25, 0.75], [0.75, 0.25]], w1=w1, w2=w2,
        expected={"bf16": exp, "mxfp8": exp, "mxfp4": exp}))

    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "fc1_topk_cases.json")
    with open(path, "w") as f:
        json.dump(dict(about="apply_topk_in_fc1 hand cases; see make_fc1_topk_cases.py",
                       cases=cases), f, separators=(",", ":"))
    print(f"wrote {len(cases)} cases to {path}")


if __name__ == "__main__":
    main()
