"""Write mx4_blocks.json: hand cases of the MXFP4 block quantizer.

MXFP4 here = E2M1 elements (1 sign, 2 exponent bits with bias 1, 1 mantissa
bit: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6) with one E8M0 scale per 32
elements; the scale is the power-of-two ceiling of the block's max magnitude
/ 6 (the MXFP8 rule of the workloads with E2M1's largest value), and each
element is v / scale rounded to the nearest E2M1 value, ties to the even code
(the code with mantissa bit 0).  Every expected value below is worked out by
hand in its "derivation" (no oracle call).  Run
``python tests/golden/make_mx4_blocks.py`` to regenerate.
"""
import json
import os

CITE = ("MXFP4 (E2M1 + E8M0 per 32): scale = power-of-two ceiling of amax / 6; "
        "elements rounded to nearest, ties to the even code")


def block(vals):
    return list(vals) + [0.0] * (32 - len(vals))


cases = [
    dict(name="amax6", cite=CITE,
         block=block([6.0, -6.0, 3.0, 1.5, 0.75, 0.25]), scale_exp=0,
         values=block([6.0, -6.0, 3.0, 1.5, 1.0, 0.0]),
         derivation="6 <= 6 * 2^0 and 6 > 6 * 2^-1 = 3: e = 0.  0.75 is halfway between "
                    "0.5 (code 1) and 1 (code 2): 1.  0.25 is halfway between 0 (code 0) "
                    "and 0.5 (code 1): 0"),
    dict(name="amax1", cite=CITE,
         block=block([1.0, 0.3, -0.2, 0.125]), scale_exp=-2,
         values=block([1.0, 0.25, -0.25, 0.125]),
         derivation="1 <= 6 * 2^-2 = 1.5 and 1 > 6 * 2^-3 = 0.75: e = -2.  Scaled by 4: 4, "
                    "1.2 -> 1, -0.8 -> -1, 0.5 -> 0.5; times 2^-2"),
    dict(name="amax_above_6", cite=CITE,
         block=block([6.5, 1.0]), scale_exp=1,
         values=block([6.0, 1.0]),
         derivation="6 < 6.5 <= 12: e = 1.  Scaled: 3.25 -> 3 (0.25 from 3, 0.75 from 4), "
                    "0.5 -> 0.5; times 2"),
    dict(name="ties_to_even", cite=CITE,
         block=block([6.0, 1.25, 1.75, 2.5, 3.5, 5.0, -5.0, -1.25]), scale_exp=0,
         values=block([6.0, 1.0, 2.0, 2.0, 4.0, 4.0, -4.0, -1.0]),
         derivation="e = 0.  1.25: 1 (code 2) vs 1.5 (code 3) -> 1.  1.75: 1.5 (3) vs 2 (4) "
                    "-> 2.  2.5: 2 (4) vs 3 (5) -> 2.  3.5: 3 (5) vs 4 (6) -> 4.  5: 4 (6) "
                    "vs 6 (7) -> 4.  Signs are kept"),
    dict(name="zeros", cite=CITE, block=block([]), scale_exp=-127, values=block([]),
         derivation="amax = 0: the smallest scale, 2^-127; every code is 0"),
    dict(name="subnormal_amax", cite=CITE, block=block([2.0 ** -130]), scale_exp=-127,
         values=block([0.0]),
         derivation="the ceiling of 2^-130 / 6 is below 2^-127, so e clamps to -127; "
                    "2^-130 * 2^127 = 0.125 is below the 0.25 midpoint: 0"),
]

path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "mx4_blocks.json")
with open(path, "w") as f:
    json.dump(dict(about="MXFP4 block quantization hand cases; see make_mx4_blocks.py",
                   cases=cases), f, indent=1)
print("wrote", path)
