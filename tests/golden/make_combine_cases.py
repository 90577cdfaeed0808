"""Write combine_cases.json: hand cases of the two combine variants.

The pages print no numeric example of either variant, so every expected value
below follows by hand from the definitions (no oracle call, no GPU code):

* BF16 combine (Megatron-LM PR #7798, "What is changed": the BF16_RANK_PARTIALS
  unpermute adds a token's routes as fp32 fused multiply-adds of probability
  and row from zero and quantizes the sum to BF16, as FlashInfer's finalize
  does).  bf16 keeps 8 significant bits, so on [1, 2) its spacing is 2^-7:
  1 + 2^-8 lies halfway between 1 and 1 + 2^-7 and rounds to the even one, 1;
  1 + 3 * 2^-8 lies halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even).
* Row mode (Megatron-LM PR #7798, "What is changed", expert compute; Megatron-Core
  API docs, expert_value_pass): each route is a top-1 token with probability
  1.0, so the finalize returns fma(1, row, +0) = the row, except that -0 + +0
  is +0 in round-to-nearest; a dropped route leaves the zero it started from.

Run ``python tests/golden/make_combine_cases.py`` to regenerate.
"""
import json
import os
import struct


def f32_bits(v):
    return struct.unpack("<I", struct.pack("<f", v))[0]


CITE_BF16 = ("Megatron-LM PR #7798, 'What is changed' (BF16_RANK_PARTIALS: fp32 FMA "
             "chain of probability and row from zero, then quantized to BF16)")
CITE_ROWS = ("Megatron-LM PR #7798, 'What is changed' (each dispatched row as a top-1 "
             "token with probability 1.0); Megatron-Core API docs, expert_value_pass")

cases = [
    dict(name="bf16_tie_to_even_down", mode="bf16", cite=CITE_BF16,
         derivation="1 + 2^-8 is halfway between bf16 1 and 1 + 2^-7; ties go to the even mantissa: 1",
         O=[[1.0], [2.0 ** -8]], dst=[[0, 1]], probs=[[1.0, 1.0]], H=1, expected_bf16=[[0x3F80]]),
    dict(name="bf16_tie_to_even_up", mode="bf16", cite=CITE_BF16,
         derivation="1 + 3*2^-8 is halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even): 1 + 2^-6",
         O=[[1.0], [3 * 2.0 ** -8]], dst=[[0, 1]], probs=[[1.0, 1.0]], H=1, expected_bf16=[[0x3F82]]),
    dict(name="bf16_above_half", mode="bf16", cite=CITE_BF16,
         derivation="1 + 2^-8 + 2^-16 is exact in fp32 and above the midpoint: 1 + 2^-7",
         O=[[1.0], [2.0 ** -8 + 2.0 ** -16]], dst=[[0, 1]], probs=[[1.0, 1.0]], H=1,
         expected_bf16=[[0x3F81]]),
    dict(name="bf16_negative_tie", mode="bf16", cite=CITE_BF16,
         derivation="-(1 + 2^-8) rounds to -1 (the sign does not change the tie rule)",
         O=[[-1.0], [-(2.0 ** -8)]], dst=[[0, 1]], probs=[[1.0, 1.0]], H=1, expected_bf16=[[0xBF80]]),
    dict(name="bf16_negative_zero", mode="bf16", cite=CITE_BF16,
         derivation="fma(1, -0, +0) = +0: the chain starts from +0, so the bf16 is +0",
         O=[[-0.0]], dst=[[0]], probs=[[1.0]], H=1, expected_bf16=[[0x0000]]),
    dict(name="bf16_probability_weights", mode="bf16", cite=CITE_BF16,
         derivation="0.25 * 4 + 0.75 * 8 = 7, exact: bf16 0x40E0",
         O=[[4.0], [8.0]], dst=[[0, 1]], probs=[[0.25, 0.75]], H=1, expected_bf16=[[0x40E0]]),
    dict(name="bf16_dropped_route", mode="bf16", cite=CITE_BF16,
         derivation="a dropped route (dst -1) adds nothing: 1",
         O=[[1.0], [5.0]], dst=[[0, -1]], probs=[[1.0, 1.0]], H=1, expected_bf16=[[0x3F80]]),
    dict(name="bf16_order", mode="bf16", cite=CITE_BF16,
         derivation="2^24, then +1 (rounds back to 2^24, tie to even), then -2^24: 0 in this order",
         O=[[2.0 ** 24], [1.0], [-(2.0 ** 24)]], dst=[[0, 1, 2]], probs=[[1.0, 1.0, 1.0]], H=1,
         expected_bf16=[[0x0000]]),
    dict(name="rows_unscaled_signed_zero_dropped", mode="rows", cite=CITE_ROWS,
         derivation="route 0 -> O row 1 as is; route 1 -> O row 0 with -0 turned into +0; "
                    "route 2 dropped -> +0 row; probabilities play no part",
         O=[[-0.0, 3.5], [-2.25, 2.0 ** -100]], dst=[[1, 0, -1]], probs=[[0.5, 0.25, 0.25]], H=2,
         expected_rows_bits=[[[f32_bits(-2.25), f32_bits(2.0 ** -100)],
                              [f32_bits(0.0), f32_bits(3.5)],
                              [f32_bits(0.0), f32_bits(0.0)]]]),
]

out = dict(about="Hand cases of the bf16 combine and the row mode; see make_combine_cases.py",
           cases=cases)
path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "combine_cases.json")
with open(path, "w") as f:
    json.dump(out, f, indent=1)
print("wrote", path)
