"""CPU oracle of the routed SwiGLU MoE forward (ctypes binding of moe_oracle.c).

TEST INFRASTRUCTURE ONLY.  The tests, the smoke check and the benchmark's
cpu_baseline leg may import this package; the product package
``swiglu_expert_mlp_amd`` never does, and shares no code with it.

Every entry point takes and returns numpy arrays:
  * bf16 data travels as uint16 bit patterns,
  * MXFP8 data as uint8 E4M3 codes plus uint8 E8M0 scale bytes.

Functions follow the method step by step (see the C source header for the
pages and sections each one follows).  Error bits returned by the router,
prepare and forward entry points use these values:
  1 expert id outside [0, E) in a live token (the route is dropped),
  2 duplicate expert id within a live token,
  4 live count above capacity (clamped),
  8 live count below zero (treated as zero).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")

ERR_BAD_ID = 1
ERR_DUP_ID = 2
ERR_LIVE_HIGH = 4
ERR_LIVE_NEG = 8


def build(force: bool = False) -> str:
    """Compile moe_oracle.c with gcc (plain -O2, no fast-math, no fp contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
             "-fno-fast-math", "-std=c11", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i64, i32, u32 = ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32
        sig = {
            "orc_bf16_bits": (ctypes.c_uint16, [ctypes.c_float]),
            "orc_bf16_round_array": (None, [P, i64, P]),
            "orc_e4m3_decode": (ctypes.c_double, [ctypes.c_uint8]),
            "orc_e4m3_encode": (ctypes.c_uint8, [ctypes.c_double]),
            "orc_e8m0_exponent": (ctypes.c_int, [ctypes.c_float]),
            "orc_mx_quantize": (None, [P, i64, i64, P, P]),
            "orc_mx_dequantize": (None, [P, P, i64, i64, P]),
            "orc_e2m1_decode": (ctypes.c_double, [ctypes.c_uint8]),
            "orc_e2m1_encode": (ctypes.c_uint8, [ctypes.c_double]),
            "orc_e8m0_exponent_fp4": (ctypes.c_int, [ctypes.c_float]),
            "orc_mx4_quantize": (None, [P, i64, i64, P, P]),
            "orc_mx4_dequantize": (None, [P, P, i64, i64, P]),
            "orc_route": (u32, [P, i64, i32, ctypes.c_int, ctypes.c_int, P, P]),
            "orc_prepare": (u32, [P, P, i64, i32, ctypes.c_int, ctypes.c_int,
                                  P, P, P, P, P, P, P]),
            "orc_finalize": (None, [P, P, P, i32, ctypes.c_int, ctypes.c_int, P]),
            "orc_finalize_bf16": (None, [P, P, P, i32, ctypes.c_int, ctypes.c_int, P]),
            "orc_finalize_rows": (None, [P, P, i32, ctypes.c_int, ctypes.c_int, P]),
            "orc_forward_ex": (u32, [P, P, P, P, i64, i32, ctypes.c_int, P, P, P]),
            "orc_weights_create": (P, [ctypes.c_int] * 5 + [P, P]),
            "orc_weights_destroy": (None, [P]),
            "orc_forward": (u32, [P, P, P, P, i64, i32, P, P, P]),
            "orc_forward_tokens": (None, [P, P, P, P, P, i64, P]),
            "orc_forward_tokens_ex": (None, [P, P, P, P, P, i64, ctypes.c_int, P]),
            "orc_finalize_sum": (None, [P, P, i32, ctypes.c_int, ctypes.c_int, ctypes.c_int, P]),
            "orc_pack_bf16": (None, [ctypes.c_int] * 3 + [P, P, P]),
            "orc_pack_mxfp8": (None, [ctypes.c_int] * 3 + [P, P, P]),
            "orc_pack_mxfp4": (None, [ctypes.c_int] * 3 + [P, P, P]),
            "orc_pack_mx4_offsets": (None, [ctypes.c_int] * 3 + [P]),
            "orc_pack_bytes": (i64, [ctypes.c_int] * 4),
            "orc_pack_mx_offsets": (None, [ctypes.c_int] * 3 + [P]),
            "orc_set_threads": (ctypes.c_int, [ctypes.c_int]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _p(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


# ---------------------------------------------------------------- formats

def bf16_bits(v: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint16)
    lib().orc_bf16_round_array(_p(v), v.size, _p(out))
    return out


def bf16_value(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 values (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def e4m3_decode(code: int) -> float:
    return lib().orc_e4m3_decode(int(code))


def e4m3_encode(v: float) -> int:
    return lib().orc_e4m3_encode(float(v))


def e8m0_exponent(amax: float) -> int:
    return lib().orc_e8m0_exponent(float(amax))


def mx_quantize(v: np.ndarray):
    """[rows, cols] fp32 -> (codes uint8 [rows, cols], scales uint8 [rows, cols/32])."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    rows, cols = v.shape
    assert cols % 32 == 0
    codes = np.empty((rows, cols), dtype=np.uint8)
    scales = np.empty((rows, cols // 32), dtype=np.uint8)
    lib().orc_mx_quantize(_p(v), rows, cols, _p(codes), _p(scales))
    return codes, scales


def mx_dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    rows, cols = codes.shape
    out = np.empty((rows, cols), dtype=np.float64)
    lib().orc_mx_dequantize(_p(codes), _p(scales), rows, cols, _p(out))
    return out


def e2m1_decode(code: int) -> float:
    return lib().orc_e2m1_decode(int(code))


def e2m1_encode(v: float) -> int:
    return lib().orc_e2m1_encode(float(v))


def e8m0_exponent_fp4(amax: float) -> int:
    return lib().orc_e8m0_exponent_fp4(float(amax))


def mx4_quantize(v: np.ndarray):
    """[rows, cols] fp32 -> (E2M1 codes uint8 [rows, cols] one per byte,
    scales uint8 [rows, cols/32])."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    rows, cols = v.shape
    assert cols % 32 == 0
    codes = np.empty((rows, cols), dtype=np.uint8)
    scales = np.empty((rows, cols // 32), dtype=np.uint8)
    lib().orc_mx4_quantize(_p(v), rows, cols, _p(codes), _p(scales))
    return codes, scales


def mx4_dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    rows, cols = codes.shape
    out = np.empty((rows, cols), dtype=np.float64)
    lib().orc_mx4_dequantize(_p(codes), _p(scales), rows, cols, _p(out))
    return out


PRECISIONS = {"bf16": 0, "mxfp8": 1, "mxfp4": 2}


# ---------------------------------------------------------------- router / prepare

def route(logits: np.ndarray, live: int, k: int):
    """Softmax, top-k by logit (ties to lower id), renormalize, ids ascending.

    Returns (ids int32 [T_cap, k], probs fp32 [T_cap, k], err).  Rows >= live
    keep the fill value (-1 ids, NaN probs) to show they were not written.
    """
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T_cap, E = logits.shape
    ids = np.full((T_cap, k), -1, dtype=np.int32)
    probs = np.full((T_cap, k), np.nan, dtype=np.float32)
    err = lib().orc_route(_p(logits), T_cap, int(live), E, k, _p(ids), _p(probs))
    return ids, probs, err


def prepare(ids: np.ndarray, probs: np.ndarray, live: int, E: int):
    """Canonical sort and stable expert permutation.  Returns a dict."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    probs = np.ascontiguousarray(probs, dtype=np.float32)
    T_cap, k = ids.shape
    n = T_cap * k + 1
    sorted_ids = np.full(n, -7, dtype=np.int32)
    sorted_probs = np.full(n, np.nan, dtype=np.float32)
    counts = np.zeros(E, dtype=np.int32)
    offsets = np.zeros(E + 1, dtype=np.int32)
    perm_src = np.full(n, -7, dtype=np.int32)
    dst = np.full(n, -7, dtype=np.int32)
    T = np.zeros(1, dtype=np.int32)
    err = lib().orc_prepare(_p(ids), _p(probs), T_cap, int(live), E, k, _p(sorted_ids),
                            _p(sorted_probs), _p(counts), _p(offsets), _p(perm_src),
                            _p(dst), _p(T))
    T = int(T[0])
    R = T * k
    nrows = int(offsets[E])
    return dict(T=T, err=err, sorted_ids=sorted_ids[:R].reshape(T, k),
                sorted_probs=sorted_probs[:R].reshape(T, k), counts=counts,
                offsets=offsets, perm_src=perm_src[:nrows], dst=dst[:R].reshape(T, k))


def finalize(O: np.ndarray, dst: np.ndarray, sorted_probs: np.ndarray, H: int) -> np.ndarray:
    O = np.ascontiguousarray(O, dtype=np.float32)
    dst = np.ascontiguousarray(dst, dtype=np.int32)
    sorted_probs = np.ascontiguousarray(sorted_probs, dtype=np.float32)
    T, k = dst.shape
    out = np.zeros((T, H), dtype=np.float32)
    lib().orc_finalize(_p(O), _p(dst), _p(sorted_probs), T, k, H, _p(out))
    return out


def finalize_bf16(O: np.ndarray, dst: np.ndarray, sorted_probs: np.ndarray, H: int) -> np.ndarray:
    """The fp32 combine rounded to bf16: uint16 bits [T, H]."""
    O = np.ascontiguousarray(O, dtype=np.float32)
    dst = np.ascontiguousarray(dst, dtype=np.int32)
    sorted_probs = np.ascontiguousarray(sorted_probs, dtype=np.float32)
    T, k = dst.shape
    out = np.zeros((T, H), dtype=np.uint16)
    lib().orc_finalize_bf16(_p(O), _p(dst), _p(sorted_probs), T, k, H, _p(out))
    return out


def finalize_rows(O: np.ndarray, dst: np.ndarray, H: int) -> np.ndarray:
    """Row mode: each route as a top-1 token with probability 1: fp32 [T, k, H]."""
    O = np.ascontiguousarray(O, dtype=np.float32)
    dst = np.ascontiguousarray(dst, dtype=np.int32)
    T, k = dst.shape
    out = np.zeros((T, k, H), dtype=np.float32)
    lib().orc_finalize_rows(_p(O), _p(dst), T, k, H, _p(out))
    return out


COMBINES = {"fp32": 0, "bf16": 1, "rows": 2}
# added to a combine: the probabilities are applied inside FC1 (fp32 / bf16 combines)
APPLY_TOPK_IN_FC1 = 0x100


def finalize_sum(O: np.ndarray, dst: np.ndarray, H: int, to_bf16: bool = False) -> np.ndarray:
    """The apply_topk_in_fc1 finalize: each token's (already weighted) rows added
    as an fp32 chain from +0 in canonical order; fp32 [T, H] or bf16 bits."""
    O = np.ascontiguousarray(O, dtype=np.float32)
    dst = np.ascontiguousarray(dst, dtype=np.int32)
    T, k = dst.shape
    out = np.zeros((T, H), dtype=np.uint16 if to_bf16 else np.float32)
    lib().orc_finalize_sum(_p(O), _p(dst), T, k, H, int(to_bf16), _p(out))
    return out


# ---------------------------------------------------------------- forward

class Model:
    """Oracle weights: bf16 W1 [E, 2F, H] (gate rows first) and W2 [E, H, F].

    precision: "bf16", "mxfp8" (weights quantized to E4M3 per 32-block along K) or
    "mxfp4" (weights quantized to E2M1 per 32-block along K; activations MXFP8).
    """

    def __init__(self, E, H, F, k, w1_bits: np.ndarray, w2_bits: np.ndarray,
                 precision: str = "bf16"):
        assert precision in PRECISIONS
        self.E, self.H, self.F, self.k = E, H, F, k
        self.precision = precision
        self._w1 = np.ascontiguousarray(w1_bits, dtype=np.uint16)
        self._w2 = np.ascontiguousarray(w2_bits, dtype=np.uint16)
        assert self._w1.size == E * 2 * F * H and self._w2.size == E * H * F
        self._h = lib().orc_weights_create(E, H, F, k, PRECISIONS[precision],
                                           _p(self._w1), _p(self._w2))

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            lib().orc_weights_destroy(h)
            self._h = None

    def forward(self, x_bits, ids, probs, live, want_rows: bool = False, combine: str = "fp32",
                topk_in_fc1: bool = False):
        """Whole forward.  Returns (out, err, extras); out is fp32 [T_cap, H] (combine
        "fp32"), bf16 bits [T_cap, H] ("bf16") or fp32 [T_cap, k, H] ("rows"), with rows
        of tokens >= T left NaN (0xFFFF for bf16); extras holds O rows and FC2 operand
        rows when asked.  probs may be None in row mode (it does not use them)."""
        x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        if probs is None:
            assert combine == "rows"
            probs = np.ones(ids.shape, dtype=np.float32)
        probs = np.ascontiguousarray(probs, dtype=np.float32)
        T_cap = x_bits.shape[0]
        if combine == "bf16":
            out = np.full((T_cap, self.H), 0xFFFF, dtype=np.uint16)
        elif combine == "rows":
            out = np.full((T_cap, self.k, self.H), np.nan, dtype=np.float32)
        else:
            out = np.full((T_cap, self.H), np.nan, dtype=np.float32)
        extras = {}
        O = Hr = None
        if want_rows:
            n = max(1, T_cap * self.k)
            O = np.zeros((n, self.H), dtype=np.float32)
            Hr = np.zeros((n, self.F), dtype=np.float32)
        if topk_in_fc1:
            assert combine in ("fp32", "bf16"), "row mode has no probabilities to apply"
        code = COMBINES[combine] | (APPLY_TOPK_IN_FC1 if topk_in_fc1 else 0)
        err = lib().orc_forward_ex(self._h, _p(x_bits), _p(ids), _p(probs), T_cap, int(live),
                                   code, _p(out), _p(O), _p(Hr))
        if want_rows:
            extras = dict(O=O, H=Hr)
        return out, err, extras

    def forward_tokens(self, x_bits, ids, probs, tokens, topk_in_fc1: bool = False) -> np.ndarray:
        """Naive per-token loop for the listed token indices: [len(tokens), H]
        (with topk_in_fc1, the probabilities applied inside FC1)."""
        x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        probs = np.ascontiguousarray(probs, dtype=np.float32)
        tokens = np.ascontiguousarray(tokens, dtype=np.int64)
        out = np.empty((len(tokens), self.H), dtype=np.float32)
        lib().orc_forward_tokens_ex(self._h, _p(x_bits), _p(ids), _p(probs), _p(tokens),
                                    len(tokens), int(topk_in_fc1), _p(out))
        return out


def set_threads(n: int = 0) -> int:
    """Set the oracle's OpenMP thread count (n > 0); returns the count in effect."""
    return int(lib().orc_set_threads(int(n)))


def pack_bytes(E, H, F, precision="bf16") -> int:
    return int(lib().orc_pack_bytes(E, H, F, PRECISIONS[precision]))


def pack_mx_offsets(E, H, F, precision="mxfp8") -> list:
    """Byte offsets of the MXFP8 / MXFP4 buffer sections: FC1 codes, FC2 codes,
    FC1 scales, FC2 scales, end (each section's padding is part of the layout)."""
    off = np.zeros(5, dtype=np.int64)
    fn = lib().orc_pack_mx4_offsets if precision == "mxfp4" else lib().orc_pack_mx_offsets
    fn(E, H, F, _p(off))
    return [int(v) for v in off]


def pack(E, H, F, w1_bits, w2_bits, precision="bf16") -> np.ndarray:
    """Kernel-weight buffer bytes in the documented layout (independent packer)."""
    w1 = np.ascontiguousarray(w1_bits, dtype=np.uint16)
    w2 = np.ascontiguousarray(w2_bits, dtype=np.uint16)
    buf = np.zeros(pack_bytes(E, H, F, precision), dtype=np.uint8)
    fn = {"bf16": lib().orc_pack_bf16, "mxfp8": lib().orc_pack_mxfp8,
          "mxfp4": lib().orc_pack_mxfp4}[precision]
    fn(E, H, F, _p(w1), _p(w2), _p(buf))
    return buf
