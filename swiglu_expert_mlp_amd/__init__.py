"""MI355X-native routed SwiGLU MoE forward: Python binding of libmoe.so.

Argument marshalling only.  Every step of the path (routing, permutation, the
expert GEMMs, SwiGLU, quantization, the fp32 finalize) runs in the HIP kernels
of ``libmoe.so`` (C ABI in ``include/moe.h``); torch supplies device memory
and the current stream.  There is no CPU fallback: if the library is missing
or no GPU is present, the calls raise.

    moe = MoE(E=64, H=2048, F=1024, topk=6, precision="bf16")
    kbuf = moe.load_weights(w1, w2)          # w1 [E, 2F, H], w2 [E, H, F], bf16, on GPU
    ws = moe.new_workspace(T_cap)
    ids, probs = moe.route(logits, live, ws=ws)
    out = moe.forward(x, ids, probs, live, ws=ws)   # fp32 [T_cap, H]

``live`` is an int32 device tensor holding the number of live tokens.
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["MoE", "lib", "LIB_PATH", "MoEError", "DEVERR_BAD_EXPERT_ID", "DEVERR_DUP_EXPERT_ID",
           "DEVERR_LIVE_ABOVE_CAP", "DEVERR_LIVE_NEGATIVE", "DEVERR_FUSED_WAIT"]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_BF16, MOE_MXFP8, MOE_MXFP4 = 0, 1, 2
_PRECISION = {"bf16": MOE_BF16, "mxfp8": MOE_MXFP8, "mxfp4": MOE_MXFP4}
DEVERR_BAD_EXPERT_ID = 1
DEVERR_DUP_EXPERT_ID = 2
DEVERR_LIVE_ABOVE_CAP = 4
DEVERR_LIVE_NEGATIVE = 8
DEVERR_FUSED_WAIT = 16
MOE_ERR_DEVICE_CONTRACT = -5
# moe_forward_ex combines (moe_combine in include/moe.h)
COMBINES = {"fp32": 0, "bf16": 1, "rows": 2}
# added to a combine: probabilities applied inside FC1 (MOE_APPLY_TOPK_IN_FC1)
APPLY_TOPK_IN_FC1 = 0x100
# added to a combine: FC1 and FC2 in one persistent launch (MOE_FUSED_FFN, bf16)
FUSED_FFN = 0x200
# added to a combine: FC1, FC2 and the finalize in one persistent launch
# (MOE_FUSED_FINALIZE, bf16; implies FUSED_FFN)
FUSED_FINALIZE = 0x400

# every symbol include/moe.h declares, with its ctypes signature
_P = ctypes.c_void_p
_SIGNATURES = {
    "moe_create": (ctypes.c_int, [ctypes.c_int] * 5 + [ctypes.POINTER(_P)]),
    "moe_destroy": (None, [_P]),
    "moe_weight_bytes": (ctypes.c_size_t, [_P]),
    "moe_load_weights": (ctypes.c_int, [_P, _P, _P, _P, ctypes.c_size_t, _P]),
    "moe_workspace_bytes": (ctypes.c_size_t, [_P, ctypes.c_int64]),
    "moe_route": (ctypes.c_int, [_P, _P, ctypes.c_int64, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "moe_forward": (ctypes.c_int, [_P, _P, _P, _P, ctypes.c_int64, _P, _P, _P, ctypes.c_size_t, _P]),
    "moe_forward_ex": (ctypes.c_int, [_P, _P, _P, _P, ctypes.c_int64, _P, ctypes.c_int, _P, _P,
                                      ctypes.c_size_t, _P]),
    "moe_forward_noalloc": (ctypes.c_int, [_P, _P, _P, _P, ctypes.c_int64, _P, ctypes.c_int, _P,
                                           _P]),
    "moe_get_indices": (ctypes.c_int, [_P, _P, ctypes.c_int64, _P, _P, _P, _P, _P, _P, _P]),
    "moe_get_rows": (ctypes.c_int, [_P, _P, ctypes.c_int64, _P, _P, _P, _P, _P, _P, _P]),
    "moe_check": (ctypes.c_int, [_P, _P, _P, ctypes.POINTER(ctypes.c_uint32)]),
    "moe_set_stage_events": (ctypes.c_int, [_P, _P, ctypes.c_int]),
    "moe_last_error": (ctypes.c_char_p, []),
}

_lib = None


class MoEError(RuntimeError):
    pass


def lib() -> ctypes.CDLL:
    """Load libmoe.so (built by ``python -m swiglu_expert_mlp_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m swiglu_expert_mlp_amd.build` (there is no fallback)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(status: int, what: str):
    if status == 0:
        return
    msg = lib().moe_last_error().decode(errors="replace")
    if status == -1:
        raise ValueError(f"{what}: {msg}")
    if status == -2:
        raise NotImplementedError(f"{what}: {msg}")
    raise MoEError(f"{what} failed ({status}): {msg}")


def _torch():
    import torch
    return torch


def _stream(stream=None) -> int:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _dev(t, name, dtypes, shape=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must have dtype in {dtypes}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t.data_ptr()


class MoE:
    """Handle of one routed SwiGLU MoE layer (E experts, hidden H, FFN F, top-k)."""

    def __init__(self, E: int, H: int, F: int, topk: int, precision: str = "bf16"):
        if precision not in _PRECISION:
            raise NotImplementedError(f"precision {precision!r} is not supported (bf16, mxfp8, mxfp4)")
        h = _P()
        _check(lib().moe_create(E, H, F, topk, _PRECISION[precision], ctypes.byref(h)),
               "moe_create")
        self._h = h
        # kept on the handle: at interpreter exit the module's globals may be
        # cleared before the last handle is collected
        self._destroy = lib().moe_destroy
        self.E, self.H, self.F, self.topk, self.precision = E, H, F, topk, precision
        self.kbuf = None

    def __del__(self):
        h = getattr(self, "_h", None)
        destroy = getattr(self, "_destroy", None)
        if h is not None and h.value and destroy is not None:
            destroy(h)
            self._h = None

    # ------------------------------------------------------------- sizes

    @property
    def weight_bytes(self) -> int:
        return int(lib().moe_weight_bytes(self._h))

    def workspace_bytes(self, T_cap: int) -> int:
        return int(lib().moe_workspace_bytes(self._h, int(T_cap)))

    def new_workspace(self, T_cap: int, device=None):
        """A workspace for capacity T_cap (no initial contents are required)."""
        torch = _torch()
        return torch.empty(self.workspace_bytes(T_cap), dtype=torch.uint8,
                           device=device or "cuda")

    # ------------------------------------------------------------- calls

    def load_weights(self, w1, w2, kbuf=None, stream=None):
        """Pack bf16 w1 [E, 2F, H] (gate rows first) and w2 [E, H, F] into kbuf
        (allocated if None).  Calling again with the same kbuf is the refit."""
        torch = _torch()
        bf = (torch.bfloat16, torch.int16, torch.uint16)
        p1 = _dev(w1, "w1", bf, (self.E, 2 * self.F, self.H))
        p2 = _dev(w2, "w2", bf, (self.E, self.H, self.F))
        if kbuf is None:
            kbuf = torch.empty(self.weight_bytes, dtype=torch.uint8, device=w1.device)
        pk = _dev(kbuf, "kbuf", (torch.uint8,))
        _check(lib().moe_load_weights(self._h, p1, p2, pk, kbuf.numel(), _stream(stream)),
               "moe_load_weights")
        self.kbuf = kbuf          # keep the buffer alive as long as the handle reads it
        return kbuf

    def route(self, logits, live, ids=None, probs=None, ws=None, stream=None):
        torch = _torch()
        T_cap = logits.shape[0]
        pl = _dev(logits, "logits", (torch.float32,), (T_cap, self.E))
        plive = _dev(live, "live", (torch.int32,))
        if ids is None:
            ids = torch.empty((T_cap, self.topk), dtype=torch.int32, device=logits.device)
        if probs is None:
            probs = torch.empty((T_cap, self.topk), dtype=torch.float32, device=logits.device)
        if ws is None:
            ws = self.new_workspace(T_cap, logits.device)
        pi = _dev(ids, "ids", (torch.int32,), (T_cap, self.topk))
        pp = _dev(probs, "probs", (torch.float32,), (T_cap, self.topk))
        pw = _dev(ws, "ws", (torch.uint8,))
        _check(lib().moe_route(self._h, pl, T_cap, plive, pi, pp, pw, ws.numel(), _stream(stream)),
               "moe_route")
        return ids, probs

    def _out_spec(self, T_cap: int, combine: str):
        """(dtypes, shape, allocation dtype) of the output of a combine."""
        torch = _torch()
        if combine == "fp32":
            return (torch.float32,), (T_cap, self.H), torch.float32
        if combine == "bf16":
            return (torch.bfloat16, torch.int16, torch.uint16), (T_cap, self.H), torch.bfloat16
        if combine == "rows":
            return (torch.float32,), (T_cap, self.topk, self.H), torch.float32
        raise ValueError(f"combine must be one of {sorted(COMBINES)}")

    @staticmethod
    def _combine_code(combine: str, topk_in_fc1: bool, fused_ffn: bool = False,
                      fused_finalize: bool = False) -> int:
        if combine not in COMBINES:
            raise ValueError(f"combine must be one of {sorted(COMBINES)}")
        return (COMBINES[combine] | (APPLY_TOPK_IN_FC1 if topk_in_fc1 else 0) |
                (FUSED_FFN if fused_ffn else 0) | (FUSED_FINALIZE if fused_finalize else 0))

    def forward(self, x, ids, probs, live, out=None, ws=None, stream=None, combine="fp32",
                topk_in_fc1=False, fused_ffn=False, fused_finalize=False):
        """The forward (moe_forward_ex).  combine: "fp32" (out fp32 [T_cap, H]), "bf16"
        (out bf16 [T_cap, H]) or "rows" (out fp32 [T_cap, topk, H]; probs may be None).
        topk_in_fc1: apply the probabilities inside FC1 (fp32 and bf16 combines).
        fused_ffn: FC1 and FC2 in one persistent launch (bf16 weights).
        fused_finalize: FC1, FC2 and the finalize in one persistent launch (bf16 weights)."""
        torch = _torch()
        T_cap = x.shape[0]
        dts, shape, alloc = self._out_spec(T_cap, combine)
        px = _dev(x, "x", (torch.bfloat16, torch.int16, torch.uint16), (T_cap, self.H))
        pi = _dev(ids, "expert_ids", (torch.int32,), (T_cap, self.topk))
        pp = None if probs is None else _dev(probs, "probs", (torch.float32,), (T_cap, self.topk))
        plive = _dev(live, "live", (torch.int32,))
        if out is None:
            out = torch.empty(shape, dtype=alloc, device=x.device)
        po = _dev(out, "out", dts, shape)
        if ws is None:
            ws = self.new_workspace(T_cap, x.device)
        pw = _dev(ws, "ws", (torch.uint8,))
        _check(lib().moe_forward_ex(self._h, px, pi, pp, T_cap, plive,
                                    self._combine_code(combine, topk_in_fc1, fused_ffn, fused_finalize), po, pw,
                                    ws.numel(), _stream(stream)), "moe_forward")
        return out

    def forward_noalloc(self, x, ids, probs, live, out=None, stream=None, combine="fp32",
                        topk_in_fc1=False, fused_ffn=False, fused_finalize=False):
        """moe_forward_noalloc: the forward with the library's own per-GPU scratch
        as workspace (no caller workspace, nothing allocated by the library).
        Calls that overlap on one GPU race; the capacity is bounded."""
        torch = _torch()
        T_cap = x.shape[0]
        dts, shape, alloc = self._out_spec(T_cap, combine)
        px = _dev(x, "x", (torch.bfloat16, torch.int16, torch.uint16), (T_cap, self.H))
        pi = _dev(ids, "expert_ids", (torch.int32,), (T_cap, self.topk))
        pp = None if probs is None else _dev(probs, "probs", (torch.float32,), (T_cap, self.topk))
        plive = _dev(live, "live", (torch.int32,))
        if out is None:
            out = torch.empty(shape, dtype=alloc, device=x.device)
        po = _dev(out, "out", dts, shape)
        _check(lib().moe_forward_noalloc(self._h, px, pi, pp, T_cap, plive,
                                         self._combine_code(combine, topk_in_fc1, fused_ffn, fused_finalize), po,
                                         _stream(stream)), "moe_forward_noalloc")
        return out

    # ------------------------------------------------------------- inspection

    def get_indices(self, ws, T_cap: int, stream=None) -> dict:
        import numpy as np
        counts = np.zeros(self.E, np.int32)
        offsets = np.zeros(self.E + 1, np.int32)
        n = max(1, T_cap * self.topk)
        perm = np.full(n, -7, np.int32)
        dst = np.full(n, -7, np.int32)
        n_rows = ctypes.c_int32(0)
        T = ctypes.c_int32(0)
        c = lambda a: a.ctypes.data_as(_P)
        _check(lib().moe_get_indices(self._h, _dev(ws, "ws", (_torch().uint8,)), T_cap, c(counts),
                                     c(offsets), c(perm), c(dst), ctypes.byref(n_rows),
                                     ctypes.byref(T), _stream(stream)), "moe_get_indices")
        T = T.value
        return dict(counts=counts, offsets=offsets, perm_src=perm[: n_rows.value],
                    dst=dst[: T * self.topk].reshape(T, self.topk), T=T, n_rows=n_rows.value)

    def get_rows(self, ws, T_cap: int, n_rows: int, T: int, stream=None) -> dict:
        """Intermediate rows of the last forward (moe_get_rows); for MXFP8 / MXFP4
        also the quantized activations x_codes [T, H] and x_scales [T, H/32]."""
        import numpy as np
        O = np.zeros((max(1, n_rows), self.H), np.float32)
        if self.precision == "bf16":
            hr = np.zeros((max(1, n_rows), self.F), np.uint16)
        else:
            hr = np.zeros(max(1, n_rows) * (self.F + self.F // 32), np.uint8)
        sid = np.zeros((max(1, T), self.topk), np.int32)
        sp = np.zeros((max(1, T), self.topk), np.float32)
        mx = self.precision != "bf16"
        xc = np.zeros((max(1, T), self.H), np.uint8) if mx else None
        xs = np.zeros((max(1, T), self.H // 32), np.uint8) if mx else None
        c = lambda a: None if a is None else a.ctypes.data_as(_P)
        _check(lib().moe_get_rows(self._h, _dev(ws, "ws", (_torch().uint8,)), T_cap, c(O), c(hr),
                                  c(sid), c(sp), c(xc), c(xs), _stream(stream)), "moe_get_rows")
        res = dict(fc2_rows=O[:n_rows], sorted_ids=sid[:T], sorted_probs=sp[:T])
        if self.precision == "bf16":
            res["fc1_out"] = hr[:n_rows]
        else:
            res["fc1_codes"] = hr[: n_rows * self.F].reshape(n_rows, self.F)
            res["fc1_scales"] = hr[n_rows * self.F: n_rows * (self.F + self.F // 32)].reshape(
                n_rows, self.F // 32)
            res["x_codes"] = xc[:T]
            res["x_scales"] = xs[:T]
        return res

    STAGES = ("permute", "quant_x", "fc1_swiglu", "fc2", "finalize")

    def set_stage_events(self, events):
        """Record 6 events at the forward's stage boundaries (before the first
        kernel, then after each of STAGES); entries may be None (skipped), raw
        hipEvent_t handles (int) or torch.cuda.Event objects.  None stops."""
        if events is None:
            _check(lib().moe_set_stage_events(self._h, None, 0), "moe_set_stage_events")
            return
        if len(events) != 6:
            raise ValueError("need 6 events")
        handles = []
        for ev in events:
            if ev is None or isinstance(ev, int):
                handles.append(_P(ev or 0))
                continue
            if not ev.cuda_event:        # torch creates the HIP event at its first record
                ev.record()
            handles.append(_P(ev.cuda_event))
        arr = (_P * 6)(*handles)
        _check(lib().moe_set_stage_events(self._h, arr, 6), "moe_set_stage_events")

    def bind_forward(self, x, ids, probs, live, out, ws, stream=None, combine="fp32",
                     topk_in_fc1=False, fused_ffn=False, fused_finalize=False):
        """Check the arguments once and return a no-argument callable that
        enqueues this forward (for launch loops where per-call checks would
        cost more host time than the GPU work)."""
        torch = _torch()
        T_cap = x.shape[0]
        dts, shape, _ = self._out_spec(T_cap, combine)
        args = (self._h, _dev(x, "x", (torch.bfloat16, torch.int16, torch.uint16), (T_cap, self.H)),
                _dev(ids, "expert_ids", (torch.int32,), (T_cap, self.topk)),
                None if probs is None else _dev(probs, "probs", (torch.float32,), (T_cap, self.topk)),
                T_cap, _dev(live, "live", (torch.int32,)),
                self._combine_code(combine, topk_in_fc1, fused_ffn, fused_finalize),
                _dev(out, "out", dts, shape),
                _dev(ws, "ws", (torch.uint8,)), ws.numel(), _stream(stream))
        fn = lib().moe_forward_ex
        keep = (x, ids, probs, live, out, ws)

        def call():
            _check(fn(*args), "moe_forward")
        call.keep = keep
        return call

    def bind_route(self, logits, live, ids, probs, ws, stream=None):
        """As bind_forward, for the router."""
        torch = _torch()
        T_cap = logits.shape[0]
        args = (self._h, _dev(logits, "logits", (torch.float32,), (T_cap, self.E)), T_cap,
                _dev(live, "live", (torch.int32,)),
                _dev(ids, "ids", (torch.int32,), (T_cap, self.topk)),
                _dev(probs, "probs", (torch.float32,), (T_cap, self.topk)),
                _dev(ws, "ws", (torch.uint8,)), ws.numel(), _stream(stream))
        fn = lib().moe_route
        keep = (logits, live, ids, probs, ws)

        def call():
            _check(fn(*args), "moe_route")
        call.keep = keep
        return call

    def check(self, ws, stream=None) -> int:
        """moe_check: the contract-violation bits (DEVERR_*) of the last route and
        forward on ws, cleared afterwards; 0 when there were none."""
        bits = ctypes.c_uint32(0)
        st = lib().moe_check(self._h, _dev(ws, "ws", (_torch().uint8,)), _stream(stream),
                             ctypes.byref(bits))
        if st == MOE_ERR_DEVICE_CONTRACT:
            return int(bits.value)
        _check(st, "moe_check")
        return int(bits.value)
