"""The C-ABI library loads without a GPU, exports every symbol include/moe.h
declares, and its host-side checks behave as documented (no compute calls)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    import swiglu_expert_mlp_amd as m
    return m.lib()


def test_header_declares_the_boundary():
    names = _declared()
    for required in ("moe_create", "moe_destroy", "moe_weight_bytes", "moe_load_weights",
                     "moe_workspace_bytes", "moe_route", "moe_forward", "moe_get_indices",
                     "moe_get_rows", "moe_check", "moe_last_error"):
        assert required in names


def test_library_exports_every_declared_symbol(L):
    import swiglu_expert_mlp_amd as m
    out = subprocess.run(["nm", "-D", "--defined-only", m.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    for name in _declared():
        assert name in exported, name
        assert getattr(L, name) is not None
    # the binding wraps exactly the declared set
    assert set(m._SIGNATURES) == set(_declared())


def _create(L, E, H, F, k, p):
    h = ctypes.c_void_p()
    st = L.moe_create(E, H, F, k, p, ctypes.byref(h))
    return st, h


@pytest.mark.parametrize("args,status", [
    ((8, 128, 256, 2, 0), 0),
    ((8, 128, 256, 2, 1), 0),
    ((128, 2688, 1856, 6, 0), 0),
    ((0, 128, 256, 1, 0), -1),
    ((8, 100, 256, 2, 0), -1),
    ((8, 128, 250, 2, 0), -1),
    ((8, 128, 256, 0, 0), -1),
    ((8, 128, 256, 9, 0), -1),
    ((64, 128, 256, 17, 0), -1),
    ((2000, 128, 256, 2, 0), -1),
    ((8, 128, 256, 2, 2), 0),             # MXFP4 weights
    ((8, 128, 256, 2, 3), -2),
    ((8, 128, 256, 2, -1), -2),
])
def test_create_status(L, args, status):
    st, h = _create(L, *args)
    assert st == status, L.moe_last_error()
    if st == 0:
        assert h.value
        L.moe_destroy(h)
    else:
        assert L.moe_last_error()


def test_sizes(L):
    st, h = _create(L, 8, 128, 256, 2, 0)
    assert L.moe_weight_bytes(h) == 2 * (8 * 512 * 128 + 8 * 128 * 256)
    sizes = [L.moe_workspace_bytes(h, T) for T in (0, 1, 64, 1000, 65536)]
    assert sizes == sorted(sizes) and all(s % 256 == 0 for s in sizes)
    L.moe_destroy(h)
    st, h = _create(L, 8, 128, 256, 2, 1)
    import oracle
    assert L.moe_weight_bytes(h) == oracle.pack_bytes(8, 128, 256, "mxfp8")
    L.moe_destroy(h)


def test_forward_before_load_and_bad_sizes(L):
    st, h = _create(L, 8, 128, 256, 2, 0)
    P = ctypes.c_void_p
    fake = P(1 << 20)
    st = L.moe_forward(h, fake, fake, fake, 64, fake, fake, fake, 1 << 30, None)
    assert st == -3 and b"load" in L.moe_last_error()
    st = L.moe_load_weights(h, fake, fake, fake, 16, None)
    assert st == -1 and b"kbuf_bytes" in L.moe_last_error()
    st = L.moe_load_weights(h, P(3), fake, fake, 1 << 30, None)
    assert st == -1 and b"aligned" in L.moe_last_error()
    st = L.moe_route(h, None, 64, fake, fake, fake, fake, 1 << 20, None)
    assert st == -1
    L.moe_destroy(h)
    L.moe_destroy(None)


def test_python_binding_errors():
    from swiglu_expert_mlp_amd import MoE
    with pytest.raises(NotImplementedError):
        MoE(8, 128, 256, 2, "nvfp4")
    with pytest.raises(ValueError):
        MoE(8, 130, 256, 2, "bf16")


def _enum_values():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    return {n: int(v) for n, v in re.findall(r"\b(MOE_[A-Z0-9_]+)\s*=\s*(-?\d+)", text)}


def test_status_codes_match_the_boundary():
    """The status codes of the C boundary, including the device-contract code
    that moe_check returns when the device set violation bits."""
    v = _enum_values()
    assert v["MOE_OK"] == 0 and v["MOE_ERR_INVALID_ARG"] == -1
    assert v["MOE_ERR_UNSUPPORTED"] == -2 and v["MOE_ERR_NOT_LOADED"] == -3
    assert v["MOE_ERR_HIP"] == -4 and v["MOE_ERR_DEVICE_CONTRACT"] == -5
    import swiglu_expert_mlp_amd as m
    assert m.MOE_ERR_DEVICE_CONTRACT == v["MOE_ERR_DEVICE_CONTRACT"]


def test_forward_flags_match_the_boundary():
    """The binding's combine codes and option flags are the header's values,
    and the options are distinct bits above every combine code."""
    text = open(HEADER).read()
    defs = {n: int(v, 0) for n, v in re.findall(r"#define\s+(MOE_[A-Z0-9_]+)\s+(0x[0-9a-fA-F]+|\d+)u?\b", text)}
    v = _enum_values()
    import swiglu_expert_mlp_amd as m
    assert m.APPLY_TOPK_IN_FC1 == defs["MOE_APPLY_TOPK_IN_FC1"]
    assert m.FUSED_FFN == defs["MOE_FUSED_FFN"]
    assert m.FUSED_FINALIZE == defs["MOE_FUSED_FINALIZE"]
    flags = [defs["MOE_APPLY_TOPK_IN_FC1"], defs["MOE_FUSED_FFN"], defs["MOE_FUSED_FINALIZE"]]
    assert all(f & (f - 1) == 0 for f in flags) and len(set(flags)) == 3
    combines = [v["MOE_COMBINE_FP32"], v["MOE_COMBINE_BF16"], v["MOE_COMBINE_ROWS"]]
    assert max(combines) < min(flags)
    code = m.MoE._combine_code("bf16", True, False, True)
    assert code == v["MOE_COMBINE_BF16"] | defs["MOE_APPLY_TOPK_IN_FC1"] | defs["MOE_FUSED_FINALIZE"]


def test_host_checks_of_inspection_calls(L):
    """moe_check / moe_get_rows reject NULL arguments on the host, and
    moe_get_rows refuses activation codes for bf16 (there are none), without
    touching the (fake) workspace."""
    st, h = _create(L, 8, 128, 256, 2, 0)
    P = ctypes.c_void_p
    fake = P(1 << 20)
    bits = ctypes.c_uint32(7)
    assert L.moe_check(h, None, None, ctypes.byref(bits)) == -1
    assert L.moe_check(None, fake, None, ctypes.byref(bits)) == -1
    assert L.moe_get_rows(h, None, 64, None, None, None, None, None, None, None) == -1
    st = L.moe_get_rows(h, fake, 64, None, None, None, None, fake, None, None)
    assert st == -1 and b"bf16" in L.moe_last_error()
    L.moe_destroy(h)


def test_workspace_needs_no_initialisation_documented():
    """The header documents that a workspace needs no initial contents (the
    launches of one call write everything a later launch reads); the GPU test
    test_garbage_workspace_gives_identical_results checks the behaviour."""
    text = open(HEADER).read()
    i = text.index("size_t moe_workspace_bytes")
    doc = " ".join(text[text.rindex("/*", 0, i): i].replace("*", " ").split())
    assert "no required initial contents" in doc
    assert "must be zero" not in text
