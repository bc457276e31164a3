"""libmoe.so loads, exports every symbol include/moe.h declares, and rejects
bad arguments on the host (no device memory is touched: every call here fails
validation before anything is enqueued)."""
import ctypes
import os
import re

import pytest

from routing_grouped_gemm_softmax_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

pytestmark = pytest.mark.skipif(not os.path.exists(L.LIB_PATH), reason="libmoe.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(\w+)\s*\(", text, flags=re.M)))


def test_header_and_binding_agree():
    names = declared_functions()
    assert len(names) >= 15
    assert set(names) == set(L.SIGNATURES), set(names) ^ set(L.SIGNATURES)


def test_every_declared_symbol_is_exported():
    lib = L.load()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings():
    lib = L.load()
    assert lib.moe_abi_version() == 8
    for code, name in [(0, b"MOE_OK"), (-1, b"MOE_ERR_INVALID_ARG"), (-2, b"MOE_ERR_UNSUPPORTED"),
                       (-3, b"MOE_ERR_MISALIGNED"), (-4, b"MOE_ERR_WORKSPACE"), (-5, b"MOE_ERR_HIP")]:
        assert lib.moe_status_string(code) == name


def shape(**kw):
    base = dict(T=256, d=64, E=8, k=4, f=128, dtype="f32")
    base.update(kw)
    return L.MoeShape.make(**base)


def test_workspace_queries():
    s = shape()
    assert L.workspace_size(L.MOE_OP_DISPATCH, s) > 256
    assert L.workspace_size(L.MOE_OP_FFN_BWD, s) == 256 * 4 * 2 * 128 * 4
    assert L.save_size(s) == 3 * 256 * 4 * 128 * 4
    assert L.save_size(shape(dtype="bf16")) == 3 * 256 * 4 * 128 * 2
    # MXFP8 layers save G, U as 24-bit planes over the rows padded per expert
    # (P = S + 63 E rounded up to 64), beside the E4M3 weight copies.
    mx = shape(dtype="mxfp8", d=128)
    P = (256 * 4 + 63 * 8 + 63) // 64 * 64
    assert L.save_size(mx) > 2 * P * 128 * 3 + 3 * 8 * 128 * 128
    assert L.workspace_size(L.MOE_OP_FFN_BWD, mx) > 256 * 4 * 2 * 128 * 4
    with pytest.raises(L.MoeError):
        L.workspace_size(L.MOE_OP_DISPATCH, shape(k=9, E=16))
    assert L.load().moe_workspace_size(99, ctypes.byref(s)) == ctypes.c_size_t(-1).value


@pytest.mark.parametrize("bad,code", [
    (dict(k=9, E=8), L.MOE_ERR_INVALID_ARG),       # k > E
    (dict(T=0), L.MOE_ERR_INVALID_ARG),
    (dict(E=300, k=4), L.MOE_ERR_UNSUPPORTED),
    (dict(k=9, E=16), L.MOE_ERR_UNSUPPORTED),
    (dict(d=96), L.MOE_ERR_UNSUPPORTED),
    (dict(f=100), L.MOE_ERR_UNSUPPORTED),
    (dict(dtype=7), L.MOE_ERR_INVALID_ARG),
])
def test_shape_validation(bad, code):
    s = shape(**bad)
    fake = ctypes.c_void_p(0x100000)
    rc = L.load().moe_route(fake, fake, ctypes.byref(s), fake, fake, fake, fake, 1 << 30, None)
    assert rc == code, L.last_error()
    assert L.last_error()


def test_null_and_misaligned_pointers():
    lib = L.load()
    s = shape()
    ok = ctypes.c_void_p(0x100000)
    assert lib.moe_route(None, ok, ctypes.byref(s), ok, ok, ok, ok, 1 << 30, None) == L.MOE_ERR_INVALID_ARG
    assert "x is NULL" in L.last_error()
    assert lib.moe_route(ctypes.c_void_p(0x100008), ok, ctypes.byref(s), ok, ok, ok, ok, 1 << 30, None) == L.MOE_ERR_MISALIGNED
    assert lib.moe_combine(ok, ok, None, ctypes.byref(s), ok, None) == L.MOE_ERR_INVALID_ARG
    rc = lib.moe_dispatch_bwd(ok, ok, ok, None, ctypes.byref(s), ok, None, 0, None)
    assert rc == L.MOE_ERR_INVALID_ARG  # dlogits without w_router
    assert lib.mxfp8_quantize(ok, 10, 48, 0, ok, ok, None) == L.MOE_ERR_INVALID_ARG  # 48 % 32
    assert lib.mxfp8_quantize(ok, 10, 64, 2, ok, ok, None) == L.MOE_ERR_INVALID_ARG


def test_workspace_too_small():
    lib = L.load()
    s = shape()
    p = ctypes.c_void_p(0x100000)
    rc = lib.moe_dispatch(p, p, ctypes.byref(s), p, p, p, p, p, None, p, 16, None)
    assert rc == L.MOE_ERR_WORKSPACE
    rc = lib.moe_dispatch(p, p, ctypes.byref(s), p, p, p, p, p, None, ctypes.c_void_p(0x100010), 1 << 20, None)
    assert rc == L.MOE_ERR_MISALIGNED  # ws must be 256-byte aligned
    rc = lib.moe_grouped_ffn_fwd(p, None, p, p, p, p, ctypes.byref(s), p, 10, p, None, 0, None)
    assert rc == L.MOE_ERR_WORKSPACE
    rc = lib.moe_grouped_ffn_bwd(p, None, p, None, p, p, p, p, ctypes.byref(s), p, p, p, p, p, p, 10, None)
    assert rc == L.MOE_ERR_WORKSPACE
    rc = lib.moe_route_bwd(p, p, p, p, p, ctypes.byref(s), p, p, p, 0, None)
    assert rc == L.MOE_ERR_WORKSPACE
    sb = shape(dtype="bf16")
    rc = lib.moe_route(p, p, ctypes.byref(sb), p, p, p, p, 16, None)  # bf16 router needs W_r^T space
    assert rc == L.MOE_ERR_WORKSPACE
    assert L.workspace_size(L.MOE_OP_ROUTE, s) == 0 and L.workspace_size(L.MOE_OP_ROUTE, sb) == 16 * 64 * 2


def test_mxfp8_layer_needs_multiples_of_128_and_a_workspace():
    lib = L.load()
    p = ctypes.c_void_p(0x100000)
    s = shape(dtype="mxfp8", d=64)
    rc = lib.moe_grouped_ffn_fwd(p, None, p, p, p, p, ctypes.byref(s), p, 1 << 40, p, p, 1 << 40, None)
    assert rc == L.MOE_ERR_UNSUPPORTED
    s = shape(dtype="mxfp8", d=128)
    assert L.workspace_size(L.MOE_OP_FFN_FWD, s) > 0
    assert L.workspace_size(L.MOE_OP_FFN_BWD, s) > L.workspace_size(L.MOE_OP_FFN_BWD, shape(dtype="bf16", d=128))
    rc = lib.moe_grouped_ffn_fwd(p, None, p, p, p, p, ctypes.byref(s), p, 1 << 40, p, p, 16, None)
    assert rc == L.MOE_ERR_WORKSPACE


def test_mx_image_arguments_are_checked_on_the_host():
    """The MXFP8 images of xp and d_o: sized by moe_mx_image_size, accepted only
    for MXFP8 layers and only 256-byte aligned; nothing is enqueued on error."""
    lib = L.load()
    assert L.mx_image_size(1024, 4096) == (1024 * 4096 + 16 + 255) // 256 * 256 + (1024 * 128 + 16 + 255) // 256 * 256
    assert lib.moe_mx_image_size(0, 64) == ctypes.c_size_t(-1).value
    assert lib.moe_mx_image_size(32, 96) == ctypes.c_size_t(-1).value
    p = ctypes.c_void_p(0x100000)
    bf = shape(dtype="bf16", d=128)
    mx = shape(dtype="mxfp8", d=128, f=128)
    ws = L.workspace_size(L.MOE_OP_DISPATCH, mx)
    rc = lib.moe_dispatch(p, p, ctypes.byref(bf), p, p, p, p, p, p, p, 1 << 20, None)
    assert rc == L.MOE_ERR_INVALID_ARG and "MXFP8" in L.last_error()
    rc = lib.moe_dispatch(p, p, ctypes.byref(mx), p, p, p, p, p, ctypes.c_void_p(0x100080), p, ws, None)
    assert rc == L.MOE_ERR_MISALIGNED
    rc = lib.moe_combine_bwd(p, p, p, p, None, None, ctypes.byref(bf), p, p, p, None)
    assert rc == L.MOE_ERR_INVALID_ARG
    rc = lib.moe_combine_bwd(p, p, p, p, p, p, ctypes.byref(mx), p, ctypes.c_void_p(0x100010), p, None)
    assert rc == L.MOE_ERR_MISALIGNED
    # The MXFP8 operands of d_o need the permutation and the offsets.
    rc = lib.moe_combine_bwd(p, p, p, p, None, p, ctypes.byref(mx), None, p, p, None)
    assert rc == L.MOE_ERR_INVALID_ARG and "token_of_row" in L.last_error()
    assert L.mx_dout_image_size(mx) > L.mx_image_size(mx.T * mx.k, mx.d)
    # xp's operands: the image along d, then the one along each expert's
    # tokens (every expert's rows padded to 64), the layout of d_o's first two.
    S, P = mx.T * mx.k, (mx.T * mx.k + 63 * mx.E + 63) // 64 * 64
    part = lambda n: (n + 16 + 255) // 256 * 256  # noqa: E731
    assert L.mx_xp_image_size(mx) == L.mx_image_size(S, mx.d) + part(P * mx.d) + part(P * mx.d // 32)
    assert L.mx_dout_image_size(mx) == L.mx_xp_image_size(mx) + part(S * 4)
    assert lib.moe_mx_xp_image_size(ctypes.byref(bf)) == ctypes.c_size_t(-1).value
    # xp may be NULL only beside its images.
    rc = lib.moe_dispatch(p, p, ctypes.byref(mx), p, p, p, p, None, None, p, ws, None)
    assert rc == L.MOE_ERR_INVALID_ARG and "xp_out" in L.last_error()
    rc = lib.moe_grouped_ffn_fwd(None, None, p, p, p, p, ctypes.byref(mx), p, 1 << 40, p, p, 1 << 40, None)
    assert rc == L.MOE_ERR_INVALID_ARG and "xp" in L.last_error()
    rc = lib.moe_grouped_ffn_bwd(p, None, None, None, p, p, p, p, ctypes.byref(mx), p, p, p, p, p, p, 1 << 40, None)
    assert rc == L.MOE_ERR_INVALID_ARG and "xp" in L.last_error()
    rc = lib.moe_grouped_ffn_bwd(p, None, None, p, p, p, p, p, ctypes.byref(bf), p, p, p, p, p, p, 1 << 40, None)
    assert rc == L.MOE_ERR_INVALID_ARG and "MXFP8" in L.last_error()
    rc = lib.moe_grouped_ffn_fwd(p, p, p, p, p, p, ctypes.byref(bf), p, 1 << 40, p, p, 1 << 40, None)
    assert rc == L.MOE_ERR_INVALID_ARG
    rc = lib.moe_grouped_ffn_bwd(p, ctypes.c_void_p(0x100040), p, None, p, p, p, p, ctypes.byref(mx), p, p, p, p, p,
                                 p, 1 << 40, None)
    assert rc == L.MOE_ERR_MISALIGNED


def test_recompute_flag_sizes_and_checks():
    """MOE_FLAG_RECOMPUTE moves G, U, H from the save buffer into the FFN
    workspaces (MXFP8: G, U and H's token-major operand; the save buffer keeps
    only the dgrad weight copies); unknown flag bits are rejected."""
    T, d, E, k, f = 256, 128, 8, 4, 128
    S = T * k
    for dt, b in (("f32", 4), ("bf16", 2)):
        plain = shape(T=T, d=d, E=E, k=k, f=f, dtype=dt)
        rec = L.MoeShape.make(T, d, E, k, f, dt, L.MOE_FLAG_RECOMPUTE)
        guh = (3 * S * f * b + 255) // 256 * 256
        assert L.save_size(plain) == guh and L.save_size(rec) == 0
        assert L.workspace_size(L.MOE_OP_FFN_FWD, plain) == 0
        assert L.workspace_size(L.MOE_OP_FFN_FWD, rec) == guh
        assert L.workspace_size(L.MOE_OP_FFN_BWD, rec) == L.workspace_size(L.MOE_OP_FFN_BWD, plain) + guh
    lib = L.load()
    bad = L.MoeShape.make(T, d, E, k, f, "bf16", 2)
    assert lib.moe_save_size(ctypes.byref(bad)) == ctypes.c_size_t(-1).value
    mxp = L.MoeShape.make(T, d, E, k, f, "mxfp8")
    mxr = L.MoeShape.make(T, d, E, k, f, "mxfp8", L.MOE_FLAG_RECOMPUTE)
    P = (S + 63 * E + 63) // 64 * 64
    gu = 2 * ((P * f * 3 + 255) // 256 * 256)  # the blocked 24-bit G, U planes
    ht = (P * f + 16 + 255) // 256 * 256 + (P * f // 32 + 16 + 255) // 256 * 256  # H along the tokens
    assert L.save_size(mxr) == L.save_size(mxp) - gu - ht
    assert L.workspace_size(L.MOE_OP_FFN_FWD, mxr) == L.workspace_size(L.MOE_OP_FFN_FWD, mxp) + ht + gu
    assert L.workspace_size(L.MOE_OP_FFN_BWD, mxr) > L.workspace_size(L.MOE_OP_FFN_BWD, mxp) + gu
    # A recompute layer's forward needs its workspace (G, U, H live there).
    rec = L.MoeShape.make(T, d, E, k, f, "bf16", L.MOE_FLAG_RECOMPUTE)
    p = ctypes.c_void_p(0x100000)
    rc = lib.moe_grouped_ffn_fwd(p, None, p, p, p, p, ctypes.byref(rec), None, 0, p, p, 16, None)
    assert rc == L.MOE_ERR_WORKSPACE


def test_load_stats_argument_checks():
    lib = L.load()
    p = ctypes.c_void_p(0x100000)
    assert lib.moe_load_stats(None, 8, p, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_load_stats(p, 0, p, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_load_stats(p, 257, p, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_load_stats(p, 8, ctypes.c_void_p(0x100008), None) == L.MOE_ERR_MISALIGNED


def test_grouped_quantize_argument_checks():
    lib = L.load()
    p = ctypes.c_void_p(0x100000)
    assert lib.mxfp8_quantize_grouped(None, 64, 64, p, 2, p, p, None) == L.MOE_ERR_INVALID_ARG
    assert lib.mxfp8_quantize_grouped(p, 0, 64, p, 2, p, p, None) == L.MOE_ERR_INVALID_ARG
    assert lib.mxfp8_quantize_grouped(p, 64, 64, p, 0, p, p, None) == L.MOE_ERR_INVALID_ARG
    assert lib.mxfp8_quantize_grouped(p, 64, 64, p, 257, p, p, None) == L.MOE_ERR_INVALID_ARG
    assert lib.mxfp8_quantize_grouped(p, 1 << 31, 1, p, 1, p, p, None) == L.MOE_ERR_UNSUPPORTED


def test_mxfp8_routed_rows_limit():
    """MXFP8 layers address a weight-gradient tile's 256 token-major rows (P
    bytes each, P = T*k + 63 E + 63 rounded down to 64) with 32-bit offsets:
    P must stay below 2^23, i.e. T*k + 63 E + 63 < 2^23. The bf16 layer of
    the same size is accepted."""
    lim = (1 << 23) - 64 - 63 * 8  # T*k + 63 E + 63 = 2^23 - 1 at E = 8 and T*k = lim + 56
    ok = L.MoeShape.make(lim // 4, 128, 8, 4, 128, "mxfp8")
    assert L.workspace_size(L.MOE_OP_FFN_FWD, ok) > 0
    big = L.MoeShape.make((lim + 64) // 4, 128, 8, 4, 128, "mxfp8")
    with pytest.raises(L.MoeError, match="MXFP8 layers support"):
        L.workspace_size(L.MOE_OP_FFN_FWD, big)
    assert L.workspace_size(L.MOE_OP_FFN_FWD, L.MoeShape.make((lim + 64) // 4, 128, 8, 4, 128, "bf16")) >= 0
