"""moe_dispatch_noalloc (the dispatch whose workspace is the library's own
device array) against moe_dispatch with a caller workspace, through the C
ABI: every output bit for bit, on two calls in a row, the second with fewer
tokens (the array keeps the first call's contents); MXFP8 with and without
xp's bf16 rows beside its E4M3 operands."""
import numpy as np
import pytest
import torch

import routing_grouped_gemm_softmax_amd as pkg
from routing_grouped_gemm_softmax_amd import _lib as L

pytestmark = pytest.mark.gpu


def _routing(T, E, k, seed):
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    return torch.from_numpy(idx).cuda()


def _run(fn_name, x, idx, shape, mx, rows=True):
    T, d, E, k = shape.T, shape.d, shape.E, shape.k
    S = T * k
    out = dict(
        counts=torch.full((E,), -7, dtype=torch.int32, device="cuda"),
        offsets=torch.full((E + 1,), -7, dtype=torch.int32, device="cuda"),
        row_of_slot=torch.full((T * k,), -7, dtype=torch.int32, device="cuda"),
        token_of_row=torch.full((S,), -7, dtype=torch.int32, device="cuda"),
    )
    if rows:  # else (MXFP8) the dispatch writes only xp's two E4M3 operands
        out["xp"] = torch.full((S, d), 3.0, dtype=x.dtype, device="cuda")
    xp_mx = torch.full((L.mx_xp_image_size(shape),), 0x55, dtype=torch.uint8, device="cuda") if mx else None
    if fn_name == "moe_dispatch":
        ws = torch.empty(L.workspace_size(L.MOE_OP_DISPATCH, shape), dtype=torch.uint8, device="cuda")
        L.moe_dispatch(x, idx, shape, out["counts"], out["offsets"], out["row_of_slot"], out["token_of_row"],
                       out.get("xp"), ws, xp_mx=xp_mx)
    else:
        L.moe_dispatch_noalloc(x, idx, shape, out["counts"], out["offsets"], out["row_of_slot"],
                               out["token_of_row"], out.get("xp"), xp_mx=xp_mx)
    torch.cuda.synchronize()
    if mx:
        out["xp_mx"] = xp_mx
    return {n: t.cpu() for n, t in out.items()}


@pytest.mark.parametrize("dtype", ["bf16", "mxfp8", "f32"])
def test_noalloc_dispatch_matches_dispatch_twice(dtype):
    torch.manual_seed(0)
    E, k, d = 128, 4, 256
    for call, T in enumerate((5000, 700)):  # 40 chunks of 128 tokens, then 6
        print(f"dispatch_noalloc dtype={dtype} call={call} T={T} E={E} k={k} d={d}", flush=True)
        shape = L.MoeShape.make(T, d, E, k, 128, dtype)
        tdt = torch.float32 if dtype == "f32" else torch.bfloat16
        x = torch.randn(T, d, device="cuda").to(tdt)
        idx = _routing(T, E, k, seed=call)
        mx = dtype == "mxfp8"
        for rows in ((True, False) if mx else (True,)):
            ref = _run("moe_dispatch", x, idx, shape, mx, rows)
            got = _run("moe_dispatch_noalloc", x, idx, shape, mx, rows)
            assert set(got) == set(ref)
            for name in ref:
                assert torch.equal(got[name].view(torch.uint8) if got[name].dtype == torch.bfloat16 else got[name],
                                   ref[name].view(torch.uint8) if ref[name].dtype == torch.bfloat16 else ref[name]), \
                    f"{name} differs (call {call}, T={T}, xp rows {rows})"
            assert int(got["offsets"][-1]) == T * k


def test_noalloc_refuses_shapes_beyond_its_array():
    shape = L.MoeShape.make(1 << 22, 128, 256, 4, 128, "bf16")
    fake = torch.empty(16, dtype=torch.int32, device="cuda")
    rc = L.load().moe_dispatch_noalloc(fake.data_ptr(), fake.data_ptr(), __import__("ctypes").byref(shape),
                                       fake.data_ptr(), fake.data_ptr(), fake.data_ptr(), fake.data_ptr(),
                                       fake.data_ptr(), None, None)
    assert rc == L.MOE_ERR_WORKSPACE
    assert "1048576" in L.last_error()
