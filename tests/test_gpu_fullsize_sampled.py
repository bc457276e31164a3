"""Full-size GPU parity for the workloads whose complete fp64 oracle would take
too long on the host: the skewed Zipf(1.2) bf16 layer (T=16384, d=4096,
E=128, k=4, f=1536) and the MXFP8 layer (T=32768, d=4096, E=128, k=4,
f=1536), in the launch configuration the benchmark times.

Checked in full (bit-exact): counts, offsets, row_of_slot, token_of_row, and
zero weight gradients of every empty expert. Against the oracle computed
from the inputs alone (end to end): every output of whole experts (G, U, H,
O, dO, dG, dU, every dXp row and the expert's three weight gradients) - for
the Zipf layer the coldest non-empty expert, a median one and the hottest
one (about 12k rows: the longest K of the weight-gradient GEMMs and the
cost-cut schedule), for the MXFP8 layer two experts; y and dx of 24 random
tokens through all k of their experts; the xp bytes of 512 random rows (for
the MXFP8 layer, which keeps xp only as E4M3 operands, their codes). For
the MXFP8 layer also stage by stage (the oracle fed the device's stored fp32
intermediates, 2e-2) and, byte for byte, the E4M3 images of the two experts'
rows (K-major H and dG | dU; token-major H, dO, Xp, dG | dU). Each piece is
an exact sub-problem of the full layer: rows are independent in the forward
and in dXp (every row operand is quantised along its own row), and an
expert's weight gradients use only that expert's rows. Tolerances: 2e-2 for
bf16, 6e-2 for MXFP8 end to end.
"""
import numpy as np
import pytest
import torch

from moe_inputs import WORKLOADS, make_inputs
from oracle import moe_oracle as O

from gpu_util import dev, host, rel_err
import mx_layout as ML

pytestmark = pytest.mark.gpu


def _rows(t, sel):
    """Rows `sel` of a device tensor, on the host in fp64."""
    return host(t[torch.as_tensor(np.asarray(sel, dtype=np.int64), device=t.device)]).astype(np.float64)


class _Full:
    def __init__(self, name):
        from routing_grouped_gemm_softmax_amd import MoELayer
        self.wl = wl = WORKLOADS[name]
        self.mx = wl.dtype == "mxfp8"
        print(f"[gpu] full-size sampled {name}: T={wl.T} d={wl.d} E={wl.E} k={wl.k} f={wl.f} {wl.dtype}",
              flush=True)
        self.inp = inp = make_inputs(wl, 0)
        layer = MoELayer(wl.T, wl.d, wl.E, wl.k, wl.f, wl.dtype, learned_routing=False)
        bf = torch.bfloat16
        t = {n: dev(inp[n], bf) for n in ("x", "dy", "w_gate", "w_up", "w_down")}
        layer.forward(t["x"], t["w_gate"], t["w_up"], t["w_down"], topk_idx=dev(inp["topk_idx"], torch.int32),
                      topk_gate=dev(inp["topk_gate"], torch.float32))
        layer.backward(t["dy"])
        torch.cuda.synchronize()
        del t
        self.layer = layer
        self.counts, self.offsets, self.row_of_slot, self.token_of_row = O.dispatch_plan(inp["topk_idx"], wl.E)
        self.slot_of_row = np.empty(wl.T * wl.k, dtype=np.int64)
        self.slot_of_row[self.row_of_slot.reshape(-1)] = np.arange(wl.T * wl.k)

    def w(self, e):
        return tuple(self.inp[n][e:e + 1] for n in ("w_gate", "w_up", "w_down"))

    def xp(self, rows):
        return self.inp["x"][self.token_of_row[rows]].astype(np.float64)

    def d_o(self, rows):
        """Oracle dO rows: g[t, j] dy[t] for the slot (t, j) of each row."""
        t, j = np.divmod(self.slot_of_row[rows], self.wl.k)
        return self.inp["topk_gate"][t, j].astype(np.float64)[:, None] * self.inp["dy"][t].astype(np.float64)

    def fwd(self, xp, e, h_in=None):
        one = np.array([0, len(xp)])
        if self.mx:
            return O.ffn_forward_mx(xp, *self.w(e), one, h_in=h_in)
        return O.ffn_forward(xp, *self.w(e), one)

    def bwd(self, d_o, xp, e, G, U, H, dgdu_in=None, dgdu_w_in=None):
        one = np.array([0, len(xp)])
        if self.mx:
            return O.ffn_backward_mx(d_o, xp, *self.w(e), one, G, U, H, dgdu_in=dgdu_in, dgdu_w_in=dgdu_w_in)
        return O.ffn_backward(d_o, xp, *self.w(e), one, G, U, H)


def _expert_device(F, e):
    """Expert e's rows of the device's stored tensors (host, fp64)."""
    L = F.layer
    a, b = int(F.offsets[e]), int(F.offsets[e + 1])
    rows = np.arange(a, b)
    dv = dict(O=_rows(L.o, rows), dXp=_rows(L.dxp, rows),
              dW_gate=host(L.dw_gate[e]), dW_up=host(L.dw_up[e]), dW_down=host(L.dw_down[e]))
    if F.mx:
        # MXFP8: 24-bit G, U blocked in the save buffer; H, dG | dU and dO
        # exist only as E4M3 operands (checked as images); dO's values are
        # the fp32 products of the gates and dy that the device encodes.
        wl = F.wl
        t, j = np.divmod(F.slot_of_row[rows], wl.k)
        dv["dO"] = (F.inp["topk_gate"][t, j].astype(np.float32)[:, None]
                    * F.inp["dy"][t].astype(np.float32)).astype(np.float64)
        dv["G"], dv["U"] = (ML.blocked_rows(L.save, n, rows, F.offsets, wl.T * wl.k, wl.f, wl.E) for n in "GU")
    else:
        dv["dO"] = _rows(L.d_o, rows)
        dv["G"], dv["U"], dv["H"] = (_rows(t, rows) for t in L.saved())
        dv["dG"], dv["dU"] = (_rows(t, rows) for t in L.dgu())
    return rows, dv


def _check_expert(F, e):
    """Every output of expert e's rows and its weight gradients, against the
    oracle's forward and backward of those rows from the inputs alone."""
    rows, dv = _expert_device(F, e)
    xp = F.xp(rows)
    d_o_ref = F.d_o(rows)
    Gr, Ur, Hr, Or = F.fwd(xp, e)
    bwd = F.bwd(d_o_ref, xp, e, Gr, Ur, Hr)
    ref = dict(G=Gr, U=Ur, H=Hr, O=Or, dO=d_o_ref, dG=bwd[4], dU=bwd[5], dXp=bwd[0],
               dW_gate=bwd[1][0], dW_up=bwd[2][0], dW_down=bwd[3][0])
    return {n: rel_err(dv[n], ref[n]) for n in ref if n in dv}, (rows, dv, xp)


def _images_of(F, e, rows, ws, pieces, kq, ks, tq, ts, K):
    """An operand of expert e's rows as the device holds it, dequantised: its
    K-major image (kq, ks; None to skip) and its token-major one (tq, ts), both
    in workspace or save buffer `ws`."""
    wl = F.wl
    S = wl.T * wl.k
    a, b = int(rows[0]), int(rows[-1]) + 1
    k_major = None
    if kq is not None:
        qo, _ = pieces[kq]
        so, _ = pieces[ks]
        codes = host(ws[qo + a * K:qo + b * K]).reshape(b - a, K)
        sc = host(ws[so:so + S * K // 32].view(K // 64, S, 2)[:, a:b, :]).transpose(1, 0, 2)
        k_major = O.mx_dequantize(codes, sc.reshape(b - a, K // 32), "cols")
    if tq is None:
        return k_major, None
    p0 = int(ML.padded_offsets(F.offsets)[e])
    P = ML.padded_rows(S, wl.E)
    qo, _ = pieces[tq]
    so, _ = pieces[ts]
    n64 = (b - a + 63) // 64 * 64
    tc = host(ws[qo:qo + K * P].view(K, P)[:, p0:p0 + n64])
    tsc = host(ws[so:so + P * K // 32].view(P // 64, K, 2)[p0 // 64:(p0 + n64) // 64])
    tsc = tsc.transpose(1, 0, 2).reshape(K, -1)
    t_major = O.mx_dequantize(tc, tsc, "cols")[:, :b - a].T
    return k_major, t_major


def _check_expert_stage(F, e, rows, dv, xp):
    """MXFP8: each GEMM stage of expert e on the device's own operands: its
    stored G, U, H, dO, and its dG | dU images for the dXp GEMM and the
    weight gradients. The oracle's dG, dU from the device's G, U, dO are
    returned for the image checks."""
    L, wl = F.layer, F.wl
    S, d, f, E = wl.T * wl.k, wl.d, wl.f, wl.E
    pf, pb, ps = ML.fwd_pieces(S, d, f, E), ML.bwd_pieces(S, d, f, E), ML.save_pieces(S, d, f, E)
    hk, ht = _images_of(F, e, rows, L.ws_ffn_fwd, pf, "hq", "hs", None, None, f)[0], \
        _images_of(F, e, rows, L.save, ps, None, None, "ht", "hts", f)[1]
    k_major, t_major = _images_of(F, e, rows, L.ws_ffn_bwd, pb, "dguq", "dgus", "dgut", "dguts", 2 * f)
    Gr, Ur, Hr, Or = F.fwd(xp, e, h_in=hk)
    bwd = F.bwd(dv["dO"], xp, e, dv["G"], dv["U"], ht, dgdu_in=(k_major[:, :f], k_major[:, f:]),
                dgdu_w_in=(t_major[:, :f], t_major[:, f:]))
    ref = dict(G=Gr, U=Ur, O=Or, dXp=bwd[0], dW_gate=bwd[1][0], dW_up=bwd[2][0], dW_down=bwd[3][0])
    return {n: rel_err(dv[n], ref[n]) for n in ref}, (bwd[4], bwd[5])


def _check_expert_images(F, e, rows, dv, xp, dgdu):
    """MXFP8: the E4M3 images of expert e's rows against the oracle's encoding:
    byte for byte where the device stored the values it quantised (dO, Xp),
    and as the same decisions up to the device's rounding for H (the exact
    SwiGLU of the device's G, U) and dG | dU (the oracle's values from the
    device's stored G, U, dO), which the device keeps only as images."""
    L, wl = F.layer, F.wl
    S, d, f, E = wl.T * wl.k, wl.d, wl.f, wl.E
    pf, pb = ML.fwd_pieces(S, d, f, E), ML.bwd_pieces(S, d, f, E)
    a = int(rows[0])
    dgu = np.concatenate(dgdu, axis=1)
    atol = np.concatenate([np.full(f, 2e-4 * np.abs(dgdu[0]).max()), np.full(f, 2e-4 * np.abs(dgdu[1]).max())])
    H = dv["G"] * O.sigmoid(dv["G"]) * dv["U"]  # the exact SwiGLU of the device's G, U
    atol_h = 1e-5 * np.abs(H).max()
    ps = ML.save_pieces(S, d, f, E)
    ML.check_kmajor(L.ws_ffn_fwd, pf, "hq", "hs", H, f"q(H) expert {e}", S=S, row0=a, near=True, atol=atol_h)
    ML.check_token_major(L.save, ps, "ht", "hts", H, F.offsets, "q(ht)", experts=[e], S=S, C=f, near=True,
                         atol=np.full(f, atol_h))
    ML.check_kmajor(L.ws_ffn_bwd, pb, "dguq", "dgus", dgu, f"q(dG|dU) expert {e}", S=S, row0=a, near=True,
                    atol=atol)
    ML.check_token_major(L.d_o_mx, ML.dout_pieces(S, d, E), "dot", "dots", dv["dO"], F.offsets, "q(dot)",
                         experts=[e], S=S, C=d)
    # Xp along the tokens: written by the dispatch pass from x.
    ML.check_token_major(L.xp_mx, ML.xp_pieces(S, d, E), "xt", "xts", xp, F.offsets, "q(xt)", experts=[e], S=S,
                         C=d)
    ML.check_token_major(L.ws_ffn_bwd, pb, "dgut", "dguts", dgu, F.offsets, "q(dgut)", experts=[e], S=S, C=2 * f,
                         near=True, atol=atol)


def _check_rows_fwd(F, e, rows):
    L, wl = F.layer, F.wl
    xp = F.xp(rows)
    Gr, Ur, Hr, Or = F.fwd(xp, e)
    if F.mx:
        G, U = (ML.blocked_rows(L.save, n, rows, F.offsets, wl.T * wl.k, wl.f, wl.E) for n in "GU")
        return {"G": rel_err(G, Gr), "U": rel_err(U, Ur), "O": rel_err(_rows(L.o, rows), Or)}
    G, U, H = (_rows(t, rows) for t in L.saved())
    return {"G": rel_err(G, Gr), "U": rel_err(U, Ur), "H": rel_err(H, Hr), "O": rel_err(_rows(L.o, rows), Or)}


def _check_tokens(F, toks):
    """y and dx of tokens `toks` from the oracle's own forward and backward
    of their rows (end to end: no device intermediates fed in)."""
    wl, L = F.wl, F.layer
    y_ref = np.zeros((len(toks), wl.d)); dx_ref = np.zeros((len(toks), wl.d))
    gates = F.inp["topk_gate"].astype(np.float64)
    idx = F.inp["topk_idx"]
    pairs = [(n, j) for n in range(len(toks)) for j in range(wl.k)]
    by_e = {}
    for n, j in pairs:
        by_e.setdefault(int(idx[toks[n], j]), []).append((n, j))
    for e, lst in by_e.items():
        rows = np.array([F.row_of_slot[toks[n], j] for n, j in lst])
        xp = F.xp(rows)
        G, U, H, Ov = F.fwd(xp, e)
        dXp = F.bwd(F.d_o(rows), xp, e, G, U, H)[0]
        for i, (n, j) in enumerate(lst):
            y_ref[n] += gates[toks[n], j] * Ov[i]
            dx_ref[n] += dXp[i]
    return {"y": rel_err(_rows(L.y, toks), y_ref), "dx": rel_err(_rows(L.dx, toks), dx_ref)}


def _run_checks(name):
    F = _Full(name)
    L, wl = F.layer, F.wl
    np.testing.assert_array_equal(host(L.topk_idx), F.inp["topk_idx"])
    np.testing.assert_array_equal(host(L.counts), F.counts)
    np.testing.assert_array_equal(host(L.offsets), F.offsets)
    np.testing.assert_array_equal(host(L.row_of_slot), F.row_of_slot)
    np.testing.assert_array_equal(host(L.token_of_row), F.token_of_row)
    rng = np.random.default_rng(0)
    S = wl.T * wl.k
    rows = np.sort(rng.choice(S, 512, replace=False))
    if L.xp is not None:
        np.testing.assert_array_equal(_rows(L.xp, rows), F.xp(rows))
    else:
        # MXFP8: xp exists only as its two E4M3 operands; these rows of the
        # one along d, byte for byte (each row is quantised on its own).
        qo, _ = ML.xp_pieces(S, wl.d, wl.E)["xq"]
        so, _ = ML.xp_pieces(S, wl.d, wl.E)["xs"]
        sel = torch.as_tensor(rows, device=L.xp_mx.device)
        codes = host(L.xp_mx[qo:qo + S * wl.d].view(S, wl.d)[sel])
        sc = host(L.xp_mx[so:so + S * wl.d // 32].view(wl.d // 64, S, 2)[:, sel, :]).transpose(1, 0, 2)
        rq, rs = O.mx_quantize(F.xp(rows), "cols")
        np.testing.assert_array_equal(codes, rq)
        np.testing.assert_array_equal(sc.reshape(len(rows), -1), rs)
    empty = np.nonzero(F.counts == 0)[0]
    for e in empty:
        assert not host(L.dw_gate[e]).any() and not host(L.dw_up[e]).any() and not host(L.dw_down[e]).any()
    print(f"counts: min {F.counts.min()} max {F.counts.max()} empty {len(empty)}", flush=True)

    tol = 6e-2 if F.mx else 2e-2
    nonempty = np.nonzero(F.counts)[0]
    order = nonempty[np.argsort(F.counts[nonempty], kind="stable")]
    experts = [int(order[0]), int(order[len(order) // 2])]
    if not F.mx:
        experts.append(int(order[-1]))  # the hottest expert: every row, its weight gradients
    for e in experts:
        errs, (rows, dv, xp) = _check_expert(F, e)
        print(f"expert {e} (n={F.counts[e]}), end to end:", {n: f"{v:.2e}" for n, v in errs.items()}, flush=True)
        bad = {n: v for n, v in errs.items() if not v <= tol}
        assert not bad, (e, bad)
        if F.mx:
            stage, dgdu = _check_expert_stage(F, e, rows, dv, xp)
            print(f"expert {e}, stage by stage:", {n: f"{v:.2e}" for n, v in stage.items()}, flush=True)
            bad = {n: v for n, v in stage.items() if not v <= 2e-2}
            assert not bad, (e, bad)
            _check_expert_images(F, e, rows, dv, xp, dgdu)
        del dv, xp
    if F.mx:
        hot = int(order[-1])
        hot_rows = np.sort(F.offsets[hot] + rng.choice(F.counts[hot], min(128, F.counts[hot]), replace=False))
        errs = _check_rows_fwd(F, hot, hot_rows)
        print(f"expert {hot}, {len(hot_rows)} rows:", {n: f"{v:.2e}" for n, v in errs.items()}, flush=True)
        assert all(v <= tol for v in errs.values()), errs

    toks = np.sort(rng.choice(wl.T, 24, replace=False))
    e2e = _check_tokens(F, toks)
    print("24 sampled tokens:", {n: f"{v:.2e}" for n, v in e2e.items()}, flush=True)
    assert all(v <= tol for v in e2e.values()), e2e


@pytest.mark.timeout(600)
def test_zipf_full_size_sampled():
    _run_checks("bf16_zipf")


@pytest.mark.timeout(600)
def test_mxfp8_full_size_sampled():
    _run_checks("mxfp8_balanced")
