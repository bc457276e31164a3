"""Pins for the oracle's MXFP8 expert FFN (ffn_forward_mx / ffn_backward_mx).

Every GEMM operand is MXFP8-quantised along that GEMM's reduction axis, at
its exact value (computed operands H, dO, dG, dU are never rounded to a
storage type first). The pins: (1) a brute-force re-implementation of that
definition with explicit loops and an exhaustive nearest-code E4M3 search
(independent of the oracle's encoder), on ragged expert ranges that
exercise the per-expert padding of the weight gradients; (2) operands that
are already exactly representable leave every GEMM unchanged, so G, U and
the weight gradients equal the unquantised FFN; (3) quantising along the
wrong axis is caught by operands whose blocks along the two axes have very
different magnitudes; (4) the whole MXFP8 layer stays within a bound of the
unquantised layer that follows from the E4M3 rounding error, tensor by
tensor.
"""
import numpy as np
import pytest

from oracle import moe_oracle as O


def _e4m3_mags():
    """Non-negative finite E4M3 magnitudes (codes 0x00..0x7E), from the format
    definition: bias 7, 3 mantissa bits, exponent field 0 subnormal."""
    out = []
    for c in range(0x7F):
        e, m = c >> 3, c & 7
        out.append(m / 8.0 * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7))
    return np.array(out)


MAGS = _e4m3_mags()


def _q_block(v):
    """Dequantised MXFP8 block of 32: scale 2^(floor(log2 amax) - 8) clamped
    to 2^-127..2^127; each element -> nearest magnitude (ties: even code),
    saturating at 448, sign kept."""
    amax = max(abs(x) for x in v)
    if amax == 0:
        return [0.0] * len(v)
    e = int(np.floor(np.log2(amax)))
    while 2.0 ** e > amax:
        e -= 1
    while 2.0 ** (e + 1) <= amax:
        e += 1
    sc = 2.0 ** min(max(e - 8, -127), 127)
    res = []
    for x in v:
        a = abs(x) / sc
        dist = np.abs(MAGS - a)
        cand = np.nonzero(dist == dist.min())[0]
        even = [c for c in cand if c % 2 == 0]
        code = even[0] if even else cand[0]
        res.append(np.copysign(MAGS[code] * sc, x))
    return res


def _q_rows(a):  # blocks of 32 inside each row
    a = np.array(a, dtype=np.float64)
    out = np.zeros_like(a)
    for r in range(a.shape[0]):
        for j in range(0, a.shape[1], 32):
            out[r, j:j + 32] = _q_block(list(a[r, j:j + 32]))
    return out


def _q_cols(a):  # blocks of 32 down each column
    return _q_rows(np.asarray(a).T).T


def _q_cols_grouped(a, offsets):  # per expert range, zero-padded to 32
    a = np.asarray(a, dtype=np.float64)
    out = np.zeros_like(a)
    for e in range(len(offsets) - 1):
        lo, hi = offsets[e], offsets[e + 1]
        n = hi - lo
        if n == 0:
            continue
        pad = np.zeros(((n + 31) // 32 * 32, a.shape[1]))
        pad[:n] = a[lo:hi]
        out[lo:hi] = _q_cols(pad)[:n]
    return out


def _brute_ffn(xp, wg, wu, wd, off, do):
    E = len(off) - 1
    S, d = xp.shape
    f = wg.shape[2]
    sig = lambda z: 1.0 / (1.0 + np.exp(-z))
    xq = _q_rows(xp)
    G = np.zeros((S, f)); U = np.zeros((S, f)); H = np.zeros((S, f)); Ov = np.zeros((S, d))
    for e in range(E):
        lo, hi = off[e], off[e + 1]
        qg, qu = _q_cols(wg[e]), _q_cols(wu[e])
        for r in range(lo, hi):
            for c in range(f):
                G[r, c] = sum(xq[r, i] * qg[i, c] for i in range(d))
                U[r, c] = sum(xq[r, i] * qu[i, c] for i in range(d))
                H[r, c] = G[r, c] * sig(G[r, c]) * U[r, c]
    hq = _q_rows(H)
    for e in range(E):
        lo, hi = off[e], off[e + 1]
        qd = _q_cols(wd[e])
        for r in range(lo, hi):
            for c in range(d):
                Ov[r, c] = sum(hq[r, i] * qd[i, c] for i in range(f))
    # backward
    doq = _q_rows(do)
    dG = np.zeros((S, f)); dU = np.zeros((S, f))
    for e in range(E):
        lo, hi = off[e], off[e + 1]
        qdk = _q_rows(wd[e])               # W_down [f][d] along d
        for r in range(lo, hi):
            for c in range(f):
                dh = sum(doq[r, i] * qdk[c, i] for i in range(d))
                g, u = G[r, c], U[r, c]
                s = sig(g)
                dU[r, c] = dh * g * s
                dG[r, c] = dh * u * s * (1 + g * (1 - s))
    dgq, duq = _q_rows(dG), _q_rows(dU)
    hg, dog, xg = _q_cols_grouped(H, off), _q_cols_grouped(do, off), _q_cols_grouped(xp, off)
    dgg, dug = _q_cols_grouped(dG, off), _q_cols_grouped(dU, off)
    dxp = np.zeros((S, d)); dwg = np.zeros((E, d, f)); dwu = np.zeros((E, d, f)); dwd = np.zeros((E, f, d))
    for e in range(E):
        lo, hi = off[e], off[e + 1]
        qg, qu = _q_rows(wg[e]), _q_rows(wu[e])   # W [d][f] along f
        for r in range(lo, hi):
            for c in range(d):
                dxp[r, c] = sum(dgq[r, i] * qg[c, i] + duq[r, i] * qu[c, i] for i in range(f))
        for i in range(f):
            for c in range(d):
                dwd[e, i, c] = sum(hg[r, i] * dog[r, c] for r in range(lo, hi))
        for i in range(d):
            for c in range(f):
                dwg[e, i, c] = sum(xg[r, i] * dgg[r, c] for r in range(lo, hi))
                dwu[e, i, c] = sum(xg[r, i] * dug[r, c] for r in range(lo, hi))
    return (G, U, H, Ov), (dxp, dwg, dwu, dwd, dG, dU)


def _inputs(rng, E, d, f, counts, scale_rows=False):
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    S = int(off[-1])
    xp = rng.standard_normal((S, d))
    if scale_rows:  # very different magnitudes per block along each axis
        xp *= np.exp2(rng.integers(-6, 6, size=(S, 1))) * np.exp2(rng.integers(-6, 6, size=(1, d)))
    wg = rng.standard_normal((E, d, f)) * 0.05
    wu = rng.standard_normal((E, d, f)) * 0.05
    wd = rng.standard_normal((E, f, d)) * 0.05
    do = rng.standard_normal((S, d))
    return xp, wg, wu, wd, off, do


def _rel(a, b):
    den = np.abs(b).max()
    return float(np.abs(a - b).max() / (den if den else 1.0))


@pytest.mark.parametrize("scale_rows", [False, True])
def test_mx_ffn_matches_brute_force(scale_rows):
    rng = np.random.default_rng(11)
    xp, wg, wu, wd, off, do = _inputs(rng, 3, 64, 32, [17, 0, 23], scale_rows)
    fwd_b, bwd_b = _brute_ffn(xp, wg, wu, wd, off, do)
    fwd = O.ffn_forward_mx(xp, wg, wu, wd, off)
    bwd = O.ffn_backward_mx(do, xp, wg, wu, wd, off, fwd[0], fwd[1], fwd[2])
    for got, want in zip(fwd + bwd, fwd_b + bwd_b):
        assert _rel(got, want) < 1e-12
    # The empty expert gets exact zero weight gradients.
    assert not bwd[1][1].any() and not bwd[3][1].any()


def test_representable_operands_leave_the_gemms_unchanged():
    rng = np.random.default_rng(5)
    xp, wg, wu, wd, off, do = _inputs(rng, 2, 64, 64, [32, 64])
    # Make every operand exactly MXFP8-representable along every axis used.
    xp = O.mx_roundtrip(O.mx_roundtrip(xp, "cols"), "rows")
    xp = O.mx_roundtrip(xp, "cols")
    assert np.array_equal(O.mx_roundtrip(xp, "cols"), xp)
    wg = np.stack([O.mx_roundtrip(w, "rows") for w in wg])
    wu = np.stack([O.mx_roundtrip(w, "rows") for w in wu])
    G, U, H, _ = O.ffn_forward_mx(xp, wg, wu, wd, off)
    G0, U0, _, _ = O.ffn_forward(xp, wg, wu, wd, off)
    assert _rel(G, G0) < 1e-14 and _rel(U, U0) < 1e-14


def test_quantisation_is_idempotent_and_bounded():
    rng = np.random.default_rng(3)
    a = rng.standard_normal((64, 96)) * np.exp2(rng.integers(-8, 8, size=(64, 1)))
    for along in ("cols", "rows"):
        q = O.mx_roundtrip(a, along)
        assert np.array_equal(O.mx_roundtrip(q, along), q)
        # Per block of 32 with scale s = 2^(floor(log2 amax) - 8): an element
        # below 448 s is off by at most half its E4M3 spacing, 2^-4 of its
        # magnitude in the normal range and 2^-10 s in the subnormal range;
        # one above 448 s saturates to 448 s (at most 1/8 of it).
        blocks = (a if along == "cols" else a.T).reshape(-1, 32)
        qb = (q if along == "cols" else q.T).reshape(-1, 32)
        s = np.exp2(np.floor(np.log2(np.abs(blocks).max(axis=1, keepdims=True))) - 8)
        err = np.abs(qb - blocks)
        sat = np.abs(blocks) > 448 * s
        assert np.all(err[~sat] <= np.maximum(2.0 ** -4 * np.abs(blocks), 2.0 ** -10 * s)[~sat] * (1 + 1e-12))
        assert np.all(np.abs(qb[sat]) == (448 * s * np.ones_like(blocks))[sat])


def test_grouped_rows_pad_inside_each_range():
    rng = np.random.default_rng(8)
    a = rng.standard_normal((50, 64))
    off = np.array([0, 20, 50])
    g = O.mx_rows_grouped(a, off)
    assert np.array_equal(g[:20], O.mx_roundtrip(np.vstack([a[:20], np.zeros((12, 64))]), "rows")[:20])
    assert np.array_equal(g[20:], O.mx_roundtrip(np.vstack([a[20:], np.zeros((2, 64))]), "rows")[:30])


def test_stage_inputs_replace_the_computed_operands():
    """h_in and dgdu_in are what the later GEMMs quantise: feeding the exact
    values back gives the same results, feeding other values changes them."""
    rng = np.random.default_rng(4)
    xp, wg, wu, wd, off, do = _inputs(rng, 2, 64, 64, [40, 24])
    G, U, H, Ov = O.ffn_forward_mx(xp, wg, wu, wd, off)
    assert np.array_equal(O.ffn_forward_mx(xp, wg, wu, wd, off, h_in=H)[3], Ov)
    assert not np.array_equal(O.ffn_forward_mx(xp, wg, wu, wd, off, h_in=H * 1.3)[3], Ov)
    b = O.ffn_backward_mx(do, xp, wg, wu, wd, off, G, U, H)
    b2 = O.ffn_backward_mx(do, xp, wg, wu, wd, off, G, U, H, dgdu_in=(b[4], b[5]))
    for x, y in zip(b, b2):
        assert np.array_equal(x, y)
    # dgdu_w_in feeds the weight gradients only; MXFP8 numbers in the weight
    # gradient's blocking (the dequantised token-major operand) pass through.
    wq = (O.mx_rows_grouped(b[4], off), O.mx_rows_grouped(b[5], off))
    b3 = O.ffn_backward_mx(do, xp, wg, wu, wd, off, G, U, H, dgdu_w_in=wq)
    for x, y in zip(b, b3):
        assert np.array_equal(x, y)
    b4 = O.ffn_backward_mx(do, xp, wg, wu, wd, off, G, U, H, dgdu_w_in=(b[4] * 1.3, b[5]))
    assert np.array_equal(b4[0], b[0]) and np.array_equal(b4[2], b[2]) and np.array_equal(b4[3], b[3])
    assert not np.array_equal(b4[1], b[1])
    b5 = O.ffn_backward_mx(do, xp, wg, wu, wd, off, G, U, H, dgdu_in=(b[4] * 1.3, b[5]), dgdu_w_in=wq)
    assert not np.array_equal(b5[0], b[0])
    for i in (1, 2, 3):
        assert np.array_equal(b5[i], b[i])


# Distance of the MXFP8 layer from the unquantised one, max|mx - exact| /
# max|exact| per tensor. Each quantised element carries a relative rounding
# error of at most 2^-4 (1/8 where a block maximum saturates), i.e. an RMS
# of about 2.6% per operand, and every output passes through two to four
# quantised GEMM operands (y: Xp, W_gate|W_up, H, W_down; the weight
# gradients add dO and dG|dU), with the SwiGLU nonlinearity between. The
# measured distances are 4-13% at these shapes and up to 19% for weight
# gradients whose K runs over only 16 tokens per expert (fewer terms to
# average the rounding errors out). A dropped quantisation shows as exactly
# zero; a mis-scaled block exponent or a wrong operand is caught exactly by
# the brute-force pin above, this bound only catches gross departures.
MX_LAYER_BOUND = 0.25


@pytest.mark.parametrize("over", [dict(T=256, d=128, E=8, f=128), dict(T=512, d=256, E=16, f=256)],
                         ids=["T256_E8", "T512_E16"])
def test_mx_layer_distance_from_unquantised(over):
    from moe_inputs import WORKLOADS, make_inputs
    wl = WORKLOADS["mxfp8_balanced"].with_shape(**over)
    inp = make_inputs(wl, 0)
    fm = O.layer_forward(inp, wl.k, mx=True)
    bm = O.layer_backward(inp, fm, mx=True)
    fu = O.layer_forward(inp, wl.k)
    bu = O.layer_backward(inp, fu)
    dist = {n: _rel(fm[n], fu[n]) for n in ("G", "U", "H", "O", "y")}
    dist.update({n: _rel(bm[n], bu[n]) for n in ("dgate", "dG", "dU", "dXp", "dx",
                                                "dw_gate", "dw_up", "dw_down")})
    print("MXFP8 layer vs unquantised:", {n: f"{v:.3f}" for n, v in dist.items()})
    for n, v in dist.items():
        assert 0 < v < MX_LAYER_BOUND, (n, v)
    # dO = g dy passes through no quantised GEMM: identical in both layers.
    assert np.array_equal(bm["dO"], bu["dO"])
