"""Where an MXFP8 layer's workspaces hold the quantised GEMM operands, and
how to read them back for byte-for-byte comparison with the oracle's
encoder. The layout is the library's documented one: every piece starts
256-byte aligned with at least 16 bytes of slack after it; K-major operands
are E4M3 codes [rows][K] with E8M0 scales [K/64][rows][2]; token-major
(weight-gradient) operands are codes [C][P] with scales [P/64][C][2], each
expert's rows padded with zero rows to a multiple of 64 inside P.
"""
from __future__ import annotations

import numpy as np

from oracle import moe_oracle as O


def _a256(n: int) -> int:
    return (n + 255) // 256 * 256


def _carve(sizes):
    """Offsets of consecutive pieces of the given byte sizes."""
    out, used = [], 0
    for n in sizes:
        out.append(used)
        used += _a256(n + 16)
    return out, used


def padded_rows(S: int, E: int) -> int:
    return (S + 63 * E + 63) // 64 * 64


def fwd_pieces(S, d, f, E):
    """Forward workspace: xq, xs, wgq, wgs, wuq, wus, hq, hs, wdq, wds."""
    w = E * d * f
    names = ["xq", "xs", "wgq", "wgs", "wuq", "wus", "hq", "hs", "wdq", "wds"]
    sizes = [S * d, S * d // 32, w, w // 32, w, w // 32, S * f, S * f // 32, w, w // 32]
    off, _ = _carve(sizes)
    return {n: (o, s) for n, o, s in zip(names, off, sizes)}


def bwd_pieces(S, d, f, E):
    """Backward workspace (after the fp32 dG|dU rows): doq, dos, dguq, dgus,
    poff, blk, ht, hts, dot, dots, xt, xts, dgut, dguts."""
    P = padded_rows(S, E)
    names = ["doq", "dos", "dguq", "dgus", "poff", "blk", "ht", "hts", "dot", "dots", "xt", "xts", "dgut", "dguts"]
    sizes = [S * d, S * d // 32, S * 2 * f, S * 2 * f // 32, (E + 1) * 4, P // 64 * 8,
             P * f, P * f // 32, P * d, P * d // 32, P * d, P * d // 32, P * 2 * f, P * 2 * f // 32]
    off, _ = _carve(sizes)
    base = _a256(S * 2 * f * 4)
    return {n: (base + o, s) for n, o, s in zip(names, off, sizes)}


def _np(t):
    return t.cpu().numpy()


def check_kmajor(ws, pieces, q, s, vals, what, S=None, row0=0):
    """Rows row0 .. row0 + len(vals) of a K-major image in workspace `ws` (a
    uint8 device tensor; the image has S rows, default len(vals)) equal the
    oracle's codes of `vals` (blocks of 32 along each row)."""
    rows, K = vals.shape
    S = rows if S is None else S
    qo, _ = pieces[q]
    so, _ = pieces[s]
    codes = _np(ws[qo + row0 * K:qo + (row0 + rows) * K]).reshape(rows, K)
    sc = _np(ws[so:so + S * K // 32].view(K // 64, S, 2)[:, row0:row0 + rows, :])
    sc = sc.transpose(1, 0, 2).reshape(rows, K // 32)
    rq, rs = O.mx_quantize(vals, "cols")
    np.testing.assert_array_equal(codes, rq, err_msg=f"{what} codes")
    np.testing.assert_array_equal(sc, rs, err_msg=f"{what} scales")


def check_token_major(ws, pieces, q, s, vals, offsets, what, experts=None, S=None, C=None):
    """The token-major image in workspace `ws` of an [S][C] operand: for each
    expert (all, or those listed), its rows padded with zeros to a multiple
    of 64, blocked in 32 rows down each column, equal the oracle's codes and
    scales. `vals` holds all S rows, or, with `experts` given, only the
    listed experts' rows one after the other (then S and C must be given)."""
    E = len(offsets) - 1
    S = vals.shape[0] if S is None else S
    C = vals.shape[1] if C is None else C
    P = padded_rows(S, E)
    qo, _ = pieces[q]
    so, _ = pieces[s]
    codes = ws[qo:qo + C * P].view(C, P)
    sc = ws[so:so + P * C // 32].view(P // 64, C, 2)
    n = np.diff(offsets)
    poff = np.concatenate([[0], np.cumsum((n + 63) // 64 * 64)])
    at = 0
    for e in (range(E) if experts is None else experts):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            continue
        n64 = (b - a + 63) // 64 * 64
        pad = np.zeros((n64, C))
        if experts is None:
            pad[:b - a] = vals[a:b]
        else:
            pad[:b - a] = vals[at:at + b - a]
            at += b - a
        rq, rs = O.mx_quantize(pad, "rows")
        p0 = int(poff[e])
        np.testing.assert_array_equal(_np(codes[:, p0:p0 + n64]), rq.T, err_msg=f"{what} codes, expert {e}")
        dev_s = _np(sc[p0 // 64:(p0 + n64) // 64]).transpose(0, 2, 1).reshape(n64 // 32, C)
        np.testing.assert_array_equal(dev_s, rs, err_msg=f"{what} scales, expert {e}")
