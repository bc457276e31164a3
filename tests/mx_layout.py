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
    """Forward workspace: xq, xs, wgq, wgs, wuq, wus, hq, hs, wdq, wds, poff."""
    w = E * d * f
    names = ["xq", "xs", "wgq", "wgs", "wuq", "wus", "hq", "hs", "wdq", "wds", "poff"]
    sizes = [S * d, S * d // 32, w, w // 32, w, w // 32, S * f, S * f // 32, w, w // 32, (E + 1) * 4]
    off, _ = _carve(sizes)
    return {n: (o, s) for n, o, s in zip(names, off, sizes)}


def save_pieces(S, d, f, E):
    """Save buffer of an MXFP8 layer: the blocked G and U planes (24-bit
    words), then wgq, wgs, wuq, wus, wdq, wds (the dgrad weight copies) and
    ht, hts (H along each expert's tokens)."""
    P = padded_rows(S, E)
    plane = _a256(P * f * 3)
    w = E * d * f
    names = ["wgq", "wgs", "wuq", "wus", "wdq", "wds", "ht", "hts"]
    sizes = [w, w // 32, w, w // 32, w, w // 32, P * f, P * f // 32]
    off, _ = _carve(sizes)
    out = {"G": (0, P * f * 3), "U": (plane, P * f * 3)}
    out.update({n: (2 * plane + o, s) for n, o, s in zip(names, off, sizes)})
    return out


def dout_pieces(S, d, E):
    """The d_o operand buffer of an MXFP8 layer (moe_combine_bwd's d_o_mx):
    the K-major image (codes [S][d], scales [d/64][S][2]) then the
    token-major one: dot (codes [d][P]), dots (scales [P/64][d][2])."""
    P = padded_rows(S, E)
    off, _ = _carve([S * d, S * d // 32, P * d, P * d // 32])
    return {"doq": (off[0], S * d), "dos": (off[1], S * d // 32), "dot": (off[2], P * d), "dots": (off[3], P * d // 32)}


def xp_pieces(S, d, E):
    """The xp operand buffer of an MXFP8 layer (moe_dispatch's xp_mx): the
    K-major image (xq codes [S][d], xs scales [d/64][S][2]) then the
    token-major one: xt (codes [d][P]), xts (scales [P/64][d][2]); the
    layout of the first two parts of the d_o buffer."""
    p = dout_pieces(S, d, E)
    return {"xq": p["doq"], "xs": p["dos"], "xt": p["dot"], "xts": p["dots"]}


def dout_f32(gate, dy, row_of_slot, token_of_row):
    """The fp32 dO rows an MXFP8 layer encodes, in expert-sorted row order:
    gate(t, j) * dy[t] for the slot (t, j) of each row, one fp32 rounding of
    the product of the fp32 gate and the bf16 dy (as fp64 values)."""
    row_of_slot = np.asarray(row_of_slot)
    k = row_of_slot.shape[1]
    flat = row_of_slot.reshape(-1)
    ok = flat >= 0
    slot = np.zeros(len(token_of_row), np.int64)
    slot[flat[ok]] = np.nonzero(ok)[0]
    t, j = np.divmod(slot, k)
    g = np.asarray(gate, np.float32)[t, j]
    return (g[:, None] * np.asarray(dy, np.float32)[t]).astype(np.float64)


def padded_offsets(offsets):
    n = np.diff(np.asarray(offsets))
    return np.concatenate([[0], np.cumsum((n + 63) // 64 * 64)])


def blocked_rows(save, which, rows, offsets, S, f, E):
    """Rows `rows` (expert-sorted row ids, host array) of the blocked G or U
    plane of an MXFP8 layer's save buffer (a uint8 device tensor), as a host
    fp64 [len(rows)][f] array. Values are 24-bit words, the top three bytes
    of an fp32 (little-endian). Block (padded row / 32, column / 32) is
    3 KB; lane l of it holds row l % 32, columns 8 Q + 4 (l / 32) .. +3 as
    four words at byte 768 Q + 12 l."""
    import torch
    o, n = save_pieces(S, 1, f, E)[which]
    plane = save[o:o + n]
    rows = np.asarray(rows)
    offsets = np.asarray(offsets)
    e = np.searchsorted(offsets, rows, side="right") - 1
    pr = padded_offsets(offsets)[e] + rows - offsets[e]
    c = np.arange(f)
    fb = f // 32
    byte = ((pr[:, None] // 32) * fb + c[None, :] // 32) * 3072 + ((c[None, :] % 32) // 8) * 768 \
        + (((c[None, :] // 4) % 2) * 32 + pr[:, None] % 32) * 12 + (c[None, :] % 4) * 3
    t = torch.from_numpy(byte.reshape(-1).astype(np.int64)).to(plane.device)
    b = torch.stack([plane[t + i] for i in range(3)], 1).cpu().numpy().astype(np.uint32)
    bits = (b[:, 0] << 8) | (b[:, 1] << 16) | (b[:, 2] << 24)
    return bits.view(np.float32).astype(np.float64).reshape(len(rows), f)


def bwd_pieces(S, d, f, E):
    """Backward workspace of an MXFP8 layer: doq, dos, dguq, dgus, poff, blk,
    dot, dots, xt, xts, dgut, dguts."""
    P = padded_rows(S, E)
    names = ["doq", "dos", "dguq", "dgus", "poff", "blk", "dot", "dots", "xt", "xts", "dgut", "dguts"]
    sizes = [S * d, S * d // 32, S * 2 * f, S * 2 * f // 32, (E + 1) * 4, P // 64 * 8,
             P * d, P * d // 32, P * d, P * d // 32, P * 2 * f, P * 2 * f // 32]
    off, _ = _carve(sizes)
    return {n: (o, s) for n, o, s in zip(names, off, sizes)}


def _np(t):
    return t.cpu().numpy()


def assert_codes_near(codes, scales, vals, what, atol=None, tol=1e-5, max_frac=1e-2):
    """Codes and scale codes (blocks of 32 along each row) that a device
    decided on its own fp32 values of an operand whose exact values are
    `vals`: the two sets of values differ only by the rounding of the
    device's arithmetic, so every decision must be the oracle's except where
    the exact value sits within that rounding of the decision's boundary: a
    block scale one step off where the block maximum lies that close to a
    power of two, a neighbouring code where the value lies that close to the
    midpoint of two codes. The allowance is `atol` in value units (a scalar,
    or an array broadcast against `vals`), else `tol` times the block's
    largest value. At most max_frac of the codes may differ."""
    vals = np.asarray(vals, np.float64)
    R, C = vals.shape
    blocks = vals.reshape(R, C // 32, 32)
    amax = np.abs(blocks).max(axis=2)
    if atol is None:
        slack = np.repeat(tol * amax, 32, axis=1)
    else:
        slack = np.broadcast_to(np.asarray(atol, np.float64), vals.shape)
    slack_blk = slack.reshape(R, C // 32, 32).max(axis=2)
    rq, rs = O.mx_quantize(vals, "cols")
    sdiff = scales.astype(np.int64) - rs.astype(np.int64)
    off = np.nonzero(sdiff)
    if off[0].size:
        assert np.all(np.abs(sdiff[off]) == 1), f"{what}: a block scale more than one step off"
        a = amax[off]
        p2 = np.exp2(np.round(np.log2(np.maximum(a, 1e-300))))
        assert np.all(np.abs(a - p2) <= slack_blk[off]), \
            f"{what}: block scales differ away from a power of two ({off[0].size} blocks)"
    # Codes under the device's own scales, errors in value units.
    sv = np.repeat(np.exp2(scales.astype(np.float64) - 127.0), 32, axis=1)
    y = vals / sv
    ref = O.e4m3_encode(y)
    bad = codes != ref
    nbad = int(bad.sum())
    if nbad:
        assert nbad <= max(8, max_frac * codes.size), f"{what}: {nbad} of {codes.size} codes differ"
        yc = np.clip(y, -448, 448)
        e_dev = np.abs(O.e4m3_decode(codes) - yc) * sv
        e_ref = np.abs(O.e4m3_decode(ref) - yc) * sv
        ok = e_dev <= e_ref + slack
        if not np.all(ok[bad]):
            sel = bad & ~ok
            worst = ((e_dev - e_ref) / slack)[sel]
            idx = np.argwhere(sel)[:5]
            detail = [(int(r), int(c), float(vals[r, c]), int(codes[r, c]), int(ref[r, c])) for r, c in idx]
            raise AssertionError(f"{what}: {int(sel.sum())} of {nbad} differing codes are not a nearest rounding "
                                 f"of the value within the allowance (excess / allowance: max {worst.max():.2f}); "
                                 f"first (row, col, value, dev, ref): {detail}")


def read_kmajor(ws, pieces, q, s, S, K):
    """The values [S][K] (fp64) of a K-major image in workspace `ws`."""
    qo, _ = pieces[q]
    so, _ = pieces[s]
    codes = _np(ws[qo:qo + S * K]).reshape(S, K)
    sc = _np(ws[so:so + S * K // 32].view(K // 64, S, 2)).transpose(1, 0, 2).reshape(S, K // 32)
    return O.mx_dequantize(codes, sc, "cols")


def read_token_major(ws, pieces, q, s, offsets, S, C):
    """The values [S][C] (fp64, rows in expert order, padding dropped) of a
    token-major image in workspace `ws`."""
    E = len(offsets) - 1
    P = padded_rows(S, E)
    qo, _ = pieces[q]
    so, _ = pieces[s]
    codes = _np(ws[qo:qo + C * P]).reshape(C, P)
    sc = _np(ws[so:so + P * C // 32].view(P // 64, C, 2)).transpose(1, 0, 2).reshape(C, P // 32)
    vals = O.mx_dequantize(codes, sc, "cols")  # blocks of 32 along the tokens
    n = np.diff(offsets)
    poff = np.concatenate([[0], np.cumsum((n + 63) // 64 * 64)])
    out = np.zeros((S, C))
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        out[a:b] = vals[:, int(poff[e]):int(poff[e]) + b - a].T
    return out


def check_kmajor(ws, pieces, q, s, vals, what, S=None, row0=0, near=False, atol=None):
    """Rows row0 .. row0 + len(vals) of a K-major image in workspace `ws` (a
    uint8 device tensor; the image has S rows, default len(vals)) equal the
    oracle's codes of `vals` (blocks of 32 along each row). near=True: the
    device decided the codes on its own fp32 values of `vals`
    (assert_codes_near)."""
    rows, K = vals.shape
    S = rows if S is None else S
    qo, _ = pieces[q]
    so, _ = pieces[s]
    codes = _np(ws[qo + row0 * K:qo + (row0 + rows) * K]).reshape(rows, K)
    sc = _np(ws[so:so + S * K // 32].view(K // 64, S, 2)[:, row0:row0 + rows, :])
    sc = sc.transpose(1, 0, 2).reshape(rows, K // 32)
    if near:
        assert_codes_near(codes, sc, vals, what, atol=atol)
        return
    rq, rs = O.mx_quantize(vals, "cols")
    np.testing.assert_array_equal(codes, rq, err_msg=f"{what} codes")
    np.testing.assert_array_equal(sc, rs, err_msg=f"{what} scales")


def check_token_major(ws, pieces, q, s, vals, offsets, what, experts=None, S=None, C=None, near=False, atol=None):
    """The token-major image in workspace `ws` of an [S][C] operand: for each
    expert (all, or those listed), its rows padded with zeros to a multiple
    of 64, blocked in 32 rows down each column, equal the oracle's codes and
    scales. `vals` holds all S rows, or, with `experts` given, only the
    listed experts' rows one after the other (then S and C must be given).
    near=True: the device decided the codes on its own fp32 values of `vals`
    (assert_codes_near)."""
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
        p0 = int(poff[e])
        dev_q = _np(codes[:, p0:p0 + n64])
        dev_s = _np(sc[p0 // 64:(p0 + n64) // 64]).transpose(0, 2, 1).reshape(n64 // 32, C)
        if near:
            at = None if atol is None else np.asarray(atol, np.float64).reshape(-1, 1)  # per column of vals
            assert_codes_near(dev_q, np.ascontiguousarray(dev_s.T), pad.T, f"{what}, expert {e}", atol=at)
            continue
        rq, rs = O.mx_quantize(pad, "rows")
        np.testing.assert_array_equal(dev_q, rq.T, err_msg=f"{what} codes, expert {e}")
        np.testing.assert_array_equal(dev_s, rs, err_msg=f"{what} scales, expert {e}")
