"""Plain fp64 CPU oracle for the MoE expert layer (forward and backward).

TEST INFRASTRUCTURE ONLY. This module is the correctness reference for the
GPU library. Only the tests, the package's smoke check and the benchmark's
CPU-baseline leg may import it; the GPU path never calls it and shares no
code with it. It is deliberately slow and obvious: every step is the plain
definition in float64, applied to the exact stored input values (bf16 or
fp32 widened to fp64), with no blocking, fusion or intermediate rounding.
Library primitives used as single steps: numpy matmul, stable argsort,
bincount, cumsum, exp, frexp, rint.

Sources. The pages describe the layer only in words:
  [P1] "Olmo-core 3 é lançado com infraestrutura para treinar modelos MoE"
       (noticiarioia.com), sections "Mudança de arquitetura e ganhos de
       desempenho" and "Otimizações e testes em escala de trilhões";
  [P2] "Olmo-core 3 escala el entrenamiento de mixture-of-experts a billones
       de parámetros" (bytechap.com), sections "Qué ocurrió", "Cómo funciona";
  [P3] "Ai2 rilascia Olmo-Core 3, stack di addestramento aperto per MoE da
       trilioni di parametri" (unite.ai), introduction and section
       "Parallelismo, precisione e tecniche di memoria".
They state that each token activates 4 of the E experts ([P1] "Mudança de
arquitetura..."; [P3] introduction), that routed rows are written straight
into contiguous per-expert input buffers and the expert matmuls run as one
grouped GEMM scheduled on the device ([P2] "Cómo funciona"; [P3]
"Parallelismo, precisione..."), and that MXFP8 is supported ([P1]
"Otimizações..."; [P3] "Parallelismo, precisione..."). They give no formula.
The layer's specification fixes the rest: softmax over router logits, top-k
with the gates renormalised to sum to one, SwiGLU experts
(silu(x W_gate) * (x W_up)) W_down, a gate-weighted combine after the
experts, no biases, no capacity limit, no token dropping. Readings taken
where both are silent:
  * top-k is selected on the logits (softmax is monotone), in decreasing
    order, equal logits going to the lower expert index;
  * rows inside one expert's buffer are in increasing token order (a stable
    counting sort of the flattened (token, slot) pairs by expert);
  * MXFP8 follows the OCP Microscaling Formats (MX) v1.0 conversion: shared
    exponent floor(log2 amax) - 8 per block of 32, E4M3 ("FN": bias 7, max
    448, no infinities) elements rounded to nearest-even and saturated.

Parity pins: every function here is checked in tests/test_oracle_*.py
against brute force, closed forms, invariants, finite differences, an
independent autograd formulation, and an exhaustive E4M3 codebook.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=F64)


# --------------------------------------------------------------------------
# Routing: router logits, softmax, top-k, renormalised gates.
# [P1] "Mudança de arquitetura e ganhos de desempenho" and [P3] introduction:
# four experts active per token; softmax/top-k/renormalisation from the
# layer specification.
# --------------------------------------------------------------------------

def router_logits(x, w_router) -> np.ndarray:
    """logits[t, e] = sum_i x[t, i] * W_r[i, e]   (fp64)."""
    return _f64(x) @ _f64(w_router)


def softmax(logits) -> np.ndarray:
    """Row softmax with the row maximum subtracted (fp64)."""
    l = _f64(logits)
    z = np.exp(l - l.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def topk_experts(logits, k: int) -> np.ndarray:
    """S_t: indices of the k largest logits, decreasing; ties -> lower index.

    A stable sort of the negated logits keeps equal values in index order.
    """
    return np.argsort(-_f64(logits), axis=1, kind="stable")[:, :k].astype(np.int32)


def route(logits, k: int):
    """(topk_idx [T,k] int32, gates [T,k] fp64) from router logits.

    p = softmax(l); S_t = top-k; g_tj = p[S_t[j]] / sum_{i in S_t} p_i.
    """
    idx = topk_experts(logits, k)
    p = softmax(logits)
    ps = np.take_along_axis(p, idx.astype(np.int64), axis=1)
    return idx, ps / ps.sum(axis=1, keepdims=True)


# --------------------------------------------------------------------------
# Dispatch: histogram, prefix scan, stable placement, row gather.
# [P2] "Cómo funciona", [P3] "Parallelismo, precisione...": routed data is
# placed directly into the experts' input buffers and the routing metadata
# stays on the device.
# --------------------------------------------------------------------------

def dispatch_plan(topk_idx, E: int):
    """(counts[E], offsets[E+1], row_of_slot[T,k], token_of_row[S]).

    counts[e] = #{(t, j): idx[t, j] = e}; offsets = exclusive prefix sum with
    offsets[E] = S; expert e's rows are offsets[e] .. offsets[e+1]-1 holding
    its tokens in increasing t (stable counting sort of the flattened slots).
    """
    idx = np.asarray(topk_idx, dtype=np.int64)
    T, k = idx.shape
    flat = idx.reshape(-1)
    if flat.size and (flat.min() < 0 or flat.max() >= E):
        raise ValueError("expert index out of range")
    counts = np.bincount(flat, minlength=E)
    offsets = np.zeros(E + 1, dtype=np.int64)
    np.cumsum(counts, out=offsets[1:])
    order = np.argsort(flat, kind="stable")  # slot ids, grouped by expert, slot order kept
    row_of_slot = np.empty(T * k, dtype=np.int64)
    row_of_slot[order] = np.arange(T * k)
    token_of_row = order // k
    return (counts.astype(np.int32), offsets.astype(np.int32),
            row_of_slot.reshape(T, k).astype(np.int32), token_of_row.astype(np.int32))


# Expert-load diagnostics from the routed counts. [P2] "Detalles clave" and
# [P3] "Risultati Documentati" report that a score meant to favour balanced
# routing can improve while the real per-expert load grows less balanced;
# these figures measure the real load itself. The pages define no statistic;
# the reading here: p_e = n_e / S, entropy in nats with 0 ln 0 = 0.
LOAD_STATS = ("max", "min", "mean", "max_over_mean", "entropy", "entropy_norm", "empty", "cv")


def load_stats(counts) -> np.ndarray:
    """fp64 [8] in LOAD_STATS order: max n_e, min n_e, mean S/E, max/mean
    (0 when S = 0), entropy -sum p_e ln p_e (0 when S = 0), entropy / ln E
    (1 when E = 1; 0 when S = 0), experts with no rows, and the coefficient of
    variation std(n)/mean(n) with the population std (0 when S = 0)."""
    n = _f64(counts)
    E = n.size
    S = n.sum()
    mean = S / E
    out = np.zeros(8, dtype=F64)
    out[0], out[1], out[2] = n.max(), n.min(), mean
    out[6] = float((n == 0).sum())
    if S > 0:
        p = n / S
        nz = p > 0
        ent = -(p[nz] * np.log(p[nz])).sum()
        out[3] = n.max() / mean
        out[4] = ent
        out[5] = ent / np.log(E) if E > 1 else 1.0
        out[7] = np.sqrt(((n - mean) ** 2).mean()) / mean
    return out


def gather_rows(x, token_of_row) -> np.ndarray:
    """Xp[r] = x[token_of_row[r]] (a pure copy; fp64 here)."""
    return _f64(x)[np.asarray(token_of_row, dtype=np.int64)]


# --------------------------------------------------------------------------
# Expert FFN (SwiGLU) over contiguous per-expert row ranges: the grouped GEMM.
# [P2] "Cómo funciona", [P3] "Parallelismo, precisione...".
# --------------------------------------------------------------------------

def sigmoid(z) -> np.ndarray:
    z = _f64(z)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def ffn_forward(xp, w_gate, w_up, w_down, offsets):
    """Per expert e on rows offsets[e]..offsets[e+1]-1:
    G = Xp_e W_gate[e], U = Xp_e W_up[e], H = silu(G) * U with
    silu(z) = z * sigmoid(z), O = H W_down[e]. Returns (G, U, H, O)."""
    xp = _f64(xp)
    E = len(offsets) - 1
    S, f = xp.shape[0], np.shape(w_gate)[2]
    d_out = np.shape(w_down)[2]
    G = np.zeros((S, f)); U = np.zeros((S, f)); H = np.zeros((S, f)); O = np.zeros((S, d_out))
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            continue
        G[a:b] = xp[a:b] @ _f64(w_gate[e])
        U[a:b] = xp[a:b] @ _f64(w_up[e])
        H[a:b] = G[a:b] * sigmoid(G[a:b]) * U[a:b]
        O[a:b] = H[a:b] @ _f64(w_down[e])
    return G, U, H, O


def combine(o, gates, row_of_slot) -> np.ndarray:
    """y[t] = sum_j g[t, j] * O[row_of_slot[t, j]] (gates applied after the FFN)."""
    o = _f64(o)
    rs = np.asarray(row_of_slot, dtype=np.int64)
    g = _f64(gates)
    y = np.zeros((rs.shape[0], o.shape[1]))
    for j in range(rs.shape[1]):
        y += g[:, j:j + 1] * o[rs[:, j]]
    return y


# --------------------------------------------------------------------------
# Backward pass: the adjoint of every forward step above.
# --------------------------------------------------------------------------

def combine_backward(dy, o, gates, row_of_slot):
    """dO[row(t,j)] = g[t,j] dy[t];  dgate[t,j] = <dy[t], O[row(t,j)]>."""
    dy = _f64(dy); o = _f64(o); g = _f64(gates)
    rs = np.asarray(row_of_slot, dtype=np.int64)
    d_o = np.zeros_like(o)
    dgate = np.zeros(rs.shape)
    for j in range(rs.shape[1]):
        d_o[rs[:, j]] = g[:, j:j + 1] * dy
        dgate[:, j] = np.einsum("td,td->t", dy, o[rs[:, j]])
    return d_o, dgate


def ffn_backward(d_o, xp, w_gate, w_up, w_down, offsets, G, U, H):
    """Per expert e (rows a..b):
        dH = dO_e W_down[e]^T
        dU = dH * silu(G);   dG = dH * U * sigmoid(G) * (1 + G (1 - sigmoid(G)))
        dW_down[e] = H_e^T dO_e;  dW_gate[e] = Xp_e^T dG;  dW_up[e] = Xp_e^T dU
        dXp_e = dG W_gate[e]^T + dU W_up[e]^T
    An expert with no rows gets exactly zero weight gradients.
    Returns (dXp, dW_gate, dW_up, dW_down, dG, dU)."""
    d_o = _f64(d_o); xp = _f64(xp)
    E = len(offsets) - 1
    S, d = xp.shape
    f = np.shape(w_gate)[2]
    dxp = np.zeros((S, d)); dG = np.zeros((S, f)); dU = np.zeros((S, f))
    dwg = np.zeros((E, d, f)); dwu = np.zeros((E, d, f)); dwd = np.zeros((E, f, np.shape(w_down)[2]))
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            continue
        g, u = G[a:b], U[a:b]
        s = sigmoid(g)
        dh = d_o[a:b] @ _f64(w_down[e]).T
        dU[a:b] = dh * g * s
        dG[a:b] = dh * u * s * (1.0 + g * (1.0 - s))
        dwd[e] = H[a:b].T @ d_o[a:b]
        dwg[e] = xp[a:b].T @ dG[a:b]
        dwu[e] = xp[a:b].T @ dU[a:b]
        dxp[a:b] = dG[a:b] @ _f64(w_gate[e]).T + dU[a:b] @ _f64(w_up[e]).T
    return dxp, dwg, dwu, dwd, dG, dU


def route_backward(x, w_router, topk_idx, gates, dgate):
    """Router gradient through the renormalised top-k softmax.

    On S_t the gates equal a softmax over the selected logits, so for
    i in S_t: dl[t,i] = g_ti (dgate_ti - sum_j g_tj dgate_tj); dl = 0 off S_t.
    dW_r = x^T dl;  the router's share of dx is dl W_r^T.
    Returns (dlogits [T,E], dW_r [d,E], dx_router [T,d]).
    """
    x = _f64(x); w = _f64(w_router); g = _f64(gates); dg = _f64(dgate)
    idx = np.asarray(topk_idx, dtype=np.int64)
    T, E = x.shape[0], w.shape[1]
    inner = (g * dg).sum(axis=1, keepdims=True)
    dl = np.zeros((T, E))
    np.put_along_axis(dl, idx, g * (dg - inner), axis=1)
    return dl, x.T @ dl, dl @ w.T


def dispatch_backward(dxp, row_of_slot, dx_router=None) -> np.ndarray:
    """dx[t] = sum_j dXp[row_of_slot[t, j]]  (+ the router's share, if any)."""
    dxp = _f64(dxp)
    rs = np.asarray(row_of_slot, dtype=np.int64)
    dx = np.zeros((rs.shape[0], dxp.shape[1]))
    for j in range(rs.shape[1]):
        dx += dxp[rs[:, j]]
    if dx_router is not None:
        dx += _f64(dx_router)
    return dx


# --------------------------------------------------------------------------
# Whole layer.
# --------------------------------------------------------------------------

def layer_forward(inp: dict, k: int, logits=None, mx: bool = False) -> dict:
    """Forward pass on an input dict (keys as produced by moe_inputs).
    mx=True uses the MXFP8 expert FFN (ffn_forward_mx).

    Learned routing uses x W_r, unless ``logits`` is given: then the top-k
    sets and gates are computed from those values (widened exactly), which is
    how routing is compared bit for bit against a device that produced fp32
    logits. Random routing takes topk_idx/topk_gate from the inputs.
    """
    x = _f64(inp["x"])
    E = np.shape(inp["w_gate"])[0]
    out = {}
    if "w_router" in inp:
        out["logits"] = router_logits(x, inp["w_router"])
        idx, gates = route(out["logits"] if logits is None else _f64(logits), k)
    else:
        idx, gates = np.asarray(inp["topk_idx"], dtype=np.int32), _f64(inp["topk_gate"])
    counts, offsets, row_of_slot, token_of_row = dispatch_plan(idx, E)
    xp = gather_rows(x, token_of_row)
    ffn = ffn_forward_mx if mx else ffn_forward
    G, U, H, O = ffn(xp, inp["w_gate"], inp["w_up"], inp["w_down"], offsets)
    out.update(topk_idx=idx, gates=gates, counts=counts, offsets=offsets,
               row_of_slot=row_of_slot, token_of_row=token_of_row,
               xp=xp, G=G, U=U, H=H, O=O, y=combine(O, gates, row_of_slot))
    return out


def layer_backward(inp: dict, fwd: dict, dy=None, mx: bool = False) -> dict:
    """Backward pass given the forward's saved values; dy defaults to inp['dy'].
    mx=True uses the MXFP8 expert FFN backward (ffn_backward_mx)."""
    dy = _f64(inp["dy"] if dy is None else dy)
    d_o, dgate = combine_backward(dy, fwd["O"], fwd["gates"], fwd["row_of_slot"])
    ffn = ffn_backward_mx if mx else ffn_backward
    dxp, dwg, dwu, dwd, dG, dU = ffn(d_o, fwd["xp"], inp["w_gate"], inp["w_up"],
                                     inp["w_down"], fwd["offsets"], fwd["G"], fwd["U"], fwd["H"])
    out = dict(dO=d_o, dgate=dgate, dXp=dxp, dG=dG, dU=dU,
               dw_gate=dwg, dw_up=dwu, dw_down=dwd)
    dx_router = None
    if "w_router" in inp:
        dl, dwr, dx_router = route_backward(inp["x"], inp["w_router"], fwd["topk_idx"],
                                            fwd["gates"], dgate)
        out.update(dlogits=dl, dw_router=dwr)
    out["dx"] = dispatch_backward(dxp, fwd["row_of_slot"], dx_router)
    return out


# --------------------------------------------------------------------------
# MXFP8: E4M3 elements with one E8M0 scale per 32 elements along K.
# [P1] "Otimizações e testes em escala de trilhões", [P3] "Parallelismo,
# precisione e tecniche di memoria" (MXFP8 is supported; no details given).
# Encoding per OCP Microscaling Formats (MX) v1.0.
# --------------------------------------------------------------------------

E4M3_MAX = 448.0
E4M3_EMAX = 8          # exponent of the largest normal E4M3 value (448 = 1.75 * 2^8)
E4M3_MIN_NORMAL_EXP = -6
E4M3_MANT_BITS = 3
MX_BLOCK = 32


def e4m3_decode(code) -> np.ndarray:
    """Value of E4M3 ("FN") codes: sign | 4-bit exponent (bias 7) | 3-bit mantissa.
    Exponent field 0 is subnormal (m/8 * 2^-6); 0x7F and 0xFF are NaN."""
    c = np.asarray(code, dtype=np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    ef = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(ef == 0, m / 8.0 * 2.0 ** E4M3_MIN_NORMAL_EXP,
                   (1.0 + m / 8.0) * np.exp2(ef - 7.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return s * mag


def _floor_log2(a) -> np.ndarray:
    """floor(log2 a) for a > 0, exact (frexp returns a = m 2^e with m in [0.5, 1))."""
    return np.frexp(_f64(a))[1].astype(np.int64) - 1


def e4m3_encode(y) -> np.ndarray:
    """Nearest E4M3 code to each fp64 value y; ties to the even mantissa;
    magnitudes beyond 448 saturate to 448; the sign is kept (so a negative
    value that rounds to zero gives -0 = 0x80)."""
    y = _f64(y)
    a = np.abs(y)
    ex = np.where(a > 0, _floor_log2(np.where(a > 0, a, 1.0)), E4M3_MIN_NORMAL_EXP)
    ex = np.maximum(ex, E4M3_MIN_NORMAL_EXP)           # below 2^-6: subnormal spacing
    quantum = np.exp2((ex - E4M3_MANT_BITS).astype(F64))
    r = np.minimum(np.rint(a / quantum) * quantum, E4M3_MAX)
    # r is now an exactly representable magnitude; read off its fields.
    rex = np.where(r > 0, _floor_log2(np.where(r > 0, r, 1.0)), E4M3_MIN_NORMAL_EXP - 1)
    sub = rex < E4M3_MIN_NORMAL_EXP
    code_sub = np.rint(r / 2.0 ** (E4M3_MIN_NORMAL_EXP - E4M3_MANT_BITS))
    mant = np.rint(r / np.exp2(rex.astype(F64)) * 8.0) - 8.0
    code_norm = (rex + 7) * 8 + mant
    code = np.where(sub, code_sub, code_norm).astype(np.int64)
    neg = np.signbit(y)
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


def e8m0_decode(c) -> np.ndarray:
    """E8M0 scale: 2^(c - 127); code 255 is NaN."""
    c = np.asarray(c, dtype=np.int64)
    return np.where(c == 255, np.nan, np.exp2((c - 127).astype(F64)))


def mx_block_scale_code(amax) -> np.ndarray:
    """E8M0 code of a block's shared scale: 2^(floor(log2 amax) - 8), clamped
    to the codes 0..254; an all-zero block gets code 0."""
    amax = _f64(amax)
    e = np.where(amax > 0, _floor_log2(np.where(amax > 0, amax, 1.0)), -127 + E4M3_EMAX)
    return np.clip(e - E4M3_EMAX + 127, 0, 254).astype(np.uint8)


def mx_quantize(a, along: str = "cols"):
    """MXFP8-quantise a 2-D array in blocks of 32 along one axis.

    along="cols": each block is 32 consecutive elements of a row; scales have
    shape [R, C/32]. along="rows": each block is 32 consecutive rows of one
    column; scales have shape [R/32, C]. Returns (codes uint8 [R, C],
    scale codes uint8). Elements are encoded as v / 2^(c - 127)."""
    a = _f64(a)
    if along == "rows":
        q, s = mx_quantize(a.T, "cols")
        return np.ascontiguousarray(q.T), np.ascontiguousarray(s.T)
    R, C = a.shape
    if C % MX_BLOCK:
        raise ValueError("blocked axis must be a multiple of 32")
    blocks = a.reshape(R, C // MX_BLOCK, MX_BLOCK)
    sc = mx_block_scale_code(np.abs(blocks).max(axis=2))
    y = blocks / e8m0_decode(sc)[:, :, None]
    return e4m3_encode(y).reshape(R, C), sc


def mx_dequantize(codes, scales, along: str = "cols") -> np.ndarray:
    """Exact fp64 value of MXFP8 data: decode(code) * 2^(scale - 127)."""
    if along == "rows":
        return mx_dequantize(np.asarray(codes).T, np.asarray(scales).T, "cols").T
    v = e4m3_decode(codes)
    R, C = v.shape
    return (v.reshape(R, C // MX_BLOCK, MX_BLOCK)
            * e8m0_decode(scales)[:, :, None]).reshape(R, C)


# --------------------------------------------------------------------------
# MXFP8 expert FFN: every grouped-GEMM operand quantised along that GEMM's K.
# The pages only say that MXFP8 is used for the expert computation and the
# data moved between experts ([P1] "Otimizações e testes em escala de
# trilhões"; [P3] "Parallelismo, precisione e tecniche di memoria"). Reading
# taken: every operand of every grouped GEMM of the forward and the backward
# is quantised in blocks of 32 along that GEMM's reduction axis; products are
# then exact on the dequantised values (accumulation in fp64 here). For the
# weight gradients the reduction runs over one expert's tokens, so those
# operands are blocked along the rows inside each expert's range, the range
# zero-padded to a multiple of 32. Every quantised operand is taken at its
# exact value: the inputs as stored, the computed operands (H, dO, dG, dU)
# exactly as the definition gives them (fp64, never rounded to a storage
# type first); the elementwise steps (SwiGLU and its derivative) use the
# exact GEMM results.
# --------------------------------------------------------------------------

def mx_roundtrip(a, along: str) -> np.ndarray:
    """Exact fp64 value of a after MXFP8 quantisation in blocks of 32 along
    `along` ("cols": inside a row; "rows": down a column)."""
    q, s = mx_quantize(a, along)
    return mx_dequantize(q, s, along)


def mx_rows_grouped(a, offsets) -> np.ndarray:
    """mx_roundtrip along rows, blocked separately inside every row range
    [offsets[e], offsets[e+1]), each range zero-padded to a multiple of 32."""
    a = _f64(a)
    out = np.zeros_like(a)
    for e in range(len(offsets) - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if lo == hi:
            continue
        n = hi - lo
        pad = np.zeros(((n + MX_BLOCK - 1) // MX_BLOCK * MX_BLOCK, a.shape[1]))
        pad[:n] = a[lo:hi]
        out[lo:hi] = mx_roundtrip(pad, "rows")[:n]
    return out


def ffn_forward_mx(xp, w_gate, w_up, w_down, offsets, h_in=None):
    """ffn_forward with MXFP8 GEMM operands: Xp and H along the row (K = d,
    f), W_gate, W_up along d and W_down along f (down their columns).
    The down GEMM quantises the exact H, or h_in if given (a stage-by-stage
    comparison feeds a device's own stored H).
    Returns (G, U, H, O)."""
    E = len(offsets) - 1
    xq = mx_roundtrip(xp, "cols")
    S, f = xq.shape[0], np.shape(w_gate)[2]
    G = np.zeros((S, f)); U = np.zeros((S, f)); H = np.zeros((S, f))
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            continue
        G[a:b] = xq[a:b] @ mx_roundtrip(w_gate[e], "rows")
        U[a:b] = xq[a:b] @ mx_roundtrip(w_up[e], "rows")
        H[a:b] = G[a:b] * sigmoid(G[a:b]) * U[a:b]
    hq = mx_roundtrip(H if h_in is None else h_in, "cols")
    O = np.zeros((S, np.shape(w_down)[2]))
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a < b:
            O[a:b] = hq[a:b] @ mx_roundtrip(w_down[e], "rows")
    return G, U, H, O


def ffn_backward_mx(d_o, xp, w_gate, w_up, w_down, offsets, G, U, H, dgdu_in=None, dgdu_w_in=None):
    """ffn_backward with MXFP8 GEMM operands, each along its GEMM's K:
    dH = q(dO) q(W_down)^T (both along d); dXp = q(dG) q(W_gate)^T +
    q(dU) q(W_up)^T (along f); dW_down = q(H)^T q(dO), dW_gate = q(Xp)^T
    q(dG), dW_up = q(Xp)^T q(dU), each along the expert's tokens.
    dO, dG, dU and H are quantised at the values given (the exact ones
    from ffn_forward_mx and combine_backward), and the SwiGLU derivative
    reads G and U as given. For stage-by-stage comparisons with a device
    that keeps its own operands: dgdu_in, if given, replaces (dG, dU) for
    the later GEMMs, and dgdu_w_in, if given, replaces them for the weight
    gradients only (the dXp GEMM then takes dgdu_in or the computed values).
    Values that are already MXFP8 numbers in the same blocking (a device's
    dequantised operand) pass through the quantisation unchanged.
    Returns (dXp, dW_gate, dW_up, dW_down, dG, dU)."""
    E = len(offsets) - 1
    S, d = np.shape(xp)
    f = np.shape(w_gate)[2]
    d_o = _f64(d_o)
    doq = mx_roundtrip(d_o, "cols")
    dG = np.zeros((S, f)); dU = np.zeros((S, f))
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            continue
        g, u = _f64(G[a:b]), _f64(U[a:b])
        s = sigmoid(g)
        dh = doq[a:b] @ mx_roundtrip(w_down[e], "cols").T
        dU[a:b] = dh * g * s
        dG[a:b] = dh * u * s * (1.0 + g * (1.0 - s))
    dg_in, du_in = (dG, dU) if dgdu_in is None else dgdu_in
    dg_w, du_w = (dg_in, du_in) if dgdu_w_in is None else dgdu_w_in
    dgq, duq = mx_roundtrip(dg_in, "cols"), mx_roundtrip(du_in, "cols")
    hg, dog = mx_rows_grouped(H, offsets), mx_rows_grouped(d_o, offsets)
    xg, dgg, dug = mx_rows_grouped(xp, offsets), mx_rows_grouped(dg_w, offsets), mx_rows_grouped(du_w, offsets)
    dxp = np.zeros((S, d))
    dwg = np.zeros((E, d, f)); dwu = np.zeros((E, d, f)); dwd = np.zeros((E, f, np.shape(w_down)[2]))
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            continue
        dxp[a:b] = dgq[a:b] @ mx_roundtrip(w_gate[e], "cols").T + duq[a:b] @ mx_roundtrip(w_up[e], "cols").T
        dwd[e] = hg[a:b].T @ dog[a:b]
        dwg[e] = xg[a:b].T @ dgg[a:b]
        dwu[e] = xg[a:b].T @ dug[a:b]
    return dxp, dwg, dwu, dwd, dG, dU
