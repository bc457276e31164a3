"""One MoE expert layer (forward + backward) driven through libmoe's C entry points.

All device buffers are allocated once, up front, with torch; forward() and
backward() only enqueue the library's kernels on the current stream, in the
order route -> dispatch -> grouped FFN -> combine and back. Nothing is
copied to the host.
"""
from __future__ import annotations

import torch

from . import _lib as L


class MoELayer:
    def __init__(self, T: int, d: int, E: int, k: int, f: int, dtype: str = "bf16",
                 learned_routing: bool = True, device: str = "cuda", mx_images: bool = True,
                 recompute: bool = False, keep_xp: bool = False):
        """``mx_images`` (MXFP8 layers): dispatch and combine-backward write
        the MXFP8 operands of xp and d_o, which the grouped FFN calls then
        read; False leaves the quantisation of both to the FFN calls. With
        the images the layer keeps neither xp's bf16 rows (unless
        ``keep_xp``) nor an fp32 d_o.
        ``recompute``: save no G, U, H (MXFP8: G, U and H's token-major
        operand) between forward and backward; the backward recomputes them
        (MOE_FLAG_RECOMPUTE)."""
        self.T, self.d, self.E, self.k, self.f = T, d, E, k, f
        self.shape = L.MoeShape.make(T, d, E, k, f, dtype, L.MOE_FLAG_RECOMPUTE if recompute else 0)
        self.recompute = recompute
        self.dtype = L.TORCH_DTYPE[self.shape.dtype]
        # G, U and d_o: fp32 for MXFP8 layers (their E4M3 codes are
        # decided on the fp32 values), else the layer dtype.
        self.act_dtype = torch.float32 if self.shape.dtype == L.MOE_MXFP8 else self.dtype
        self.learned = learned_routing
        S = T * k
        dev = torch.device(device)
        f32, i32, dt = torch.float32, torch.int32, self.dtype

        def buf(*shape, dtype=dt):
            return torch.empty(*shape, dtype=dtype, device=dev)

        def ws(op):
            n = L.workspace_size(op, self.shape)
            return torch.empty(max(n, 256), dtype=torch.uint8, device=dev)

        # forward
        self.logits = buf(T, E, dtype=f32) if learned_routing else None
        self.ws_route = ws(L.MOE_OP_ROUTE) if learned_routing else None
        self.topk_idx = buf(T, k, dtype=i32)
        self.topk_gate = buf(T, k, dtype=f32)
        self.counts = buf(E, dtype=i32)
        self.offsets = buf(E + 1, dtype=i32)
        self.row_of_slot = buf(T, k, dtype=i32)
        self.token_of_row = buf(S, dtype=i32)
        use_mx = mx_images and self.shape.dtype == L.MOE_MXFP8
        self.xp = buf(S, d) if keep_xp or not use_mx else None
        self.xp_mx = torch.empty(L.mx_xp_image_size(self.shape), dtype=torch.uint8, device=dev) if use_mx else None
        self.d_o_mx = torch.empty(L.mx_dout_image_size(self.shape), dtype=torch.uint8, device=dev) if use_mx else None
        self.save = torch.empty(L.save_size(self.shape), dtype=torch.uint8, device=dev)
        self.ws_ffn_fwd = ws(L.MOE_OP_FFN_FWD)
        self.o = buf(S, d)
        self.y = buf(T, d)
        self.ws_dispatch = ws(L.MOE_OP_DISPATCH)
        # backward
        # An MXFP8 layer with the operand images keeps no fp32 d_o: the combine
        # backward writes both of its E4M3 layouts and the FFN backward reads
        # only those.
        self.d_o = None if use_mx else buf(S, d, dtype=self.act_dtype)
        self.dgate = buf(T, k, dtype=f32)
        self.dxp = buf(S, d)
        self.dw_gate = buf(E, d, f)
        self.dw_up = buf(E, d, f)
        self.dw_down = buf(E, f, d)
        self.dx = buf(T, d)
        self.ws_ffn_bwd = ws(L.MOE_OP_FFN_BWD)
        if learned_routing:
            self.dlogits = buf(T, E, dtype=f32)
            self.dw_router = buf(d, E)
            self.ws_route_bwd = ws(L.MOE_OP_ROUTE_BWD)
            self.ws_dispatch_bwd = ws(L.MOE_OP_DISPATCH_BWD)

    def saved(self):
        """(G, U, H), each [S][f]: views of the save buffer or, for a
        recompute layer, of the planes its last backward rebuilt in the
        backward workspace (after the dG|dU rows). fp32 and bf16 layers only:
        an MXFP8 layer saves G, U in a blocked layout and H only as an E4M3
        operand."""
        if self.shape.dtype == L.MOE_MXFP8:
            raise ValueError("MXFP8 layers save G, U blocked and H only as an E4M3 operand")
        S, f = self.T * self.k, self.f
        eb = torch.empty((), dtype=self.act_dtype).element_size()
        if self.recompute:
            off = (S * 2 * f * eb + 255) // 256 * 256
            flat = self.ws_ffn_bwd[off:off + 3 * S * f * eb].view(self.act_dtype)
        else:
            flat = self.save[:3 * S * f * eb].view(self.act_dtype)
        return tuple(flat[i * S * f:(i + 1) * S * f].view(S, f) for i in range(3))

    def dgu(self):
        """(dG, dU), each [S][f]: views of the dG|dU rows the last backward
        left at the start of its workspace (fp32 and bf16 layers; MXFP8
        layers keep dG | dU only as E4M3 operands)."""
        if self.shape.dtype == L.MOE_MXFP8:
            raise ValueError("MXFP8 layers keep no dG | dU rows")
        S, f = self.T * self.k, self.f
        eb = torch.empty((), dtype=self.act_dtype).element_size()
        rows = self.ws_ffn_bwd[:S * 2 * f * eb].view(self.act_dtype).view(S, 2 * f)
        return rows[:, :f], rows[:, f:]

    def load_stats(self, stream=None):
        """Enqueue the expert-load diagnostics of the last dispatch (moe_load_stats)
        and return the device tensor of 8 float64 (LOAD_STATS order)."""
        if not hasattr(self, "stats"):
            self.stats = torch.empty(8, dtype=torch.float64, device=self.counts.device)
        L.moe_load_stats(self.counts, self.stats, stream)
        return self.stats

    def forward(self, x, w_gate, w_up, w_down, w_router=None, topk_idx=None, topk_gate=None, stream=None,
                mark=None):
        """Enqueue the forward pass. ``mark(name)``, if given, is called after
        each library call is enqueued (the benchmark records events there)."""
        s = self.shape
        mark = mark or (lambda name: None)
        self.x, self.w_gate, self.w_up, self.w_down, self.w_router = x, w_gate, w_up, w_down, w_router
        if self.learned:
            L.moe_route(x, w_router, s, self.logits, self.topk_idx, self.topk_gate, self.ws_route, stream)
            mark("moe_route")
        else:
            self.topk_idx.copy_(topk_idx)
            self.topk_gate.copy_(topk_gate)
        L.moe_dispatch(x, self.topk_idx, s, self.counts, self.offsets, self.row_of_slot, self.token_of_row,
                       self.xp, self.ws_dispatch, stream, xp_mx=self.xp_mx)
        mark("moe_dispatch")
        L.moe_grouped_ffn_fwd(self.xp, w_gate, w_up, w_down, self.offsets, s, self.save, self.o, self.ws_ffn_fwd,
                              stream, xp_mx=self.xp_mx)
        mark("moe_grouped_ffn_fwd")
        L.moe_combine(self.o, self.topk_gate, self.row_of_slot, s, self.y, stream)
        mark("moe_combine")
        return self.y

    def backward(self, dy, stream=None, mark=None):
        s = self.shape
        mark = mark or (lambda name: None)
        L.moe_combine_bwd(dy, self.o, self.topk_gate, self.row_of_slot, s, self.d_o, self.dgate, stream,
                          d_o_mx=self.d_o_mx, token_of_row=self.token_of_row, offsets=self.offsets)
        mark("moe_combine_bwd")
        L.moe_grouped_ffn_bwd(self.d_o, self.xp, self.w_gate, self.w_up, self.w_down, self.offsets, s, self.save,
                              self.dxp, self.dw_gate, self.dw_up, self.dw_down, self.ws_ffn_bwd, stream,
                              d_o_mx=self.d_o_mx, xp_mx=self.xp_mx)
        mark("moe_grouped_ffn_bwd")
        if self.learned:
            L.moe_route_bwd(self.x, self.w_router, self.topk_idx, self.topk_gate, self.dgate, s, self.dlogits,
                            self.dw_router, self.ws_route_bwd, stream)
            mark("moe_route_bwd")
            L.moe_dispatch_bwd(self.dxp, self.row_of_slot, self.dlogits, self.w_router, s, self.dx,
                               self.ws_dispatch_bwd, stream)
        else:
            L.moe_dispatch_bwd(self.dxp, self.row_of_slot, None, None, s, self.dx, None, stream)
        mark("moe_dispatch_bwd")
        return self.dx
