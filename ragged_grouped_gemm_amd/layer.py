"""The dropless MoE expert-FFN layer composed from the C-ABI calls.

``MoEFFN`` owns every activation and gradient buffer of one layer shape, so a
forward + backward pass allocates nothing and reads nothing back to the host:
it can be captured once in a HIP graph and replayed with new inputs copied
into the same tensors (``capture``).  Every computation is a library kernel;
this module only sequences the calls.

Forward:  route top-k -> permute -> FC1 + GLU epilogue -> FC2 -> combine.
Backward: combine bwd (dY, dgate) -> route bwd (dlogits) -> FC2 dgrad + dGLU
(dH) -> FC2 wgrad (dW2, db2) -> FC1 dgrad (dXp) -> FC1 wgrad (dW1p, db1p) ->
unpermute-sum (dX).

Gather-fused permute (``fuse_permute``, the default for bf16 / float32): the
permuted copy Xp is never written; FC1 and FC1's weight gradient read each row
of x through src_row, so the forward keeps a reference to x for the backward
(x must not change in between).  ``fuse_permute=False`` materializes Xp.  The
gathering loaders address x with 31-bit byte offsets from one base, so a
layer whose x spans 2 GiB or more (e.g. 150K tokens at d = 7168 in bf16)
materializes Xp whatever ``fuse_permute`` says (``gather_fits``).

Transposed weights for the dgrads (``transpose_w2``, ``transpose_w1``): at
the start of each backward W2 and W1p are copied transposed
(``moe_transpose_weights``), so FC2's dgrad + dGLU and FC1's dgrad read both
operands contiguous along the reduction; the results are bit-identical to
reading the weights as stored.  The copies cost time in proportion to E d f,
the dgrads gain in proportion to R d f, so by default (``None``) they are
made when the layer averages at least ``TRANSPOSE_MIN_ROWS`` routed rows per
expert: measured at 4096 rows per expert (16384 tokens, top-8 of 32) both
pay (step -1.5 ms), at 1024 (8192 tokens, top-4 of 32) neither does (step
6.93-7.00 ms with both, 6.75 ms without; W2's copy alone breaks even, W1p's
alone costs 0.2 ms).

Activation recomputation (``recompute=True``): the forward does not write
the pre-activation H; the backward first runs FC1 + GLU again (from x or Xp,
and the routing the forward left in place) to rebuild H and A, then proceeds
as usual.  Between the passes the layer then needs only the routing, Y and
its inputs, at the price of one more FC1 GEMM (4·R·d·f FLOP) per backward;
the gradients are bit-identical to the stored-H path.

Fused router (``router=True``, bf16 input): the layer computes its own
logits as the router's linear map x w_router^T, fused with the top-k routing
in one launch (``moe_router_topk``); pass the router weight w_router [E, d]
where the logits would go (forward, backward, step, capture).  The backward
adds the router's share dlogits w_router to dX and writes its weight
gradient ``dWr`` [E, d] (float32, ``moe_router_bwd``).

Gates inside the activation (``gate_in_act=True``): FC1's epilogue scales
each row's activation output by its routing gate (feature scaling, gates
moved to row order by ``moe_permute_rows``), the combine sums the expert
outputs with unit weights, and the backward takes the gate gradient from the
dGLU epilogue (sum over the row of dA * act) instead of from <dOut, Y>, so
the combine's backward no longer reads Y.  Without b2 this is the same
function as the default layer; with b2 the bias is added after the gate
weighting.

Buffers (``alloc``): every buffer the layer holds is taken from
``alloc(shape, dtype, device)`` when given (caller-managed memory, guard
bands), else from ``torch.zeros``.  Their initial contents do not matter:
each pass writes every element it later reads, the padding of the MX
column copies included; the error word, whose bits are sticky, is cleared
once here.

MXFP8 variant (``gemm="mxfp8"``; ``gemm="mxfp4"`` is the same with E2M1
elements; ``mx_dxp=True`` also writes FC1's dgrad output dXp as an MX row
copy and sums dX from it): every GEMM operand is an MXFP8 copy blocked
along that GEMM's reduction axis.  Xp and dY exist only as MXFP8 row and
expert-segmented column copies written straight from x and d_out; FC1's
epilogue writes A, and the dGLU epilogue dH, as the same two copies; H stays
bf16 for the dGLU.  Weights are quantized once (``mx_weights``) into row and
transposed copies.
"""
from __future__ import annotations

import contextlib

import torch

from . import ops


class MXWeights:
    """MX copies (MXFP8, or MXFP4 with fmt="e2m1") of the expert weights: W1p
    [E, 2f, d] blocked along d (FC1) and along 2f (FC1 dgrad, stored transposed
    [E*d, 2f]); W2 [E, d, f] along f (FC2) and along d (FC2 dgrad, stored
    transposed [E*f, d])."""

    def __init__(self, W1p, W2, fmt="e4m3"):
        E, n1, d = W1p.shape
        self.fmt = fmt
        self.w1 = ops.moe_mx_quantize(W1p.reshape(E * n1, d), fmt=fmt)
        self.w1t = ops.moe_mx_quantize_transpose(W1p, fmt=fmt)
        self.w2 = ops.moe_mx_quantize(W2.reshape(-1, W2.shape[2]), fmt=fmt)
        self.w2t = ops.moe_mx_quantize_transpose(W2, fmt=fmt)


class MoEFFN:
    # largest x (bytes) the gather-fused loaders can address from one base
    TRANSPOSE_MIN_ROWS = 2048   # routed rows per expert from which the dgrads' weight copies pay

    GATHER_MAX_BYTES = 0x7FFFFFF0

    @staticmethod
    def gather_fits(T, d, dtype) -> bool:
        """Whether x [T, d] is small enough for the gather-fused permute."""
        return T * d * torch.empty((), dtype=dtype).element_size() <= MoEFFN.GATHER_MAX_BYTES

    def __init__(self, T, d, f, E, k, *, dtype=torch.bfloat16, act="swiglu", score="softmax",
                 normalize=True, clamp=0.0, alpha=1.0, gelu_tanh=False, bias=False,
                 backward=True, device="cuda", max_cus=0, gemm="bf16", fuse_permute=True,
                 recompute=False, mx_dxp=False, transpose_w2=None, transpose_w1=None,
                 router=False, alloc=None, gate_in_act=False):
        self.T, self.d, self.f, self.E, self.k = T, d, f, E, k
        if gemm not in ("bf16", "f32", "mxfp8", "mxfp4"):
            raise ValueError(gemm)
        self.mx = gemm in ("mxfp8", "mxfp4")
        self.mx_fmt = "e2m1" if gemm == "mxfp4" else "e4m3"
        if mx_dxp and not self.mx:
            raise ValueError("mx_dxp applies to the MX variants")
        self.mx_dxp = mx_dxp
        if recompute and (self.mx or not backward):
            raise ValueError("recompute applies to the bf16 / fp32 training layer")
        self.recompute = recompute
        self.W1p_saved = self.b1p_saved = None
        self.fuse_permute = fuse_permute and not self.mx and self.gather_fits(T, d, dtype)
        self.x_saved = None
        if self.mx and (bias or act == "srelu" or dtype != torch.bfloat16):
            raise ValueError("the MXFP8 variant is gated, bias-free, with bf16 activations")
        if router and dtype != torch.bfloat16:
            raise ValueError("the fused router takes a bf16 input")
        self.router = router
        self.gate_in_act = gate_in_act
        self.R = R = T * k
        self.dtype, self.act, self.score, self.normalize = dtype, act, score, normalize
        self.clamp, self.alpha, self.gelu_tanh = clamp, alpha, gelu_tanh
        self.max_cus = max_cus
        self.n1 = n1 = f if act == "srelu" else 2 * f
        dev = torch.device(device)
        i32, f32 = torch.int32, torch.float32

        def z(shape, dt):
            if alloc is not None:
                t = alloc(tuple(shape), dt, dev)
                same_dev = t.device.type == dev.type and dev.index in (None, t.device.index)
                if tuple(t.shape) != tuple(shape) or t.dtype != dt or not same_dev:
                    raise ValueError("alloc returned a tensor of another shape, type or device")
                return t
            return torch.zeros(shape, dtype=dt, device=dev)

        self.topk_idx = z((T, k), i32)
        self.topk_w = z((T, k), f32)
        self.err = z((1,), i32)
        self.err.zero_()           # the only buffer read before it is written (sticky bits)
        self.counts = z((E,), i32)
        self.offsets = z((E + 1,), i32)
        self.row_map = z((T, k), i32)
        self.src_row = z((R,), i32)
        self.ws = z((ops.moe_permute_workspace_size(T, E, k),), torch.uint8)
        self.has_backward = backward
        self.logits = z((T, E), f32) if router else None
        self.dWr = z((E, d), f32) if router and backward else None
        self.timer = None          # optional OpTimer: HIP events around each library call
        # gates as FC1's feature scaling: per-row gates, their gradient and the
        # dGLU's partial sums
        self.w_row = z((R,), f32) if gate_in_act else None
        self.ds = z((R,), f32) if gate_in_act and backward else None
        self.ds_ws = (z((max(ops.moe_glu_bwd_workspace_size(R, f), 1),), torch.uint8)
                      if gate_in_act and backward else None)
        if self.mx:
            self._alloc_mx(z, dev)
            return
        self.xp = None if self.fuse_permute else z((R, d), dtype)
        self.H = z((R, n1), dtype) if backward else None
        self.A = z((R, f), dtype)
        self.Y = z((R, d), dtype)
        self.out = z((T, d), dtype)
        if backward:
            self.dY = z((R, d), dtype)
            self.dgate = z((T, k), f32)
            self.dlogits = z((T, E), f32)
            self.dH = z((R, n1), dtype)
            self.dXp = z((R, d), dtype)
            self.dX = z((T, d), dtype)
            self.dW1p = z((E, n1, d), f32)
            self.dW2 = z((E, d, f), f32)
            self.db1p = z((E, n1), f32) if bias else None
            self.db2 = z((E, d), f32) if bias else None
            # transposed weight copies for the dgrad GEMMs, refreshed every backward
            auto = R >= self.TRANSPOSE_MIN_ROWS * E
            transpose_w2 = auto if transpose_w2 is None else transpose_w2
            transpose_w1 = auto if transpose_w1 is None else transpose_w1
            self.W2t = z((E, f, d), dtype) if transpose_w2 else None
            self.W1pt = z((E, d, n1), dtype) if transpose_w1 else None

    def _alloc_mx(self, z, dev):
        T, d, f, E, R, n1 = self.T, self.d, self.f, self.E, self.R, self.n1
        L = ops.moe_mx_col_ld(R, E, self.mx_fmt)   # padded row stride of the column copies
        u8, f32, bf = torch.uint8, torch.float32, torch.bfloat16

        fmt = self.mx_fmt
        nb = (lambda ld: ld // 2) if fmt == "e2m1" else (lambda ld: ld)

        def mx(rows, ld):
            return ops.MXTensor(rows, ld, dev, z((rows, nb(ld)), u8), z((rows, ld // 32), u8),
                                fmt=fmt)

        self.pad_offsets = z((E + 1,), torch.int32)
        self.xp_row, self.xp_col = mx(R, d), mx(d, L)
        self.H = z((R, n1), bf)
        self.A_row, self.A_col = mx(R, f), mx(f, L)
        self.Y = z((R, d), bf)
        self.out = z((T, d), bf)
        if self.has_backward:
            self.dgate = z((T, self.k), f32)
            self.dlogits = z((T, E), f32)
            self.dY_row, self.dY_col = mx(R, d), mx(d, L)
            self.dH_row, self.dH_col = mx(R, n1), mx(n1, L)
            self.dXp = mx(R, d) if self.mx_dxp else z((R, d), bf)
            self.dX = z((T, d), bf)
            self.dW1p = z((E, n1, d), f32)
            self.dW2 = z((E, d, f), f32)
            self.db1p = self.db2 = None

    @staticmethod
    def mx_weights(W1p, W2, gemm="mxfp8"):
        return MXWeights(W1p, W2, "e2m1" if gemm == "mxfp4" else "e4m3")

    # ------------------------------------------------------------------ passes

    def _op(self, name):
        return self.timer.op(name) if self.timer is not None else contextlib.nullcontext()

    def _route(self, x, logits):
        """Top-k routing of the given logits, or (fused router) of x w_router^T
        with ``logits`` the router weight."""
        if self.router:
            with self._op("router_topk"):
                ops.moe_router_topk(x, logits, self.k, self.score, self.normalize,
                                    logits=self.logits, topk_idx=self.topk_idx,
                                    topk_w=self.topk_w, err_word=self.err)
            self.x_saved = x
        else:
            with self._op("route_topk"):
                ops.moe_route_topk(logits, self.k, self.score, self.normalize, self.topk_idx,
                                   self.topk_w, self.err)

    def _route_bwd(self, logits):
        with self._op("route_topk_bwd"):
            ops.moe_route_topk_bwd(self.logits if self.router else logits, self.topk_idx,
                                   self.dgate, self.score, self.normalize, d_logits=self.dlogits)

    def _router_bwd(self, logits):
        """The router's share of dX and its weight gradient (after dX is written)."""
        if self.router:
            with self._op("router_bwd"):
                ops.moe_router_bwd(self.x_saved, logits, self.dlogits, d_w_router=self.dWr,
                                   dx=self.dX)

    def forward(self, x, logits, W1p, W2, b1p=None, b2=None):
        if self.mx:
            return self._forward_mx(x, logits, W1p)
        self._route(x, logits)
        fused = self.fuse_permute
        with self._op("permute"):
            ops.moe_permute(x, self.topk_idx, self.E, counts=self.counts, offsets=self.offsets,
                            row_map=self.row_map, src_row=self.src_row, xp=self.xp, ws=self.ws,
                            err_word=self.err, gather=not fused)
        self.x_saved = x if (fused or self.router) else None
        self.b1p_saved = b1p
        self._gates_to_rows()
        with self._op("fc1_glu_fwd"):
            self._fc1(x, W1p, b1p, save_h=self.H is not None and not self.recompute)
        with self._op("fc2_fwd"):
            ops.moe_grouped_gemm_fwd(self.A, W2, self.offsets, b=b2, y=self.Y,
                                     max_cus=self.max_cus)
        with self._op("combine"):
            ops.moe_unpermute_combine(self.Y, self.row_map, self._combine_w(), out=self.out)
        return self.out

    def _gates_to_rows(self):
        if self.gate_in_act:
            with self._op("gates_to_rows"):
                ops.moe_permute_rows(self.topk_w, self.row_map, out=self.w_row)

    def _combine_w(self):
        """Gates of the combine: unit weights when they scale FC1's activation."""
        return None if self.gate_in_act else self.topk_w

    def _gate_grad(self, logits):
        """dgate from the dGLU's feature-scaling gradient, then the routing's backward."""
        with self._op("gate_grad"):
            ops.moe_permute_rows(self.ds, self.row_map, inverse=True, out=self.dgate)
        self._route_bwd(logits)

    def _fc1(self, x, W1p, b1p, save_h):
        fused = self.fuse_permute
        ops.moe_grouped_gemm_glu_fwd(x if fused else self.xp, W1p, self.offsets, b1p=b1p,
                                     act=self.act, clamp=self.clamp, alpha=self.alpha,
                                     gelu_tanh=self.gelu_tanh, save_h=save_h,
                                     h_out=self.H if save_h else None, a_out=self.A,
                                     max_cus=self.max_cus,
                                     src_row=self.src_row if fused else None,
                                     row_scale=self.w_row)

    def backward(self, d_out, logits, W1p, W2):
        if not self.has_backward:
            raise RuntimeError("layer built without backward buffers")
        if self.mx:
            return self._backward_mx(d_out, logits, W1p)
        if self.recompute:
            with self._op("fc1_recompute"):
                self._fc1(self.x_saved, W1p, self.b1p_saved, save_h=True)
        with self._op("combine_bwd"):
            if self.gate_in_act:
                # unit weights: dY rows are d_out's, Y is not read
                ops.moe_unpermute_combine_bwd(d_out, None, self.row_map, None, d_y=self.dY,
                                              want_dgate=False)
            else:
                ops.moe_unpermute_combine_bwd(d_out, self.Y, self.row_map, self.topk_w,
                                              d_y=self.dY, d_topk_w=self.dgate)
                self._route_bwd(logits)
        if self.W2t is not None:
            with self._op("transpose_w2"):
                ops.moe_transpose_weights(W2, self.W2t)
        with self._op("fc2_dgrad_dglu"):
            ops.moe_grouped_gemm_glu_bwd(self.dY, None if self.W2t is not None else W2, self.H,
                                         self.offsets, act=self.act, clamp=self.clamp,
                                         alpha=self.alpha, gelu_tanh=self.gelu_tanh, dh=self.dH,
                                         max_cus=self.max_cus, w2t=self.W2t,
                                         row_scale=self.w_row, d_row_scale=self.ds, ws=self.ds_ws)
        if self.gate_in_act:
            self._gate_grad(logits)
        with self._op("fc2_wgrad"):
            ops.moe_grouped_gemm_bwd(self.dY, self.offsets, mode="wgrad", a=self.A, out=self.dW2,
                                     db=self.db2, max_cus=self.max_cus)
        if self.W1pt is not None:
            with self._op("transpose_w1p"):
                ops.moe_transpose_weights(W1p, self.W1pt)
        with self._op("fc1_dgrad"):
            ops.moe_grouped_gemm_bwd(self.dH, self.offsets, mode="dgrad",
                                     w=None if self.W1pt is not None else W1p, out=self.dXp,
                                     max_cus=self.max_cus, wt=self.W1pt)
        with self._op("fc1_wgrad"):
            if self.fuse_permute:
                ops.moe_grouped_gemm_bwd(self.dH, self.offsets, mode="wgrad", a=self.x_saved,
                                         a_src_row=self.src_row, out=self.dW1p, db=self.db1p,
                                         max_cus=self.max_cus)
            else:
                ops.moe_grouped_gemm_bwd(self.dH, self.offsets, mode="wgrad", a=self.xp,
                                         out=self.dW1p, db=self.db1p, max_cus=self.max_cus)
        with self._op("unpermute_dx"):
            ops.moe_unpermute_combine(self.dXp, self.row_map, None, out=self.dX)
        self._router_bwd(logits)
        return self.dX

    def _forward_mx(self, x, logits, W: MXWeights):
        E, R, f, d = self.E, self.R, self.f, self.d
        self._route(x, logits)
        with self._op("permute"):
            ops.moe_permute(x, self.topk_idx, E, counts=self.counts, offsets=self.offsets,
                            pad_offsets=self.pad_offsets, row_map=self.row_map,
                            src_row=self.src_row, ws=self.ws, err_word=self.err, gather=False)
        with self._op("quantize_x"):
            ops.moe_mx_quantize_experts(x, self.offsets, self.pad_offsets, R, src_row=self.src_row,
                                        row_out=self.xp_row, col_out=self.xp_col,
                                        want_col=self.has_backward)
        self._gates_to_rows()
        with self._op("fc1_glu_fwd"):
            ops.moe_grouped_gemm_glu_fwd(self.xp_row, W.w1, self.offsets, E=E, f=f, act=self.act,
                                         clamp=self.clamp, alpha=self.alpha,
                                         gelu_tanh=self.gelu_tanh, h_out=self.H,
                                         pad_offsets=self.pad_offsets, a_row=self.A_row,
                                         a_col=self.A_col, want_col=self.has_backward,
                                         max_cus=self.max_cus, row_scale=self.w_row)
        with self._op("fc2_fwd"):
            ops.moe_grouped_gemm_fwd(self.A_row, W.w2, self.offsets, E=E, N=d, y=self.Y,
                                     max_cus=self.max_cus)
        with self._op("combine"):
            ops.moe_unpermute_combine(self.Y, self.row_map, self._combine_w(), out=self.out)
        return self.out

    def _backward_mx(self, d_out, logits, W: MXWeights):
        E, R, d = self.E, self.R, self.d
        if not self.gate_in_act:
            with self._op("combine_bwd"):
                ops.moe_unpermute_combine_bwd(d_out, self.Y, self.row_map, self.topk_w,
                                              d_topk_w=self.dgate, want_dy=False)
            self._route_bwd(logits)
        with self._op("quantize_dy"):
            ops.moe_mx_quantize_experts(d_out, self.offsets, self.pad_offsets, R,
                                        src_row=self.src_row,
                                        row_map=None if self.gate_in_act else self.row_map,
                                        topk_w=self._combine_w(), row_out=self.dY_row,
                                        col_out=self.dY_col)
        with self._op("fc2_dgrad_dglu"):
            ops.moe_grouped_gemm_glu_bwd(self.dY_row, W.w2t, self.H, self.offsets, E=E,
                                         act=self.act, clamp=self.clamp, alpha=self.alpha,
                                         gelu_tanh=self.gelu_tanh, pad_offsets=self.pad_offsets,
                                         dh_row=self.dH_row, dh_col=self.dH_col,
                                         max_cus=self.max_cus, row_scale=self.w_row,
                                         d_row_scale=self.ds, ws=self.ds_ws)
        if self.gate_in_act:
            self._gate_grad(logits)
        with self._op("fc2_wgrad"):
            ops.moe_grouped_gemm_bwd(self.dY_col, self.offsets, mode="wgrad", a=self.A_col,
                                     out=self.dW2, E=E, R=R, pad_offsets=self.pad_offsets,
                                     max_cus=self.max_cus)
        with self._op("fc1_dgrad"):
            if self.mx_dxp:
                ops.moe_grouped_gemm_bwd(self.dH_row, self.offsets, mode="dgrad", w=W.w1t,
                                         out_mx=self.dXp, E=E, K=d, max_cus=self.max_cus)
            else:
                ops.moe_grouped_gemm_bwd(self.dH_row, self.offsets, mode="dgrad", w=W.w1t,
                                         out=self.dXp, E=E, K=d, max_cus=self.max_cus)
        with self._op("fc1_wgrad"):
            ops.moe_grouped_gemm_bwd(self.dH_col, self.offsets, mode="wgrad", a=self.xp_col,
                                     out=self.dW1p, E=E, R=R, pad_offsets=self.pad_offsets,
                                     max_cus=self.max_cus)
        with self._op("unpermute_dx"):
            if self.mx_dxp:
                ops.moe_unpermute_combine_mx(self.dXp, self.row_map, None, out=self.dX)
            else:
                ops.moe_unpermute_combine(self.dXp, self.row_map, None, out=self.dX)
        self._router_bwd(logits)
        return self.dX

    def step(self, x, logits, W1p, W2, d_out, b1p=None, b2=None):
        self.forward(x, logits, W1p, W2, b1p, b2)
        if self.has_backward and d_out is not None:
            self.backward(d_out, logits, W1p, W2)

    # ------------------------------------------------------------------ graphs

    def capture(self, x, logits, W1p, W2, d_out=None, b1p=None, b2=None, warmup=1):
        """Capture one whole step (forward, and backward when d_out is given)
        into a HIP graph.  Replay with ``graph.replay()`` after writing new
        values into the same input tensors."""
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for _ in range(warmup):
                self.step(x, logits, W1p, W2, d_out, b1p, b2)
        torch.cuda.current_stream().wait_stream(s)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.step(x, logits, W1p, W2, d_out, b1p, b2)
        return g


class OpTimer:
    """HIP events recorded on the current stream around each named library call."""

    def __init__(self):
        self.events = {}

    @contextlib.contextmanager
    def op(self, name):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        yield
        b.record()
        self.events.setdefault(name, []).append((a, b))

    def summary(self):
        """{name: (launches, mean ms)} after a synchronize."""
        out = {}
        for name, evs in self.events.items():
            ms = [a.elapsed_time(b) for a, b in evs]
            out[name] = (len(ms), sum(ms) / len(ms))
        return out

    def reset(self):
        self.events = {}
