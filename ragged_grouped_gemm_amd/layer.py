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
"""
from __future__ import annotations

import contextlib

import torch

from . import ops


class MoEFFN:
    def __init__(self, T, d, f, E, k, *, dtype=torch.bfloat16, act="swiglu", score="softmax",
                 normalize=True, clamp=0.0, alpha=1.0, gelu_tanh=False, bias=False,
                 backward=True, device="cuda", max_cus=0):
        self.T, self.d, self.f, self.E, self.k = T, d, f, E, k
        self.R = R = T * k
        self.dtype, self.act, self.score, self.normalize = dtype, act, score, normalize
        self.clamp, self.alpha, self.gelu_tanh = clamp, alpha, gelu_tanh
        self.max_cus = max_cus
        self.n1 = n1 = f if act == "srelu" else 2 * f
        dev = torch.device(device)
        i32, f32 = torch.int32, torch.float32

        def z(shape, dt):
            return torch.zeros(shape, dtype=dt, device=dev)

        self.topk_idx = z((T, k), i32)
        self.topk_w = z((T, k), f32)
        self.err = z((1,), i32)
        self.counts = z((E,), i32)
        self.offsets = z((E + 1,), i32)
        self.row_map = z((T, k), i32)
        self.src_row = z((R,), i32)
        self.ws = z((ops.moe_permute_workspace_size(T, E, k),), torch.uint8)
        self.xp = z((R, d), dtype)
        self.H = z((R, n1), dtype) if backward else None
        self.A = z((R, f), dtype)
        self.Y = z((R, d), dtype)
        self.out = z((T, d), dtype)
        self.has_backward = backward
        self.timer = None          # optional OpTimer: HIP events around each library call
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

    # ------------------------------------------------------------------ passes

    def _op(self, name):
        return self.timer.op(name) if self.timer is not None else contextlib.nullcontext()

    def forward(self, x, logits, W1p, W2, b1p=None, b2=None):
        with self._op("route_topk"):
            ops.moe_route_topk(logits, self.k, self.score, self.normalize, self.topk_idx,
                               self.topk_w, self.err)
        with self._op("permute"):
            ops.moe_permute(x, self.topk_idx, self.E, counts=self.counts, offsets=self.offsets,
                            row_map=self.row_map, src_row=self.src_row, xp=self.xp, ws=self.ws,
                            err_word=self.err)
        with self._op("fc1_glu_fwd"):
            ops.moe_grouped_gemm_glu_fwd(self.xp, W1p, self.offsets, b1p=b1p, act=self.act,
                                         clamp=self.clamp, alpha=self.alpha,
                                         gelu_tanh=self.gelu_tanh, save_h=self.H is not None,
                                         h_out=self.H, a_out=self.A, max_cus=self.max_cus)
        with self._op("fc2_fwd"):
            ops.moe_grouped_gemm_fwd(self.A, W2, self.offsets, b=b2, y=self.Y,
                                     max_cus=self.max_cus)
        with self._op("combine"):
            ops.moe_unpermute_combine(self.Y, self.row_map, self.topk_w, out=self.out)
        return self.out

    def backward(self, d_out, logits, W1p, W2):
        if not self.has_backward:
            raise RuntimeError("layer built without backward buffers")
        with self._op("combine_bwd"):
            ops.moe_unpermute_combine_bwd(d_out, self.Y, self.row_map, self.topk_w, d_y=self.dY,
                                          d_topk_w=self.dgate)
        with self._op("route_topk_bwd"):
            ops.moe_route_topk_bwd(logits, self.topk_idx, self.dgate, self.score,
                                   self.normalize, d_logits=self.dlogits)
        with self._op("fc2_dgrad_dglu"):
            ops.moe_grouped_gemm_glu_bwd(self.dY, W2, self.H, self.offsets, act=self.act,
                                         clamp=self.clamp, alpha=self.alpha,
                                         gelu_tanh=self.gelu_tanh, dh=self.dH,
                                         max_cus=self.max_cus)
        with self._op("fc2_wgrad"):
            ops.moe_grouped_gemm_bwd(self.dY, self.offsets, mode="wgrad", a=self.A, out=self.dW2,
                                     db=self.db2, max_cus=self.max_cus)
        with self._op("fc1_dgrad"):
            ops.moe_grouped_gemm_bwd(self.dH, self.offsets, mode="dgrad", w=W1p, out=self.dXp,
                                     max_cus=self.max_cus)
        with self._op("fc1_wgrad"):
            ops.moe_grouped_gemm_bwd(self.dH, self.offsets, mode="wgrad", a=self.xp,
                                     out=self.dW1p, db=self.db1p, max_cus=self.max_cus)
        with self._op("unpermute_dx"):
            ops.moe_unpermute_combine(self.dXp, self.row_map, None, out=self.dX)
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
