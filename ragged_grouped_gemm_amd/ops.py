"""Python binding of the C ABI: one function per entry point, same names.

Arguments are torch tensors on the GPU; the functions only check shapes,
marshal pointers and the current stream, and call the library.  Every step of
the computation runs in the library's HIP kernels.  Output tensors may be
passed in (preallocated, e.g. for graph capture) or are allocated here.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _lib
from ._lib import ACT, SCORE, check

_DT = {torch.float32: _lib.MOE_F32, torch.bfloat16: _lib.MOE_BF16}


def _dtype(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")
    return _DT[t.dtype]


def _p(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _empty(shape, dtype, like):
    return torch.empty(shape, dtype=dtype, device=like.device)


class MXTensor:
    """An MX matrix (moe_mx_t): element codes ``data`` (uint8; E4M3 [rows, ld],
    or E2M1 packed two per byte [rows, ld / 2] when ``fmt == "e2m1"``) and E8M0
    scales ``scale`` [rows, ld / 32] (uint8)."""

    def __init__(self, rows: int, ld: int, device, data=None, scale=None, fmt: str = "e4m3"):
        if ld % 32:
            raise ValueError("ld must be a multiple of 32")
        if fmt not in ("e4m3", "e2m1"):
            raise ValueError(fmt)
        self.ld = ld
        self.fmt = fmt
        nb = ld if fmt == "e4m3" else ld // 2
        self.data = torch.empty((rows, nb), dtype=torch.uint8, device=device) if data is None else data
        self.scale = (torch.empty((rows, ld // 32), dtype=torch.uint8, device=device)
                      if scale is None else scale)

    @property
    def dtype_code(self):
        return _lib.MOE_E2M1 if self.fmt == "e2m1" else _lib.MOE_E4M3

    @property
    def rows(self):
        return self.data.shape[0]

    def c(self):
        """The ctypes moe_mx_t (keep it referenced while the call runs)."""
        return _lib.MxT(_p(self.data), _p(self.scale), self.ld)


def _mx(m: Optional[MXTensor]):
    return None if m is None else ctypes.pointer(m.c())


def moe_mx_col_len(R: int, E: int) -> int:
    return int(_lib.load().moe_mx_col_len(R, E))


def moe_mx_col_ld(R: int, E: int, fmt: str = "e4m3") -> int:
    """Leading dimension of a column copy: row stride an odd multiple of 128 bytes."""
    code = _lib.MOE_E2M1 if fmt == "e2m1" else _lib.MOE_E4M3
    return int(_lib.load().moe_mx_col_ld(R, E, code))


def _qname(base, fmt):
    return base.replace("moe_mx_", "moe_mxfp4_") if fmt == "e2m1" else base


def moe_mx_quantize(x, out: Optional[MXTensor] = None, fmt: str = "e4m3") -> MXTensor:
    """Row copy of x [rows, n] (blocks of 32 along n); fmt "e4m3" (MXFP8) or
    "e2m1" (MXFP4)."""
    x2 = x.reshape(-1, x.shape[-1])
    rows, n = x2.shape
    out = MXTensor(rows, n, x.device, fmt=fmt) if out is None else out
    name = _qname("moe_mx_quantize", out.fmt)
    check(getattr(_lib.load(), name)(_p(x2), _dtype(x), rows, n, _mx(out), _stream()), name)
    return out


def moe_mx_quantize_transpose(x, out: Optional[MXTensor] = None, fmt: str = "e4m3") -> MXTensor:
    """Transposed copy of x [B, rows, n]: row b*n + c = column c of x[b], blocked along rows."""
    B, rows, n = x.shape
    out = MXTensor(B * n, rows, x.device, fmt=fmt) if out is None else out
    name = _qname("moe_mx_quantize_transpose", out.fmt)
    check(getattr(_lib.load(), name)(_p(x), _dtype(x), B, rows, n, _mx(out), _stream()), name)
    return out


def moe_mx_quantize_experts(x, offsets, pad_offsets, R, *, src_row=None, row_map=None,
                            topk_w=None, want_row=True, want_col=True, row_out=None,
                            col_out=None, fmt: str = "e4m3"):
    """Row and/or expert-segmented column copies of v[r] = x[src_row[r]] (* gate)."""
    n = x.shape[1]
    E = offsets.shape[0] - 1
    k = row_map.shape[1] if row_map is not None else 0
    if want_row and row_out is None:
        row_out = MXTensor(R, n, x.device, fmt=fmt)
    if want_col and col_out is None:
        col_out = MXTensor(n, moe_mx_col_ld(R, E, fmt), x.device, fmt=fmt)
    fmt = (row_out if want_row else col_out).fmt
    name = _qname("moe_mx_quantize_experts", fmt)
    check(getattr(_lib.load(), name)(
        _p(x), _dtype(x), _p(src_row), _p(row_map), _p(topk_w), k, _p(offsets),
        _p(pad_offsets), E, R, n, _mx(row_out if want_row else None),
        _mx(col_out if want_col else None), _stream()), name)
    return (row_out if want_row else None), (col_out if want_col else None)


def moe_version() -> str:
    return _lib.load().moe_version().decode()


def moe_glu_granularity() -> int:
    return _lib.load().moe_glu_granularity()


def moe_route_topk(logits, k, score="softmax", normalize=True, topk_idx=None, topk_w=None,
                   err_word=None):
    T, E = logits.shape
    if logits.dtype != torch.float32:
        raise TypeError("logits must be float32")
    topk_idx = _empty((T, k), torch.int32, logits) if topk_idx is None else topk_idx
    topk_w = _empty((T, k), torch.float32, logits) if topk_w is None else topk_w
    check(_lib.load().moe_route_topk(_p(logits), T, E, k, SCORE[score], int(normalize),
                                     _p(topk_idx), _p(topk_w), _p(err_word), _stream()),
          "moe_route_topk")
    return topk_idx, topk_w


def moe_route_topk_bwd(logits, topk_idx, d_topk_w, score="softmax", normalize=True,
                       d_logits=None):
    T, E = logits.shape
    k = topk_idx.shape[1]
    d_logits = _empty((T, E), torch.float32, logits) if d_logits is None else d_logits
    check(_lib.load().moe_route_topk_bwd(_p(logits), _p(topk_idx), _p(d_topk_w), T, E, k,
                                         SCORE[score], int(normalize), _p(d_logits), _stream()),
          "moe_route_topk_bwd")
    return d_logits


def moe_router_topk(x, w_router, k, score="softmax", normalize=True, logits=None, topk_idx=None,
                    topk_w=None, err_word=None, want_logits=True, route=True):
    """The router's logits x w_router^T with the top-k routing of the same
    launch.  Returns (logits or None, topk_idx or None, topk_w or None)."""
    T, d = x.shape
    E = w_router.shape[0]
    if w_router.shape[1] != d:
        raise ValueError("w_router must be [E, d]")
    if want_logits and logits is None:
        logits = _empty((T, E), torch.float32, x)
    if route:
        topk_idx = _empty((T, k), torch.int32, x) if topk_idx is None else topk_idx
        topk_w = _empty((T, k), torch.float32, x) if topk_w is None else topk_w
    else:
        topk_idx = topk_w = None
    check(_lib.load().moe_router_topk(_p(x), _p(w_router), _dtype(x), T, d, E, k, SCORE[score],
                                      int(normalize), _p(logits), _p(topk_idx), _p(topk_w),
                                      _p(err_word), _stream()),
          "moe_router_topk")
    return logits, topk_idx, topk_w


def moe_router_bwd(x, w_router, d_logits, d_w_router=None, want_dw=True, accumulate=False,
                   dx=None):
    """d_w_router = d_logits^T x (float32) and dx += d_logits w_router (dx bf16,
    in place, when given).  Returns d_w_router."""
    T, d = x.shape
    E = w_router.shape[0]
    if want_dw and d_w_router is None:
        d_w_router = _empty((E, d), torch.float32, x)
    check(_lib.load().moe_router_bwd(_p(x), _p(w_router), _dtype(x), _p(d_logits), T, d, E,
                                     _p(d_w_router), int(accumulate), _p(dx), _stream()),
          "moe_router_bwd")
    return d_w_router


def moe_permute_workspace_size(T, E, k) -> int:
    return int(_lib.load().moe_permute_workspace_size(T, E, k))


def moe_permute(x, topk_idx, E, *, counts=None, offsets=None, pad_offsets=None, row_map=None,
                src_row=None, xp=None, ws=None, err_word=None, gather=True, want_pad=False):
    """Returns (counts, offsets, pad_offsets, row_map, src_row, xp)."""
    T, k = topk_idx.shape
    dev = topk_idx
    counts = _empty((E,), torch.int32, dev) if counts is None else counts
    offsets = _empty((E + 1,), torch.int32, dev) if offsets is None else offsets
    if want_pad and pad_offsets is None:
        pad_offsets = _empty((E + 1,), torch.int32, dev)
    row_map = _empty((T, k), torch.int32, dev) if row_map is None else row_map
    src_row = _empty((T * k,), torch.int32, dev) if src_row is None else src_row
    d = 0
    dt = _lib.MOE_BF16
    if gather:
        d = x.shape[1]
        dt = _dtype(x)
        xp = _empty((T * k, d), x.dtype, x) if xp is None else xp
    else:
        xp = None
    nbytes = moe_permute_workspace_size(T, E, k)
    if ws is None:
        ws = _empty((nbytes,), torch.uint8, dev)
    check(_lib.load().moe_permute(_p(x) if gather else None, dt, T, d, _p(topk_idx), k, E,
                                  _p(counts), _p(offsets), _p(pad_offsets), _p(row_map),
                                  _p(src_row), _p(xp), _p(ws), ws.numel() * ws.element_size(),
                                  _p(err_word), _stream()),
          "moe_permute")
    return counts, offsets, pad_offsets, row_map, src_row, xp


def moe_permute_noalloc(x, topk_idx, E, *, counts, offsets, row_map, src_row, pad_offsets=None,
                        xp=None, err_word=None):
    """moe_permute with the library's static scratch instead of a workspace:
    every output is the caller's preallocated tensor and the call allocates
    nothing (the first call on a device looks up the scratch address).  With
    xp given, x is gathered into it."""
    T, k = topk_idx.shape
    d = x.shape[1] if xp is not None else 0
    dt = _dtype(x) if xp is not None else _lib.MOE_BF16
    check(_lib.load().moe_permute_noalloc(_p(x) if xp is not None else None, dt, T, d,
                                          _p(topk_idx), k, E, _p(counts), _p(offsets),
                                          _p(pad_offsets), _p(row_map), _p(src_row), _p(xp),
                                          _p(err_word), _stream()),
          "moe_permute_noalloc")
    return counts, offsets, pad_offsets, row_map, src_row, xp


def moe_repack_glu_weights(w, b=None, inverse=False, w_out=None, b_out=None):
    E, n1, d = w.shape
    f = n1 // 2
    w_out = torch.empty_like(w) if w_out is None else w_out
    if b is not None and b_out is None:
        b_out = torch.empty_like(b)
    check(_lib.load().moe_repack_glu_weights(_p(w), _p(b), _dtype(w), E, f, d, int(inverse),
                                             _p(w_out), _p(b_out), _stream()),
          "moe_repack_glu_weights")
    return w_out, b_out


def moe_transpose_weights(w, wt=None):
    """wt [E, cols, rows] with wt[e][j][i] = w[e][i][j] (w [E, rows, cols])."""
    E, rows, cols = w.shape
    wt = torch.empty((E, cols, rows), dtype=w.dtype, device=w.device) if wt is None else wt
    if tuple(wt.shape) != (E, cols, rows) or wt.dtype != w.dtype:
        raise ValueError(f"wt must be {(E, cols, rows)} {w.dtype}, got {tuple(wt.shape)} {wt.dtype}")
    check(_lib.load().moe_transpose_weights(_p(w), _dtype(w), E, rows, cols, _p(wt), _stream()),
          "moe_transpose_weights")
    return wt


def moe_grouped_gemm_glu_fwd(xp, w1p, offsets, *, b1p=None, act="swiglu", clamp=0.0, alpha=1.0,
                             gelu_tanh=False, save_h=True, h_out=None, a_out=None, max_cus=0,
                             E=None, f=None, pad_offsets=None, a_row=None, a_col=None,
                             want_row=True, want_col=True, src_row=None, row_scale=None):
    """FC1 + GLU epilogue.  Returns (A [R, f], H [R, n1] or None).

    src_row (gather-fused permute): xp is the unpermuted x [T, d] and row r
    of the product reads x[src_row[r]] (R = src_row.numel()).
    row_scale (float32 [R], optional): feature scaling, A[r] = row_scale[r] * act.
    MXFP8 operands (xp, w1p MXTensor row copies along d; E and f given):
    returns ((A row copy, A column copy), H bf16)."""
    if isinstance(xp, MXTensor):
        R, d = xp.rows, xp.ld
        n1 = 2 * f
        dev = xp.data.device
        if want_row and a_row is None:
            a_row = MXTensor(R, f, dev, fmt=xp.fmt)
        if want_col and a_col is None:
            a_col = MXTensor(f, moe_mx_col_ld(R, E, xp.fmt), dev, fmt=xp.fmt)
        if save_h and h_out is None:
            h_out = torch.empty((R, n1), dtype=torch.bfloat16, device=dev)
        args = _lib.GluFwdArgs(ctypes.sizeof(_lib.GluFwdArgs), xp.dtype_code, None, None, None,
                               _p(offsets), E, R, d, f, ACT[act], clamp, alpha, int(gelu_tanh),
                               _p(h_out) if save_h else None, None, max_cus, _mx(xp), _mx(w1p),
                               _mx(a_row if want_row else None),
                               _mx(a_col if want_col else None), _p(pad_offsets))
        args.row_scale = _p(row_scale)
        check(_lib.load().moe_grouped_gemm_glu_fwd(ctypes.byref(args), _stream()),
              "moe_grouped_gemm_glu_fwd")
        return ((a_row if want_row else None), (a_col if want_col else None)), \
            (h_out if save_h else None)
    T, d = xp.shape
    R = T if src_row is None else src_row.numel()
    E, n1, _ = w1p.shape
    f = n1 if act == "srelu" else n1 // 2
    a_out = _empty((R, f), xp.dtype, xp) if a_out is None else a_out
    if save_h and h_out is None:
        h_out = _empty((R, n1), xp.dtype, xp)
    args = _lib.GluFwdArgs(ctypes.sizeof(_lib.GluFwdArgs), _dtype(xp), _p(xp), _p(w1p), _p(b1p),
                           _p(offsets), E, R, d, f, ACT[act], clamp, alpha, int(gelu_tanh),
                           _p(h_out) if save_h else None, _p(a_out), max_cus)
    if src_row is not None:
        args.src_row = _p(src_row)
        args.src_rows = T
    args.row_scale = _p(row_scale)
    check(_lib.load().moe_grouped_gemm_glu_fwd(ctypes.byref(args), _stream()),
          "moe_grouped_gemm_glu_fwd")
    return a_out, (h_out if save_h else None)


def moe_grouped_gemm_fwd(a, w, offsets, *, b=None, y=None, max_cus=0, E=None, N=None,
                         y_mx: Optional[MXTensor] = None):
    """y[r] = a[r] @ w[e]^T (+ b[e]).  MX operands (a, w MXTensor row copies
    along K; E and N given): y is bf16, or, with ``y_mx``, an MX row copy in
    the operands' format (returned instead)."""
    if isinstance(a, MXTensor):
        R, K = a.rows, a.ld
        if y_mx is None and y is None:
            y = torch.empty((R, N), dtype=torch.bfloat16, device=a.data.device)
        args = _lib.GemmFwdArgs(ctypes.sizeof(_lib.GemmFwdArgs), a.dtype_code, None, None, None,
                                _p(offsets), E, R, N, K, _p(y), max_cus, _mx(a), _mx(w),
                                _mx(y_mx))
        check(_lib.load().moe_grouped_gemm_fwd(ctypes.byref(args), _stream()),
              "moe_grouped_gemm_fwd")
        return y if y_mx is None else y_mx
    R, K = a.shape
    E, N, _ = w.shape
    y = _empty((R, N), a.dtype, a) if y is None else y
    args = _lib.GemmFwdArgs(ctypes.sizeof(_lib.GemmFwdArgs), _dtype(a), _p(a), _p(w), _p(b),
                            _p(offsets), E, R, N, K, _p(y), max_cus)
    check(_lib.load().moe_grouped_gemm_fwd(ctypes.byref(args), _stream()), "moe_grouped_gemm_fwd")
    return y


def moe_grouped_gemm_glu_bwd(dy, w2, h, offsets, *, act="swiglu", clamp=0.0, alpha=1.0,
                             gelu_tanh=False, dh=None, max_cus=0, E=None, pad_offsets=None,
                             dh_row=None, dh_col=None, want_row=True, want_col=True, w2t=None,
                             row_scale=None, d_row_scale=None, ws=None):
    """FC2 dgrad + dGLU epilogue -> dH [R, n1] (packed like h).

    w2t (bf16 / fp32, optional): W2 transposed [E, f, d] (moe_transpose_weights),
    read instead of w2 (which may then be None).
    row_scale (float32 [R], optional): the forward's feature scaling;
    d_row_scale (float32 [R], optional, written): its gradient, with the
    partial sums in ws (allocated here when not given).

    MXFP8 operands (dy row copy along d, w2 the transposed copy [E*f, d]; E
    given; h bf16): returns (dH row copy, dH column copy)."""
    if isinstance(dy, MXTensor):
        R, d = dy.rows, dy.ld
        n1 = h.shape[1]
        f = n1 // 2
        dev = h.device
        if want_row and dh_row is None:
            dh_row = MXTensor(R, n1, dev, fmt=dy.fmt)
        if want_col and dh_col is None:
            dh_col = MXTensor(n1, moe_mx_col_ld(R, E, dy.fmt), dev, fmt=dy.fmt)
        args = _lib.GluBwdArgs(ctypes.sizeof(_lib.GluBwdArgs), dy.dtype_code, None, None, _p(h),
                               _p(offsets), E, R, d, f, ACT[act], clamp, alpha, int(gelu_tanh),
                               None, max_cus, _mx(dy), _mx(w2), _mx(dh_row if want_row else None),
                               _mx(dh_col if want_col else None), _p(pad_offsets))
        _row_scale_bwd(args, R, f, row_scale, d_row_scale, ws, dev)
        check(_lib.load().moe_grouped_gemm_glu_bwd(ctypes.byref(args), _stream()),
              "moe_grouped_gemm_glu_bwd")
        return (dh_row if want_row else None), (dh_col if want_col else None)
    R, d = dy.shape
    if w2t is not None:
        E, f, d2 = w2t.shape
    else:
        E, d2, f = w2.shape
    if d2 != d:
        raise ValueError(f"the weight's d ({d2}) differs from dy's ({d})")
    dh = torch.empty_like(h) if dh is None else dh
    args = _lib.GluBwdArgs(ctypes.sizeof(_lib.GluBwdArgs), _dtype(dy), _p(dy), _p(w2), _p(h),
                           _p(offsets), E, R, d, f, ACT[act], clamp, alpha, int(gelu_tanh),
                           _p(dh), max_cus)
    args.w2t = _p(w2t)
    _row_scale_bwd(args, R, f, row_scale, d_row_scale, ws, dy.device)
    check(_lib.load().moe_grouped_gemm_glu_bwd(ctypes.byref(args), _stream()),
          "moe_grouped_gemm_glu_bwd")
    return dh


def moe_glu_bwd_workspace_size(R, f):
    return int(_lib.load().moe_glu_bwd_workspace_size(R, f))


def _row_scale_bwd(args, R, f, row_scale, d_row_scale, ws, dev):
    args.row_scale = _p(row_scale)
    if d_row_scale is not None:
        nbytes = moe_glu_bwd_workspace_size(R, f)
        if ws is None:
            ws = torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=dev)
        args.d_row_scale = _p(d_row_scale)
        args.ws = _p(ws)
        args.ws_bytes = ws.numel() * ws.element_size()


def moe_permute_rows(src, row_map, inverse=False, out=None):
    """A float per assignment to the row order (out[row_map[i]] = src[i]) or,
    with inverse, back (out[i] = src[row_map[i]]); src [T, k] or [T*k]."""
    n = row_map.numel()
    if out is None:
        out = _empty(tuple(row_map.shape) if inverse else (n,), torch.float32, row_map)
    check(_lib.load().moe_permute_rows(_p(src), _p(row_map), n, int(inverse), _p(out),
                                       _stream()),
          "moe_permute_rows")
    return out


def moe_grouped_gemm_bwd(g, offsets, *, mode, w=None, a=None, out=None, db=None, want_db=False,
                         accumulate=False, max_cus=0, E=None, R=None, N=None, K=None,
                         pad_offsets=None, a_src_row=None, out_mx: Optional[MXTensor] = None,
                         wt=None):
    """mode "dgrad": da = g @ w[e];  mode "wgrad": dw[e] = g[seg]^T @ a[seg] (+ db).

    wt (dgrad, bf16 / fp32, optional): w transposed [E, K, N]
    (moe_transpose_weights), read instead of w (which may then be None).

    a_src_row (wgrad, gather-fused permute): a is the unpermuted [T, K] and
    row r of the segments reads a[a_src_row[r]].

    MXFP8 operands: dgrad takes g [R, N] row copy and w transposed [E*K, N]
    (E, K given; da bf16); wgrad takes g [N, L] and a [K, L] column copies
    (E, R given, pad_offsets)."""
    if isinstance(g, MXTensor):
        dev = g.data.device
        if mode == "dgrad":
            R, N = g.rows, g.ld
            if out_mx is None and out is None:
                out = torch.empty((R, K), dtype=torch.bfloat16, device=dev)
            m = _lib.MOE_BWD_DGRAD
            args = _lib.GemmBwdArgs(ctypes.sizeof(_lib.GemmBwdArgs), g.dtype_code, m, None, None,
                                    None, _p(offsets), E, R, N, K, _p(out), None, 0, max_cus,
                                    _mx(g), None, _mx(w), None)
            args.out_mx = _mx(out_mx)
        elif mode == "wgrad":
            N, K = g.rows, a.rows
            out = torch.empty((E, N, K), dtype=torch.float32, device=dev) if out is None else out
            m = _lib.MOE_BWD_WGRAD
            args = _lib.GemmBwdArgs(ctypes.sizeof(_lib.GemmBwdArgs), g.dtype_code, m, None, None,
                                    None, _p(offsets), E, R, N, K, _p(out), None, int(accumulate),
                                    max_cus, _mx(g), _mx(a), None, _p(pad_offsets))
        else:
            raise ValueError(mode)
        check(_lib.load().moe_grouped_gemm_bwd(ctypes.byref(args), _stream()),
              "moe_grouped_gemm_bwd")
        return out if out_mx is None else out_mx
    R, N = g.shape
    if mode == "dgrad":
        if wt is not None:
            E, K, N2 = wt.shape
        else:
            E, N2, K = w.shape
        if N2 != N:
            raise ValueError(f"the weight's N ({N2}) differs from g's ({N})")
        out = _empty((R, K), g.dtype, g) if out is None else out
        m = _lib.MOE_BWD_DGRAD
    elif mode == "wgrad":
        K = a.shape[1]
        E = offsets.shape[0] - 1
        out = _empty((E, N, K), torch.float32, g) if out is None else out
        if want_db and db is None:
            db = _empty((E, N), torch.float32, g)
        m = _lib.MOE_BWD_WGRAD
    else:
        raise ValueError(mode)
    args = _lib.GemmBwdArgs(ctypes.sizeof(_lib.GemmBwdArgs), _dtype(g), m, _p(g), _p(a), _p(w),
                            _p(offsets), E, R, N, K, _p(out), _p(db), int(accumulate), max_cus)
    args.wt = _p(wt)
    if a_src_row is not None:
        args.a_src_row = _p(a_src_row)
        args.a_src_rows = a.shape[0]
    check(_lib.load().moe_grouped_gemm_bwd(ctypes.byref(args), _stream()),
          "moe_grouped_gemm_bwd")
    return (out, db) if mode == "wgrad" else out


def moe_unpermute_combine(y, row_map, topk_w=None, out=None):
    T, k = row_map.shape
    d = y.shape[1]
    out = _empty((T, d), y.dtype, y) if out is None else out
    check(_lib.load().moe_unpermute_combine(_p(y), _dtype(y), _p(row_map), _p(topk_w), T, k, d,
                                            _p(out), _stream()),
          "moe_unpermute_combine")
    return out


def moe_unpermute_combine_mx(y_mx: MXTensor, row_map, topk_w=None, out=None,
                             out_dtype=torch.bfloat16):
    """out[t] = sum_j w[t,j] * decode(y_mx)[row_map[t,j]] (float32 sum, one rounding)."""
    T, k = row_map.shape
    d = y_mx.ld
    out = torch.empty((T, d), dtype=out_dtype, device=row_map.device) if out is None else out
    check(_lib.load().moe_unpermute_combine_mx(_mx(y_mx), y_mx.dtype_code, _p(row_map),
                                               _p(topk_w), T, k, d, _p(out), _dtype(out),
                                               _stream()),
          "moe_unpermute_combine_mx")
    return out


def moe_unpermute_combine_bwd(d_out, y, row_map, topk_w, d_y=None, d_topk_w=None, want_dy=True,
                              want_dgate=True):
    """dY rows (topk_w None: unit weights) and the gate gradient (want_dgate;
    y is read only for it and may be None without it)."""
    T, k = row_map.shape
    d = d_out.shape[1]
    if want_dy and d_y is None:
        d_y = _empty((T * k, d), d_out.dtype, d_out)
    if want_dgate and d_topk_w is None:
        d_topk_w = _empty((T, k), torch.float32, d_out)
    check(_lib.load().moe_unpermute_combine_bwd(_p(d_out), _p(y), _dtype(d_out), _p(row_map),
                                                _p(topk_w), T, k, d, _p(d_y), _p(d_topk_w),
                                                _stream()),
          "moe_unpermute_combine_bwd")
    return d_y, d_topk_w
