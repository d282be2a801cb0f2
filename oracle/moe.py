"""CPU oracle of the dropless MoE expert-FFN layer, forward and backward.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no
code with the HIP library and never imports it; the library never imports it.

Everything here is plain numpy in float64, one expert at a time, written from
the definitions on the pages (and, where the pages only name a function, from
its published definition).  Nothing is blocked, fused or reordered beyond what
the definition states; library primitives (matmul, stable sort, bincount) serve
as single steps.

Sources, cited by page title and section:

[P1] "高度な融合カーネルによる MoE 学習スループットの向上" (NVIDIA developer-blog
     post on CuTe-DSL fused MoE/MLP kernels, Japanese rendering).
     - [P1 Bottlenecks]  "MoE ブロックにおけるトレーニングのボトルネック克服":
       per-expert token counts are computed at run time; the three kernel
       families GroupGemm + Quantize, GroupGemm + Activation +
       Quantize/Transpose, GroupGemm + dActivation + Quantize/Transpose;
       activations SwiGLU, GeGLU, sReLU with clamp and scaling options.
     - [P1 GLU] "融合された GEMM エピローグによる GLU 活性化関数の最適化" and its
       Figure 2: a GLU splits the FC1 output into two chunks (input and gate)
       and combines them; weights are repacked into input and gate columns so
       one tile sees half a tile of each; the backward epilogue reads the GEMM
       output and computes dSwiGLU; epilogues also do feature scaling, clamp
       and bias-vector add.
     - [P1 Sync] "ホストとデバイスの同期および CPU 起動オーバーヘッドの排除":
       tokens per group live in device memory.
     - [P1 Quant] "MXFP8 および NVFP4 量子化の融合による露出メモリオーバーヘッドの削減":
       MXFP8 output plus a transposed copy for the backward pass.
[P2] "JAXとNVIDIA Transformer EngineによるDropless MoE学習の高速化",
     section "主張と根拠": dropless MoE, ragged tensors whose per-expert group
     sizes vary, one grouped GEMM call over the ragged groups.
[GLUvar] N. Shazeer, "GLU Variants Improve Transformer" (2020): SwiGLU and
     GeGLU, FFN(x) = (act(x W) * x V) W2.
[Primer] D. So et al., "Primer" (2021): squared ReLU, relu(x)^2.
[GELU] D. Hendrycks, K. Gimpel, "Gaussian Error Linear Units" (2016).

Readings of points the pages leave open (each is listed in the design doc):
 * Routing keys are the fp32 logits; ties go to the lower expert id; slots are
   in descending-logit order; NaN logits rank as -inf and are reported.
 * Softmax gates are the softmax over the selected logits (= the full softmax
   renormalised over the selection); sigmoid gates are sigmoid(l) / sum over
   the selection.  ``normalize=False`` keeps the unrenormalised probabilities.
 * The expert-contiguous order is a stable counting sort of the flat
   assignment index t*k + j.
 * Canonical FC1 rows [0, f) are the gate (activated) chunk, rows [f, 2f) the
   linear ("input") chunk.  The packed layout alternates G-row chunks:
   gate chunk c, then linear chunk c.
 * Clamp with limit L > 0: gate <- min(gate, L), lin <- clip(lin, -L, L); the
   gradient passes where the raw value lies inside the closed interval.
 * alpha scales the sigmoid argument: silu_a(g) = g * sigmoid(a g).
 * b2 is added to each expert output before the gate weighting.
 * Feature scaling ([P1 GLU]: the epilogues also scale): a per-row float32
   factor s[r] multiplying the activation output, A[r] = s[r] * act(H[r]);
   its gradient is ds[r] = sum over c of dA[r, c] * act(H[r])[c], and the
   activation's input gradient is taken at s[r] * dA.  With the gates as the
   factors (``LayerSpec(gate_in_act=True)``: s[r] = w[t, j] for the row r of
   assignment (t, j)) the combine sums the expert outputs with unit weights
   and the gate gradient is ds; a bias b2 is then added after the weighting
   instead of before it.
 * MXFP8 operands ([P1 Quant]; format in ``oracle/mx.py``): every GEMM operand
   is quantized in blocks of 32 along that GEMM's reduction axis.  Row copies
   (blocks along features) feed the forward and dgrad GEMMs; column copies
   (blocks along tokens, anchored at each expert's segment start, the last
   block zero-padded) feed the weight gradients.  A and dH are quantized from
   their exact epilogue values, Xp from the stored x, dY from the product
   w * dOut; H stays a bf16 tensor for the backward epilogue.  Biases are not
   part of the MXFP8 variant.  The MXFP4 variant (``gemm="mxfp4"``) quantizes
   the same tensors at the same points with E2M1 elements.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

from . import mx as _mx

# ---------------------------------------------------------------------------
# Storage rounding


def round_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (ties to even).

    bf16 keeps 8 significant bits and the float32 exponent range, so the
    quantum of a normal value 2^e * m (0.5 <= |m| < 1) is 2^(e-8), and below
    the smallest normal it is the subnormal quantum 2^-133.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    q = np.maximum(e - 8, -133)
    r = np.ldexp(np.rint(np.ldexp(x, -q)), q)
    big = np.abs(r) >= 2.0 ** 128
    if np.any(big):
        r = np.where(big, np.copysign(np.inf, x), r)
    return r


def round_f32(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def storage_round(dtype: str):
    """The rounding applied where the layer stores a tensor in ``dtype``."""
    if dtype == "bf16":
        return round_bf16
    if dtype == "f32":
        return round_f32
    if dtype == "f64":
        return lambda a: np.asarray(a, dtype=np.float64)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# a1: routing  [P1 Bottlenecks: counts are a run-time quantity]


def route_topk(logits, k: int, score: str = "softmax", normalize: bool = True):
    """Top-k expert selection and gate weights.

    Returns ``(idx [T,k] int32, w [T,k] float64, nan_seen: bool)``.  Experts
    are ranked by the float32 logit, descending, with the lower expert id first
    among equal logits.
    """
    val = np.asarray(logits, dtype=np.float64)
    lg = val.astype(np.float32)
    T, E = lg.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    nan = np.isnan(lg)
    key = np.where(nan, -np.inf, lg.astype(np.float64))
    ids = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((ids, -key), axis=-1)          # primary: -logit, then id
    idx = order[:, :k].astype(np.int32)
    # Gates use the logit values themselves (identical to the keys for float32
    # input; float64 input keeps its extra bits so gradients can be checked).
    vals = np.where(nan, -np.inf, val)
    sel = np.take_along_axis(vals, idx.astype(np.int64), axis=1)
    w = gates_from_logits(vals, sel, score, normalize)
    return idx, w, bool(nan.any())


def gates_from_logits(all_logits, sel, score: str, normalize: bool):
    """Gate weights of the selected logits ``sel`` [T,k] (rows of ``all_logits`` [T,E])."""
    if score == "softmax":
        if normalize:
            m = sel.max(axis=1, keepdims=True)
            ex = np.exp(sel - m)
            return ex / ex.sum(axis=1, keepdims=True)
        m = all_logits.max(axis=1, keepdims=True)
        return np.exp(sel - m) / np.exp(all_logits - m).sum(axis=1, keepdims=True)
    if score == "sigmoid":
        s = 1.0 / (1.0 + np.exp(-sel))
        return s / s.sum(axis=1, keepdims=True) if normalize else s
    raise ValueError(score)


def route_topk_bwd(logits, idx, dw, score: str = "softmax", normalize: bool = True):
    """Gradient of the gate weights w.r.t. all logits, given ``dw`` = dL/dw [T,k].

    The selection itself is piecewise constant, so only the gate formula is
    differentiated; unselected experts get 0 except for the unrenormalised
    softmax, whose denominator involves every logit.
    """
    lg = np.asarray(logits, dtype=np.float64)
    T, E = lg.shape
    idx = np.asarray(idx, dtype=np.int64)
    dw = np.asarray(dw, dtype=np.float64)
    sel = np.take_along_axis(lg, idx, axis=1)
    w = gates_from_logits(lg, sel, score, normalize)
    dl = np.zeros((T, E))
    rows = np.arange(T)[:, None]
    if score == "softmax" and normalize:
        # w_j = exp(l_j) / sum_sel exp  =>  dl_j = w_j (dw_j - sum_i w_i dw_i)
        inner = (w * dw).sum(axis=1, keepdims=True)
        np.add.at(dl, (rows, idx), w * (dw - inner))
    elif score == "softmax":
        # p_m = exp(l_m) / sum_all exp  =>  dl_m = p_m (dw_m [m selected] - sum_j p_j dw_j)
        m = lg.max(axis=1, keepdims=True)
        p = np.exp(lg - m) / np.exp(lg - m).sum(axis=1, keepdims=True)
        g = np.zeros((T, E))
        np.add.at(g, (rows, idx), dw)
        dl = p * (g - (p * g).sum(axis=1, keepdims=True))
    elif score == "sigmoid" and normalize:
        # w_j = s_j / S  =>  dl_m = s_m (1 - s_m) / S * (dw_m - sum_j w_j dw_j)
        s = 1.0 / (1.0 + np.exp(-sel))
        S = s.sum(axis=1, keepdims=True)
        inner = (w * dw).sum(axis=1, keepdims=True)
        np.add.at(dl, (rows, idx), s * (1.0 - s) / S * (dw - inner))
    elif score == "sigmoid":
        s = 1.0 / (1.0 + np.exp(-sel))
        np.add.at(dl, (rows, idx), dw * s * (1.0 - s))
    else:
        raise ValueError(score)
    return dl


def router_logits(x, Wr):
    """The router's linear map: logits[t, e] = <x[t], Wr[e]> (no bias).

    [P1 Bottlenecks]: routing decides at run time which experts each token
    reaches; the logits it ranks come from this map of the layer's own input.
    """
    return _f64(x) @ _f64(Wr).T


def router_backward(dlogits, x, Wr):
    """Gradients of :func:`router_logits` given dL/dlogits:
    dWr[e] = sum_t dlogits[t, e] x[t],  dx[t] = sum_e dlogits[t, e] Wr[e]."""
    dl = _f64(dlogits)
    return dl.T @ _f64(x), dl @ _f64(Wr)


# ---------------------------------------------------------------------------
# a2: permute into expert-contiguous rows  [P2 "主張と根拠": ragged groups;
#     P1 Sync: counts in device memory]


def permute_indices(topk_idx, E: int):
    """Counts, offsets and the row maps of the expert-contiguous layout.

    Row of assignment i = t*k + j (expert e_i): offsets[e_i] + #{i' < i with
    e_i' = e_i}, i.e. a stable counting sort by expert.

    Returns ``counts [E], offsets [E+1], row_map [T,k], src_row [R]`` (int32).
    """
    topk_idx = np.asarray(topk_idx)
    T, k = topk_idx.shape
    flat = topk_idx.reshape(-1).astype(np.int64)
    if flat.size and (flat.min() < 0 or flat.max() >= E):
        raise ValueError("expert id out of range")
    counts = np.bincount(flat, minlength=E)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    order = np.argsort(flat, kind="stable")       # order[row] = flat assignment index
    row_map = np.empty(T * k, dtype=np.int64)
    row_map[order] = np.arange(T * k)
    src_row = order // k
    return (counts.astype(np.int32), offsets.astype(np.int32),
            row_map.reshape(T, k).astype(np.int32), src_row.astype(np.int32))


def pad_offsets(counts, block: int = 32):
    """Offsets of the expert segments when each is padded to a multiple of ``block`` rows."""
    counts = np.asarray(counts, dtype=np.int64)
    p = np.zeros(counts.size + 1, dtype=np.int64)
    p[1:] = np.cumsum((counts + block - 1) // block * block)
    return p.astype(np.int32)


def gather_rows(x, src_row):
    """Xp[r] = x[src_row[r]] (a copy: the values are not changed)."""
    return np.asarray(x)[np.asarray(src_row, dtype=np.int64)]


# ---------------------------------------------------------------------------
# a13: repack of the FC1 weights  [P1 GLU, Figure 2]


def glu_pack_rows(f: int, G: int) -> np.ndarray:
    """Packed position of each canonical FC1 row (length 2f).

    Canonical rows [0, f) are the gate chunk and [f, 2f) the linear chunk.
    Packed rows alternate G-row chunks: gate chunk c occupies packed rows
    [2Gc, 2Gc + G) and linear chunk c occupies [2Gc + G, 2Gc + 2G).
    """
    if G <= 0 or f % G:
        raise ValueError("G must divide f")
    pos = np.empty(2 * f, dtype=np.int64)
    for i in range(f):
        c, w = divmod(i, G)
        pos[i] = 2 * G * c + w            # gate row i
        pos[f + i] = 2 * G * c + G + w    # linear row i
    return pos


def repack_glu(W1, b1=None, G: int = 64, axis: int = 1):
    """Canonical [E, 2f, ...] -> packed layout along ``axis`` (bit-exact copy)."""
    W1 = np.asarray(W1)
    f2 = W1.shape[axis]
    pos = glu_pack_rows(f2 // 2, G)
    out = np.empty_like(W1)
    idx_out = [slice(None)] * W1.ndim
    idx_out[axis] = pos
    out[tuple(idx_out)] = W1
    if b1 is None:
        return out
    b1 = np.asarray(b1)
    bo = np.empty_like(b1)
    bo[:, pos] = b1
    return out, bo


def unpack_glu(W1p, b1p=None, G: int = 64, axis: int = 1):
    """Inverse of :func:`repack_glu`."""
    W1p = np.asarray(W1p)
    pos = glu_pack_rows(W1p.shape[axis] // 2, G)
    idx_in = [slice(None)] * W1p.ndim
    idx_in[axis] = pos
    out = W1p[tuple(idx_in)]
    if b1p is None:
        return out
    return out, np.asarray(b1p)[:, pos]


# ---------------------------------------------------------------------------
# Activations  [P1 Bottlenecks / GLU: SwiGLU, GeGLU, sReLU; GLUvar; Primer; GELU]


def sigmoid(a):
    return 1.0 / (1.0 + np.exp(-a))


def act_fn(g, act: str, alpha: float = 1.0, gelu_tanh: bool = False):
    """The activation applied to the gate chunk (or to the whole output for sReLU)."""
    g = np.asarray(g, dtype=np.float64)
    if act == "swiglu":
        return g * sigmoid(alpha * g)
    if act == "geglu":
        if gelu_tanh:
            c = math.sqrt(2.0 / math.pi)
            return 0.5 * g * (1.0 + np.tanh(c * (g + 0.044715 * g ** 3)))
        # Phi(g) = (1 + erf(g / sqrt 2)) / 2, written with erfc to avoid cancellation for g << 0
        erfc = np.vectorize(math.erfc, otypes=[np.float64])
        return 0.5 * g * erfc(-g / math.sqrt(2.0))
    if act == "srelu":
        return np.maximum(g, 0.0) ** 2
    raise ValueError(act)


def act_grad(g, act: str, alpha: float = 1.0, gelu_tanh: bool = False):
    """d act / d g."""
    g = np.asarray(g, dtype=np.float64)
    if act == "swiglu":
        s = sigmoid(alpha * g)
        return s + alpha * g * s * (1.0 - s)
    if act == "geglu":
        if gelu_tanh:
            c = math.sqrt(2.0 / math.pi)
            u = c * (g + 0.044715 * g ** 3)
            th = np.tanh(u)
            return 0.5 * (1.0 + th) + 0.5 * g * (1.0 - th ** 2) * c * (1.0 + 3 * 0.044715 * g ** 2)
        erfc = np.vectorize(math.erfc, otypes=[np.float64])
        return 0.5 * erfc(-g / math.sqrt(2.0)) + g * np.exp(-0.5 * g * g) / math.sqrt(2.0 * math.pi)
    if act == "srelu":
        return 2.0 * np.maximum(g, 0.0)
    raise ValueError(act)


def glu_forward(gate, lin, act: str = "swiglu", clamp: float = 0.0, alpha: float = 1.0,
                gelu_tanh: bool = False):
    """GLU output act(gate) * lin, with the optional clamp.  [P1 GLU; GLUvar]"""
    gate = np.asarray(gate, dtype=np.float64)
    lin = np.asarray(lin, dtype=np.float64)
    if clamp > 0:
        gate = np.minimum(gate, clamp)
        lin = np.clip(lin, -clamp, clamp)
    return act_fn(gate, act, alpha, gelu_tanh) * lin


def glu_backward(dA, gate, lin, act: str = "swiglu", clamp: float = 0.0, alpha: float = 1.0,
                 gelu_tanh: bool = False):
    """(d gate, d lin) of act(gate) * lin given dA.  [P1 GLU: dSwiGLU epilogue]"""
    dA = np.asarray(dA, dtype=np.float64)
    gate = np.asarray(gate, dtype=np.float64)
    lin = np.asarray(lin, dtype=np.float64)
    mg = np.ones_like(gate)
    ml = np.ones_like(lin)
    if clamp > 0:
        mg = (gate <= clamp).astype(np.float64)
        ml = ((lin >= -clamp) & (lin <= clamp)).astype(np.float64)
        gate = np.minimum(gate, clamp)
        lin = np.clip(lin, -clamp, clamp)
    dg = dA * lin * act_grad(gate, act, alpha, gelu_tanh) * mg
    dl = dA * act_fn(gate, act, alpha, gelu_tanh) * ml
    return dg, dl


def srelu_forward(h, clamp: float = 0.0):
    h = np.asarray(h, dtype=np.float64)
    if clamp > 0:
        h = np.minimum(h, clamp)
    return act_fn(h, "srelu")


def srelu_backward(dA, h, clamp: float = 0.0):
    h = np.asarray(h, dtype=np.float64)
    m = np.ones_like(h)
    if clamp > 0:
        m = (h <= clamp).astype(np.float64)
        h = np.minimum(h, clamp)
    return np.asarray(dA, dtype=np.float64) * act_grad(h, "srelu") * m


def row_scale_forward(A, s):
    """Feature scaling of the activation output: A[r] * s[r].  [P1 GLU]"""
    return np.asarray(s, dtype=np.float64)[:, None] * np.asarray(A, dtype=np.float64)


def row_scale_backward(dA, A, s):
    """Backward of :func:`row_scale_forward` at the unscaled activation A:
    (s[r] * dA[r], the gradient the activation receives;  ds[r] = <dA[r], A[r]>)."""
    dA = np.asarray(dA, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    return np.asarray(s, dtype=np.float64)[:, None] * dA, (dA * A).sum(axis=1)


def rows_of_assignments(v, row_map):
    """v[t, j] moved to the row of assignment (t, j): out[row_map[t, j]] = v[t, j]."""
    v = np.asarray(v, dtype=np.float64)
    row_map = np.asarray(row_map, dtype=np.int64)
    out = np.zeros(row_map.size)
    out[row_map.reshape(-1)] = v.reshape(-1)
    return out


# ---------------------------------------------------------------------------
# Grouped GEMMs over the ragged expert segments  [P2 "主張と根拠"; P1 Sync]


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def grouped_linear(a, W, offsets, bias=None):
    """out[s:t] = a[s:t] @ W[e]^T (+ bias[e]) for each expert segment [s, t)."""
    a = np.asarray(a)
    E = len(offsets) - 1
    N = W.shape[1]
    out = np.zeros((a.shape[0], N))
    for e in range(E):
        s, t = int(offsets[e]), int(offsets[e + 1])
        if t > s:
            out[s:t] = _f64(a[s:t]) @ _f64(W[e]).T
            if bias is not None:
                out[s:t] += _f64(bias[e])[None, :]
    return out


def grouped_dgrad(g, W, offsets):
    """out[s:t] = g[s:t] @ W[e] for each expert segment (the input gradient of a linear map)."""
    g = np.asarray(g)
    E = len(offsets) - 1
    out = np.zeros((g.shape[0], W.shape[2]))
    for e in range(E):
        s, t = int(offsets[e]), int(offsets[e + 1])
        if t > s:
            out[s:t] = _f64(g[s:t]) @ _f64(W[e])
    return out


def grouped_wgrad(g, a, offsets, with_bias: bool = False):
    """dW[e] = g[s:t]^T @ a[s:t] and db[e] = sum of g[s:t] rows; empty segments give 0."""
    g = np.asarray(g)
    a = np.asarray(a)
    E = len(offsets) - 1
    dW = np.zeros((E, g.shape[1], a.shape[1]))
    db = np.zeros((E, g.shape[1]))
    for e in range(E):
        s, t = int(offsets[e]), int(offsets[e + 1])
        if t > s:
            ge = _f64(g[s:t])
            dW[e] = ge.T @ _f64(a[s:t])
            db[e] = ge.sum(axis=0)
    return (dW, db) if with_bias else dW


# ---------------------------------------------------------------------------
# a5 / a6 / a12: combine and its backward


def combine(Y, row_map, w=None):
    """out[t] = sum_j w[t,j] * Y[row_map[t,j]], summed over j = 0..k-1 (w = 1 if None)."""
    Y = _f64(Y)
    row_map = np.asarray(row_map, dtype=np.int64)
    T, k = row_map.shape
    out = np.zeros((T, Y.shape[1]))
    for j in range(k):
        wj = 1.0 if w is None else _f64(w)[:, j:j + 1]
        out += wj * Y[row_map[:, j]]
    return out


def combine_bwd(dout, Y, row_map, w):
    """dY[row_map[t,j]] = w[t,j] * dout[t];  dw[t,j] = <dout[t], Y[row_map[t,j]]>."""
    dout = _f64(dout)
    Y = _f64(Y)
    w = _f64(w)
    row_map = np.asarray(row_map, dtype=np.int64)
    T, k = row_map.shape
    dY = np.zeros((T * k, dout.shape[1]))
    dw = np.zeros((T, k))
    for j in range(k):
        r = row_map[:, j]
        dY[r] = w[:, j:j + 1] * dout
        dw[:, j] = (dout * Y[r]).sum(axis=1)
    return dY, dw


# ---------------------------------------------------------------------------
# The whole layer: the plain definition, and the chain with storage rounding


def ffn_dense(x, logits, W1, W2, b1=None, b2=None, *, k, score="softmax", normalize=True,
              act="swiglu", clamp=0.0, alpha=1.0, gelu_tanh=False):
    """The plain definition, token by token: y_t = sum_j w_tj * FFN_{e_tj}(x_t).

    FFN_e(x) = act(W1_e[gate] x + b1_e[gate], W1_e[lin] x + b1_e[lin]) W2_e^T + b2_e
    for gated activations, relu(W1_e x + b1_e)^2 W2_e^T + b2_e for sReLU.
    No permutation and no grouping: used to pin the grouped formulation.
    """
    x = _f64(x)
    idx, w, _ = route_topk(logits, k, score, normalize)
    T, d = x.shape
    f = W2.shape[2]
    y = np.zeros((T, d))
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            h = _f64(W1[e]) @ x[t] + (0.0 if b1 is None else _f64(b1[e]))
            if act == "srelu":
                a = srelu_forward(h, clamp)
            else:
                a = glu_forward(h[:f], h[f:], act, clamp, alpha, gelu_tanh)
            o = _f64(W2[e]) @ a + (0.0 if b2 is None else _f64(b2[e]))
            y[t] += w[t, j] * o
    return y


class LayerSpec:
    """Options of the layer (what the configs vary)."""

    def __init__(self, k, score="softmax", normalize=True, act="swiglu", clamp=0.0,
                 alpha=1.0, gelu_tanh=False, store="bf16", gemm="bf16", mx_dxp=False,
                 gate_in_act=False):
        self.k = k
        self.score = score
        self.normalize = normalize
        self.act = act
        self.clamp = clamp
        self.alpha = alpha
        self.gelu_tanh = gelu_tanh
        self.store = store      # dtype of every stored activation: "bf16", "f32" or "f64"
        self.gemm = gemm        # GEMM operands: "bf16"/"f32" (the stored tensors), "mxfp8"
        #                         or "mxfp4" (same quantization points, E2M1 elements)
        # MX variants: FC1's dgrad output dXp is stored as an MX row copy (blocks
        # along d, from the exact values) instead of bf16, as for a quantized
        # backward dispatch; the unpermute-sum then adds the decoded rows
        self.mx_dxp = mx_dxp
        # the gates scale FC1's activation output (feature scaling) and the
        # combine sums with unit weights
        self.gate_in_act = gate_in_act

    @property
    def gated(self):
        return self.act in ("swiglu", "geglu")

    @property
    def mx(self):
        return self.gemm in ("mxfp8", "mxfp4")

    @property
    def fmt(self):
        """Element format of the MX operands."""
        return "e2m1" if self.gemm == "mxfp4" else "e4m3"


def layer_forward(x, logits, W1, W2, b1=None, b2=None, *, spec: LayerSpec):
    """Forward chain in the grouped formulation with storage rounding.

    ``x``, ``W1`` (canonical [E, n1, d]), ``W2`` are the stored input values (as
    floats).  Each tensor the layer stores (H, A, Y, out) is rounded to
    ``spec.store``; arithmetic is float64.  Returns a dict of every
    intermediate, in canonical (unpacked) FC1 column order.
    """
    rnd = storage_round(spec.store)
    E = W1.shape[0]
    idx, w, nan = route_topk(logits, spec.k, spec.score, spec.normalize)
    counts, offsets, row_map, src_row = permute_indices(idx, E)
    xp = gather_rows(_f64(x), src_row)
    q = spec.mx
    if q and (b1 is not None or b2 is not None):
        raise ValueError("the MXFP8 variant has no biases")
    pad = pad_offsets(counts) if q else None
    # FC1 reduces over d: activations and weights blocked along d
    H = grouped_linear(_mx.mx_qdq(xp, 1, fmt=spec.fmt) if q else xp,
                       _mx.mx_qdq(_f64(W1), 2, fmt=spec.fmt) if q else W1,
                       offsets, b1)
    if spec.gated:
        f = W1.shape[1] // 2
        A = glu_forward(H[:, :f], H[:, f:], spec.act, spec.clamp, spec.alpha, spec.gelu_tanh)
    else:
        A = srelu_forward(H, spec.clamp)
    res = {}
    if spec.gate_in_act:
        w_row = rows_of_assignments(w, row_map)
        res.update(w_row=w_row, A_unscaled=A)
        A = row_scale_forward(A, w_row)
    H_s = rnd(H)
    if q:
        # A from its exact values: row copy along f for FC2, column copy along
        # tokens for the FC2 weight gradient
        A_fc2 = _mx.mx_qdq(A, 1, fmt=spec.fmt)
        res.update(A_row=A_fc2,
                   A_col=_mx.mx_qdq_segments_colwise(A, offsets, pad, fmt=spec.fmt),
                   xp_col=_mx.mx_qdq_segments_colwise(xp, offsets, pad, fmt=spec.fmt),
                   pad_offsets=pad)
        A_s = A_fc2
    else:
        A_s = A_fc2 = rnd(A)
    Y = grouped_linear(A_fc2, _mx.mx_qdq(_f64(W2), 2, fmt=spec.fmt) if q else W2, offsets, b2)
    Y_s = rnd(Y)
    out = combine(Y_s, row_map, None if spec.gate_in_act else w)
    res.update(topk_idx=idx, topk_w=w, nan=nan, counts=counts, offsets=offsets,
               row_map=row_map, src_row=src_row, xp=xp, H=H_s, A=A_s, Y=Y_s,
               out=rnd(out), H_exact=H, A_exact=A, Y_exact=Y, out_exact=out)
    return res


def layer_backward(fwd: dict, dout, logits, W1, W2, *, spec: LayerSpec, has_bias=False,
                   router=None):
    """Backward chain matching :func:`layer_forward`: the exact gradient of the
    grouped formulation, with the stored tensors (dY, dH, dXp, dX) rounded to
    ``spec.store`` and the weight / bias / gate gradients kept in float64.

    ``router=(x, Wr)`` when the logits are the router's map of x
    (:func:`router_logits`): the router's gradients are added -- dWr, and
    its share of dx, added to the experts' dX after that is stored:
    dX = rnd(rnd(dX_experts) + dlogits Wr)."""
    rnd = storage_round(spec.store)
    offsets, row_map = fwd["offsets"], fwd["row_map"]
    q = spec.mx
    dout = _f64(dout)
    T, k = row_map.shape
    if spec.gate_in_act:
        # unit-weight combine: every row of token t receives d_out[t]
        dY, _ = combine_bwd(dout, fwd["Y"], row_map, np.ones((T, k)))
    else:
        dY, dgate = combine_bwd(dout, fwd["Y"], row_map, fwd["topk_w"])
    if q:
        pad = fwd["pad_offsets"]
        # dY from the product w * dOut: row copy along d (FC2 dgrad), column
        # copy along tokens (FC2 weight gradient); W2 blocked along d
        dY_s = _mx.mx_qdq(dY, 1, fmt=spec.fmt)
        dY_col = _mx.mx_qdq_segments_colwise(dY, offsets, pad, fmt=spec.fmt)
        dW2, db2 = grouped_wgrad(dY_col, fwd["A_col"], offsets, with_bias=True)
        dA = grouped_dgrad(dY_s, _mx.mx_qdq(_f64(W2), 1, fmt=spec.fmt), offsets)
    else:
        dY_s = rnd(dY)
        dW2, db2 = grouped_wgrad(dY_s, fwd["A"], offsets, with_bias=True)
        dA = grouped_dgrad(dY_s, W2, offsets)
    H = fwd["H"]
    dA_act = dA
    if spec.gate_in_act:
        # the gate gradient comes out of the activation's feature scaling, at
        # the activation of the stored H (which the backward epilogue reads)
        if spec.gated:
            f = W1.shape[1] // 2
            A_h = glu_forward(H[:, :f], H[:, f:], spec.act, spec.clamp, spec.alpha,
                              spec.gelu_tanh)
        else:
            A_h = srelu_forward(H, spec.clamp)
        dA_act, ds = row_scale_backward(dA, A_h, fwd["w_row"])
        dgate = ds[row_map]
    dlogits = route_topk_bwd(logits, fwd["topk_idx"], dgate, spec.score, spec.normalize)
    if spec.gated:
        f = W1.shape[1] // 2
        dg, dl = glu_backward(dA_act, H[:, :f], H[:, f:], spec.act, spec.clamp, spec.alpha,
                              spec.gelu_tanh)
        dH = np.concatenate([dg, dl], axis=1)
    else:
        dH = srelu_backward(dA_act, H, spec.clamp)
    if q:
        # dH from its exact values: row copy along 2f (FC1 dgrad; with f a
        # multiple of 32 its blocks are the same in packed and canonical
        # order), column copy along tokens (FC1 weight gradient); W1 blocked
        # along 2f for the dgrad
        dH_s = _mx.mx_qdq(dH, 1, fmt=spec.fmt)
        dH_col = _mx.mx_qdq_segments_colwise(dH, offsets, pad, fmt=spec.fmt)
        dW1, db1 = grouped_wgrad(dH_col, fwd["xp_col"], offsets, with_bias=True)
        dXp = grouped_dgrad(dH_s, _mx.mx_qdq(_f64(W1), 1, fmt=spec.fmt), offsets)
    else:
        dH_s = rnd(dH)
        dW1, db1 = grouped_wgrad(dH_s, fwd["xp"], offsets, with_bias=True)
        dXp = grouped_dgrad(dH_s, W1, offsets)
    dXp_s = _mx.mx_qdq(dXp, 1, fmt=spec.fmt) if (q and spec.mx_dxp) else rnd(dXp)
    dX = combine(dXp_s, row_map, None)
    out = dict(dY=dY_s, dgate=dgate, dlogits=dlogits, dA=dA, dH=dH_s, dW2=dW2, dXp=dXp_s,
               dW1=dW1, dX=rnd(dX), dY_exact=dY, dH_exact=dH, dXp_exact=dXp, dX_exact=dX)
    if router is not None:
        dWr, dx_r = router_backward(dlogits, router[0], router[1])
        out.update(dWr=dWr, dX_router=dx_r, dX_experts=out["dX"],
                   dX_exact=out["dX"] + dx_r, dX=rnd(out["dX"] + dx_r))
    if q:
        out.update(dY_col=dY_col, dH_col=dH_col)
    if has_bias:
        out["db1"] = db1
        out["db2"] = db2
    return out


# ---------------------------------------------------------------------------
# Comparison metric


def norm_max_err(got, ref) -> float:
    """max |got - ref| / rms(ref) over the whole tensor (0 if ref is all zero and got matches)."""
    got = _f64(got)
    ref = _f64(ref)
    if got.shape != ref.shape:
        raise ValueError(f"shape {got.shape} vs {ref.shape}")
    if ref.size == 0:
        return 0.0
    rms = math.sqrt(float(np.mean(ref * ref)))
    diff = float(np.max(np.abs(got - ref)))
    if rms == 0.0:
        return 0.0 if diff == 0.0 else math.inf
    return diff / rms
