"""The oracle's MX layer chain evaluated on the GPU's own quantization decisions.

In the MXFP8 / MXFP4 layer, FC1's epilogue quantizes A and the dGLU epilogue
quantizes dH from float32 values that the scaled fp8 MFMA accumulates with
about 2^-13 relative precision, where the oracle has float64 values.  An
element that close to a rounding midpoint of its element format may round
either way, and a block maximum just under a power of two may pick either
scale: several codes are correct there, and a downstream output that sums
over f (or 2f) terms moves by one element step of one term when such a code
differs -- up to ~0.1 of its rms at f = 256.

The same holds for dY, quantized from the float32 product w * dOut on the
GPU and from the float64 product in the oracle (an E2M1 step is a quarter to
a half of the value), and for the bf16 roundings of H, Y and dXp, whose
float32 values the MX GEMMs accumulate to about 6e-5 of the sum: a few
percent of them land on the neighbouring bf16 value, one ulp away.

So the comparison takes those decisions apart:
  * check_codes / check_stored: every GPU code of A, dY and dH (row and
    token-axis column copies) is a valid rounding of the exact value -- within
    half a quantum of its element format (in the GPU's own block scale) plus
    the MFMA's accumulation error, scales within one code -- and differs from
    the oracle's own code in few elements; every stored bf16 H, Y, dXp is
    within a few ulps of its exact value;
  * conditioned chain: the oracle chain evaluated with those checked GPU
    decisions in place of its own, so each output is unique again and held to
    the plain 2e-2 max-abs / rms bound.
The oracle's unconditioned chain is reported beside it.
"""
import numpy as np
import torch

import synth
from oracle import moe as om
from oracle import mx as omx

G = 32


def codes_of(m, fmt):
    """(codes [rows, ld] int64, unpacked; scales [rows, ld/32] int64) of an MXTensor."""
    data = m.data.detach().cpu().numpy()
    c = omx.unpack_fp4(data) if fmt == "e2m1" else data
    return c.astype(np.int64), m.scale.detach().cpu().numpy().astype(np.int64)


def decode(codes, scales, fmt):
    return omx.mx_dequantize_blocks(codes, scales, fmt=fmt)


def check_codes(gc, gs, exact, fmt, what):
    """GPU codes / scales (blocks of 32 along the last axis) against the
    oracle's codes of the exact values.  Returns (scale flips, element flips)
    as fractions."""
    exact = np.asarray(exact, np.float64)
    oc, os_ = omx.mx_quantize_blocks(exact, fmt=fmt)
    gc, gs, oc, os_ = (np.asarray(a, np.int64) for a in (gc, gs, oc, os_))
    sd = gs != os_
    assert np.all(np.abs(gs - os_) <= 1), (what, "scale more than one code away")
    assert sd.mean() <= 1e-3, (what, "scale flips", sd.mean())
    rows, n = gc.shape
    vmax = 6.0 if fmt == "e2m1" else 448.0
    mant = 1 if fmt == "e2m1" else 3            # mantissa bits
    sub = -1 if fmt == "e2m1" else -9           # exponent of the subnormal quantum
    # each GPU element against the exact value in the GPU's own block scale
    # (where the scale flipped, the two sides saturate at different points)
    sc = np.ldexp(1.0, np.repeat(gs, 32, axis=1) - 127)
    v = np.clip(exact / sc, -vmax, vmax)
    g = decode(gc, gs, fmt) / sc
    bmax = np.repeat(np.abs(v).reshape(rows, n // 32, 32).max(-1), 32, axis=1)
    a = np.abs(v)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    half = 0.5 * np.ldexp(1.0, np.maximum(ex - 1 - mant, sub))   # half a quantum at |v|
    dev = np.abs(g - v) - half
    # values much smaller than their block maximum carry the MFMA's absolute
    # error (relative to the products, not to the value): rare beyond 2^-9
    assert (dev > 2.0 ** -9 * bmax).mean() <= 1e-5, (what, int((dev > 2.0 ** -9 * bmax).sum()))
    assert not (dev > 2.0 ** -4 * bmax).any(), (what, np.argwhere(dev > 2.0 ** -4 * bmax)[:5])
    flips = float((gc != oc)[~np.repeat(sd, 32, axis=1)].mean())
    assert flips <= 1e-2, (what, "element flips", flips)
    return float(sd.mean()), flips


def seg_cols(v, off, pad):
    """[R, n] values laid out like a token-axis column copy: [n, pad[-1]], zero padding."""
    out = np.zeros((v.shape[1], int(pad[-1])))
    for e in range(len(off) - 1):
        c = int(off[e + 1] - off[e])
        out[:, pad[e]:pad[e] + c] = v[off[e]:off[e + 1]].T
    return out


def cols_to_rows(vc, off, pad):
    """Inverse of seg_cols: a column copy [n, >= pad[-1]] back to [R, n] rows."""
    R = int(off[-1])
    out = np.zeros((R, vc.shape[0]))
    for e in range(len(off) - 1):
        c = int(off[e + 1] - off[e])
        out[off[e]:off[e + 1]] = vc[:, pad[e]:pad[e] + c].T
    return out


def packed_to_canonical(a, axis):
    """Packed GLU column (or row) order -> canonical [gate | linear] order."""
    pos = om.glu_pack_rows(a.shape[axis] // 2, G)
    return np.take(a, pos, axis=axis)


def check_stored(got, exact, what, max_ulps):
    """A stored bf16 intermediate (H, Y, dXp) against its exact value: each
    element within max_ulps bf16 ulps (+1e-3 rms, for values that cancel).
    Returns the largest distance in ulps."""
    from gpu_util import ulp_err
    e = ulp_err(got, exact)
    assert e <= max_ulps, (what, e)
    return e


def conditioned_layer(inp, L, fmt, k, score, normalize, act="swiglu"):
    """Whole-layer chain (forward + backward, every element) on a small MX
    layer L after L.forward / L.backward.

    Every decision the layer takes in floating point is taken from the GPU
    after checking that it is a valid one: the codes of A, dY and dH (row and
    token-axis copies) and the bf16 roundings of H, Y and dXp, each against
    its exact value computed from the (already checked) decisions before it;
    the codes of Xp, quantized from the exact input x, must equal the
    oracle's.  Every layer output is then the oracle's product, sum or
    gradient of those checked values.  Returns (got, cond, plain, flips): the
    GPU's outputs, the conditioned chain, the oracle's own chain, and the
    flip fractions / ulp distances of the decisions."""
    x, W1, W2, dout = (synth.as_f64(inp[n], "bf16") for n in ("x", "W1", "W2", "dOut"))
    lg = inp["logits"]
    host = lambda t: t.detach().cpu().to(torch.float64).numpy()
    spec = om.LayerSpec(k, score, normalize, act, store="bf16",
                        gemm="mxfp4" if fmt == "e2m1" else "mxfp8")
    fwd = om.layer_forward(x, lg, W1, W2, spec=spec)
    bwd = om.layer_backward(fwd, dout, lg, W1, W2, spec=spec)
    off, pad, row_map, w = fwd["offsets"], fwd["pad_offsets"], fwd["row_map"], fwd["topk_w"]
    f, R, Rp = W2.shape[2], int(fwd["offsets"][-1]), int(fwd["pad_offsets"][-1])
    q = lambda v, ax: omx.mx_qdq(v, ax, fmt=fmt)
    pos = om.glu_pack_rows(f, G)

    def to_packed(a):
        out = np.empty_like(a)
        out[:, pos] = a
        return out

    dec = {}

    def take(m, exact_rows, what, cols=None):
        """GPU row copy m [R, >= n] checked against exact [R, n]; its values."""
        n = exact_rows.shape[1]
        gc, gs = codes_of(m, fmt)
        dec[what] = check_codes(gc[:, :n], gs[:, :n // 32], exact_rows, fmt, what)
        return decode(gc, gs, fmt)[:, :n]

    def take_col(m, exact_rows, what):
        """GPU token-axis copy m [n, >= Rp] checked against exact [R, n] rows."""
        gc, gs = codes_of(m, fmt)
        dec[what] = check_codes(gc[:, :Rp], gs[:, :Rp // 32], seg_cols(exact_rows, off, pad), fmt,
                                what)
        return cols_to_rows(decode(gc, gs, fmt), off, pad)

    # Xp: quantized from the exact input, so its codes are unique
    for m, (oc, os_) in ((L.xp_row, omx.mx_quantize_blocks(fwd["xp"], fmt=fmt)),
                         (L.xp_col, omx.mx_quantize_segments_colwise(fwd["xp"], off, pad,
                                                                     fmt=fmt))):
        gc, gs = codes_of(m, fmt)
        n = oc.shape[1]
        assert np.array_equal(gc[:, :n], oc) and np.array_equal(gs[:, :n // 32], os_), "Xp codes"
    # ---- forward
    H = packed_to_canonical(host(L.H), 1)
    dec["H"] = check_stored(H, fwd["H_exact"], "H", 8.0)
    A_row = take(L.A_row, fwd["A_exact"], "A row copy")
    A_col = take_col(L.A_col, fwd["A_exact"], "A column copy")
    Y = host(L.Y)
    dec["Y"] = check_stored(Y, om.grouped_linear(A_row, q(W2, 2), off), "Y", 4.0)
    out = om.combine(Y, row_map, w)
    # ---- backward
    dY_exact, dgate = om.combine_bwd(dout, Y, row_map, w)
    dlogits = om.route_topk_bwd(lg, fwd["topk_idx"], dgate, score, normalize)
    dY_row = take(L.dY_row, dY_exact, "dY row copy")
    dY_col = take_col(L.dY_col, dY_exact, "dY column copy")
    dW2 = om.grouped_wgrad(dY_col, A_col, off)
    dA = om.grouped_dgrad(dY_row, q(W2, 1), off)
    dg, dl = om.glu_backward(dA, H[:, :f], H[:, f:], act)
    dH_exact = to_packed(np.concatenate([dg, dl], axis=1))   # the order the GPU blocks in
    dH_row = packed_to_canonical(take(L.dH_row, dH_exact, "dH row copy"), 1)
    dH_col = packed_to_canonical(take_col(L.dH_col, dH_exact, "dH column copy"), 1)
    dW1 = om.grouped_wgrad(dH_col, fwd["xp_col"], off)
    dXp = host(L.dXp)
    dec["dXp"] = check_stored(dXp, om.grouped_dgrad(dH_row, q(W1, 1), off), "dXp", 4.0)
    dX = om.combine(dXp, row_map, None)
    cond = dict(out=out, dX=dX, dW1=dW1, dW2=dW2, dgate=dgate, dlogits=dlogits)
    plain = dict(out=fwd["out_exact"], dX=bwd["dX_exact"], dW1=bwd["dW1"], dW2=bwd["dW2"],
                 dgate=bwd["dgate"], dlogits=bwd["dlogits"])
    got = dict(out=host(L.out), dX=host(L.dX), dW1=om.unpack_glu(host(L.dW1p), None, G),
               dW2=host(L.dW2), dgate=host(L.dgate), dlogits=host(L.dlogits))
    assert R == A_row.shape[0]
    return got, cond, plain, dec
