"""Pin of the oracle's MXFP8 layer chain by brute force on a tiny workload.

The brute force below is written per expert in the dense per-token form and
shares nothing with ``oracle.mx`` except the E4M3 format itself: elements are
rounded by torch's float8_e4m3fn cast (after clamping to +-448, which the
OCP conversion saturates to), block scales come from torch.frexp, and the
token-axis blocks are built by listing each expert's assignments in (t, j)
order and padding the list with zero rows to a multiple of 32.  It checks
where the chain quantizes (which tensors, along which axis, from exact or
stored values) against the reading in the oracle's header:

  FC1:  QDQ_d(Xp) . QDQ_d(W1)^T -> H (bf16 kept) -> A exact
  FC2:  QDQ_f(A) . QDQ_f(W2)^T -> Y (bf16) -> out = sum_j w Y (bf16)
  bwd:  dY = w dOut; dA = QDQ_d(dY) . QDQ_d(W2); dH exact from bf16 H;
        dXp = QDQ_2f(dH) . QDQ_2f(W1) (bf16, or QDQ_d of it with mx_dxp); dX = sum_j dXp (bf16);
        dW2 = QDQ_tok(dY)^T QDQ_tok(A);  dW1 = QDQ_tok(dH)^T QDQ_tok(Xp).

torch's cast rounds float64 through float32 first, which differs from a
direct round-to-nearest-even only within 2^-24 (relative) of a rounding
midpoint; the fixed inputs here avoid that (about 1e-6 chance per element).
"""
import numpy as np
import pytest
import torch

import synth
from oracle import moe as om

T, D, F, E, K = 40, 64, 64, 3, 2


def qdq_last(v):
    """QDQ along the last axis in blocks of 32 (torch float8 cast + frexp scales)."""
    t = torch.as_tensor(np.ascontiguousarray(v), dtype=torch.float64)
    n = t.shape[-1]
    b = t.reshape(*t.shape[:-1], n // 32, 32)
    amax = b.abs().amax(-1, keepdim=True)
    _, ex = torch.frexp(torch.where(amax > 0, amax, torch.ones_like(amax)))
    e = torch.clamp(ex - 1 - 8, -127, 127)
    e = torch.where(amax > 0, e, torch.full_like(e, -127)).to(torch.float64)
    scaled = torch.clamp(b / torch.pow(2.0, e), -448.0, 448.0)
    q = scaled.to(torch.float8_e4m3fn).to(torch.float64) * torch.pow(2.0, e)
    return q.reshape(t.shape).numpy()


E2M1_MAGS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def qdq_last_fp4(v):
    """E2M1 QDQ along the last axis in blocks of 32: frexp scales (exponent of
    amax minus 2) and the nearest of the eight E2M1 magnitudes by search (ties
    to the even code), saturating at 6."""
    t = np.asarray(v, dtype=np.float64)
    n = t.shape[-1]
    b = t.reshape(*t.shape[:-1], n // 32, 32)
    amax = np.abs(b).max(-1, keepdims=True)
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))
    e = np.where(amax > 0, np.clip(ex - 1 - 2, -127, 127), -127).astype(np.float64)
    a = np.abs(b) / 2.0 ** e
    d = np.abs(a[..., None] - E2M1_MAGS)                      # [..., 32, 8]
    d = d + (np.arange(8) & 1) * 1e-12 * (d.min(-1, keepdims=True) + 1)   # ties: even code
    m = E2M1_MAGS[np.argmin(d, axis=-1)]
    m = np.where(a > 6.0, 6.0, m)
    q = np.copysign(m, b) * 2.0 ** e
    return q.reshape(t.shape)


QLAST = {"e4m3": qdq_last, "e2m1": qdq_last_fp4}
_fmt = ["e4m3"]


def qdq_axis(v, axis):
    return np.moveaxis(QLAST[_fmt[0]](np.moveaxis(v, axis, -1)), -1, axis)


def qdq_tokens(rows):
    """Token-axis QDQ of one expert's rows [c, n]: blocks of 32 rows from the first."""
    c, n = rows.shape
    cp = (c + 31) // 32 * 32
    buf = np.zeros((cp, n))
    buf[:c] = rows
    return qdq_axis(buf, 0)[:c]


def qlast(v):
    return QLAST[_fmt[0]](v)


def bf16(v):
    return synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(np.asarray(v, np.float32))).astype(np.float64)


def brute(x, logits, W1, W2, dout, spec):
    idx, w, _ = om.route_topk(logits, K, spec.score, spec.normalize)
    out = np.zeros((T, D))
    dX = np.zeros((T, D))
    dW1 = np.zeros((E, 2 * F, D))
    dW2 = np.zeros((E, D, F))
    Ys = {}
    W1q_d, W2q_f = qdq_axis(W1, 2), qdq_axis(W2, 2)
    W1q_2f, W2q_d = qdq_axis(W1, 1), qdq_axis(W2, 1)
    per_expert = {}
    for e in range(E):
        assign = [(t, j) for t in range(T) for j in range(K) if idx[t, j] == e]
        if not assign:
            continue
        toks = [t for t, _ in assign]
        X = x[toks]
        H = qlast(X) @ W1q_d[e].T
        A = om.glu_forward(H[:, :F], H[:, F:], spec.act)
        Y = bf16(qlast(A) @ W2q_f[e].T)
        for r, (t, j) in enumerate(assign):
            Ys[(t, j)] = Y[r]
        per_expert[e] = (assign, X, bf16(H), A)
    for t in range(T):
        out[t] = sum(w[t, j] * Ys[(t, j)] for j in range(K))
    for e, (assign, X, Hs, A) in per_expert.items():
        wr = np.array([w[t, j] for t, j in assign])
        dY = wr[:, None] * dout[[t for t, _ in assign]]
        dA = qlast(dY) @ W2q_d[e]
        dg, dl = om.glu_backward(dA, Hs[:, :F], Hs[:, F:], spec.act)
        dH = np.concatenate([dg, dl], 1)
        dXp = qlast(dH) @ W1q_2f[e]
        dXp = qlast(dXp) if spec.mx_dxp else bf16(dXp)
        for r, (t, j) in enumerate(assign):
            dX[t] += dXp[r]
        dW2[e] = qdq_tokens(dY).T @ qdq_tokens(A)
        dW1[e] = qdq_tokens(dH).T @ qdq_tokens(X)
    return dict(out=bf16(out), dX=bf16(dX), dW1=dW1, dW2=dW2, Y=Ys)


@pytest.fixture(scope="module")
def case():
    cfg = synth.MoEConfig("mx_tiny", T=T, d=D, f=F, E=E, k=K, gemm="mxfp8", score="sigmoid",
                          zipf=0.5, seed=11, backward=True)
    inp = synth.make_inputs(cfg)
    f = lambda a: synth.bf16_bits_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a
    return cfg, f(inp["x"]), inp["logits"], f(inp["W1"]), f(inp["W2"]), f(inp["dOut"])


@pytest.mark.parametrize("gemm,fmt,mx_dxp", [("mxfp8", "e4m3", False), ("mxfp4", "e2m1", False),
                                            ("mxfp8", "e4m3", True), ("mxfp4", "e2m1", True)])
def test_mx_chain_matches_brute_force(case, gemm, fmt, mx_dxp):
    cfg, x, logits, W1, W2, dout = case
    spec = om.LayerSpec(K, "sigmoid", True, "swiglu", store="bf16", gemm=gemm, mx_dxp=mx_dxp)
    fwd = om.layer_forward(x, logits, W1, W2, spec=spec)
    bwd = om.layer_backward(fwd, dout, logits, W1, W2, spec=spec)
    _fmt[0] = fmt
    try:
        ref = brute(x, logits, W1, W2, dout, spec)
    finally:
        _fmt[0] = "e4m3"
    rel = lambda a, b: float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))
    assert rel(fwd["out"], ref["out"]) < 1e-12
    assert rel(bwd["dX"], ref["dX"]) < 1e-12
    assert rel(bwd["dW1"], ref["dW1"]) < 1e-12
    assert rel(bwd["dW2"], ref["dW2"]) < 1e-12


def test_fp4_brute_force_qdq_agrees_with_torch_free_table():
    """The brute-force E2M1 QDQ above, on values whose result the table fixes."""
    v = np.zeros(32)
    v[:8] = [6.0, 0.3, 0.75, 1.25, 2.6, -3.5, 5.0, -0.2]
    np.testing.assert_array_equal(qdq_last_fp4(v)[:8], [6.0, 0.5, 1.0, 1.0, 3.0, -4.0, 4.0, -0.0])


@pytest.mark.parametrize("gemm,lo,hi", [("mxfp8", 1e-3, 0.5), ("mxfp4", 2e-2, 0.6)])
def test_mx_chain_differs_from_plain_chain_by_quantization_size(case, gemm, lo, hi):
    """The MX chain sits a few percent (E4M3 has 4 significant bits; E2M1 two,
    so tens of percent) from the bf16 chain: far above fp64 noise, below the
    signal."""
    cfg, x, logits, W1, W2, dout = case
    sp_mx = om.LayerSpec(K, "sigmoid", True, "swiglu", store="bf16", gemm=gemm)
    sp_bf = om.LayerSpec(K, "sigmoid", True, "swiglu", store="bf16")
    a = om.layer_forward(x, logits, W1, W2, spec=sp_mx)["out"]
    b = om.layer_forward(x, logits, W1, W2, spec=sp_bf)["out"]
    # MXFP8: max error / rms; MXFP4 (one mantissa bit): rms error / rms
    r = om.norm_max_err(a, b) if gemm == "mxfp8" else \
        float(np.sqrt(np.mean((a - b) ** 2) / np.mean(b ** 2)))
    assert lo < r < hi
