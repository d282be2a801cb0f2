"""Calibration of the layer-level tolerances on stored bf16 intermediates.

The GPU layer tests hold each tensor the library stores in bf16 (H, A, Y, dY,
dH, dXp) to within 8 bf16 ulps (+1e-3 RMS) of the oracle chain's exact value,
elementwise, and the layer outputs (out, dX) and float32 gradients to
max-abs/RMS <= 2e-2.  The bound is looser than one ulp because the chain
rounds to bf16 six times: where the library's float32 value and the oracle's
float64 value of a stored tensor round to neighbouring bf16 values, every
later product sees a one-ulp different input, and heavy-tailed elements
downstream move by more than their own half ulp.

This test is the CPU emulation behind that bound: the same chain in float32
arithmetic (float32 matrix products, the GLU in float32), rounding to bf16 at
the library's storage points, on a small DeepSeek-V3-like workload.  It is
checked against the oracle chain with exactly the metrics of the GPU layer
test.  It also shows that a bound of one ulp would be too tight: the
emulated chain is more than one ulp away somewhere, although every one of
its operations is correctly rounded float32.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import moe as om
from gpu_util import bf16_excess, norm_err, ulp_err


def _bf16(a):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def _silu32(g):
    g = g.astype(np.float32)
    return g / (np.float32(1) + np.exp(-g))


def _emulate(cfg, inp, fwd):
    """The layer chain in float32 with bf16 storage, on the oracle's routing."""
    f32 = np.float32
    x = synth.as_f64(inp["x"], "bf16").astype(f32)
    W1 = synth.as_f64(inp["W1"], "bf16").astype(f32)
    W2 = synth.as_f64(inp["W2"], "bf16").astype(f32)
    dout = synth.as_f64(inp["dOut"], "bf16").astype(f32)
    off, row_map, src = fwd["offsets"], fwd["row_map"], fwd["src_row"]
    w = fwd["topk_w"].astype(f32)
    E, f = cfg.E, cfg.f
    Xp = x[src]
    R = Xp.shape[0]
    H = np.zeros((R, 2 * f), f32)
    Y = np.zeros((R, cfg.d), f32)
    for e in range(E):
        s, t = off[e], off[e + 1]
        H[s:t] = Xp[s:t] @ W1[e].T
    A = _silu32(H[:, :f]) * H[:, f:]
    Hs, As = _bf16(H), _bf16(A)
    for e in range(E):
        s, t = off[e], off[e + 1]
        Y[s:t] = As[s:t] @ W2[e].T
    Ys = _bf16(Y)
    out = np.zeros((cfg.T, cfg.d), f32)
    for j in range(cfg.k):
        out += w[:, j:j + 1] * Ys[row_map[:, j]]
    # backward
    dY = np.zeros_like(Y)
    for j in range(cfg.k):
        dY[row_map[:, j]] = w[:, j:j + 1] * dout
    dYs = _bf16(dY)
    dA = np.zeros((R, f), f32)
    dW2 = np.zeros((E, cfg.d, f), f32)
    for e in range(E):
        s, t = off[e], off[e + 1]
        dA[s:t] = dYs[s:t] @ W2[e]
        dW2[e] = dYs[s:t].T @ As[s:t]
    g, lin = Hs[:, :f], Hs[:, f:]
    sg = f32(1) / (f32(1) + np.exp(-g))
    dH = np.concatenate([dA * lin * (sg + g * sg * (f32(1) - sg)), dA * g * sg], axis=1)
    dHs = _bf16(dH)
    dXp = np.zeros_like(Xp)
    dW1 = np.zeros((E, 2 * f, cfg.d), f32)
    for e in range(E):
        s, t = off[e], off[e + 1]
        dXp[s:t] = dHs[s:t] @ W1[e]
        dW1[e] = dHs[s:t].T @ Xp[s:t]
    dXps = _bf16(dXp)
    dX = np.zeros_like(x)
    for j in range(cfg.k):
        dX += dXps[row_map[:, j]]
    return dict(H=Hs, A=As, Y=Ys, out=_bf16(out), dY=dYs, dH=dHs, dXp=dXps, dX=_bf16(dX),
                dW1=dW1, dW2=dW2)


def test_float32_chain_meets_the_layer_tolerances():
    # the dsv3_small case of the GPU layer test (SwiGLU, sigmoid gates, Zipf routing)
    cfg = synth.workload("dsv3_fwdbwd", T=1024, d=512, f=256, E=16, k=8)
    inp = synth.make_inputs(cfg)
    f64 = lambda a: synth.as_f64(a, "bf16")
    spec = om.LayerSpec(cfg.k, cfg.score, cfg.normalize, cfg.act, store="bf16")
    fwd = om.layer_forward(f64(inp["x"]), inp["logits"], f64(inp["W1"]), f64(inp["W2"]),
                           spec=spec)
    bwd = om.layer_backward(fwd, f64(inp["dOut"]), inp["logits"], f64(inp["W1"]),
                            f64(inp["W2"]), spec=spec)
    em = _emulate(cfg, inp, fwd)
    ulps = {n: ulp_err(em[n], ref) for n, ref in
            (("H", fwd["H_exact"]), ("A", fwd["A_exact"]), ("Y", fwd["Y_exact"]),
             ("dY", bwd["dY_exact"]), ("dH", bwd["dH_exact"]), ("dXp", bwd["dXp_exact"]))}
    outs = {"out": bf16_excess(em["out"], fwd["out_exact"]),
            "dX": bf16_excess(em["dX"], bwd["dX_exact"]),
            "dW1": norm_err(em["dW1"], bwd["dW1"]), "dW2": norm_err(em["dW2"], bwd["dW2"])}
    print("emulated float32 chain, bf16 ulps:", {k: round(v, 2) for k, v in ulps.items()},
          "outputs:", {k: f"{v:.2e}" for k, v in outs.items()})
    assert all(v <= 8.0 for v in ulps.values()), ulps
    assert all(v <= 2e-2 for v in outs.values()), outs
    # a one-ulp bound would reject this correctly rounded float32 chain
    assert max(ulps.values()) > 1.0, ulps
