"""GPU parity of the quantized plain-GEMM outputs ("GroupGemm + Quantize"):
the MX grouped GEMM writing its product as an MX row copy (FC2 forward,
FC1 dgrad), the unpermute-sum over MX rows, and the MX layers with dXp
stored as an MX row copy (``mx_dxp``).

* GEMM MX outputs against the oracle's codes of the float64 products of the
  GPU's own quantized operands, with the criteria of the MX epilogue tests
  (tests/test_gpu_mx.py for E4M3, tests/test_gpu_mx4.py for E2M1).
* The MX unpermute-sum against float64 sums of the decoded rows: float32
  output relative L2 <= 1e-6, bf16 output within 5e-3 of the rms beyond its
  own rounding.
* Layers against the oracle chain with ``mx_dxp``, routing bit-exact, with
  the tolerances of the MX layer tests of each format.
"""
import numpy as np
import pytest
import torch

from gpu_util import bf16_excess, dev, host, note, offsets_of, rand_bf16, rel_l2
from oracle import moe as om
from oracle import mx as omx

pytestmark = pytest.mark.gpu
G = 32
COUNTS_SMALL = [0, 1, 31, 32, 33, 255, 256, 257, 0, 130]
COUNTS_BIG = [0, 700, 1300, 300, 513]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from ragged_grouped_gemm_amd import ops
    ops.moe_version()


def ops_():
    from ragged_grouped_gemm_amd import ops
    return ops


def u8(t):
    return t.detach().cpu().numpy().astype(np.int64)


def deq(m):
    c = u8(m.data)
    if m.fmt == "e2m1":
        c = omx.unpack_fp4(c.astype(np.uint8))
    return omx.mx_dequantize_blocks(c, u8(m.scale), fmt=m.fmt)


def close(m, exact, what):
    """MX output codes vs the oracle's codes of the exact values."""
    oc, os_ = omx.mx_quantize_blocks(exact, fmt=m.fmt)
    if m.fmt == "e2m1":
        from test_gpu_mx4 import _fp4_close
        return _fp4_close(u8(m.data), u8(m.scale), oc, os_, exact, what)
    from test_gpu_mx import _mx_close
    return _mx_close(u8(m.data), u8(m.scale), oc, os_, exact, what)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
@pytest.mark.parametrize("counts,N,K", [(COUNTS_SMALL, 512, 256), (COUNTS_BIG, 1024, 1024)])
def test_dgrad_mx_output(fmt, counts, N, K):
    note(f"dgrad with MX output {fmt} counts={counts} N={N} K={K}")
    ops = ops_()
    rng = np.random.default_rng(31)
    E, R = len(counts), sum(counts)
    off = offsets_of(counts)
    _, gd = rand_bf16(rng, (R, N))
    _, wd = rand_bf16(rng, (E, N, K), N ** -0.5)
    gq = ops.moe_mx_quantize(gd, fmt=fmt)
    wt = ops.moe_mx_quantize_transpose(wd, fmt=fmt)
    out = ops.MXTensor(R, K, gd.device, fmt=fmt)
    ops.moe_grouped_gemm_bwd(gq, dev(off), mode="dgrad", w=wt, E=E, K=K, out_mx=out)
    torch.cuda.synchronize()
    Gq, WT = deq(gq), deq(wt).reshape(E, K, N)
    exact = np.concatenate([Gq[off[e]:off[e + 1]] @ WT[e].T for e in range(E)])
    close(out, exact, f"dgrad {fmt} MX row copy")


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_fwd_mx_output(fmt):
    counts, N, K = COUNTS_BIG, 1024, 512
    note(f"fwd with MX output {fmt}")
    ops = ops_()
    rng = np.random.default_rng(32)
    E, R = len(counts), sum(counts)
    off = offsets_of(counts)
    _, ad = rand_bf16(rng, (R, K))
    _, wd = rand_bf16(rng, (E, N, K), K ** -0.5)
    aq = ops.moe_mx_quantize(ad, fmt=fmt)
    wq = ops.moe_mx_quantize(wd.reshape(E * N, K), fmt=fmt)
    y = ops.MXTensor(R, N, ad.device, fmt=fmt)
    ops.moe_grouped_gemm_fwd(aq, wq, dev(off), E=E, N=N, y_mx=y)
    torch.cuda.synchronize()
    Aq, Wq = deq(aq), deq(wq).reshape(E, N, K)
    exact = np.concatenate([Aq[off[e]:off[e + 1]] @ Wq[e].T for e in range(E)])
    close(y, exact, f"fwd {fmt} MX row copy")


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
@pytest.mark.parametrize("k,weighted", [(8, False), (2, True), (3, True), (1, False)])
def test_unpermute_combine_mx(fmt, k, weighted):
    note(f"unpermute-sum from MX rows {fmt} k={k} weighted={weighted}")
    ops = ops_()
    rng = np.random.default_rng(33 + k)
    T, d = 300, 2048
    R = T * k
    _, yd = rand_bf16(rng, (R, d))
    ym = ops.moe_mx_quantize(yd, fmt=fmt)
    perm = rng.permutation(R).astype(np.int32).reshape(T, k)
    w = rng.random((T, k)).astype(np.float32) if weighted else None
    rmd, wd = dev(perm), (dev(w) if weighted else None)
    out_bf = ops.moe_unpermute_combine_mx(ym, rmd, wd)
    out_f = ops.moe_unpermute_combine_mx(ym, rmd, wd, out_dtype=torch.float32)
    torch.cuda.synchronize()
    Y = deq(ym)
    ref = om.combine(Y, perm, w.astype(np.float64) if weighted else None)
    assert rel_l2(host(out_f), ref) <= 1e-6
    assert bf16_excess(host(out_bf), ref) <= 5e-3


LAYER = dict(T=512, d=256, f=256, E=8, k=2, zipf=1.2, forced_empty=1, seed=21)


@pytest.mark.parametrize("gemm,rms_tol,max_tol", [("mxfp8", 5e-3, 0.25), ("mxfp4", 1e-4, 2e-2)])
def test_layer_with_mx_dxp(gemm, rms_tol, max_tol):
    import synth
    from test_gpu_mx import mx_errors
    from ragged_grouped_gemm_amd.layer import MoEFFN
    note(f"layer {gemm} with dXp as an MX row copy")
    ops = ops_()
    cfg = synth.MoEConfig("mx_dxp_layer", gemm=gemm, score="sigmoid", backward=True, **LAYER)
    inp = synth.make_inputs(cfg)
    t = lambda a: synth.to_torch(a, "cuda")
    x, lg, W1, W2, dout = t(inp["x"]), t(inp["logits"]), t(inp["W1"]), t(inp["W2"]), t(inp["dOut"])
    W1p, _ = ops.moe_repack_glu_weights(W1)
    L = MoEFFN(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, score="sigmoid", gemm=gemm, mx_dxp=True)
    Wmx = MoEFFN.mx_weights(W1p, W2, gemm)
    L.forward(x, lg, Wmx, None)
    L.backward(dout, lg, Wmx, None)
    torch.cuda.synchronize()
    f64 = lambda a: synth.bf16_bits_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a
    spec = om.LayerSpec(cfg.k, "sigmoid", True, "swiglu", store="bf16", gemm=gemm, mx_dxp=True)
    fwd = om.layer_forward(f64(inp["x"]), inp["logits"], f64(inp["W1"]), f64(inp["W2"]), spec=spec)
    bwd = om.layer_backward(fwd, f64(inp["dOut"]), inp["logits"], f64(inp["W1"]), f64(inp["W2"]),
                            spec=spec)
    np.testing.assert_array_equal(host(L.topk_idx), fwd["topk_idx"])
    # dXp itself: the GPU's MX row copy against the oracle's codes of the exact
    # products of the operands the GPU stored (its dH row copy, the W1 copy);
    # the chain's own dH codes differ at the rare epilogue flips
    off = host(L.offsets)
    dH, W1T = deq(L.dH_row), deq(Wmx.w1t).reshape(cfg.E, cfg.d, 2 * cfg.f)
    exact = np.concatenate([dH[off[e]:off[e + 1]] @ W1T[e].T for e in range(cfg.E)])
    close(L.dXp, exact, f"{gemm} layer dXp")
    rep = {"dX": mx_errors(host(L.dX), bwd["dX_exact"], bf16=True),
           "out": mx_errors(host(L.out), fwd["out_exact"], bf16=True)}
    print(gemm, "mx_dxp layer", {k_: f"rms {a:.2e} max {b:.2e}" for k_, (a, b) in rep.items()},
          flush=True)
    for name, (r_, mx) in rep.items():
        assert r_ <= rms_tol and mx <= max_tol, (name, rep)
