"""GPU parity of the feature scaling (a per-row factor on the GLU / sReLU
output, and its gradient from the dGLU epilogue) against the oracle, of the
row-order moves of the gates, of the unit-weight combine backward, and of the
layer whose gates scale FC1's activation (``gate_in_act``).

Tolerances as in the per-op and layer tests: bf16 outputs within 5e-3 (per
op) or 2e-2 (layer) of the rms beyond their own rounding, float32 results
relative L2 <= 1e-5 and max |err| / rms <= 1e-4 (per op) or 2e-2 (layer
gradients from bf16 operands); stored layer intermediates within 8 bf16 ulps;
index moves bit-exact."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import (bf16_excess, dev, host, norm_err, note, offsets_of, rand_bf16, rand_f32,
                      rel_l2, ulp_err)
from oracle import moe as om

pytestmark = pytest.mark.gpu
G = 32
ops = None


@pytest.fixture(scope="module", autouse=True)
def _lib():
    global ops
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from ragged_grouped_gemm_amd import ops as _ops
    ops = _ops
    ops.moe_version()


def f32_ok(got, ref, tol=1e-5, tol_max=1e-4):
    return rel_l2(got, ref) <= tol and norm_err(got, ref) <= tol_max


COUNTS_SMALL = [0, 1, 31, 32, 33, 255, 256, 257, 0, 130]
COUNTS_BIG = [0, 700, 1300, 300, 513]


def _scales(rng, R):
    s = rng.uniform(0.05, 1.0, R).astype(np.float32)
    s[::7] = 0.0                      # a zero gate scales the row to zero
    return s.astype(np.float64), synth.to_torch(s, "cuda")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("counts,d,f", [(COUNTS_SMALL, 256, 256), (COUNTS_BIG, 512, 512)])
@pytest.mark.parametrize("act,clamp,gather", [("swiglu", 0.0, False), ("geglu", 1.5, True),
                                              ("srelu", 0.0, False), ("swiglu", 0.8, True)])
def test_glu_fwd_row_scale(dtype, counts, d, f, act, clamp, gather):
    note(f"glu_fwd row_scale {dtype} R={sum(counts)} d={d} f={f} {act} clamp={clamp} "
         f"gather={gather}")
    rng = np.random.default_rng(sum(counts) + d + f)
    E, R = len(counts), sum(counts)
    off = offsets_of(counts)
    n1 = f if act == "srelu" else 2 * f
    mk = rand_bf16 if dtype == "bf16" else rand_f32
    T = R // 2 + 3
    xh, xd = mk(rng, (T if gather else R, d))
    src = rng.integers(0, T, R).astype(np.int32) if gather else None
    Wh, Wd = mk(rng, (E, n1, d), d ** -0.5)
    bh, bd = rand_f32(rng, (E, n1))
    sh, sd = _scales(rng, R)
    Wpd, bpd = (Wd, bd) if act == "srelu" else ops.moe_repack_glu_weights(Wd, bd)
    A, H = ops.moe_grouped_gemm_glu_fwd(xd, Wpd, dev(off), b1p=bpd, act=act, clamp=clamp,
                                        src_row=dev(src) if gather else None, row_scale=sd)
    A0, _ = ops.moe_grouped_gemm_glu_fwd(xd, Wpd, dev(off), b1p=bpd, act=act, clamp=clamp,
                                         src_row=dev(src) if gather else None, save_h=False)
    torch.cuda.synchronize()
    Xp = xh[src] if gather else xh
    Hc = om.grouped_linear(Xp, Wh, off, bh)
    Au = om.srelu_forward(Hc, clamp) if act == "srelu" else \
        om.glu_forward(Hc[:, :f], Hc[:, f:], act, clamp)
    ref = om.row_scale_forward(Au, sh)
    if dtype == "bf16":
        assert bf16_excess(host(A), ref) <= 5e-3
    else:
        assert f32_ok(host(A), ref)
    assert not host(A)[sh == 0].any()
    # the unscaled kernel is unchanged
    if dtype == "bf16":
        assert bf16_excess(host(A0), Au) <= 5e-3
    else:
        assert f32_ok(host(A0), Au)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("counts,d,f", [(COUNTS_SMALL, 256, 256), (COUNTS_BIG, 512, 512)])
@pytest.mark.parametrize("act,clamp,w2t", [("swiglu", 0.0, True), ("swiglu", 1.0, False),
                                           ("geglu", 0.0, True), ("srelu", 0.7, True)])
def test_glu_bwd_row_scale(dtype, counts, d, f, act, clamp, w2t):
    note(f"glu_bwd row_scale {dtype} R={sum(counts)} d={d} f={f} {act} clamp={clamp} w2t={w2t}")
    rng = np.random.default_rng(3 * sum(counts) + d + f)
    E, R = len(counts), sum(counts)
    Rcap = R + 45                      # rows past offsets[E]: ds must be zero there
    off = offsets_of(counts)
    n1 = f if act == "srelu" else 2 * f
    mk = rand_bf16 if dtype == "bf16" else rand_f32
    dyh, dyd = mk(rng, (Rcap, d))
    w2h, w2d = mk(rng, (E, d, f), d ** -0.5)
    hh, hd = mk(rng, (Rcap, n1))
    sh, sd = _scales(rng, Rcap)
    ds = torch.full((Rcap,), float("nan"), dtype=torch.float32, device="cuda")
    kw = dict(w2t=ops.moe_transpose_weights(w2d)) if w2t else {}
    dh = ops.moe_grouped_gemm_glu_bwd(dyd, None if w2t else w2d, hd, dev(off), act=act,
                                      clamp=clamp, row_scale=sd, d_row_scale=ds, **kw)
    torch.cuda.synchronize()
    dA = om.grouped_dgrad(dyh[:R], w2h, off)
    h = hh[:R]
    if act == "srelu":
        Au = om.srelu_forward(h, clamp)
        dA_act, ds_ref = om.row_scale_backward(dA, Au, sh[:R])
        ref = om.srelu_backward(dA_act, h, clamp)
    else:
        hc = om.unpack_glu(h[None], G=G, axis=2)[0]
        Au = om.glu_forward(hc[:, :f], hc[:, f:], act, clamp)
        dA_act, ds_ref = om.row_scale_backward(dA, Au, sh[:R])
        dg, dl = om.glu_backward(dA_act, hc[:, :f], hc[:, f:], act, clamp)
        ref = om.repack_glu(np.concatenate([dg, dl], 1)[None], G=G, axis=2)[0]
    got = host(dh)[:R]
    if dtype == "bf16":
        assert bf16_excess(got, ref) <= 5e-3
    else:
        assert f32_ok(got, ref)
    g_ds = host(ds)
    assert f32_ok(g_ds[:R], ds_ref), (rel_l2(g_ds[:R], ds_ref), norm_err(g_ds[:R], ds_ref))
    assert not g_ds[R:].any()
    # the workspace is checked before anything runs
    from ragged_grouped_gemm_amd._lib import MoEError
    with pytest.raises(MoEError, match="WORKSPACE"):
        ops.moe_grouped_gemm_glu_bwd(dyd, None if w2t else w2d, hd, dev(off), act=act,
                                     clamp=clamp, row_scale=sd, d_row_scale=ds,
                                     ws=torch.empty(8, dtype=torch.uint8, device="cuda"), **kw)


@pytest.mark.parametrize("T,k,E", [(1, 1, 1), (333, 4, 8), (4096, 8, 32)])
def test_permute_rows_bitexact(T, k, E):
    note(f"permute_rows T={T} k={k} E={E}")
    rng = np.random.default_rng(T + k)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    _, _, row_map, _ = om.permute_indices(idx, E)
    w = rng.standard_normal((T, k)).astype(np.float32)
    rm = dev(row_map.astype(np.int32))
    w_row = ops.moe_permute_rows(dev(w), rm)
    back = ops.moe_permute_rows(w_row, rm, inverse=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(w_row), om.rows_of_assignments(w, row_map).astype(np.float32))
    np.testing.assert_array_equal(host(back), w)


def test_combine_bwd_unit_weights_is_a_row_copy():
    note("combine_bwd unit weights")
    rng = np.random.default_rng(5)
    T, k, E, d = 300, 4, 8, 256
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    _, _, row_map, src_row = om.permute_indices(idx, E)
    dh, dd = rand_bf16(rng, (T, d))
    dy, _ = ops.moe_unpermute_combine_bwd(dd, None, dev(row_map.astype(np.int32)), None,
                                          want_dgate=False)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(dy), dh[src_row])


# ------------------------------------------------------------------ layer

LAYER_CASES = {
    "dsv3_small": (synth.workload("dsv3_fwdbwd", T=1024, d=512, f=256, E=16, k=8), {}),
    "gptoss_small_bias": (synth.workload("gptoss_fwdbwd", T=512, d=256, f=256, E=8, k=4), {}),
    "srelu_small": (synth.workload("dsv3_fwdbwd", T=300, d=128, f=96, E=6, k=3, act="srelu",
                                   forced_empty=1), {}),
    "dsv3_small_router": (synth.workload("dsv3_fwdbwd", T=512, d=256, f=256, E=8, k=4),
                          {"router": True}),
}


@pytest.mark.parametrize("name", sorted(LAYER_CASES))
def test_layer_gate_in_act(name):
    from ragged_grouped_gemm_amd.layer import MoEFFN
    cfg, extra = LAYER_CASES[name]
    router = extra.get("router", False)
    note(f"layer gate_in_act {name}")
    inp = synth.make_inputs(cfg)
    t = lambda a: synth.to_torch(a, "cuda")
    x, lg, W1, W2, dout = t(inp["x"]), t(inp["logits"]), t(inp["W1"]), t(inp["W2"]), t(inp["dOut"])
    b1 = t(inp["b1"]) if cfg.bias else None
    b2 = t(inp["b2"]) if cfg.bias else None
    W1p, b1p = ops.moe_repack_glu_weights(W1, b1) if cfg.gated else (W1, b1)
    if router:
        wr_bits = synth.draw_router_weights(cfg)
        lg = t(wr_bits)
    L = MoEFFN(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, act=cfg.act, score=cfg.score,
               normalize=cfg.normalize, clamp=cfg.clamp, alpha=cfg.alpha, bias=cfg.bias,
               gate_in_act=True, router=router)
    L.forward(x, lg, W1p, W2, b1p, b2)
    L.backward(dout, lg, W1p, W2)
    torch.cuda.synchronize()
    f64 = lambda a: synth.as_f64(a, "bf16")
    spec = om.LayerSpec(cfg.k, cfg.score, cfg.normalize, cfg.act, cfg.clamp, cfg.alpha,
                        store="bf16", gate_in_act=True)
    b1h = inp["b1"] if cfg.bias else None
    b2h = inp["b2"] if cfg.bias else None
    if router:
        xh = f64(inp["x"])
        logits = host(L.logits).astype(np.float32)       # the routing decision's input
        rt = (xh, f64(wr_bits))
    else:
        logits, rt = inp["logits"], None
    fwd = om.layer_forward(f64(inp["x"]), logits, f64(inp["W1"]), f64(inp["W2"]), b1h, b2h,
                           spec=spec)
    bwd = om.layer_backward(fwd, f64(inp["dOut"]), logits, f64(inp["W1"]), f64(inp["W2"]),
                            spec=spec, has_bias=cfg.bias, router=rt)
    np.testing.assert_array_equal(host(L.topk_idx), fwd["topk_idx"])
    np.testing.assert_array_equal(host(L.row_map), fwd["row_map"])
    # the gates moved to row order bit for bit (the gates themselves are
    # checked against the oracle's by the routing tests)
    np.testing.assert_array_equal(host(L.w_row),
                                  om.rows_of_assignments(host(L.topk_w), fwd["row_map"]))
    unpack = (lambda a: om.unpack_glu(a, None, G)) if cfg.gated else (lambda a: a)
    unpack_c = (lambda a: om.unpack_glu(a[None], None, G, axis=2)[0]) if cfg.gated else \
        (lambda a: a)
    # stored intermediates: each within 8 bf16 ulps of the chain's exact value
    g_A, g_dH = host(L.A), unpack_c(host(L.dH))
    assert ulp_err(g_A, fwd["A_exact"]) <= 8.0
    assert ulp_err(g_dH, bwd["dH_exact"]) <= 8.0
    # weight gradients: the oracle's weight gradient of the GPU's (checked)
    # stored dY, A and dH.  One dH element that rounds the other way (its
    # float32 and float64 values straddle a bf16 rounding point) moves a
    # dW1 element by one bf16 step of |dH| times |x|, up to ~2e-2 of the rms
    # here; the unconditioned errors are printed beside.
    off = fwd["offsets"]
    ref_dW1 = om.grouped_wgrad(g_dH, fwd["xp"], off)
    ref_dW2 = om.grouped_wgrad(host(L.dY), g_A, off)
    rep = {"out": bf16_excess(host(L.out), fwd["out_exact"]),
           "dX": bf16_excess(host(L.dX), bwd["dX_exact"]),
           "dgate": norm_err(host(L.dgate), bwd["dgate"]),
           "dlogits": norm_err(host(L.dlogits), bwd["dlogits"]),
           "dW1": norm_err(unpack(host(L.dW1p)), ref_dW1),
           "dW2": norm_err(host(L.dW2), ref_dW2)}
    free = {"dW1": norm_err(unpack(host(L.dW1p)), bwd["dW1"]),
            "dW2": norm_err(host(L.dW2), bwd["dW2"])}
    if cfg.bias:
        rep["db1"] = norm_err(unpack_c(host(L.db1p)), bwd["db1"])
        rep["db2"] = norm_err(host(L.db2), bwd["db2"])
    if router:
        rep["dWr"] = norm_err(host(L.dWr), bwd["dWr"])
    print(name, {k_: f"{v:.2e}" for k_, v in rep.items()},
          "unconditioned", {k_: f"{v:.2e}" for k_, v in free.items()}, flush=True)
    for k_, v in rep.items():
        assert v <= 2e-2, (k_, rep)
