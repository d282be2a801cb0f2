"""GPU parity of the fused router (logits = x Wr^T with top-k routing in one
launch) and of its backward, against the oracle.

Tolerances:
  * logits (float32 sums of d bf16 products): max |err| / rms <= 1e-5 against
    the float64 products;
  * routing: the selection is taken on the GPU's float32 logits (a near tie of
    two logits may order either way in another precision), so topk_idx must
    equal the oracle's selection on those logits bit for bit, and topk_idx /
    topk_w equal moe_route_topk's on the same logits bit for bit (the same
    selection and gate code); gates within 2e-6 relative of the oracle's;
  * dWr (float32 sums over tokens): max |err| / rms <= 1e-5; dx (bf16, one
    rounding of dx + dlogits Wr): beyond its own rounding <= 1e-3 of the rms;
  * the layer with the fused router: as test_gpu_layer (bf16 outputs 2e-2
    beyond their rounding, float32 gradients 2e-2), dWr and the total dX
    included, on the oracle chain run from the GPU's (checked) logits.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_util import bf16_excess, host, norm_err, note, rel_l2
from oracle import moe as om

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from ragged_grouped_gemm_amd import ops
    ops.moe_version()


def _bf16(rng, shape, scale=1.0):
    bits = synth.f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) *
                                  np.float32(scale))
    return synth.bf16_bits_to_f32(bits).astype(np.float64), synth.to_torch(bits, "cuda")


# (T, d, E, k, score): tails of the 32-token blocks, every expert-tile count
# of the fused path (E <= 32, 64, 128, 256), k > 8, and the passes beyond 256
# experts (selected by moe_route_topk's kernel)
CASES = [(1000, 256, 8, 2, "softmax"), (333, 2880, 32, 4, "softmax"),
         (2048, 7168, 32, 8, "sigmoid"), (500, 512, 64, 6, "sigmoid"),
         (257, 256, 128, 12, "softmax"), (300, 1024, 256, 8, "sigmoid"),
         (129, 128, 300, 6, "softmax"), (64, 64, 1024, 32, "sigmoid"), (1, 32, 5, 5, "softmax")]


@pytest.mark.parametrize("T,d,E,k,score", CASES)
def test_router_topk(T, d, E, k, score):
    note(f"router_topk T={T} d={d} E={E} k={k} {score}")
    from ragged_grouped_gemm_amd import ops
    rng = np.random.default_rng(T + d + E)
    xh, xd = _bf16(rng, (T, d))
    wh, wd = _bf16(rng, (E, d), d ** -0.5)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    lg, idx, w = ops.moe_router_topk(xd, wd, k, score, True, err_word=err)
    # logits only, and routing without writing the logits (fused path only)
    lg2, _, _ = ops.moe_router_topk(xd, wd, k, score, True, route=False)
    if E <= 256:
        _, idx3, w3 = ops.moe_router_topk(xd, wd, k, score, True, want_logits=False)
    idx_r, w_r = ops.moe_route_topk(lg, k, score, True)
    torch.cuda.synchronize()
    ref = om.router_logits(xh, wh)
    g = host(lg)
    assert norm_err(g, ref) <= 1e-5, norm_err(g, ref)
    assert torch.equal(lg, lg2)
    # the selection on the GPU's logits: the oracle's, and moe_route_topk's bit for bit
    idx_o, w_o, _ = om.route_topk(g.astype(np.float32), k, score, True)
    np.testing.assert_array_equal(host(idx), idx_o)
    assert torch.equal(idx, idx_r) and torch.equal(w, w_r)
    if E <= 256:
        assert torch.equal(idx, idx3) and torch.equal(w, w3)
    assert rel_l2(host(w), w_o) <= 2e-6
    assert int(err.item()) == 0


@pytest.mark.parametrize("T,d,E", [(1000, 256, 8), (2048, 7168, 32), (333, 2880, 32),
                                   (300, 512, 300), (64, 64, 1024)])
def test_router_bwd(T, d, E):
    note(f"router_bwd T={T} d={d} E={E}")
    from ragged_grouped_gemm_amd import ops
    rng = np.random.default_rng(7 * T + E)
    xh, xd = _bf16(rng, (T, d))
    wh, wd = _bf16(rng, (E, d), d ** -0.5)
    dl = rng.standard_normal((T, E)).astype(np.float32)
    dl[:, ::3] = 0.0                                   # unselected experts
    dld = synth.to_torch(dl, "cuda")
    dxh, dxd = _bf16(rng, (T, d))
    dw = ops.moe_router_bwd(xd, wd, dld, dx=dxd)
    dw2 = dw.clone()
    ops.moe_router_bwd(xd, wd, dld, d_w_router=dw2, accumulate=True)
    torch.cuda.synchronize()
    ref_dw, ref_dx = om.router_backward(dl.astype(np.float64), xh, wh)
    assert norm_err(host(dw), ref_dw) <= 1e-5, norm_err(host(dw), ref_dw)
    assert norm_err(host(dw2), 2 * ref_dw) <= 1e-5
    assert bf16_excess(host(dxd), dxh + ref_dx) <= 1e-3


@pytest.mark.parametrize("name,gemm", [("dsv3", "bf16"), ("gptoss", "bf16"), ("dsv3", "mxfp8")])
def test_layer_with_fused_router(name, gemm):
    """The whole layer computing its own logits: forward + backward against
    the oracle chain run from the GPU's logits (checked against x Wr^T),
    with the router's gradients (dWr, its share of dX) included."""
    from ragged_grouped_gemm_amd import ops
    from ragged_grouped_gemm_amd.layer import MoEFFN
    cfg = (synth.workload("dsv3_fwdbwd", T=1024, d=512, f=256, E=16, k=8) if name == "dsv3" else
           synth.workload("gptoss_fwdbwd", T=512, d=256, f=256, E=8, k=4, bias=False))
    note(f"layer with fused router {name} {gemm}")
    inp = synth.make_inputs(cfg)
    wr_bits = synth.draw_router_weights(cfg)
    t = lambda a: synth.to_torch(a, "cuda")
    x, W1, W2, dout, Wr = t(inp["x"]), t(inp["W1"]), t(inp["W2"]), t(inp["dOut"]), t(wr_bits)
    W1p, _ = ops.moe_repack_glu_weights(W1)
    L = MoEFFN(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, act=cfg.act, score=cfg.score,
               normalize=cfg.normalize, clamp=cfg.clamp, alpha=cfg.alpha, gemm=gemm, router=True)
    Wl = MoEFFN.mx_weights(W1p, W2, gemm) if gemm != "bf16" else W1p
    W2l = None if gemm != "bf16" else W2
    L.forward(x, Wr, Wl, W2l)
    L.backward(dout, Wr, Wl, W2l)
    torch.cuda.synchronize()
    f64 = lambda a: synth.as_f64(a, "bf16")
    xh, wh = f64(inp["x"]), f64(wr_bits)
    g_lg = host(L.logits)
    assert norm_err(g_lg, om.router_logits(xh, wh)) <= 1e-5
    lg32 = g_lg.astype(np.float32)                     # the routing decision's input
    spec = om.LayerSpec(cfg.k, cfg.score, cfg.normalize, cfg.act, cfg.clamp, cfg.alpha,
                        store="bf16", gemm=gemm)
    fwd = om.layer_forward(xh, lg32, f64(inp["W1"]), f64(inp["W2"]), spec=spec)
    bwd = om.layer_backward(fwd, f64(inp["dOut"]), lg32, f64(inp["W1"]), f64(inp["W2"]),
                            spec=spec, router=(xh, wh))
    np.testing.assert_array_equal(host(L.topk_idx), fwd["topk_idx"])
    np.testing.assert_array_equal(host(L.row_map), fwd["row_map"])
    if gemm == "bf16":
        rep = {"dWr": norm_err(host(L.dWr), bwd["dWr"]),
               "dlogits": norm_err(host(L.dlogits), bwd["dlogits"]),
               "out": bf16_excess(host(L.out), fwd["out_exact"]),
               "dX": bf16_excess(host(L.dX), bwd["dX_exact"]),
               "dW1": norm_err(om.unpack_glu(host(L.dW1p), None, 32), bwd["dW1"]),
               "dW2": norm_err(host(L.dW2), bwd["dW2"])}
    else:
        # MX: the experts' share (and the dlogits it feeds) is held to its
        # bound by the MX layer tests; here the router's backward on the
        # GPU's own dlogits and on top of the GPU's own expert dX
        g_dl = host(L.dlogits)
        ref_dw, ref_dx = om.router_backward(g_dl, xh, wh)
        rep = {"dWr": norm_err(host(L.dWr), ref_dw),
               "dX": bf16_excess(host(L.dX), _experts_dx(L, fwd) + ref_dx)}
    print(name, gemm, {k_: f"{v:.2e}" for k_, v in rep.items()}, flush=True)
    for k_, v in rep.items():
        assert v <= 2e-2, (k_, rep)


def _experts_dx(L, fwd):
    """The experts' share of dX as the GPU summed it (unpermute-sum of its own
    dXp), for checking the router's addition on top of it."""
    dXp = host(L.dXp)
    return om.round_bf16(om.combine(dXp, fwd["row_map"], None))
