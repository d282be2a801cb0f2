"""Pins of the oracle's feature scaling (a per-row factor on the activation
output) and of the layer variant whose gates scale FC1's activation
(``LayerSpec(gate_in_act=True)``): finite differences of the scaled GLU,
torch float64 autograd through a dense token-by-token model, and the
identity with the standard layer when there is no b2 (the gate then
multiplies a linear map either before or after it)."""
import numpy as np
import pytest
import torch

from oracle import moe as om

F = torch.nn.functional


def _inputs(seed, T=19, d=12, f=8, E=5, k=2, gated=True):
    rng = np.random.default_rng(seed)
    n1 = 2 * f if gated else f
    return dict(x=rng.standard_normal((T, d)), logits=rng.standard_normal((T, E)),
                W1=rng.standard_normal((E, n1, d)) / np.sqrt(d),
                W2=rng.standard_normal((E, d, f)) / np.sqrt(f),
                b1=rng.standard_normal((E, n1)), b2=rng.standard_normal((E, d)),
                dout=rng.standard_normal((T, d)), k=k)


def _run(inp, score, act, clamp, gate_in_act, b2=True, store="f64"):
    spec = om.LayerSpec(inp["k"], score, True, act, clamp, store=store, gate_in_act=gate_in_act)
    b2v = inp["b2"] if b2 else None
    fwd = om.layer_forward(inp["x"], inp["logits"], inp["W1"], inp["W2"], inp["b1"], b2v,
                           spec=spec)
    bwd = om.layer_backward(fwd, inp["dout"], inp["logits"], inp["W1"], inp["W2"], spec=spec,
                            has_bias=True)
    return fwd, bwd


@pytest.mark.parametrize("score,act,clamp", [("softmax", "swiglu", 0.0),
                                             ("sigmoid", "swiglu", 0.8),
                                             ("softmax", "geglu", 0.0),
                                             ("sigmoid", "srelu", 0.9)])
def test_gate_in_act_equals_standard_layer_without_b2(score, act, clamp):
    """w * (W2 a) == W2 (w * a): without b2 both layers compute the same
    function, so the outputs and every gradient must agree to rounding."""
    inp = _inputs(11, gated=act != "srelu")
    f0, b0 = _run(inp, score, act, clamp, False, b2=False)
    f1, b1 = _run(inp, score, act, clamp, True, b2=False)
    np.testing.assert_allclose(f1["out"], f0["out"], rtol=1e-12, atol=1e-12)
    for name in ("dX", "dW1", "dW2", "db1", "dgate", "dlogits"):
        np.testing.assert_allclose(b1[name], b0[name], rtol=1e-10, atol=1e-12, err_msg=name)
    # the scaled activation really carries the gate
    assert np.abs(f1["A"] - f0["A"]).max() > 1e-3


def _torch_layer(inp, score, act, clamp):
    """Token by token: y_t = sum_j (W2_e (w_tj act(W1_e x_t + b1_e)) + b2_e);
    torch autograd for every gradient, the gates' included."""
    t = {n: torch.tensor(inp[n], requires_grad=True) for n in ("x", "logits", "W1", "W2", "b1",
                                                                "b2")}
    k = inp["k"]
    lg = t["logits"]
    _, idx = torch.topk(lg.detach(), k, dim=1)
    sel = lg.gather(1, idx)
    w = torch.softmax(sel, 1) if score == "softmax" else \
        torch.sigmoid(sel) / torch.sigmoid(sel).sum(1, keepdim=True)
    f = inp["W2"].shape[2]
    out = torch.zeros_like(t["x"])
    for j in range(k):
        e = idx[:, j]
        h = torch.einsum("tnd,td->tn", t["W1"][e], t["x"]) + t["b1"][e]
        if act == "srelu":
            hh = torch.clamp(h, max=clamp) if clamp > 0 else h
            a = torch.relu(hh) ** 2
        else:
            g, li = h[:, :f], h[:, f:]
            if clamp > 0:
                g, li = torch.clamp(g, max=clamp), torch.clamp(li, -clamp, clamp)
            a = (F.silu(g) if act == "swiglu" else F.gelu(g)) * li
        a = w[:, j:j + 1] * a
        out = out + torch.einsum("tdf,tf->td", t["W2"][e], a) + t["b2"][e]
    (out * torch.tensor(inp["dout"])).sum().backward()
    return idx.numpy(), out.detach().numpy(), {n: v.grad.numpy() for n, v in t.items()}


@pytest.mark.parametrize("score,act,clamp", [("softmax", "swiglu", 0.0),
                                             ("sigmoid", "geglu", 0.7),
                                             ("softmax", "srelu", 0.0)])
def test_gate_in_act_layer_matches_torch_autograd(score, act, clamp):
    inp = _inputs(12, gated=act != "srelu")
    fwd, bwd = _run(inp, score, act, clamp, True, b2=True)
    idx, out, g = _torch_layer(inp, score, act, clamp)
    np.testing.assert_array_equal(fwd["topk_idx"], idx)
    np.testing.assert_allclose(fwd["out"], out, rtol=1e-10, atol=1e-12)
    tol = dict(rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(bwd["dX"], g["x"], **tol)
    np.testing.assert_allclose(bwd["dW1"], g["W1"], **tol)
    np.testing.assert_allclose(bwd["dW2"], g["W2"], **tol)
    np.testing.assert_allclose(bwd["db1"], g["b1"], **tol)
    np.testing.assert_allclose(bwd["db2"], g["b2"], **tol)
    np.testing.assert_allclose(bwd["dlogits"], g["logits"], **tol)


def test_scaled_glu_matches_finite_differences():
    """L = <dA, s * glu(gate, lin)>: d/ds from row_scale_backward, d/dgate and
    d/dlin from glu_backward at s * dA, against central differences."""
    rng = np.random.default_rng(13)
    n, f = 5, 6
    gate, lin = rng.standard_normal((n, f)), rng.standard_normal((n, f))
    s, dA = rng.uniform(0.1, 1.0, n), rng.standard_normal((n, f))

    def loss(g, l, sc):
        return float((dA * om.row_scale_forward(om.glu_forward(g, l, "swiglu", 0.9), sc)).sum())

    dA_act, ds = om.row_scale_backward(dA, om.glu_forward(gate, lin, "swiglu", 0.9), s)
    dg, dl = om.glu_backward(dA_act, gate, lin, "swiglu", 0.9)
    eps = 1e-6
    for arr, grad in ((s, ds), (gate, dg), (lin, dl)):
        flat, gf = arr.reshape(-1), grad.reshape(-1)
        for i in range(flat.size):
            old = flat[i]
            flat[i] = old + eps
            lp = loss(gate, lin, s)
            flat[i] = old - eps
            lm = loss(gate, lin, s)
            flat[i] = old
            assert abs(gf[i] - (lp - lm) / (2 * eps)) <= 1e-6 * max(1.0, abs(gf[i])), i


def test_rows_of_assignments_is_the_row_map_permutation():
    topk_idx = np.array([[2, 0], [0, 1], [2, 1]])
    _, _, row_map, _ = om.permute_indices(topk_idx, 3)
    v = np.array([[0.1, 0.2], [0.3, 0.4], [0.5, 0.6]])
    w_row = om.rows_of_assignments(v, row_map)
    # expert 0 rows: (0,1), (1,0); expert 1: (1,1), (2,1); expert 2: (0,0), (2,0)
    np.testing.assert_array_equal(w_row, [0.2, 0.3, 0.4, 0.6, 0.1, 0.5])
    np.testing.assert_array_equal(w_row[row_map], v)


def test_gate_in_act_storage_rounding_points():
    """bf16 storage: A is rounded after the scaling; dY is the unweighted
    d_out (exact in bf16); the gate gradient uses the stored H."""
    inp = _inputs(14)
    rb = om.round_bf16
    inp = {n: (rb(v) if isinstance(v, np.ndarray) and n not in ("logits",) else v)
           for n, v in inp.items()}
    fwd, bwd = _run(inp, "softmax", "swiglu", 0.0, True, b2=False, store="bf16")
    np.testing.assert_array_equal(fwd["A"], rb(fwd["A_exact"]))
    np.testing.assert_array_equal(fwd["A_exact"], fwd["w_row"][:, None] * fwd["A_unscaled"])
    np.testing.assert_array_equal(bwd["dY"], inp["dout"][fwd["src_row"]])
    # a gate gradient from the unrounded H would differ
    f = inp["W2"].shape[2]
    H = fwd["H_exact"]
    a_exact = om.glu_forward(H[:, :f], H[:, f:])
    ds_exact = (bwd["dA"] * a_exact).sum(axis=1)[fwd["row_map"]]
    assert np.abs(bwd["dgate"] - ds_exact).max() > 0
    np.testing.assert_allclose(bwd["dgate"], ds_exact, rtol=1e-2, atol=1e-2)
