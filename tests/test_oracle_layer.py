"""Pins of the oracle's whole-layer chain: the grouped formulation against the
token-by-token definition, special cases that reduce to a dense MLP (checked
with torch float64), invariants, and finite-difference / autograd gradients."""
import numpy as np
import pytest
import torch

from oracle import moe as om


def _rand_layer(rng, T, d, f, E, k, act="swiglu", bias=True):
    n1 = 2 * f if act != "srelu" else f
    x = rng.standard_normal((T, d))
    lg = rng.standard_normal((T, E)).astype(np.float32)
    W1 = rng.standard_normal((E, n1, d)) / np.sqrt(d)
    W2 = rng.standard_normal((E, d, f)) / np.sqrt(f)
    b1 = rng.standard_normal((E, n1)) * 0.3 if bias else None
    b2 = rng.standard_normal((E, d)) * 0.3 if bias else None
    return x, lg, W1, W2, b1, b2


CASES = [
    dict(act="swiglu", score="softmax", clamp=0.0, alpha=1.0),
    dict(act="swiglu", score="sigmoid", clamp=1.5, alpha=1.0),
    dict(act="swiglu", score="softmax", clamp=0.0, alpha=1.702),
    dict(act="geglu", score="softmax", clamp=0.0, alpha=1.0),
    dict(act="srelu", score="sigmoid", clamp=0.0, alpha=1.0),
]


@pytest.mark.parametrize("case", CASES)
def test_grouped_equals_definition(case):
    rng = np.random.default_rng(11)
    T, d, f, E, k = 23, 12, 8, 5, 2
    x, lg, W1, W2, b1, b2 = _rand_layer(rng, T, d, f, E, k, case["act"])
    spec = om.LayerSpec(k, case["score"], True, case["act"], case["clamp"], case["alpha"], store="f64")
    fwd = om.layer_forward(x, lg, W1, W2, b1, b2, spec=spec)
    ref = om.ffn_dense(x, lg, W1, W2, b1, b2, k=k, score=case["score"], act=case["act"],
                       clamp=case["clamp"], alpha=case["alpha"])
    np.testing.assert_allclose(fwd["out"], ref, rtol=1e-12, atol=1e-12)


def test_single_expert_is_dense_mlp_torch():
    rng = np.random.default_rng(12)
    T, d, f = 19, 16, 24
    x, lg, W1, W2, b1, b2 = _rand_layer(rng, T, d, f, 1, 1)
    spec = om.LayerSpec(1, store="f64")
    fwd = om.layer_forward(x, lg, W1, W2, b1, b2, spec=spec)
    F = torch.nn.functional
    xt = torch.from_numpy(x)
    h = F.linear(xt, torch.from_numpy(W1[0]), torch.from_numpy(b1[0]))
    a = F.silu(h[:, :f]) * h[:, f:]
    y = F.linear(a, torch.from_numpy(W2[0]), torch.from_numpy(b2[0]))
    np.testing.assert_allclose(fwd["out"], y.numpy(), rtol=1e-12, atol=1e-13)
    assert np.all(fwd["topk_w"] == 1.0)


def test_identical_experts_make_routing_irrelevant():
    rng = np.random.default_rng(13)
    T, d, f, E, k = 31, 8, 16, 6, 3
    x, lg, W1, W2, b1, b2 = _rand_layer(rng, T, d, f, E, k)
    W1[:] = W1[0]; W2[:] = W2[0]; b1[:] = b1[0]; b2[:] = b2[0]
    spec = om.LayerSpec(k, "sigmoid", store="f64")
    out = om.layer_forward(x, lg, W1, W2, b1, b2, spec=spec)["out"]
    lg2 = rng.standard_normal(lg.shape).astype(np.float32)
    out2 = om.layer_forward(x, lg2, W1, W2, b1, b2, spec=spec)["out"]
    np.testing.assert_allclose(out, out2, rtol=1e-12, atol=1e-12)


def test_empty_expert_rows_untouched_and_zero_grads():
    rng = np.random.default_rng(14)
    T, d, f, E, k = 20, 8, 8, 4, 2
    x, lg, W1, W2, b1, b2 = _rand_layer(rng, T, d, f, E, k)
    lg[:, 2] = -100.0
    spec = om.LayerSpec(k, store="f64")
    fwd = om.layer_forward(x, lg, W1, W2, b1, b2, spec=spec)
    assert fwd["counts"][2] == 0
    W1b = W1.copy(); W1b[2] += 1000.0
    out2 = om.layer_forward(x, lg, W1b, W2, b1, b2, spec=spec)["out"]
    np.testing.assert_array_equal(out2, fwd["out"])
    bwd = om.layer_backward(fwd, rng.standard_normal((T, d)), lg, W1, W2, spec=spec, has_bias=True)
    assert np.all(bwd["dW1"][2] == 0) and np.all(bwd["dW2"][2] == 0)
    assert np.all(bwd["db1"][2] == 0) and np.all(bwd["db2"][2] == 0)


def _loss_fn(x, lg, W1, W2, b1, b2, dout, spec):
    return float((om.layer_forward(x, lg, W1, W2, b1, b2, spec=spec)["out"] * dout).sum())


@pytest.mark.parametrize("case", CASES)
def test_backward_finite_differences(case):
    rng = np.random.default_rng(21)
    T, d, f, E, k = 9, 6, 4, 4, 2
    x, lg, W1, W2, b1, b2 = _rand_layer(rng, T, d, f, E, k, case["act"])
    lg = lg.astype(np.float64)
    spec = om.LayerSpec(k, case["score"], True, case["act"], case["clamp"], case["alpha"], store="f64")
    dout = rng.standard_normal((T, d))
    fwd = om.layer_forward(x, lg, W1, W2, b1, b2, spec=spec)
    bwd = om.layer_backward(fwd, dout, lg, W1, W2, spec=spec, has_bias=True)
    n1 = W1.shape[1]
    eps = 1e-6
    params = dict(x=x, W1=W1, W2=W2, b1=b1, b2=b2, lg=lg)
    grads = dict(x=bwd["dX"], W1=bwd["dW1"], W2=bwd["dW2"], b1=bwd["db1"], b2=bwd["db2"],
                 lg=bwd["dlogits"])
    pick = np.random.default_rng(3)
    for name, p in params.items():
        flat = p.reshape(-1)
        for i in pick.choice(flat.size, size=min(12, flat.size), replace=False):
            old = flat[i]
            flat[i] = old + eps
            lp = _loss_fn(x, lg, W1, W2, b1, b2, dout, spec)
            flat[i] = old - eps
            lm = _loss_fn(x, lg, W1, W2, b1, b2, dout, spec)
            flat[i] = old
            fd = (lp - lm) / (2 * eps)
            g = grads[name].reshape(-1)[i]
            assert abs(g - fd) <= 1e-6 * max(1.0, abs(fd)), (name, i, g, fd)
    assert n1 == (2 * f if case["act"] != "srelu" else f)


def test_backward_adjoint_identity():
    rng = np.random.default_rng(22)
    T, d, f, E, k = 11, 8, 8, 3, 2
    x, lg, W1, W2, b1, b2 = _rand_layer(rng, T, d, f, E, k)
    spec = om.LayerSpec(k, "sigmoid", store="f64")
    dout = rng.standard_normal((T, d))
    fwd = om.layer_forward(x, lg, W1, W2, b1, b2, spec=spec)
    bwd = om.layer_backward(fwd, dout, lg, W1, W2, spec=spec, has_bias=True)
    v = dict(x=rng.standard_normal(x.shape), W1=rng.standard_normal(W1.shape),
             W2=rng.standard_normal(W2.shape))
    eps = 1e-6

    def out_at(s):
        return om.layer_forward(x + s * v["x"], lg, W1 + s * v["W1"], W2 + s * v["W2"], b1, b2,
                                spec=spec)["out"]

    jv = (out_at(eps) - out_at(-eps)) / (2 * eps)
    lhs = float((dout * jv).sum())
    rhs = float((bwd["dX"] * v["x"]).sum() + (bwd["dW1"] * v["W1"]).sum() + (bwd["dW2"] * v["W2"]).sum())
    assert lhs == pytest.approx(rhs, rel=1e-7)


def test_single_expert_backward_vs_torch_autograd():
    rng = np.random.default_rng(23)
    T, d, f = 13, 10, 12
    x, lg, W1, W2, b1, b2 = _rand_layer(rng, T, d, f, 1, 1)
    spec = om.LayerSpec(1, clamp=0.8, store="f64")
    dout = rng.standard_normal((T, d))
    fwd = om.layer_forward(x, lg, W1, W2, b1, b2, spec=spec)
    bwd = om.layer_backward(fwd, dout, lg, W1, W2, spec=spec, has_bias=True)
    t = {n: torch.tensor(a, requires_grad=True) for n, a in
         dict(x=x, W1=W1[0], W2=W2[0], b1=b1[0], b2=b2[0]).items()}
    F = torch.nn.functional
    h = F.linear(t["x"], t["W1"], t["b1"])
    gate = torch.clamp(h[:, :f], max=0.8)
    lin = torch.clamp(h[:, f:], -0.8, 0.8)
    y = F.linear(F.silu(gate) * lin, t["W2"], t["b2"])
    y.backward(torch.from_numpy(dout))
    np.testing.assert_allclose(bwd["dX"], t["x"].grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(bwd["dW1"][0], t["W1"].grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(bwd["dW2"][0], t["W2"].grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(bwd["db1"][0], t["b1"].grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(bwd["db2"][0], t["b2"].grad.numpy(), rtol=1e-11, atol=1e-12)


def test_storage_rounding_points():
    rng = np.random.default_rng(24)
    T, d, f, E, k = 16, 8, 8, 3, 2
    x, lg, W1, W2, b1, b2 = _rand_layer(rng, T, d, f, E, k)
    x = om.round_bf16(x)
    spec = om.LayerSpec(k, store="bf16")
    fwd = om.layer_forward(x, lg, W1, W2, b1, b2, spec=spec)
    for name in ("H", "A", "Y", "out"):
        np.testing.assert_array_equal(fwd[name], om.round_bf16(fwd[name]))
    # Y is computed from the rounded A, not from the exact one
    Yref = om.grouped_linear(fwd["A"], W2, fwd["offsets"], b2)
    np.testing.assert_array_equal(fwd["Y_exact"], Yref)


def test_norm_max_err():
    assert om.norm_max_err([1.0, -1.0], [1.0, -1.0]) == 0.0
    assert om.norm_max_err([1.1, -1.0], [1.0, -1.0]) == pytest.approx(0.1)
