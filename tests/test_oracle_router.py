"""Pins of the oracle's router (logits = x Wr^T) and of its gradients inside
the layer: torch float64 autograd through a dense, token-by-token layer whose
logits come from the router, and central finite differences of the layer's
loss with respect to Wr and x (the input gradient then has the experts' share
and the router's)."""
import numpy as np
import pytest
import torch

from oracle import moe as om

F = torch.nn.functional


def _inputs(seed, T=17, d=12, f=8, E=5, k=2):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d))
    Wr = rng.standard_normal((E, d)) / np.sqrt(d)
    W1 = rng.standard_normal((E, 2 * f, d)) / np.sqrt(d)
    W2 = rng.standard_normal((E, d, f)) / np.sqrt(f)
    dout = rng.standard_normal((T, d))
    return x, Wr, W1, W2, dout, k


def _oracle(x, Wr, W1, W2, dout, k, score):
    spec = om.LayerSpec(k, score, True, "swiglu", store="f64")
    lg = om.router_logits(x, Wr)
    fwd = om.layer_forward(x, lg, W1, W2, spec=spec)
    bwd = om.layer_backward(fwd, dout, lg, W1, W2, spec=spec, router=(x, Wr))
    return fwd, bwd


def _torch_layer(x, Wr, W1, W2, dout, k, score):
    """The layer by definition, every token through its k experts, logits from
    the router; torch autograd for every gradient."""
    t = {n: torch.tensor(a, requires_grad=True) for n, a in
         dict(x=x, Wr=Wr, W1=W1, W2=W2).items()}
    logits = t["x"] @ t["Wr"].T
    _, idx = torch.topk(logits.detach(), k, dim=1)
    sel = logits.gather(1, idx)
    w = torch.softmax(sel, 1) if score == "softmax" else \
        torch.sigmoid(sel) / torch.sigmoid(sel).sum(1, keepdim=True)
    f = W2.shape[2]
    out = torch.zeros_like(t["x"])
    for j in range(k):
        W1e, W2e = t["W1"][idx[:, j]], t["W2"][idx[:, j]]        # per token
        h = torch.einsum("tnd,td->tn", W1e, t["x"])
        a = F.silu(h[:, :f]) * h[:, f:]
        out = out + w[:, j:j + 1] * torch.einsum("tdf,tf->td", W2e, a)
    (out * torch.tensor(dout)).sum().backward()
    return idx.numpy(), {n: v.grad.numpy() for n, v in t.items()}


@pytest.mark.parametrize("score", ["softmax", "sigmoid"])
def test_router_layer_gradients_match_torch_autograd(score):
    x, Wr, W1, W2, dout, k = _inputs(3)
    fwd, bwd = _oracle(x, Wr, W1, W2, dout, k, score)
    idx, g = _torch_layer(x, Wr, W1, W2, dout, k, score)
    np.testing.assert_array_equal(fwd["topk_idx"], idx)
    np.testing.assert_allclose(bwd["dWr"], g["Wr"], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(bwd["dX"], g["x"], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(bwd["dW1"], g["W1"], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(bwd["dW2"], g["W2"], rtol=1e-10, atol=1e-12)
    # the router's share of dx is not negligible here
    assert np.abs(bwd["dX_router"]).max() > 1e-2 * np.abs(bwd["dX_experts"]).max()


def test_router_layer_gradients_match_finite_differences():
    x, Wr, W1, W2, dout, k = _inputs(4, T=9, d=6, f=4, E=4)
    score = "sigmoid"
    _, bwd = _oracle(x, Wr, W1, W2, dout, k, score)

    def loss():
        spec = om.LayerSpec(k, score, True, "swiglu", store="f64")
        out = om.layer_forward(x, om.router_logits(x, Wr), W1, W2, spec=spec)["out"]
        return float((out * dout).sum())

    eps = 1e-6
    pick = np.random.default_rng(5)
    for name, p, grad in (("Wr", Wr, bwd["dWr"]), ("x", x, bwd["dX"])):
        flat, gflat = p.reshape(-1), grad.reshape(-1)
        for i in pick.choice(flat.size, size=12, replace=False):
            old = flat[i]
            flat[i] = old + eps
            lp = loss()
            flat[i] = old - eps
            lm = loss()
            flat[i] = old
            fd = (lp - lm) / (2 * eps)
            assert abs(gflat[i] - fd) <= 1e-6 * max(1.0, abs(fd)), (name, i, gflat[i], fd)


def test_router_logits_and_backward_definitions():
    """Closed forms on a hand-checkable case: one token, two experts."""
    x = np.array([[1.0, 2.0, -1.0]])
    Wr = np.array([[0.5, 0.0, 1.0], [-1.0, 1.0, 0.0]])
    np.testing.assert_array_equal(om.router_logits(x, Wr), [[-0.5, 1.0]])
    dWr, dx = om.router_backward(np.array([[2.0, -1.0]]), x, Wr)
    np.testing.assert_array_equal(dWr, [[2.0, 4.0, -2.0], [-1.0, -2.0, 1.0]])
    np.testing.assert_array_equal(dx, [[2.0, -1.0, 2.0]])
