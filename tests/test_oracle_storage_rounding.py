"""Pins of the oracle chain's storage rounding, forward and backward.

The layer stores H, A, Y and out in the forward and dY, dH, dXp and dX in the
backward in its activation dtype (bf16, or float32 for the tiny workload);
every product downstream of a stored tensor reads the stored value, and the
dGLU of the backward is evaluated at the stored (rounded) H ([P1]
"融合された GEMM エピローグによる GLU 活性化関数の最適化": the backward epilogue
reads the pre-activation the forward kept).  The oracle's ``layer_forward`` /
``layer_backward`` with ``store="bf16"`` or ``"f32"`` implement that chain.

Here the same chain is written a second, independent way: torch float64
autograd through the dense per-expert products, with torch's own bf16 /
float32 casts applied by straight-through functions at the storage points
(value rounded, gradient passed on; or value passed on, gradient rounded).
Routing is torch.topk, the expert-contiguous order a stable torch.sort.  The
two must agree to float64 rounding, and for every storage point a variant of
the torch chain that skips it must disagree -- so each rounding point of the
oracle is pinned by something other than itself.
"""
import numpy as np
import pytest
import torch

from oracle import moe as om

F = torch.nn.functional


def _cast(store):
    dt = torch.bfloat16 if store == "bf16" else torch.float32
    return lambda t: t.to(dt).to(torch.float64)


class _GradRound(torch.autograd.Function):
    """Identity on the value; the incoming gradient is rounded to the storage type."""

    @staticmethod
    def forward(ctx, x, store):
        ctx.store = store
        return x.clone()

    @staticmethod
    def backward(ctx, g):
        return _cast(ctx.store)(g), None


def _value_round(x, store):
    """The value rounded to the storage type; the gradient passes unchanged."""
    return x + (_cast(store)(x) - x).detach()


def _act(h, f, act, clamp, alpha):
    if act == "srelu":
        hh = torch.clamp(h, max=clamp) if clamp > 0 else h
        return torch.relu(hh) ** 2
    g, lin = h[:, :f], h[:, f:]
    if clamp > 0:
        g = torch.clamp(g, max=clamp)
        lin = torch.clamp(lin, -clamp, clamp)
    a = g * torch.sigmoid(alpha * g) if act == "swiglu" else F.gelu(g)
    return a * lin


SKIP = (None, "H", "A_from_H", "dGLU_at_H", "A", "Y", "dY", "dH", "dXp")


def torch_chain(x, lg, W1, W2, b1, b2, dout, *, k, score, act, clamp, alpha, store, skip=None):
    """The layer forward + backward by torch autograd with rounding at the
    storage points.  ``skip`` names one storage point to leave out (for the
    sensitivity checks): "H" (H stored unrounded), "A_from_H" (A computed from
    the rounded H), "dGLU_at_H" (dGLU evaluated at the exact H), "A", "Y",
    "dY", "dH", "dXp"."""
    rnd = _cast(store)
    t64 = lambda a: torch.tensor(np.asarray(a, dtype=np.float64))
    xt = t64(x).requires_grad_(True)
    lgt = t64(np.asarray(lg, dtype=np.float32)).requires_grad_(True)
    W1t, W2t = t64(W1).requires_grad_(True), t64(W2).requires_grad_(True)
    b1t = t64(b1).requires_grad_(True) if b1 is not None else None
    b2t = t64(b2).requires_grad_(True) if b2 is not None else None
    E, n1, d = W1.shape
    f = W2.shape[2]
    T = x.shape[0]
    # routing: top-k by logit (descending), gates from the selected logits
    sel, idx = torch.topk(lgt.detach(), k, dim=1, largest=True, sorted=True)
    lsel = lgt.gather(1, idx)
    if score == "softmax":
        w = torch.softmax(lsel, dim=1)
    else:
        s = torch.sigmoid(lsel)
        w = s / s.sum(dim=1, keepdim=True)
    # expert-contiguous rows: stable sort of the flat assignments by expert
    flat = idx.reshape(-1)
    order = torch.sort(flat, stable=True).indices          # row r <- assignment order[r]
    src = order // k
    row_of = torch.empty_like(order)
    row_of[order] = torch.arange(order.numel())
    counts = torch.bincount(flat, minlength=E)
    bounds = [0] + torch.cumsum(counts, 0).tolist()
    Xp = xt[src]
    if skip != "dXp":
        Xp = _GradRound.apply(Xp, store)
    Hraw = torch.cat([Xp[bounds[e]:bounds[e + 1]] @ W1t[e].T +
                      (b1t[e] if b1t is not None else 0.0) for e in range(E)])
    H = Hraw if skip == "dH" else _GradRound.apply(Hraw, store)
    Hs = H if skip == "H" else _value_round(H, store)        # the stored H
    # A's value from the exact H; its derivative (dGLU) at the stored H
    a_grad = _act(H if skip == "dGLU_at_H" else Hs, f, act, clamp, alpha)
    a_val = _act((Hs if skip == "A_from_H" else H).detach(), f, act, clamp, alpha)
    A = a_grad + (a_val - a_grad).detach()
    As = A if skip == "A" else _value_round(A, store)
    Yraw = torch.cat([As[bounds[e]:bounds[e + 1]] @ W2t[e].T +
                      (b2t[e] if b2t is not None else 0.0) for e in range(E)])
    Ys = Yraw if skip == "Y" else _value_round(Yraw, store)
    Yg = Ys if skip == "dY" else _GradRound.apply(Ys, store)
    rows = row_of.reshape(T, k)
    out = sum(w[:, j:j + 1] * Yg[rows[:, j]] for j in range(k))
    # keep the gradients of the stored tensors
    grads = {}
    # (the gradient at Ys is dY after its rounding; at Hraw, dH after its rounding)
    for name, tns in (("dY", Ys), ("dH", Hraw)):
        tns.register_hook(lambda g, name=name: grads.__setitem__(name, g.detach().clone()))
    out.backward(t64(dout))
    res = dict(idx=idx.numpy(), row_map=rows.numpy(), H=Hs.detach().numpy(),
               A=As.detach().numpy(), Y=Ys.detach().numpy(), out=rnd(out.detach()).numpy(),
               dX=rnd(xt.grad).numpy(), dW1=W1t.grad.numpy(), dW2=W2t.grad.numpy(),
               dlogits=lgt.grad.numpy())
    res["dY"] = grads["dY"].numpy()
    res["dH"] = grads["dH"].numpy()
    if b1t is not None:
        res["db1"] = b1t.grad.numpy()
        res["db2"] = b2t.grad.numpy()
    return res


CASES = [
    dict(store="bf16", score="softmax", act="swiglu", clamp=0.9, alpha=1.0, bias=True),
    dict(store="bf16", score="sigmoid", act="geglu", clamp=0.0, alpha=1.0, bias=False),
    dict(store="bf16", score="sigmoid", act="srelu", clamp=0.0, alpha=1.0, bias=True),
    dict(store="f32", score="softmax", act="swiglu", clamp=0.0, alpha=1.702, bias=True),
]


def _inputs(case, seed=5):
    rng = np.random.default_rng(seed)
    T, d, f, E, k = 40, 24, 16, 5, 2
    n1 = f if case["act"] == "srelu" else 2 * f
    cast = _cast(case["store"])
    r = lambda *s: cast(torch.tensor(rng.standard_normal(s))).numpy()
    x = r(T, d)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    W1 = r(E, n1, d) / 4.0
    W2 = r(E, d, f) / 4.0
    b1 = r(E, n1) * 0.3 if case["bias"] else None
    b2 = r(E, d) * 0.3 if case["bias"] else None
    dout = r(T, d)
    return dict(x=x, lg=lg, W1=W1, W2=W2, b1=b1, b2=b2, dout=dout, k=k)


def _oracle(case, inp):
    spec = om.LayerSpec(inp["k"], case["score"], True, case["act"], case["clamp"], case["alpha"],
                        store=case["store"])
    fwd = om.layer_forward(inp["x"], inp["lg"], inp["W1"], inp["W2"], inp["b1"], inp["b2"],
                           spec=spec)
    bwd = om.layer_backward(fwd, inp["dout"], inp["lg"], inp["W1"], inp["W2"], spec=spec,
                            has_bias=case["bias"])
    return fwd, bwd


def _compare(fwd, bwd, ref):
    """Largest relative difference over every stored tensor and gradient."""
    pairs = dict(H=fwd["H"], A=fwd["A"], Y=fwd["Y"], out=fwd["out"], dX=bwd["dX"],
                 dW1=bwd["dW1"], dW2=bwd["dW2"], dlogits=bwd["dlogits"], dY=bwd["dY"],
                 dH=bwd["dH"])
    if "db1" in ref:
        pairs.update(db1=bwd["db1"], db2=bwd["db2"])
    worst = {}
    for name, o in pairs.items():
        if name not in ref:
            continue
        g = ref[name]
        scale = max(float(np.max(np.abs(o))), 1e-300)
        worst[name] = float(np.max(np.abs(g - o))) / scale
    return worst


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c['store']}-{c['act']}-{c['score']}")
def test_oracle_storage_rounding_matches_torch_autograd(case):
    inp = _inputs(case)
    fwd, bwd = _oracle(case, inp)
    ref = torch_chain(inp["x"], inp["lg"], inp["W1"], inp["W2"], inp["b1"], inp["b2"],
                      inp["dout"], k=inp["k"], score=case["score"], act=case["act"],
                      clamp=case["clamp"], alpha=case["alpha"], store=case["store"])
    np.testing.assert_array_equal(ref["idx"], fwd["topk_idx"])
    np.testing.assert_array_equal(ref["row_map"], fwd["row_map"])
    worst = _compare(fwd, bwd, ref)
    bad = {n: v for n, v in worst.items() if v > 1e-12}
    assert not bad, worst
    # every stored tensor is representable in the storage type
    cast = _cast(case["store"])
    for name, v in (("H", fwd["H"]), ("A", fwd["A"]), ("Y", fwd["Y"]), ("out", fwd["out"]),
                    ("dY", bwd["dY"]), ("dH", bwd["dH"]), ("dXp", bwd["dXp"]), ("dX", bwd["dX"])):
        t = torch.tensor(v)
        assert torch.equal(cast(t), t), name


@pytest.mark.parametrize("skip", [s for s in SKIP if s is not None])
@pytest.mark.parametrize("case", [CASES[0], CASES[3]], ids=["bf16", "f32"])
def test_each_rounding_point_is_observable(case, skip):
    """Leaving any one storage point out of the torch chain moves some
    compared tensor well beyond float64 rounding: the comparison above pins
    every rounding point of the oracle, forward and backward."""
    inp = _inputs(case)
    fwd, bwd = _oracle(case, inp)
    ref = torch_chain(inp["x"], inp["lg"], inp["W1"], inp["W2"], inp["b1"], inp["b2"],
                      inp["dout"], k=inp["k"], score=case["score"], act=case["act"],
                      clamp=case["clamp"], alpha=case["alpha"], store=case["store"], skip=skip)
    worst = _compare(fwd, bwd, ref)
    assert max(worst.values()) > 1e-9, (skip, worst)
