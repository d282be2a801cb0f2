"""Pins of the CPU oracle against facts that do not come from the oracle itself:
library routines computing the same quantity by another route, brute force on
tiny inputs, closed forms, invariants and finite differences."""
import json
import math
import os

import numpy as np
import pytest
import torch

import synth
from oracle import moe as om

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- bf16 rounding

def test_round_bf16_matches_torch_cast():
    rng = np.random.default_rng(0)
    v = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-39).astype(np.float32),     # subnormal range
        (rng.standard_normal(2000) * 1e37).astype(np.float32),
        np.array([1 + 2**-8, 1 + 3 * 2**-8, -(1 + 2**-8), 3.3895314e38, 0.0, -0.0], np.float32),
    ])
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    got = om.round_bf16(v.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


def test_round_bf16_ties_to_even():
    assert om.round_bf16(1 + 2**-8) == 1.0
    assert om.round_bf16(1 + 3 * 2**-8) == 1 + 2**-6
    assert om.round_bf16(-(1 + 2**-8)) == -1.0


def test_generator_bf16_cast_matches_torch():
    rng = np.random.default_rng(1)
    v = rng.standard_normal(5000).astype(np.float32)
    bits = synth.f32_to_bf16_bits(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, ref)


# ---------------------------------------------------------------- routing

def _route_brute(logits, k):
    T, E = logits.shape
    idx = np.zeros((T, k), np.int64)
    for t in range(T):
        keyed = [(-(-math.inf if math.isnan(v) else float(v)), e) for e, v in enumerate(logits[t])]
        keyed.sort()
        idx[t] = [e for _, e in keyed[:k]]
    return idx


@pytest.mark.parametrize("E,k", [(8, 2), (5, 5), (16, 3), (1, 1)])
def test_route_topk_brute_force(E, k):
    rng = np.random.default_rng(E * 10 + k)
    lg = rng.standard_normal((64, E)).astype(np.float32)
    lg[::7, 0] = lg[::7, -1]          # exact ties
    lg = np.round(lg * 4) / 4           # many ties
    idx, w, nan = om.route_topk(lg, k)
    np.testing.assert_array_equal(idx, _route_brute(lg, k))
    assert not nan
    for t in range(64):
        assert len(set(idx[t].tolist())) == k
    np.testing.assert_allclose(w.sum(1), 1.0, atol=1e-12)


def test_route_tie_goes_to_lower_id():
    lg = np.array([[0.5, 1.0, 1.0, 1.0]], np.float32)
    idx, _, _ = om.route_topk(lg, 2)
    assert idx.tolist() == [[1, 2]]


def test_route_softmax_closed_form():
    lg = np.array([[2.0, 1.0, 0.0, -1.0]], np.float32)
    idx, w, _ = om.route_topk(lg, 2, "softmax", True)
    assert idx.tolist() == [[0, 1]]
    # e^2/(e^2+e^1) = 1/(1+e^-1) = 0.7310585786300049
    np.testing.assert_allclose(w[0], [0.7310585786300049, 0.2689414213699951], rtol=1e-15)


def test_route_gates_vs_torch():
    rng = np.random.default_rng(3)
    lg = rng.standard_normal((32, 12)).astype(np.float32)
    t = torch.from_numpy(lg).double()
    for k in (1, 4):
        idx, w, _ = om.route_topk(lg, k, "softmax", True)
        ii = torch.from_numpy(idx.astype(np.int64))
        full = torch.softmax(t, dim=1)
        ref = torch.gather(full, 1, ii)
        np.testing.assert_allclose(w, (ref / ref.sum(1, keepdim=True)).numpy(), rtol=1e-13)
        _, w0, _ = om.route_topk(lg, k, "softmax", False)
        np.testing.assert_allclose(w0, ref.numpy(), rtol=1e-13)
        _, ws, _ = om.route_topk(lg, k, "sigmoid", True)
        s = torch.gather(torch.sigmoid(t), 1, ii)
        np.testing.assert_allclose(ws, (s / s.sum(1, keepdim=True)).numpy(), rtol=1e-13)
        _, ws0, _ = om.route_topk(lg, k, "sigmoid", False)
        np.testing.assert_allclose(ws0, s.numpy(), rtol=1e-13)


def test_route_k_equals_E_and_nan():
    lg = np.array([[0.1, np.nan, -0.3], [1, 2, 3]], np.float32)
    idx, w, nan = om.route_topk(lg, 3)
    assert nan
    assert sorted(idx[0].tolist()) == [0, 1, 2]
    assert idx[0, -1] == 1            # NaN ranks last
    assert w[0, -1] == 0.0
    assert idx[1].tolist() == [2, 1, 0]


# Per-expert token counts of the seeded workloads, computed independently of
# this oracle (a separate simulation of the generator recipe and routing rule).
COUNT_PINS = {
    "tiny_fp32": [79, 63, 84, 84, 64, 73, 65, 0],
    "mixtral_fwd": [264, 363, 182, 1148, 710, 477, 3155, 1893],
    "gptoss_fwdbwd": [44, 31, 3216, 161, 34, 54, 411, 44, 533, 101, 20, 7526, 73, 246, 469, 325,
                      879, 665, 141, 1357, 5959, 4388, 53, 204, 242, 2405, 1076, 68, 1782, 94,
                      114, 53],
    "dsv3_fwdbwd": [15824, 0, 235, 5629, 412, 508, 6748, 276, 16352, 3897, 2299, 3161, 1025, 1466,
                    391, 1654, 4673, 9687, 755, 1247, 383, 14786, 8136, 919, 0, 594, 11310, 13035,
                    2792, 661, 283, 1934],
}


@pytest.mark.parametrize("name", sorted(COUNT_PINS))
def test_generator_count_pins(name):
    cfg = synth.WORKLOADS[name]
    lg = synth.draw_router(cfg)
    idx, w, _ = om.route_topk(lg, cfg.k, cfg.score, cfg.normalize)
    counts, offsets, _, _ = om.permute_indices(idx, cfg.E)
    assert counts.tolist() == COUNT_PINS[name]
    assert offsets[-1] == cfg.T * cfg.k


# ---------------------------------------------------------------- route backward

def _fd(fun, x, eps=1e-6):
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        xp = x.copy(); xp[i] += eps
        xm = x.copy(); xm[i] -= eps
        g[i] = (fun(xp) - fun(xm)) / (2 * eps)
    return g


@pytest.mark.parametrize("score", ["softmax", "sigmoid"])
@pytest.mark.parametrize("normalize", [True, False])
def test_route_bwd_finite_differences(score, normalize):
    rng = np.random.default_rng(5)
    T, E, k = 6, 7, 3
    lg = rng.standard_normal((T, E))
    idx, _, _ = om.route_topk(lg.astype(np.float32), k, score, normalize)
    dw = rng.standard_normal((T, k))
    lg64 = lg.astype(np.float32).astype(np.float64)

    def loss(l):
        sel = np.take_along_axis(l, idx.astype(np.int64), 1)
        return float((om.gates_from_logits(l, sel, score, normalize) * dw).sum())

    ref = _fd(loss, lg64)
    got = om.route_topk_bwd(lg64, idx, dw, score, normalize)
    np.testing.assert_allclose(got, ref, atol=1e-8)


def test_route_bwd_softmax_closed_form():
    # two selected experts with w = (p, 1-p): dl_0 = p (1-p) (dw_0 - dw_1) = -dl_1
    lg = np.array([[1.0, 0.0, -5.0]])
    dw = np.array([[1.0, 0.0]])
    got = om.route_topk_bwd(lg, np.array([[0, 1]]), dw, "softmax", True)
    p = 1 / (1 + math.exp(-1))
    np.testing.assert_allclose(got, [[p * (1 - p), -p * (1 - p), 0.0]], rtol=1e-14)


# ---------------------------------------------------------------- permute

def _permute_brute(idx, E):
    T, k = idx.shape
    rows = []
    for e in range(E):
        for t in range(T):
            for j in range(k):
                if idx[t, j] == e:
                    rows.append((t, j))
    row_map = np.zeros((T, k), np.int64)
    for r, (t, j) in enumerate(rows):
        row_map[t, j] = r
    return row_map, np.array([t for t, _ in rows])


@pytest.mark.parametrize("T,E,k", [(40, 6, 2), (33, 1, 1), (17, 9, 9), (50, 5, 1), (29, 3, 3)])
def test_permute_brute_force_and_invariants(T, E, k):
    rng = np.random.default_rng(T + E + k)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    if E > 2:
        lg[:, 1] -= 50        # expert 1 stays empty unless k forces it
    idx, _, _ = om.route_topk(lg, k)
    counts, offsets, row_map, src_row = om.permute_indices(idx, E)
    rm, sr = _permute_brute(idx, E)
    np.testing.assert_array_equal(row_map, rm)
    np.testing.assert_array_equal(src_row, sr)
    R = T * k
    assert counts.sum() == R and offsets[0] == 0 and offsets[-1] == R
    np.testing.assert_array_equal(np.diff(offsets), counts)
    assert sorted(row_map.ravel().tolist()) == list(range(R))          # bijection
    for t in range(T):
        for j in range(k):
            r = row_map[t, j]
            assert src_row[r] == t
            e = idx[t, j]
            assert offsets[e] <= r < offsets[e + 1]
    if E == 1:
        np.testing.assert_array_equal(row_map.ravel(), np.arange(R))
    # rows inside an expert ascend in (t, j)
    for e in range(E):
        seg = [(src_row[r], r) for r in range(offsets[e], offsets[e + 1])]
        assert seg == sorted(seg)


@pytest.mark.parametrize("k", [2, 4, 8])
def test_unit_unpermute_is_exact_multiple(k):
    cfg = synth.workload("tiny_fp32", T=64, d=32, E=16, k=k, dtype="bf16")
    inp = synth.make_inputs(cfg, parts=("x", "logits"))
    x = synth.as_f64(inp["x"], "bf16")
    idx, _, _ = om.route_topk(inp["logits"], k)
    _, _, row_map, src_row = om.permute_indices(idx, cfg.E)
    xp = om.gather_rows(x, src_row)
    np.testing.assert_array_equal(xp[row_map[:, 0]], x)
    s = om.combine(om.round_f32(xp), row_map, None)     # fp32-exact partial sums
    np.testing.assert_array_equal(om.round_bf16(s), k * x)


def test_pad_offsets():
    np.testing.assert_array_equal(om.pad_offsets([0, 1, 32, 33, 64]), [0, 0, 32, 64, 128, 192])


# ---------------------------------------------------------------- repack

def test_repack_layout_small():
    # f = 4, G = 2: one tile of width 2G sees G gate rows and G linear rows.
    f, G = 4, 2
    W = np.arange(2 * f)[None, :, None].astype(float)     # row i holds value i
    Wp = om.repack_glu(W, G=G)
    # canonical gate rows 0..3 = values 0..3, linear rows = values 4..7
    assert Wp[0, :, 0].tolist() == [0, 1, 4, 5, 2, 3, 6, 7]
    np.testing.assert_array_equal(om.unpack_glu(Wp, G=G), W)


@pytest.mark.parametrize("G", [32, 64])
def test_repack_roundtrip_and_gemm_equivalence(G):
    rng = np.random.default_rng(G)
    E, f, d = 3, 128, 16
    W = rng.standard_normal((E, 2 * f, d))
    b = rng.standard_normal((E, 2 * f))
    Wp, bp = om.repack_glu(W, b, G)
    W2, b2 = om.unpack_glu(Wp, bp, G)
    np.testing.assert_array_equal(W2, W)
    np.testing.assert_array_equal(b2, b)
    x = rng.standard_normal((5, d))
    h = x @ W[1].T
    hp = x @ Wp[1].T
    for c in range(f // G):
        np.testing.assert_array_equal(hp[:, 2 * G * c: 2 * G * c + G], h[:, G * c: G * c + G])
        np.testing.assert_array_equal(hp[:, 2 * G * c + G: 2 * G * c + 2 * G],
                                      h[:, f + G * c: f + G * c + G])


# ---------------------------------------------------------------- activations

def _golden():
    with open(os.path.join(GOLDEN, "closed_forms.json")) as fh:
        return json.load(fh)


def test_activation_closed_forms():
    g = _golden()
    for x, v in g["silu"]:
        assert om.act_fn(x, "swiglu") == pytest.approx(v, rel=1e-15, abs=1e-300)
    for x, v in g["silu_grad"]:
        assert om.act_grad(x, "swiglu") == pytest.approx(v, rel=1e-15)
    for x, v in g["gelu"]:
        assert om.act_fn(x, "geglu") == pytest.approx(v, rel=1e-15, abs=1e-300)
    for x, v in g["gelu_grad"]:
        assert om.act_grad(x, "geglu") == pytest.approx(v, rel=1e-15)
    for x, v in g["srelu"]:
        assert om.act_fn(x, "srelu") == v
    for x, v in g["srelu_grad"]:
        assert om.act_grad(x, "srelu") == v
    s = g["swiglu_gate1_lin2"]
    assert om.glu_forward(1.0, 2.0) == pytest.approx(s["value"], rel=1e-15)
    dg, dl = om.glu_backward(1.0, 1.0, 2.0)
    assert dg == pytest.approx(s["d_gate"], rel=1e-15)
    assert dl == pytest.approx(s["d_lin"], rel=1e-15)


def test_activations_vs_torch():
    x = np.linspace(-6, 6, 241)
    t = torch.from_numpy(x)
    np.testing.assert_allclose(om.act_fn(x, "swiglu"), torch.nn.functional.silu(t).numpy(), rtol=1e-14, atol=1e-300)
    np.testing.assert_allclose(om.act_fn(x, "swiglu", alpha=1.702), (t * torch.sigmoid(1.702 * t)).numpy(), rtol=1e-14)
    from scipy.special import ndtr      # standard normal CDF, computed without cancellation
    np.testing.assert_allclose(om.act_fn(x, "geglu"), x * ndtr(x), rtol=1e-14, atol=1e-300)
    np.testing.assert_allclose(om.act_fn(x, "geglu"), torch.nn.functional.gelu(t).numpy(), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(om.act_fn(x, "geglu", gelu_tanh=True),
                               torch.nn.functional.gelu(t, approximate="tanh").numpy(), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(om.act_fn(x, "srelu"), (torch.relu(t) ** 2).numpy())


@pytest.mark.parametrize("act,alpha,tanh", [("swiglu", 1.0, False), ("swiglu", 1.702, False),
                                            ("geglu", 1.0, False), ("geglu", 1.0, True),
                                            ("srelu", 1.0, False)])
def test_activation_derivatives_finite_differences(act, alpha, tanh):
    x = np.linspace(-5, 5, 101) + 0.013
    eps = 1e-6
    fd = (om.act_fn(x + eps, act, alpha, tanh) - om.act_fn(x - eps, act, alpha, tanh)) / (2 * eps)
    np.testing.assert_allclose(om.act_grad(x, act, alpha, tanh), fd, rtol=1e-7, atol=1e-8)


def test_clamp_semantics():
    # gate 9 clamps to 7 with zero gate gradient; lin 9 clamps to 7 with zero lin gradient
    assert om.glu_forward(9.0, 1.0, clamp=7.0) == pytest.approx(6.993622641639195, rel=1e-15)
    dg, dl = om.glu_backward(1.0, 9.0, 1.0, clamp=7.0)
    assert dg == 0.0 and dl == pytest.approx(6.993622641639195, rel=1e-15)
    assert om.glu_forward(1.0, 9.0, clamp=7.0) == pytest.approx(7 * 0.7310585786300049, rel=1e-15)
    dg, dl = om.glu_backward(1.0, 1.0, -9.0, clamp=7.0)
    assert dl == 0.0 and dg == pytest.approx(-7 * 0.9276705118714869, rel=1e-15)
    # gate below the limit is untouched (one-sided clamp of the gate)
    assert om.glu_forward(-9.0, 1.0, clamp=7.0) == pytest.approx(float(om.act_fn(-9.0, "swiglu")), rel=1e-15)
