"""Parity at the workloads' full sizes, in the launch configuration bench.py
times (MoEFFN, eager, default tile choice and grid).

The full oracle chain is too slow at these sizes, so the oracle computes
sampled outputs one at a time, following the same chain (fp64 arithmetic,
the library's storage rounding at H, A, Y, dY, dH, dXp):
  * whole output rows out[t], dX[t], dgate[t], dlogits[t] for sampled tokens,
    including tokens routed to the heaviest and to the lightest expert;
  * whole weight-gradient slices: dW2[e][:, j] and the packed dW1 rows of the
    gate and linear halves of column j, db1/db2 where present, for the
    heaviest, a light and a random expert;
  * exact zeros for every empty expert's weight gradients;
  * routing, counts and offsets bit-exact over all tokens.
Tolerances as in test_gpu_layer: bf16 outputs by max error beyond their own
half-ulp / rms <= 2e-2, float32 gradients max |err| / rms <= 2e-2, both
normalised by the rms of the sampled reference values."""

import numpy as np
import pytest
import torch

import synth
from oracle import moe as om
from gpu_util import bf16_excess, host, norm_err, note

pytestmark = [pytest.mark.gpu, pytest.mark.slow]
G = 32


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from ragged_grouped_gemm_amd import ops
    ops.moe_version()


def _f32(a):
    return synth.bf16_bits_to_f32(a) if a.dtype == np.uint16 else np.asarray(a, np.float32)


class Chain:
    """The oracle chain evaluated row by row for chosen tokens / experts."""

    def __init__(self, cfg, inp, fwd_idx, fwd_w):
        self.cfg = cfg
        self.x = _f32(inp["x"])
        self.W1 = _f32(inp["W1"])
        self.W2 = _f32(inp["W2"])
        self.b1 = inp.get("b1") if cfg.bias else None
        self.b2 = inp.get("b2") if cfg.bias else None
        self.dout = _f32(inp["dOut"]) if cfg.backward else None
        self.idx = fwd_idx
        self.w = fwd_w
        self.rnd = om.round_bf16 if cfg.dtype == "bf16" else om.round_f32
        self.f = cfg.f

    def expert_rows(self, xs, e):
        """H (exact), H stored, A exact, A stored for rows xs [n, d] on expert e."""
        W1 = self.W1[e].astype(np.float64)
        H = xs.astype(np.float64) @ W1.T
        if self.b1 is not None:
            H += self.b1[e]
        f = self.f
        A = om.glu_forward(H[:, :f], H[:, f:], self.cfg.act, self.cfg.clamp, self.cfg.alpha)
        return H, self.rnd(H), A, self.rnd(A)

    def token(self, t):
        """out[t] (exact, before its final rounding) and, with backward, dX[t], dgate[t], dlogits[t]."""
        cfg, f = self.cfg, self.f
        Ys, Hs = [], []
        for j in range(cfg.k):
            e = int(self.idx[t, j])
            _, H_s, _, A_s = self.expert_rows(self.x[t:t + 1], e)
            Y = A_s @ self.W2[e].astype(np.float64).T
            if self.b2 is not None:
                Y += self.b2[e]
            Ys.append(self.rnd(Y)[0])
            Hs.append(H_s[0])
        out = sum(self.w[t, j] * Ys[j] for j in range(cfg.k))
        res = {"out": out}
        if not cfg.backward:
            return res
        g = self.dout[t].astype(np.float64)
        dX = np.zeros(cfg.d)
        dgate = np.zeros(cfg.k)
        for j in range(cfg.k):
            e = int(self.idx[t, j])
            dY = self.rnd(self.w[t, j] * g)
            dgate[j] = float(g @ Ys[j])
            dA = dY @ self.W2[e].astype(np.float64)
            dg, dl = om.glu_backward(dA, Hs[j][:f], Hs[j][f:], cfg.act, cfg.clamp, cfg.alpha)
            dH = self.rnd(np.concatenate([dg, dl]))
            dX += self.rnd(dH @ self.W1[e].astype(np.float64))
        res["dX"] = dX
        res["dgate"] = dgate
        return res


def _run(name):
    cfg = synth.WORKLOADS[name]
    note(f"full-size {name}: T={cfg.T} d={cfg.d} f={cfg.f} E={cfg.E} k={cfg.k}")
    from ragged_grouped_gemm_amd import ops
    from ragged_grouped_gemm_amd.layer import MoEFFN
    inp = synth.make_inputs(cfg)
    t = lambda a: synth.to_torch(a, "cuda")
    x, lg, W2 = t(inp["x"]), t(inp["logits"]), t(inp["W2"])
    W1p, b1p = ops.moe_repack_glu_weights(t(inp["W1"]), t(inp["b1"]) if cfg.bias else None)
    b2 = t(inp["b2"]) if cfg.bias else None
    dout = t(inp["dOut"]) if cfg.backward else None
    L = MoEFFN(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, act=cfg.act, score=cfg.score,
               normalize=cfg.normalize, clamp=cfg.clamp, alpha=cfg.alpha, bias=cfg.bias,
               backward=cfg.backward)
    L.forward(x, lg, W1p, W2, b1p, b2)
    if cfg.backward:
        L.backward(dout, lg, W1p, W2)
    torch.cuda.synchronize()
    return cfg, inp, L


def _check_routing(cfg, inp, L):
    idx, w, _ = om.route_topk(inp["logits"], cfg.k, cfg.score, cfg.normalize)
    counts, offsets, row_map, _ = om.permute_indices(idx, cfg.E)
    np.testing.assert_array_equal(host(L.topk_idx), idx)
    np.testing.assert_array_equal(host(L.counts), counts)
    np.testing.assert_array_equal(host(L.offsets), offsets)
    np.testing.assert_array_equal(host(L.row_map), row_map)
    return idx, w, counts, offsets, row_map


def _sample_tokens(idx, counts, n_random, seed):
    heavy = int(np.argmax(counts))
    nz = [e for e in range(len(counts)) if counts[e] > 0]
    light = min(nz, key=lambda e: counts[e])
    toks = [int(np.nonzero((idx == heavy).any(1))[0][0]), int(np.nonzero((idx == light).any(1))[0][-1])]
    rng = np.random.default_rng(seed)
    toks += [int(v) for v in rng.choice(idx.shape[0], size=n_random, replace=False)]
    return sorted(set(toks)), heavy, light


def _check_tokens(cfg, inp, L, idx, w, toks):
    ch = Chain(cfg, inp, idx, w)
    got_out = host(L.out)[toks]
    ref = [ch.token(tk) for tk in toks]
    ref_out = np.stack([r["out"] for r in ref])
    e_out = bf16_excess(got_out, ref_out)
    report = {"out": e_out, "out_raw": norm_err(got_out, ref_out)}
    assert e_out <= 2e-2, report
    if cfg.backward:
        ref_dx = np.stack([r["dX"] for r in ref])
        e_dx = bf16_excess(host(L.dX)[toks], ref_dx)
        report["dX"] = e_dx
        assert e_dx <= 2e-2, report
        ref_dg = np.stack([r["dgate"] for r in ref])
        e_dg = norm_err(host(L.dgate)[toks], ref_dg)
        report["dgate"] = e_dg
        assert e_dg <= 2e-2, report
        lg64 = inp["logits"][toks].astype(np.float64)
        ref_dl = om.route_topk_bwd(lg64, idx[toks], ref_dg, cfg.score, cfg.normalize)
        e_dl = norm_err(host(L.dlogits)[toks], ref_dl)
        report["dlogits"] = e_dl
        assert e_dl <= 2e-2, report
    return report


def _check_weight_grads(cfg, inp, L, idx, w, counts, offsets, row_map, experts, cols):
    """dW2[e][:, j], packed dW1 rows of column j (gate and linear), db's."""
    ch = Chain(cfg, inp, idx, w)
    f = cfg.f
    T, k = idx.shape
    src = np.empty(T * k, np.int64)
    src[row_map.reshape(-1)] = np.repeat(np.arange(T), k)
    wflat = np.empty(T * k)
    wflat[row_map.reshape(-1)] = w.reshape(-1)
    dW1 = L.dW1p
    dW2 = L.dW2
    pos = om.glu_pack_rows(f, G)
    report = {}
    db1_got, db1_ref = [], []
    for e in experts:
        s, u = int(offsets[e]), int(offsets[e + 1])
        if u == s:
            continue
        rows = src[s:u]
        xs = ch.x[rows]
        dY = ch.rnd(wflat[s:u, None] * ch.dout[rows].astype(np.float64))
        W1e = ch.W1[e].astype(np.float64)
        W2e = ch.W2[e].astype(np.float64)
        for j in cols:
            hg = xs.astype(np.float64) @ W1e[j]
            hl = xs.astype(np.float64) @ W1e[f + j]
            if ch.b1 is not None:
                hg = hg + ch.b1[e][j]
                hl = hl + ch.b1[e][f + j]
            a_s = ch.rnd(om.glu_forward(hg, hl, cfg.act, cfg.clamp, cfg.alpha))
            ref_dw2 = dY.T @ a_s                                    # dW2[e][:, j]
            got_dw2 = dW2[e, :, j].detach().cpu().numpy().astype(np.float64)
            dA = dY @ W2e[:, j]
            dg, dl = om.glu_backward(dA, ch.rnd(hg), ch.rnd(hl), cfg.act, cfg.clamp, cfg.alpha)
            dg_s, dl_s = ch.rnd(dg), ch.rnd(dl)
            ref_dw1g = dg_s @ xs.astype(np.float64)
            ref_dw1l = dl_s @ xs.astype(np.float64)
            got_dw1g = dW1[e, int(pos[j])].detach().cpu().numpy().astype(np.float64)
            got_dw1l = dW1[e, int(pos[f + j])].detach().cpu().numpy().astype(np.float64)
            for lab, g_, r_ in (("dW2", got_dw2, ref_dw2), ("dW1g", got_dw1g, ref_dw1g),
                                ("dW1l", got_dw1l, ref_dw1l)):
                err = norm_err(g_, r_)
                report[f"{lab}[{e},{j}]"] = err
                assert err <= 2e-2, (lab, e, j, err)
            if cfg.bias:
                db1_got += L.db1p[e, [int(pos[j]), int(pos[f + j])]].detach().cpu().tolist()
                db1_ref += [float(dg_s.sum()), float(dl_s.sum())]
        if cfg.bias:
            err = norm_err(host(L.db2)[e], dY.sum(0))
            report[f"db2[{e}]"] = err
            assert err <= 2e-2
    if db1_got:
        err = norm_err(np.array(db1_got), np.array(db1_ref))
        report["db1"] = err
        assert err <= 2e-2
    for e in range(cfg.E):
        if counts[e] == 0:
            assert not dW1[e].any().item() and not dW2[e].any().item()
    return report


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["mixtral_fwd", "gptoss_fwdbwd", "dsv3_fwdbwd"])
def test_fullsize_sampled(name):
    cfg, inp, L = _run(name)
    idx, w, counts, offsets, row_map = _check_routing(cfg, inp, L)
    toks, heavy, light = _sample_tokens(idx, counts, n_random=6, seed=cfg.seed)
    report = _check_tokens(cfg, inp, L, idx, w, toks)
    if cfg.backward:
        rng = np.random.default_rng(cfg.seed + 1)
        experts = sorted({heavy, light, int(rng.integers(cfg.E))})
        cols = [0, cfg.f - 1, int(rng.integers(cfg.f))]
        report.update(_check_weight_grads(cfg, inp, L, idx, w, counts, offsets, row_map,
                                          experts, cols))
    print(name, {k: f"{v:.2e}" for k, v in report.items()}, flush=True)


# ------------------------------------------------------------------ MXFP8

def _mx_err(g, o, bf16=False):
    """(99.9th percentile, max) of |g - o| / rms(o) (bf16: beyond half an ulp)."""
    from gpu_util import half_ulp_bf16, rms
    g, o = np.asarray(g, np.float64), np.asarray(o, np.float64)
    e = np.abs(g - o)
    if bf16:
        e = np.maximum(e - half_ulp_bf16(o), 0.0)
    r = rms(o)
    return float(np.quantile(e, 0.999)) / r, float(e.max()) / r


class ChainMX:
    """The oracle's MXFP8 chain (every GEMM operand QDQ'd in blocks of 32 along
    its reduction axis; A and dH from exact values; dY = w dOut) evaluated for
    chosen tokens and weight-gradient columns, one expert at a time."""

    def __init__(self, cfg, inp, idx, w, offsets, pad, src_row):
        from oracle import mx as omx
        fmt = "e2m1" if cfg.gemm == "mxfp4" else "e4m3"

        class _Q:            # the oracle's QDQ in this workload's element format
            @staticmethod
            def mx_qdq(v, axis):
                return omx.mx_qdq(v, axis, fmt=fmt)
        self.q = _Q
        self.cfg, self.idx, self.w = cfg, idx, w
        self.x = _f32(inp["x"])
        self.W1 = inp["W1"]
        self.W2 = inp["W2"]
        self.dout = _f32(inp["dOut"])
        self.off, self.pad, self.src = offsets, pad, src_row

    def weights(self, e):
        f = self.cfg.f
        W1 = _f32(self.W1[e]).astype(np.float64)
        W2 = _f32(self.W2[e]).astype(np.float64)
        return dict(w1d=self.q.mx_qdq(W1, 1), w1f=self.q.mx_qdq(W1, 0),
                    w2f=self.q.mx_qdq(W2, 1), w2d=self.q.mx_qdq(W2, 0))

    def tokens(self, toks):
        cfg, f, q = self.cfg, self.cfg.f, self.q
        out = {t: np.zeros(cfg.d) for t in toks}
        dX = {t: np.zeros(cfg.d) for t in toks}
        for e in sorted({int(self.idx[t, j]) for t in toks for j in range(cfg.k)}):
            W = self.weights(e)
            for t in toks:
                for j in range(cfg.k):
                    if int(self.idx[t, j]) != e:
                        continue
                    H = q.mx_qdq(self.x[t:t + 1].astype(np.float64), 1) @ W["w1d"].T
                    A = om.glu_forward(H[:, :f], H[:, f:], cfg.act)
                    Y = om.round_bf16(q.mx_qdq(A, 1) @ W["w2f"].T)[0]
                    out[t] += self.w[t, j] * Y
                    dY = self.w[t, j] * self.dout[t:t + 1].astype(np.float64)
                    dA = q.mx_qdq(dY, 1) @ W["w2d"]
                    Hs = om.round_bf16(H)
                    dg, dl = om.glu_backward(dA, Hs[:, :f], Hs[:, f:], cfg.act)
                    dH = np.concatenate([dg, dl], 1)
                    dX[t] += om.round_bf16(q.mx_qdq(dH, 1) @ W["w1f"])[0]
        return out, dX

    def wgrad_cols(self, e, cols):
        """dW2[e][:, j] and canonical dW1[e] rows j (gate) and f + j (linear)."""
        cfg, f, q = self.cfg, self.cfg.f, self.q
        s, u = int(self.off[e]), int(self.off[e + 1])
        rows = self.src[s:u]
        W = self.weights(e)
        X = self.x[rows].astype(np.float64)
        Hx = q.mx_qdq(X, 1)
        # gate of each routed row (a token reaches expert e through one slot)
        wr_rows = np.array([self.w[t, int(np.nonzero(self.idx[t] == e)[0][0])] for t in rows])
        dY = wr_rows[:, None] * self.dout[rows].astype(np.float64)
        tq = lambda v: _tok_qdq(q, v)
        dYc = tq(dY)
        Xc = tq(X)
        dYr = q.mx_qdq(dY, 1)
        res = {}
        for j in cols:
            H2 = Hx @ W["w1d"][[j, f + j]].T            # gate j, linear j for every row
            A = om.glu_forward(H2[:, :1], H2[:, 1:], cfg.act)
            res[("dW2", j)] = dYc.T @ tq(A)[:, 0]
            dA = dYr @ W["w2d"][:, j]
            Hs = om.round_bf16(H2)
            dg, dl = om.glu_backward(dA[:, None], Hs[:, :1], Hs[:, 1:], cfg.act)
            res[("dW1g", j)] = tq(dg)[:, 0] @ Xc
            res[("dW1l", j)] = tq(dl)[:, 0] @ Xc
        return res


def _tok_qdq(q, v):
    """QDQ of one expert's rows [c, n] along the tokens, blocks from the first row."""
    c = v.shape[0]
    cp = (c + 31) // 32 * 32
    buf = np.zeros((cp,) + v.shape[1:])
    buf[:c] = v
    return q.mx_qdq(buf, 0)[:c]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["dsv3_mxfp8_fwdbwd", "dsv3_mxfp4_fwdbwd"])
def test_fullsize_mx_sampled(name):
    """dsv3_mxfp8_fwdbwd / dsv3_mxfp4_fwdbwd at full size: sampled token rows
    of out and dX, and weight-gradient columns of a heavy and a light expert,
    against the oracle's MX chain in the same element format; routing, offsets
    and padded offsets bit-exact."""
    cfg = synth.WORKLOADS[name]
    note(f"full-size {cfg.name}: T={cfg.T} d={cfg.d} f={cfg.f} E={cfg.E} k={cfg.k}")
    from ragged_grouped_gemm_amd import ops
    from ragged_grouped_gemm_amd.layer import MoEFFN
    inp = synth.make_inputs(cfg)
    t = lambda a: synth.to_torch(a, "cuda")
    x, lg, dout = t(inp["x"]), t(inp["logits"]), t(inp["dOut"])
    W1p, _ = ops.moe_repack_glu_weights(t(inp["W1"]))
    Wm = MoEFFN.mx_weights(W1p, t(inp["W2"]), cfg.gemm)
    del W1p
    L = MoEFFN(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, score=cfg.score, normalize=cfg.normalize,
               gemm=cfg.gemm)
    L.forward(x, lg, Wm, None)
    L.backward(dout, lg, Wm, None)
    torch.cuda.synchronize()
    idx, w, counts, offsets, row_map = _check_routing(cfg, inp, L)
    pad = om.pad_offsets(counts)
    np.testing.assert_array_equal(host(L.pad_offsets), pad)
    toks, heavy, light = _sample_tokens(idx, counts, n_random=3, seed=cfg.seed)
    ch = ChainMX(cfg, inp, idx, w, offsets, pad, host(L.src_row))
    ref_out, ref_dx = ch.tokens(toks)
    rep = {"out": _mx_err(host(L.out)[toks], np.stack([ref_out[k_] for k_ in toks]), bf16=True),
           "dX": _mx_err(host(L.dX)[toks], np.stack([ref_dx[k_] for k_ in toks]), bf16=True)}
    f = cfg.f
    pos = om.glu_pack_rows(f, G)
    cols = [0, f - 1]
    for e in (heavy, light):
        res = ch.wgrad_cols(e, cols)
        for j in cols:
            rep[f"dW2[{e}][:,{j}]"] = _mx_err(host(L.dW2[e, :, j]), res[("dW2", j)])
            rep[f"dW1g[{e},{j}]"] = _mx_err(host(L.dW1p[e, int(pos[j])]), res[("dW1g", j)])
            rep[f"dW1l[{e},{j}]"] = _mx_err(host(L.dW1p[e, int(pos[f + j])]), res[("dW1l", j)])
    for e in range(cfg.E):
        if counts[e] == 0:
            assert not L.dW1p[e].any().item() and not L.dW2[e].any().item()
    print(cfg.name, {k_: f"q999 {a:.2e} max {b:.2e}" for k_, (a, b) in rep.items()}, flush=True)
    for name, (qv, mv) in rep.items():
        assert mv <= 2e-2, (name, rep)
