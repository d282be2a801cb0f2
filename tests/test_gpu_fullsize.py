"""Parity at the workloads' full sizes, in the launch configuration bench.py
times (MoEFFN, eager, default tile choice and grid).

The full oracle chain is too slow at these sizes, so the oracle computes
sampled outputs one at a time, following the same chain (fp64 arithmetic,
the library's storage rounding at H, A, Y, dY, dH, dXp):
  * whole output rows out[t], dX[t], dgate[t], dlogits[t] for 64 random
    tokens plus tokens routed to the heaviest and to the lightest expert;
  * whole weight-gradient slices: dW2[e][:, j] and the packed dW1 rows of the
    gate and linear halves of column j (8 columns), db1/db2 where present, for
    the heaviest, a light and a random expert;
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
    toks, heavy, light = _sample_tokens(idx, counts, n_random=64, seed=cfg.seed)
    report = _check_tokens(cfg, inp, L, idx, w, toks)
    if cfg.backward:
        rng = np.random.default_rng(cfg.seed + 1)
        experts = sorted({heavy, light, int(rng.integers(cfg.E))})
        cols = sorted({0, cfg.f - 1, *(int(v) for v in rng.integers(cfg.f, size=6))})
        report.update(_check_weight_grads(cfg, inp, L, idx, w, counts, offsets, row_map,
                                          experts, cols))
    print(name, {k: f"{v:.2e}" for k, v in report.items()}, flush=True)


# ------------------------------------------------------------------ MXFP8 / MXFP4

def _mx_err(g, o, bf16=False):
    """(99.9th percentile, max) of |g - o| / rms(o) (bf16: beyond half an ulp)."""
    from gpu_util import half_ulp_bf16, rms
    g, o = np.asarray(g, np.float64), np.asarray(o, np.float64)
    e = np.abs(g - o)
    if bf16:
        e = np.maximum(e - half_ulp_bf16(o), 0.0)
    r = rms(o)
    return float(np.quantile(e, 0.999)) / r, float(e.max()) / r


POOL_THREADS = 16          # the host cores of one GPU's share


def _par_qdq(pool, fmt, v, axis):
    """The oracle's QDQ of a 2-D array along ``axis`` (blocks of 32 from index
    0, zero-padded), computed in independent slices on a thread pool: rows for
    axis 1, columns for axis 0 (the blocks never span two slices)."""
    from oracle import mx as omx
    v = np.asarray(v, np.float64)
    n = v.shape[axis]
    npad = (n + 31) // 32 * 32
    if npad != n:
        pad = [(0, 0), (0, 0)]
        pad[axis] = (0, npad - n)
        v = np.pad(v, pad)
    other = v.shape[1 - axis]
    step = max(1, -(-other // POOL_THREADS))
    sl = [slice(i, min(i + step, other)) for i in range(0, other, step)]
    take = (lambda s_: v[s_]) if axis == 1 else (lambda s_: v[:, s_])
    parts = list(pool.map(lambda s_: omx.mx_qdq(take(s_), axis, fmt=fmt), sl))
    out = np.concatenate(parts, axis=1 - axis)
    return out[:, :n] if axis == 1 else out[:n]


def _rows_mx(m, rows, fmt):
    """Codes (unpacked) and scales of chosen rows of an MXTensor, as int64."""
    from oracle import mx as omx
    ri = torch.as_tensor(np.asarray(rows, np.int64), device=m.data.device)
    data = m.data.index_select(0, ri).cpu().numpy()
    c = omx.unpack_fp4(data) if fmt == "e2m1" else data
    return c.astype(np.int64), m.scale.index_select(0, ri).cpu().numpy().astype(np.int64)


def _window_mx(m, p0, n, fmt):
    """Codes (unpacked) and scales of columns [p0, p0 + n) of every row of an
    MXTensor (p0, n multiples of 32), as int64."""
    from oracle import mx as omx
    if fmt == "e2m1":
        c = omx.unpack_fp4(m.data[:, p0 // 2:(p0 + n) // 2].contiguous().cpu().numpy())
    else:
        c = m.data[:, p0:p0 + n].contiguous().cpu().numpy()
    sc = m.scale[:, p0 // 32:(p0 + n) // 32].contiguous().cpu().numpy()
    return c.astype(np.int64), sc.astype(np.int64)


def _blocks(a):
    """[..., 32k] -> [n, 32] (one block of 32 per row) for check_codes."""
    return np.asarray(a).reshape(-1, 32)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["dsv3_mxfp8_fwdbwd", "dsv3_mxfp4_fwdbwd"])
def test_fullsize_mx_dense(name):
    """dsv3_mxfp8_fwdbwd / dsv3_mxfp4_fwdbwd at full size, in bench.py's launch
    configuration: 512 token rows of out, dX, dgate and dlogits spread over
    every non-empty expert, and 32 whole columns of dW2 and the matching gate
    and linear rows of dW1 for the heaviest, a middle and the lightest
    non-empty expert, each held to max-abs / rms <= 2e-2 against the oracle's
    chain in the same element format, evaluated on the GPU's own checked
    decisions (codes of A, dY, dH; bf16 roundings of H, Y, dXp -- each first
    checked against its exact value; see tests/mx_chain.py).  The errors
    against the oracle's unconditioned chain are printed beside them.
    Routing, offsets and padded offsets bit-exact; empty experts' weight
    gradients exactly zero."""
    from concurrent.futures import ThreadPoolExecutor
    import mx_chain
    from oracle import mx as omx
    cfg = synth.WORKLOADS[name]
    fmt = "e2m1" if cfg.gemm == "mxfp4" else "e4m3"
    note(f"full-size dense {cfg.name}: T={cfg.T} d={cfg.d} f={cfg.f} E={cfg.E} k={cfg.k}")
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
    for e in range(cfg.E):
        if counts[e] == 0:
            assert not L.dW1p[e].any().item() and not L.dW2[e].any().item()
    f, d, k = cfg.f, cfg.d, cfg.k
    pos = om.glu_pack_rows(f, G)
    X = _f32(inp["x"])
    DO = _f32(inp["dOut"])
    gw = lambda e: (_f32(inp["W1"][e]).astype(np.float64), _f32(inp["W2"][e]).astype(np.float64))
    src = host(L.src_row)
    pool = ThreadPoolExecutor(max_workers=POOL_THREADS)
    q = lambda v, ax: _par_qdq(pool, fmt, v, ax)
    rows_of = lambda tns, r_: host(tns[torch.as_tensor(np.asarray(r_, np.int64), device="cuda")])
    rep, plain, dec = {}, {}, {}

    # ---- 512 tokens: the first 8 of every non-empty expert, then random ones
    rng = np.random.default_rng(cfg.seed + 7)
    toks = set()
    for e in range(cfg.E):
        toks.update(int(v) for v in np.nonzero((idx == e).any(1))[0][:8])
    rest = np.setdiff1d(np.arange(cfg.T), sorted(toks))
    toks.update(int(v) for v in rng.choice(rest, size=max(0, 512 - len(toks)), replace=False))
    toks = np.array(sorted(toks))
    flat = row_map[toks].reshape(-1)                       # routed rows, token-major
    Ac, As = _rows_mx(L.A_row, flat, fmt)
    Yc, Ys_ = _rows_mx(L.dY_row, flat, fmt)
    Dc, Ds = _rows_mx(L.dH_row, flat, fmt)
    Hg = mx_chain.packed_to_canonical(rows_of(L.H, flat), 1)
    Yg = rows_of(L.Y, flat)
    dXpg = rows_of(L.dXp, flat)
    nr = flat.size
    H_ex, A_ex = np.zeros((nr, 2 * f)), np.zeros((nr, f))
    Y_ex, dY_ex = np.zeros((nr, d)), np.zeros((nr, d))
    dH_ex, dXp_ex = np.zeros((nr, 2 * f)), np.zeros((nr, d))   # dH_ex in packed order
    Yp, dXpp = np.zeros((nr, d)), np.zeros((nr, d))
    tok_of = np.repeat(toks, k)
    slot_of = np.tile(np.arange(k), toks.size)
    for e in sorted(set(idx[toks].reshape(-1).tolist())):
        sel = np.nonzero(idx[tok_of, slot_of] == e)[0]
        W1, W2 = gw(e)
        w1d, w1f, w2f, w2d = q(W1, 1), q(W1, 0), q(W2, 1), q(W2, 0)
        tt = tok_of[sel]
        H = omx.mx_qdq(X[tt].astype(np.float64), 1, fmt=fmt) @ w1d.T
        H_ex[sel] = H
        A = om.glu_forward(H[:, :f], H[:, f:], cfg.act)
        A_ex[sel] = A
        Y_ex[sel] = mx_chain.decode(Ac[sel], As[sel], fmt)[:, :f] @ w2f.T
        Yp[sel] = om.round_bf16(omx.mx_qdq(A, 1, fmt=fmt) @ w2f.T)
        dY = w[tt, slot_of[sel]][:, None] * DO[tt].astype(np.float64)
        dY_ex[sel] = dY
        dA = mx_chain.decode(Yc[sel], Ys_[sel], fmt)[:, :d] @ w2d
        dg, dl = om.glu_backward(dA, Hg[sel][:, :f], Hg[sel][:, f:], cfg.act)
        dH_ex[sel[:, None], pos[None, :]] = np.concatenate([dg, dl], 1)
        dH_gpu = mx_chain.packed_to_canonical(mx_chain.decode(Dc[sel], Ds[sel], fmt)[:, :2 * f], 1)
        dXp_ex[sel] = dH_gpu @ w1f
        Hs = om.round_bf16(H)
        dAp = omx.mx_qdq(dY, 1, fmt=fmt) @ w2d
        dgp, dlp = om.glu_backward(dAp, Hs[:, :f], Hs[:, f:], cfg.act)
        dXpp[sel] = om.round_bf16(omx.mx_qdq(np.concatenate([dgp, dlp], 1), 1, fmt=fmt) @ w1f)
    blk = lambda c_, s_, n_: (_blocks(c_[:, :n_]), s_[:, :n_ // 32].reshape(-1, 1))
    dec["H"] = mx_chain.check_stored(Hg, H_ex, "H (sampled rows)", 8.0)
    dec["A_row"] = mx_chain.check_codes(*blk(Ac, As, f), _blocks(A_ex), fmt, "A row copy")
    dec["Y"] = mx_chain.check_stored(Yg, Y_ex, "Y (sampled rows)", 4.0)
    dec["dY_row"] = mx_chain.check_codes(*blk(Yc, Ys_, d), _blocks(dY_ex), fmt, "dY row copy")
    dec["dH_row"] = mx_chain.check_codes(*blk(Dc, Ds, 2 * f), _blocks(dH_ex), fmt, "dH row copy")
    dec["dXp"] = mx_chain.check_stored(dXpg, dXp_ex, "dXp (sampled rows)", 4.0)
    n = toks.size
    wt = w[toks]
    out = np.einsum("tj,tjd->td", wt, Yg.reshape(n, k, d))
    outp = np.einsum("tj,tjd->td", wt, Yp.reshape(n, k, d))
    dX = dXpg.reshape(n, k, d).sum(1)
    dXpl = dXpp.reshape(n, k, d).sum(1)
    dgate = np.einsum("td,tjd->tj", DO[toks].astype(np.float64), Yg.reshape(n, k, d))
    lg64 = inp["logits"][toks].astype(np.float64)
    dlog = om.route_topk_bwd(lg64, idx[toks], dgate, cfg.score, cfg.normalize)
    rep["out"] = _mx_err(host(L.out)[toks], out, bf16=True)
    rep["dX"] = _mx_err(host(L.dX)[toks], dX, bf16=True)
    rep["dgate"] = _mx_err(host(L.dgate)[toks], dgate)
    rep["dlogits"] = _mx_err(host(L.dlogits)[toks], dlog)
    plain["out"] = _mx_err(host(L.out)[toks], outp, bf16=True)
    plain["dX"] = _mx_err(host(L.dX)[toks], dXpl, bf16=True)

    # ---- whole weight-gradient columns of the heaviest, a middle and the lightest expert
    nz = [e for e in range(cfg.E) if counts[e] > 0]
    by = sorted(nz, key=lambda e: (counts[e], e))
    experts = sorted({by[-1], by[len(by) // 2], by[0]})
    cols = np.unique(np.linspace(0, f - 1, 32).round().astype(int))
    wcodes = {k_: ([], [], []) for k_ in ("A", "dH", "dY_row", "dY_col")}

    def add(key, c_, s_, ex):
        wcodes[key][0].append(_blocks(c_))
        wcodes[key][1].append(s_.reshape(-1, 1))
        wcodes[key][2].append(_blocks(ex))

    for e in experts:
        s_, u_ = int(offsets[e]), int(offsets[e + 1])
        c = u_ - s_
        cp = (c + 31) // 32 * 32
        p0 = int(pad[e])
        tk = src[s_:u_]
        slot = np.array([int(np.nonzero(idx[t_] == e)[0][0]) for t_ in tk])
        Xe = X[tk].astype(np.float64)
        Xq, Xc = q(Xe, 1), q(Xe, 0)
        dY = w[tk, slot][:, None] * DO[tk].astype(np.float64)
        # the GPU's dY codes of the segment: row copy (FC2 dgrad) and token-axis copy (FC2 wgrad)
        rc, rs = _rows_mx(L.dY_row, np.arange(s_, u_), fmt)
        add("dY_row", rc[:, :d], rs[:, :d // 32], dY)
        dYr = mx_chain.decode(rc, rs, fmt)[:, :d]
        cc, cs = _window_mx(L.dY_col, p0, cp, fmt)
        dYpad = np.zeros((cp, d))
        dYpad[:c] = dY
        add("dY_col", cc, cs, dYpad.T)
        dYc = mx_chain.decode(cc, cs, fmt)[:, :c].T                  # [c, d]
        dYr_o, dYc_o = q(dY, 1), q(dY, 0)                            # the oracle's own codes
        W1, W2 = gw(e)
        Hseg = mx_chain.packed_to_canonical(host(L.H[s_:u_]), 1)
        for j in cols:
            w1rows = omx.mx_qdq(W1[[j, f + j]], 1, fmt=fmt)          # blocks along d
            H2 = Xq @ w1rows.T
            A = om.glu_forward(H2[:, :1], H2[:, 1:], cfg.act)[:, 0]
            Ap = np.zeros(cp)
            Ap[:c] = A
            ac, as_ = _rows_mx(L.A_col, [j], fmt)
            ac, as_ = ac[:, p0:p0 + cp], as_[:, p0 // 32:(p0 + cp) // 32]
            add("A", ac, as_, Ap[None])
            A_gpu = mx_chain.decode(ac, as_, fmt)[0, :c]
            got2 = host(L.dW2[e, :, int(j)])
            rep[f"dW2[{e}][:,{j}]"] = _mx_err(got2, dYc.T @ A_gpu)
            plain[f"dW2[{e}][:,{j}]"] = _mx_err(got2, dYc_o.T @ q(A[:, None], 0)[:, 0])
            w2col = omx.mx_qdq(W2[:, j][:, None], 0, fmt=fmt)[:, 0]   # W2 column j, blocks along d
            dg, dl = om.glu_backward(dYr @ w2col, Hseg[:, j], Hseg[:, f + j], cfg.act)
            dc, ds_ = _rows_mx(L.dH_col, [int(pos[j]), int(pos[f + j])], fmt)
            dc, ds_ = dc[:, p0:p0 + cp], ds_[:, p0 // 32:(p0 + cp) // 32]
            ex = np.zeros((2, cp))
            ex[0, :c], ex[1, :c] = dg, dl
            add("dH", dc, ds_, ex)
            dH_gpu = mx_chain.decode(dc, ds_, fmt)[:, :c]
            Hs = om.round_bf16(H2)
            dgp, dlp = om.glu_backward(dYr_o @ w2col, Hs[:, 0], Hs[:, 1], cfg.act)
            for r_, lab, ref_p in ((0, "dW1g", dgp), (1, "dW1l", dlp)):
                got1 = host(L.dW1p[e, int(pos[j + r_ * f])])
                rep[f"{lab}[{e},{j}]"] = _mx_err(got1, dH_gpu[r_] @ Xc)
                plain[f"{lab}[{e},{j}]"] = _mx_err(got1, q(ref_p[:, None], 0)[:, 0] @ Xc)
    for key, (cs_, ss, es) in wcodes.items():
        dec[key + " (wgrad experts)"] = mx_chain.check_codes(
            np.concatenate(cs_), np.concatenate(ss), np.concatenate(es), fmt, key)
    pool.shutdown()
    worst = max(rep.items(), key=lambda kv: kv[1][1])
    worst_p = max(plain.items(), key=lambda kv: kv[1][1])
    fmt_dec = lambda v: f"{v[0]:.1e}/{v[1]:.1e}" if isinstance(v, tuple) else f"{v:.2f} ulp"
    print(cfg.name, f"{toks.size} tokens, experts {experts} (rows {[int(counts[e]) for e in experts]}),"
          f" {cols.size} columns;", "decisions", {k_: fmt_dec(v) for k_, v in dec.items()},
          "conditioned", {k_: f"q999 {a:.2e} max {b:.2e}" for k_, (a, b) in rep.items()
                          if "[" not in k_},
          f"worst {worst[0]} max {worst[1][1]:.2e};",
          "unconditioned", {k_: f"q999 {a:.2e} max {b:.2e}" for k_, (a, b) in plain.items()
                            if "[" not in k_},
          f"worst {worst_p[0]} max {worst_p[1][1]:.2e}", flush=True)
    for name_, (qv, mv) in rep.items():
        assert mv <= 2e-2, (name_, rep[name_])
