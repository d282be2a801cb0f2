"""GPU parity of the MXFP4 path (E2M1 elements packed two per byte, E8M0
scale per 32).

* Quantizers (row copy, transposed weight copy, expert-segmented row / column
  copies with gather and gate product): bit-exact against oracle.mx on the
  same float32 values (codes packed with oracle.mx.pack_fp4).
"""
import numpy as np
import pytest
import torch

from gpu_util import host, note
from oracle import mx as omx

pytestmark = pytest.mark.gpu


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


def fp4_values(rng, rows, n, dtype):
    """Rows at scales 2^-30 .. 2^30 with an all-zero block, a tiny block, a
    block of exact E2M1 midpoints and one whose maximum is 7 (saturates)."""
    from test_gpu_mx import wide_values
    x64, xd = wide_values(rng, rows, n, dtype)
    if rows > 3 and n >= 128:
        mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0] * 4)
        x64[3, 96:128] = mids * np.where(np.arange(32) % 3 == 0, -1.0, 1.0)
        x64[3, 100] = 7.0
        x64[3, 96:128] *= 2.0 ** 4
        xd[3, 96:128] = torch.as_tensor(x64[3, 96:128], dtype=xd.dtype, device=xd.device)
    return x64, xd


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rows,n", [(37, 256), (5, 2048)])
def test_quantize_rows_bitexact(dtype, rows, n):
    note(f"mxfp4 quantize rows {dtype} {rows}x{n}")
    rng = np.random.default_rng(rows + n)
    x64, xd = fp4_values(rng, rows, n, dtype)
    out = ops_().moe_mx_quantize(xd, fmt="e2m1")
    torch.cuda.synchronize()
    c, s = omx.mx_quantize_blocks(x64, fmt="e2m1")
    assert out.data.shape == (rows, n // 2)
    np.testing.assert_array_equal(u8(out.data), omx.pack_fp4(c))
    np.testing.assert_array_equal(u8(out.scale), s)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quantize_transpose_bitexact(dtype):
    note(f"mxfp4 quantize transpose {dtype}")
    rng = np.random.default_rng(3)
    B, rows, n = 3, 64, 96
    x64, xd = fp4_values(rng, B * rows, n, dtype)
    out = ops_().moe_mx_quantize_transpose(xd.reshape(B, rows, n), fmt="e2m1")
    torch.cuda.synchronize()
    ref = np.concatenate([x64.reshape(B, rows, n)[b].T for b in range(B)])
    c, s = omx.mx_quantize_blocks(ref, fmt="e2m1")
    np.testing.assert_array_equal(u8(out.data), omx.pack_fp4(c))
    np.testing.assert_array_equal(u8(out.scale), s)


@pytest.mark.parametrize("n", [256, 352])
@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quantize_experts_bitexact(gated, dtype, n):
    """Row and segment-column copies of x[src_row] (* gate), straight from x;
    n = 352 leaves the second 256-column chunk three blocks wide."""
    from test_gpu_mx import _routing
    note(f"mxfp4 quantize experts gated={gated} {dtype} n={n}")
    T, E, k = 300, 6, 2
    idx, w, offsets, pad, row_map, src_row = _routing(T, E, k, 5)
    rng = np.random.default_rng(7)
    x64, xd = fp4_values(rng, T, n, dtype)
    R = T * k
    kw = dict(src_row=src_row)
    if gated:
        kw.update(row_map=row_map, topk_w=w)
    row, col = ops_().moe_mx_quantize_experts(xd, offsets, pad, R, fmt="e2m1", **kw)
    torch.cuda.synchronize()
    src = host(src_row)
    v = x64[src]
    if gated:
        rm, wt = host(row_map).reshape(-1), host(w).reshape(-1)
        wr = np.empty(R)
        wr[rm] = wt
        v = (v.astype(np.float32) * wr.astype(np.float32)[:, None]).astype(np.float64)
    c, s = omx.mx_quantize_blocks(v, fmt="e2m1")
    np.testing.assert_array_equal(u8(row.data), omx.pack_fp4(c))
    np.testing.assert_array_equal(u8(row.scale), s)
    off, pd = host(offsets), host(pad)
    cc, cs = omx.mx_quantize_segments_colwise(v, off, pd, fmt="e2m1")
    Rp = int(pd[-1])
    np.testing.assert_array_equal(u8(col.data)[:, :Rp // 2], omx.pack_fp4(cc))
    np.testing.assert_array_equal(u8(col.scale)[:, :Rp // 32], cs)


# ------------------------------------------------------------------ GEMMs
#
# MXFP4 grouped GEMMs against float64 products of the GPU's own quantized
# operands (decoded by oracle.mx): bf16 outputs by their excess over bf16
# rounding (<= 5e-3 of the rms), float32 weight gradients by max |err| / rms.
# The epilogue outputs (A, dH as MXFP4 copies) against the exact values in
# the GPU's own block scale: every element within half an E2M1 quantum plus
# 2^-9 of its block maximum, scales within one code in at most 0.1 % of the
# blocks, and element codes different from the oracle's in at most 1 % (a
# value within the scaled MFMA's accumulation error of an E2M1 rounding
# midpoint may round either way).

from gpu_util import bf16_excess, dev, norm_err, offsets_of, rand_bf16, rel_l2  # noqa: E402
from oracle import moe as om  # noqa: E402

G = 32
COUNTS_SMALL = [0, 1, 31, 32, 33, 255, 256, 257, 0, 130]
COUNTS_BIG = [0, 700, 1300, 300, 513]


def deq4(m, rows=None, cols=None):
    """float64 values of an MXFP4 MXTensor (optionally a [rows, cols] window)."""
    c = omx.unpack_fp4(u8(m.data).astype(np.uint8))
    v = omx.mx_dequantize_blocks(c, u8(m.scale), fmt="e2m1")
    if rows is not None:
        v = v[:rows]
    if cols is not None:
        v = v[:, :cols]
    return v


def pad_of(counts):
    return om.pad_offsets(np.asarray(counts))


def _fp4_close(gdata, gs, oc, os_, exact, what):
    """GPU packed codes / scales vs the oracle's codes of the exact values."""
    gc = omx.unpack_fp4(np.asarray(gdata, np.uint8)).astype(np.int64)
    gs, oc, os_ = (np.asarray(a, np.int64) for a in (gs, oc, os_))
    sd = gs != os_
    assert np.all(np.abs(gs - os_) <= 1), what
    assert sd.mean() <= 1e-3, (what, "scale flips", sd.mean())
    rows, n = gc.shape
    sc = np.ldexp(1.0, np.repeat(gs, 32, axis=1) - 127)
    v = np.clip(np.asarray(exact, np.float64) / sc, -6.0, 6.0)
    g = omx.mx_dequantize_blocks(gc, gs, fmt="e2m1") / sc
    bmax = np.repeat(np.abs(v).reshape(rows, n // 32, 32).max(-1), 32, axis=1)
    a = np.abs(v)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    half = 0.5 * np.ldexp(1.0, np.maximum(ex - 2, -1))     # half an E2M1 quantum at |v|
    dev_ = np.abs(g - v) - half
    assert not (dev_ > 2.0 ** -9 * bmax).any(), (what, np.argwhere(dev_ > 2.0 ** -9 * bmax)[:5])
    flips = (gc != oc)[~np.repeat(sd, 32, axis=1)].mean()
    assert flips <= 1e-2, (what, "element flips", flips)
    print(what, "scale flips", sd.mean(), "element flips", flips, flush=True)
    return sd.mean(), flips


def _seg_cols(v, off, pad):
    out = np.zeros((v.shape[1], int(pad[-1])))
    for e in range(len(off) - 1):
        c = int(off[e + 1] - off[e])
        out[:, pad[e]:pad[e] + c] = v[off[e]:off[e + 1]].T
    return out


def _check_col_padding(data, off, pad):
    codes = omx.unpack_fp4(np.asarray(data, np.uint8))
    for e in range(len(off) - 1):
        c = int(off[e + 1] - off[e])
        assert not codes[:, pad[e] + c:pad[e + 1]].any(), ("padding not zero", e)


def _unpack_cols(f):
    pos = om.glu_pack_rows(f, G)
    return pos[:f], pos[f:]


@pytest.mark.parametrize("counts,N,K", [(COUNTS_SMALL, 256, 256), (COUNTS_BIG, 1024, 512),
                                        (COUNTS_BIG, 2048, 128)])
def test_mx4_gemm_fwd(counts, N, K):
    note(f"mxfp4 gemm fwd counts={counts} N={N} K={K}")
    ops = ops_()
    rng = np.random.default_rng(12)
    E, R = len(counts), sum(counts)
    off = offsets_of(counts)
    _, ad = rand_bf16(rng, (R, K))
    _, wd = rand_bf16(rng, (E, N, K), K ** -0.5)
    aq = ops.moe_mx_quantize(ad, fmt="e2m1")
    wq = ops.moe_mx_quantize(wd.reshape(E * N, K), fmt="e2m1")
    y = ops.moe_grouped_gemm_fwd(aq, wq, dev(off), E=E, N=N)
    torch.cuda.synchronize()
    Aq, Wq = deq4(aq), deq4(wq).reshape(E, N, K)
    ref = np.concatenate([Aq[off[e]:off[e + 1]] @ Wq[e].T for e in range(E)])
    err = bf16_excess(host(y), ref)
    print("mxfp4 fwd excess", err, flush=True)
    assert err <= 5e-3


@pytest.mark.parametrize("counts,N,K", [(COUNTS_SMALL, 512, 256), (COUNTS_BIG, 1024, 1024)])
def test_mx4_gemm_dgrad(counts, N, K):
    note(f"mxfp4 dgrad counts={counts} N={N} K={K}")
    ops = ops_()
    rng = np.random.default_rng(14)
    E, R = len(counts), sum(counts)
    off = offsets_of(counts)
    _, gd = rand_bf16(rng, (R, N))
    _, wd = rand_bf16(rng, (E, N, K), N ** -0.5)
    gq = ops.moe_mx_quantize(gd, fmt="e2m1")
    wt = ops.moe_mx_quantize_transpose(wd, fmt="e2m1")
    da = ops.moe_grouped_gemm_bwd(gq, dev(off), mode="dgrad", w=wt, E=E, K=K)
    torch.cuda.synchronize()
    Gq, WT = deq4(gq), deq4(wt).reshape(E, K, N)
    ref = np.concatenate([Gq[off[e]:off[e + 1]] @ WT[e].T for e in range(E)])
    assert bf16_excess(host(da), ref) <= 5e-3


@pytest.mark.parametrize("counts,N,K", [(COUNTS_SMALL, 512, 256), (COUNTS_BIG, 1024, 1024)])
def test_mx4_gemm_wgrad(counts, N, K):
    note(f"mxfp4 wgrad counts={counts} N={N} K={K}")
    ops = ops_()
    rng = np.random.default_rng(15)
    E, R = len(counts), sum(counts)
    off, pad = offsets_of(counts), pad_of(counts)
    _, gd = rand_bf16(rng, (R, N))
    _, ad = rand_bf16(rng, (R, K))
    doff, dpad = dev(off), dev(pad)
    _, gc = ops.moe_mx_quantize_experts(gd, doff, dpad, R, want_row=False, fmt="e2m1")
    _, ac = ops.moe_mx_quantize_experts(ad, doff, dpad, R, want_row=False, fmt="e2m1")
    dw = ops.moe_grouped_gemm_bwd(gc, doff, mode="wgrad", a=ac, E=E, R=R, pad_offsets=dpad)
    # accumulating onto zeros takes the direct float32 stores, the plain call
    # the whole rows staged through LDS (over two ring slots): the same values
    dw0 = torch.zeros_like(dw)
    ops.moe_grouped_gemm_bwd(gc, doff, mode="wgrad", a=ac, E=E, R=R, pad_offsets=dpad, out=dw0,
                             accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(dw, dw0)
    Gc, Ac = deq4(gc), deq4(ac)
    got = host(dw)
    for e in range(E):
        c = counts[e]
        if c == 0:
            assert not np.any(got[e]), e
            continue
        ref = Gc[:, pad[e]:pad[e] + c] @ Ac[:, pad[e]:pad[e] + c].T
        assert norm_err(got[e], ref) <= 1e-3, (e, norm_err(got[e], ref), rel_l2(got[e], ref))


@pytest.mark.parametrize("counts,d,f", [(COUNTS_SMALL, 256, 256), (COUNTS_BIG, 1024, 512)])
def test_mx4_glu_fwd(counts, d, f):
    note(f"mxfp4 glu fwd counts={counts} d={d} f={f}")
    ops = ops_()
    rng = np.random.default_rng(11)
    E, R, n1 = len(counts), sum(counts), 2 * f
    off = offsets_of(counts)
    pad = pad_of(counts)
    _, xd = rand_bf16(rng, (R, d))
    _, wd = rand_bf16(rng, (E, n1, d), d ** -0.5)
    xq = ops.moe_mx_quantize(xd, fmt="e2m1")
    wq = ops.moe_mx_quantize(wd.reshape(E * n1, d), fmt="e2m1")
    (a_row, a_col), H = ops.moe_grouped_gemm_glu_fwd(xq, wq, dev(off), E=E, f=f,
                                                    pad_offsets=dev(pad))
    torch.cuda.synchronize()
    assert a_row.fmt == "e2m1" and a_row.data.shape == (R, f // 2)
    X, W = deq4(xq), deq4(wq).reshape(E, n1, d)
    Href = np.concatenate([X[off[e]:off[e + 1]] @ W[e].T for e in range(E)])
    assert bf16_excess(host(H), Href) <= 5e-3
    gpos, lpos = _unpack_cols(f)
    A = om.glu_forward(Href[:, gpos], Href[:, lpos], "swiglu")
    oc, os_ = omx.mx_quantize_blocks(A, fmt="e2m1")
    _fp4_close(u8(a_row.data), u8(a_row.scale), oc, os_, A, "A row copy")
    cc, cs = omx.mx_quantize_segments_colwise(A, off, pad, fmt="e2m1")
    Rp = int(pad[-1])
    _fp4_close(u8(a_col.data)[:, :Rp // 2], u8(a_col.scale)[:, :Rp // 32], cc, cs,
               _seg_cols(A, off, pad), "A column copy")
    _check_col_padding(u8(a_col.data)[:, :Rp // 2], off, pad)


@pytest.mark.parametrize("counts,d,f", [(COUNTS_SMALL, 256, 256), (COUNTS_BIG, 1024, 512),
                                        (COUNTS_BIG, 256, 1024)])
def test_mx4_glu_bwd(counts, d, f):
    note(f"mxfp4 glu bwd counts={counts} d={d} f={f}")
    ops = ops_()
    rng = np.random.default_rng(13)
    E, R, n1 = len(counts), sum(counts), 2 * f
    off = offsets_of(counts)
    pad = pad_of(counts)
    _, dyd = rand_bf16(rng, (R, d))
    _, w2d = rand_bf16(rng, (E, d, f), d ** -0.5)
    h64, hd = rand_bf16(rng, (R, n1))
    dyq = ops.moe_mx_quantize(dyd, fmt="e2m1")
    w2t = ops.moe_mx_quantize_transpose(w2d, fmt="e2m1")
    dh_row, dh_col = ops.moe_grouped_gemm_glu_bwd(dyq, w2t, hd, dev(off), E=E,
                                                  pad_offsets=dev(pad))
    torch.cuda.synchronize()
    DY, W2T = deq4(dyq), deq4(w2t).reshape(E, f, d)
    dA = np.concatenate([DY[off[e]:off[e + 1]] @ W2T[e].T for e in range(E)])
    gpos, lpos = _unpack_cols(f)
    dg, dl = om.glu_backward(dA, h64[:, gpos], h64[:, lpos], "swiglu")
    dH = np.empty((R, n1))
    dH[:, gpos], dH[:, lpos] = dg, dl
    oc, os_ = omx.mx_quantize_blocks(dH, fmt="e2m1")
    _fp4_close(u8(dh_row.data), u8(dh_row.scale), oc, os_, dH, "dH row copy")
    cc, cs = omx.mx_quantize_segments_colwise(dH, off, pad, fmt="e2m1")
    Rp = int(pad[-1])
    _fp4_close(u8(dh_col.data)[:, :Rp // 2], u8(dh_col.scale)[:, :Rp // 32], cc, cs,
               _seg_cols(dH, off, pad), "dH column copy")
    _check_col_padding(u8(dh_col.data)[:, :Rp // 2], off, pad)


# ------------------------------------------------------------------ layer

LAYER_CASES = [
    dict(T=512, d=256, f=256, E=8, k=2, zipf=1.2, forced_empty=1, seed=21),
    dict(T=640, d=512, f=384, E=6, k=3, zipf=0.8, forced_empty=0, seed=22),
]


@pytest.mark.parametrize("case", LAYER_CASES, ids=lambda c: f"T{c['T']}d{c['d']}f{c['f']}E{c['E']}")
def test_mx4_layer_vs_oracle(case):
    from test_gpu_mx import mx_errors
    import synth
    note(f"mxfp4 layer {case}")
    from ragged_grouped_gemm_amd.layer import MoEFFN
    ops = ops_()
    cfg = synth.MoEConfig("mx4_layer", gemm="mxfp4", score="sigmoid", backward=True, **case)
    inp = synth.make_inputs(cfg)
    t = lambda a: synth.to_torch(a, "cuda")
    x, lg, W1, W2, dout = t(inp["x"]), t(inp["logits"]), t(inp["W1"]), t(inp["W2"]), t(inp["dOut"])
    W1p, _ = ops.moe_repack_glu_weights(W1)
    L = MoEFFN(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, score="sigmoid", gemm="mxfp4")
    Wmx = MoEFFN.mx_weights(W1p, W2, "mxfp4")
    L.forward(x, lg, Wmx, None)
    L.backward(dout, lg, Wmx, None)
    torch.cuda.synchronize()

    f64 = lambda a: synth.bf16_bits_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a
    spec = om.LayerSpec(cfg.k, "sigmoid", True, "swiglu", store="bf16", gemm="mxfp4")
    fwd = om.layer_forward(f64(inp["x"]), inp["logits"], f64(inp["W1"]), f64(inp["W2"]), spec=spec)
    bwd = om.layer_backward(fwd, f64(inp["dOut"]), inp["logits"], f64(inp["W1"]), f64(inp["W2"]),
                            spec=spec)
    np.testing.assert_array_equal(host(L.topk_idx), fwd["topk_idx"])
    np.testing.assert_array_equal(host(L.pad_offsets), fwd["pad_offsets"])
    dW1 = om.unpack_glu(host(L.dW1p), None, G)
    rep = {"out": mx_errors(host(L.out), fwd["out_exact"], bf16=True),
           "dX": mx_errors(host(L.dX), bwd["dX_exact"], bf16=True),
           "dW1": mx_errors(dW1, bwd["dW1"]), "dW2": mx_errors(host(L.dW2), bwd["dW2"]),
           "dgate": mx_errors(host(L.dgate), bwd["dgate"]),
           "dlogits": mx_errors(host(L.dlogits), bwd["dlogits"])}
    print("mxfp4 layer", case, {k_: f"rms {a:.2e} max {b:.2e}" for k_, (a, b) in rep.items()},
          flush=True)
    for name, (r_, mx) in rep.items():
        assert r_ <= 1e-4 and mx <= 2e-2, (name, rep)
