"""GPU parity of the MXFP8 path (E4M3 elements, E8M0 scale per 32).

* Quantizers (row copy, transposed weight copy, expert-segmented row / column
  copies with gather and gate product): bit-exact against oracle.mx on the
  same float32 values.
* MXFP8 grouped GEMMs: against float64 products of the GPU's own quantized
  operands (decoded by oracle.mx); bf16 outputs by their excess over bf16
  rounding (<= 5e-3 of the rms), float32 weight gradients by max |err| / rms.
* MXFP8 epilogue outputs (A of FC1, dH of the dGLU) are quantized on the GPU
  from float32 values that the scaled fp8 MFMA accumulates with about 2^-13
  relative precision per instruction (measured on the device: 7.7e-3 absolute
  on 64-term sums of magnitude 136, against 7.6e-6 for a float32 sum); the
  oracle quantizes float64 values.  A value that close to an E4M3 rounding
  midpoint may round either way, so each GPU element must be within half an
  E4M3 quantum of the exact value plus 2^-9 of its block's largest magnitude,
  scales within one code, and codes different from the oracle's in at most 1 %
  of elements (about 0.14 % measured).
* The layer's MXFP8 variant against the oracle's MXFP8 chain, routing and
  padded offsets bit-exact.  Those isolated one-step flips of A and dH move a
  downstream output by at most one E4M3 step of one term, which at small
  widths (f = 256) is up to ~0.1 of the rms; so the unconditioned small layer
  is held to rms(err) / rms <= 5e-3 (bf16 outputs beyond their own rounding)
  and max |err| / rms <= 0.25.  Every element of the layers (f = 256 and
  f = 1024, MXFP8 and MXFP4) meets the plain 2e-2 max-abs bound against the
  oracle chain conditioned on the GPU's validated A / dH codes
  (test_mx_layer_every_element, tests/mx_chain.py); so does the full-size
  workload on 512 tokens and whole weight-gradient columns
  (test_gpu_fullsize.py).
"""
import numpy as np
import pytest
import torch

import synth
from gpu_util import bf16_excess, dev, host, norm_err, note, offsets_of, rand_bf16, rel_l2
from oracle import moe as om
from oracle import mx as omx

pytestmark = pytest.mark.gpu
G = 32


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


def deq(m, rows=None, cols=None):
    """float64 values of an MXTensor (optionally a [rows, cols] window)."""
    c, s = u8(m.data), u8(m.scale)
    v = omx.mx_dequantize_blocks(c, s)
    if rows is not None:
        v = v[:rows]
    if cols is not None:
        v = v[:, :cols]
    return v


def wide_values(rng, rows, n, dtype):
    """Rows at scales 2^-30 .. 2^30, with an all-zero block, a tiny block and
    blocks whose maximum sits exactly on a power of two."""
    v = rng.standard_normal((rows, n)).astype(np.float32)
    v *= np.float32(2.0) ** rng.integers(-30, 30, size=(rows, 1)).astype(np.float32)
    v[0, :32] = 0.0
    if rows > 1:
        v[1, 32:64] *= np.float32(2.0 ** -100)
    if rows > 2 and n >= 96:
        v[2, 64:96] = np.float32(448.0) * np.float32(2.0 ** 5) * np.sign(v[2, 64:96])
        v[2, 70] = np.float32(2.0 ** 14)
    if dtype == "bf16":
        bits = synth.f32_to_bf16_bits(v)
        return synth.bf16_bits_to_f32(bits).astype(np.float64), synth.to_torch(bits, "cuda")
    return v.astype(np.float64), synth.to_torch(v, "cuda")


def pad_of(counts):
    return om.pad_offsets(np.asarray(counts))


# ------------------------------------------------------------------ quantizers

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rows,n", [(37, 256), (5, 2048)])
def test_quantize_rows_bitexact(dtype, rows, n):
    note(f"mx quantize rows {dtype} {rows}x{n}")
    rng = np.random.default_rng(rows + n)
    x64, xd = wide_values(rng, rows, n, dtype)
    out = ops_().moe_mx_quantize(xd)
    torch.cuda.synchronize()
    c, s = omx.mx_quantize_blocks(x64)
    np.testing.assert_array_equal(u8(out.data), c)
    np.testing.assert_array_equal(u8(out.scale), s)


def _tie_blocks(fmt):
    """float32 blocks of 32 whose largest magnitude puts the block scale at
    2^0 (E4M3: 448 leads; E2M1: 6 leads), the other 31 values walking every
    rounding tie of the element format (normal and subnormal) and the float32
    neighbours on both sides, the saturation range and signed zeros; each
    pattern block also appears scaled by 2^k for k in -24 .. 24 (same codes,
    other scale).  NaN is not included: a block holding one has no agreed
    scale (the oracle's maximum is NaN, the device's ignores it)."""
    f32 = np.float32
    vals = []
    if fmt == "e4m3":
        for E in range(-6, 9):                       # normal binades
            for m in range(8):
                t = (1.0 + (2 * m + 1) / 16.0) * 2.0 ** E  # tie between m and m + 1
                if t < 448.0:
                    vals.append(t)
        for j in range(8):                           # subnormal ties: quantum 2^-9
            vals.append((2 * j + 1) * 2.0 ** -10)
        vals += [448.0, 449.0, 463.999, 464.0, 470.0, 500.0, 511.99]
        lead = 448.0
    else:
        vals += [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 6.5, 7.0, 7.99]
        lead = 6.0
    vals = np.asarray(vals, dtype=f32)
    nb = np.concatenate([np.nextafter(vals, f32(0)), vals, np.nextafter(vals, f32(np.inf))])
    nb = np.concatenate([nb, -nb, np.array([0.0, -0.0], dtype=f32)])
    pad = (-len(nb)) % 31
    nb = np.concatenate([nb, np.zeros(pad, dtype=f32)]).reshape(-1, 31)
    blocks = np.concatenate([np.full((len(nb), 1), lead, dtype=f32), nb], axis=1)
    scaled = [blocks * f32(2.0 ** k) for k in range(-24, 25, 4)]
    return np.concatenate(scaled).reshape(1, -1).astype(np.float32)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_quantize_rounding_ties_bitexact(fmt):
    note(f"mx quantize ties {fmt}")
    x = _tie_blocks(fmt)
    n = x.shape[1] // 128 * 128
    x = x[:, :n]
    out = ops_().moe_mx_quantize(synth.to_torch(x, "cuda"), fmt=fmt)
    torch.cuda.synchronize()
    c, s = omx.mx_quantize_blocks(x.astype(np.float64), fmt=fmt)
    got = u8(out.data)
    if fmt == "e2m1":
        got = omx.unpack_fp4(got)
    np.testing.assert_array_equal(got, c)
    np.testing.assert_array_equal(u8(out.scale), s)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quantize_transpose_bitexact(dtype):
    note(f"mx quantize transpose {dtype}")
    rng = np.random.default_rng(3)
    B, rows, n = 3, 64, 96
    x64, xd = wide_values(rng, B * rows, n, dtype)
    out = ops_().moe_mx_quantize_transpose(xd.reshape(B, rows, n))
    torch.cuda.synchronize()
    ref = np.concatenate([x64.reshape(B, rows, n)[b].T for b in range(B)])
    c, s = omx.mx_quantize_blocks(ref)
    np.testing.assert_array_equal(u8(out.data), c)
    np.testing.assert_array_equal(u8(out.scale), s)


def _routing(T, E, k, seed, empty=(1,)):
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits += (-1.5 * np.log(np.arange(1, E + 1))).astype(np.float32)
    for e in empty:
        logits[:, e] -= 30.0
    lg = synth.to_torch(logits, "cuda")
    ops = ops_()
    idx, w = ops.moe_route_topk(lg, k, "sigmoid", True)
    counts, offsets, pad, row_map, src_row, _ = ops.moe_permute(None, idx, E, gather=False,
                                                                want_pad=True)
    return idx, w, offsets, pad, row_map, src_row


@pytest.mark.parametrize("n", [256, 352])
@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quantize_experts_bitexact(gated, dtype, n):
    """Row and segment-column copies of x[src_row] (* gate), straight from x;
    n = 352 leaves the second 256-column chunk three blocks wide."""
    note(f"mx quantize experts gated={gated} {dtype} n={n}")
    T, E, k = 300, 6, 2
    idx, w, offsets, pad, row_map, src_row = _routing(T, E, k, 5)
    rng = np.random.default_rng(7)
    x64, xd = wide_values(rng, T, n, dtype)
    R = T * k
    kw = dict(src_row=src_row)
    if gated:
        kw.update(row_map=row_map, topk_w=w)
    row, col = ops_().moe_mx_quantize_experts(xd, offsets, pad, R, **kw)
    torch.cuda.synchronize()
    src = host(src_row)
    v = x64[src]
    if gated:
        rm, wt = host(row_map).reshape(-1), host(w).reshape(-1)
        wr = np.empty(R)
        wr[rm] = wt
        # the float32 product the kernel forms
        v = (v.astype(np.float32) * wr.astype(np.float32)[:, None]).astype(np.float64)
    c, s = omx.mx_quantize_blocks(v)
    np.testing.assert_array_equal(u8(row.data), c)
    np.testing.assert_array_equal(u8(row.scale), s)
    off, pd = host(offsets), host(pad)
    assert int(pd[-1]) <= col.ld
    cc, cs = omx.mx_quantize_segments_colwise(v, off, pd)
    Rp = int(pd[-1])
    np.testing.assert_array_equal(u8(col.data)[:, :Rp], cc)
    np.testing.assert_array_equal(u8(col.scale)[:, :Rp // 32], cs)


# ------------------------------------------------------------------ GEMMs

COUNTS_SMALL = [0, 1, 31, 32, 33, 255, 256, 257, 0, 130]
COUNTS_BIG = [0, 700, 1300, 300, 513]


def _mx_close(gc, gs, oc, os_, exact, what):
    """GPU codes/scales vs the oracle's codes of the exact values (blocks of 32
    along the last axis of all five arrays)."""
    gc, gs, oc, os_ = (np.asarray(a, np.int64) for a in (gc, gs, oc, os_))
    sd = gs != os_
    assert np.all(np.abs(gs - os_) <= 1), what
    assert sd.mean() <= 1e-3, (what, "scale flips", sd.mean())
    rows, n = gc.shape
    # each GPU element against the exact value in the GPU's own block scale
    # (where the scale flipped, the two sides saturate at different points)
    sc = np.ldexp(1.0, np.repeat(gs, 32, axis=1) - 127)
    v = np.clip(np.asarray(exact, np.float64) / sc, -448.0, 448.0)
    g = omx.mx_dequantize_blocks(gc, gs) / sc
    bmax = np.repeat(np.abs(v).reshape(rows, n // 32, 32).max(-1), 32, axis=1)
    a = np.abs(v)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    half = 0.5 * np.ldexp(1.0, np.maximum(ex - 4, -9))     # half an E4M3 quantum at |v|
    dev_ = np.abs(g - v) - half
    # values much smaller than their block maximum carry the MFMA's absolute
    # error (relative to the products, not to the value): rare beyond 2^-9
    assert (dev_ > 2.0 ** -9 * bmax).mean() <= 1e-5, (what, int((dev_ > 2.0 ** -9 * bmax).sum()))
    assert not (dev_ > 2.0 ** -4 * bmax).any(), (what, np.argwhere(dev_ > 2.0 ** -4 * bmax)[:5])
    flips = (gc != oc)[~np.repeat(sd, 32, axis=1)].mean()
    assert flips <= 1e-2, (what, "element flips", flips)
    return sd.mean(), flips


def _seg_cols(v, off, pad):
    """[R, n] values laid out like a column copy: [n, pad[-1]], zero padding."""
    out = np.zeros((v.shape[1], int(pad[-1])))
    for e in range(len(off) - 1):
        c = int(off[e + 1] - off[e])
        out[:, pad[e]:pad[e] + c] = v[off[e]:off[e + 1]].T
    return out


def _check_col_padding(codes, off, pad):
    for e in range(len(off) - 1):
        c = int(off[e + 1] - off[e])
        assert not codes[:, pad[e] + c:pad[e + 1]].any(), ("padding not zero", e)


def _unpack_cols(f):
    pos = om.glu_pack_rows(f, G)          # packed position of canonical column
    return pos[:f], pos[f:]


def _row_scales(rng, R):
    """Feature-scaling factors (a zero among them), float64 and on the GPU."""
    s = rng.uniform(0.05, 1.0, R).astype(np.float32)
    s[::7] = 0.0
    return s.astype(np.float64), synth.to_torch(s, "cuda")


@pytest.mark.parametrize("scaled", [False, True], ids=["plain", "row_scale"])
@pytest.mark.parametrize("counts,d,f", [(COUNTS_SMALL, 256, 256), (COUNTS_BIG, 1024, 512)])
def test_mx_glu_fwd(counts, d, f, scaled):
    note(f"mx glu fwd counts={counts} d={d} f={f} scaled={scaled}")
    ops = ops_()
    rng = np.random.default_rng(11)
    E, R, n1 = len(counts), sum(counts), 2 * f
    off = offsets_of(counts)
    pad = pad_of(counts)
    _, xd = rand_bf16(rng, (R, d))
    _, wd = rand_bf16(rng, (E, n1, d), d ** -0.5)
    sh, sd = _row_scales(rng, R) if scaled else (None, None)
    xq, wq = ops.moe_mx_quantize(xd), ops.moe_mx_quantize(wd.reshape(E * n1, d))
    (a_row, a_col), H = ops.moe_grouped_gemm_glu_fwd(xq, wq, dev(off), E=E, f=f,
                                                    pad_offsets=dev(pad), row_scale=sd)
    torch.cuda.synchronize()
    X, W = deq(xq), deq(wq).reshape(E, n1, d)
    Href = np.concatenate([X[off[e]:off[e + 1]] @ W[e].T for e in range(E)])
    assert bf16_excess(host(H), Href) <= 5e-3
    gpos, lpos = _unpack_cols(f)
    A = om.glu_forward(Href[:, gpos], Href[:, lpos], "swiglu")
    if scaled:
        A = om.row_scale_forward(A, sh)
    oc, os_ = omx.mx_quantize_blocks(A)
    _mx_close(u8(a_row.data), u8(a_row.scale), oc, os_, A, "A row copy")
    cc, cs = omx.mx_quantize_segments_colwise(A, off, pad)
    Rp = int(pad[-1])
    _mx_close(u8(a_col.data)[:, :Rp], u8(a_col.scale)[:, :Rp // 32], cc, cs, _seg_cols(A, off, pad),
              "A column copy")
    _check_col_padding(u8(a_col.data), off, pad)


@pytest.mark.parametrize("counts,N,K", [(COUNTS_SMALL, 256, 256), (COUNTS_BIG, 1024, 512),
                                        (COUNTS_BIG, 2048, 128)])
def test_mx_gemm_fwd(counts, N, K):
    note(f"mx gemm fwd counts={counts} N={N} K={K}")
    ops = ops_()
    rng = np.random.default_rng(12)
    E, R = len(counts), sum(counts)
    off = offsets_of(counts)
    _, ad = rand_bf16(rng, (R, K))
    _, wd = rand_bf16(rng, (E, N, K), K ** -0.5)
    aq, wq = ops.moe_mx_quantize(ad), ops.moe_mx_quantize(wd.reshape(E * N, K))
    y = ops.moe_grouped_gemm_fwd(aq, wq, dev(off), E=E, N=N)
    torch.cuda.synchronize()
    Aq, Wq = deq(aq), deq(wq).reshape(E, N, K)
    ref = np.concatenate([Aq[off[e]:off[e + 1]] @ Wq[e].T for e in range(E)])
    assert bf16_excess(host(y), ref) <= 5e-3


@pytest.mark.parametrize("scaled", [False, True], ids=["plain", "row_scale"])
@pytest.mark.parametrize("counts,d,f", [(COUNTS_SMALL, 256, 256), (COUNTS_BIG, 1024, 512),
                                        (COUNTS_BIG, 256, 1024)])
def test_mx_glu_bwd(counts, d, f, scaled):
    note(f"mx glu bwd counts={counts} d={d} f={f} scaled={scaled}")
    ops = ops_()
    rng = np.random.default_rng(13)
    E, R, n1 = len(counts), sum(counts), 2 * f
    off = offsets_of(counts)
    pad = pad_of(counts)
    _, dyd = rand_bf16(rng, (R, d))
    _, w2d = rand_bf16(rng, (E, d, f), d ** -0.5)
    h64, hd = rand_bf16(rng, (R, n1))
    sh, sd = _row_scales(rng, R) if scaled else (None, None)
    ds = torch.empty((R,), dtype=torch.float32, device="cuda") if scaled else None
    dyq, w2t = ops.moe_mx_quantize(dyd), ops.moe_mx_quantize_transpose(w2d)
    dh_row, dh_col = ops.moe_grouped_gemm_glu_bwd(dyq, w2t, hd, dev(off), E=E,
                                                  pad_offsets=dev(pad), row_scale=sd,
                                                  d_row_scale=ds)
    torch.cuda.synchronize()
    DY, W2T = deq(dyq), deq(w2t).reshape(E, f, d)
    dA = np.concatenate([DY[off[e]:off[e + 1]] @ W2T[e].T for e in range(E)])
    gpos, lpos = _unpack_cols(f)
    if scaled:
        dA, ds_ref = om.row_scale_backward(
            dA, om.glu_forward(h64[:, gpos], h64[:, lpos], "swiglu"), sh)
        # dA from the scaled fp8 / fp4 MFMA, whose accumulation is coarser than
        # float32 (as for the MX weight gradients: max |err| / rms <= 1e-3)
        assert rel_l2(host(ds), ds_ref) <= 1e-4 and norm_err(host(ds), ds_ref) <= 1e-3, \
            (rel_l2(host(ds), ds_ref), norm_err(host(ds), ds_ref))
    dg, dl = om.glu_backward(dA, h64[:, gpos], h64[:, lpos], "swiglu")
    dH = np.empty((R, n1))
    dH[:, gpos], dH[:, lpos] = dg, dl
    oc, os_ = omx.mx_quantize_blocks(dH)
    _mx_close(u8(dh_row.data), u8(dh_row.scale), oc, os_, dH, "dH row copy")
    cc, cs = omx.mx_quantize_segments_colwise(dH, off, pad)
    Rp = int(pad[-1])
    _mx_close(u8(dh_col.data)[:, :Rp], u8(dh_col.scale)[:, :Rp // 32], cc, cs,
              _seg_cols(dH, off, pad), "dH column copy")
    _check_col_padding(u8(dh_col.data), off, pad)


@pytest.mark.parametrize("counts,N,K", [(COUNTS_SMALL, 512, 256), (COUNTS_BIG, 1024, 1024)])
def test_mx_gemm_dgrad(counts, N, K):
    note(f"mx dgrad counts={counts} N={N} K={K}")
    ops = ops_()
    rng = np.random.default_rng(14)
    E, R = len(counts), sum(counts)
    off = offsets_of(counts)
    _, gd = rand_bf16(rng, (R, N))
    _, wd = rand_bf16(rng, (E, N, K), N ** -0.5)
    gq, wt = ops.moe_mx_quantize(gd), ops.moe_mx_quantize_transpose(wd)
    da = ops.moe_grouped_gemm_bwd(gq, dev(off), mode="dgrad", w=wt, E=E, K=K)
    torch.cuda.synchronize()
    Gq, WT = deq(gq), deq(wt).reshape(E, K, N)
    ref = np.concatenate([Gq[off[e]:off[e + 1]] @ WT[e].T for e in range(E)])
    assert bf16_excess(host(da), ref) <= 5e-3


@pytest.mark.parametrize("counts,N,K", [(COUNTS_SMALL, 512, 256), (COUNTS_BIG, 1024, 1024)])
def test_mx_gemm_wgrad(counts, N, K):
    note(f"mx wgrad counts={counts} N={N} K={K}")
    ops = ops_()
    rng = np.random.default_rng(15)
    E, R = len(counts), sum(counts)
    off, pad = offsets_of(counts), pad_of(counts)
    _, gd = rand_bf16(rng, (R, N))
    _, ad = rand_bf16(rng, (R, K))
    doff, dpad = dev(off), dev(pad)
    _, gc = ops.moe_mx_quantize_experts(gd, doff, dpad, R, want_row=False)
    _, ac = ops.moe_mx_quantize_experts(ad, doff, dpad, R, want_row=False)
    dw = ops.moe_grouped_gemm_bwd(gc, doff, mode="wgrad", a=ac, E=E, R=R, pad_offsets=dpad)
    # accumulating onto zeros takes the direct float32 stores, the plain call
    # the whole rows staged through LDS: the same values
    dw0 = torch.zeros_like(dw)
    ops.moe_grouped_gemm_bwd(gc, doff, mode="wgrad", a=ac, E=E, R=R, pad_offsets=dpad, out=dw0,
                             accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(dw, dw0)
    Gc, Ac = deq(gc), deq(ac)
    got = host(dw)
    for e in range(E):
        c = counts[e]
        if c == 0:
            assert not np.any(got[e]), e
            continue
        ref = Gc[:, pad[e]:pad[e] + c] @ Ac[:, pad[e]:pad[e] + c].T
        assert norm_err(got[e], ref) <= 1e-3, (e, norm_err(got[e], ref), rel_l2(got[e], ref))


# ------------------------------------------------------------------ layer

def mx_errors(g, o, bf16=False):
    """(rms, max) of |g - o| / rms(o); bf16 results measured beyond their own
    half-ulp rounding."""
    from gpu_util import half_ulp_bf16, rms
    g, o = np.asarray(g, np.float64), np.asarray(o, np.float64)
    e = np.abs(g - o)
    if bf16:
        e = np.maximum(e - half_ulp_bf16(o), 0.0)
    r = rms(o)
    return rms(e) / r, float(e.max()) / r


# The unconditioned comparison at f = 256: one isolated flip of a large A or
# dH code moves an output by one E4M3 step of one of only 256 terms, up to
# ~0.1 of the rms, so it is held to rms(err) / rms <= 5e-3 and max <= 0.25.
# The stated 2e-2 bound is checked over every element by
# test_mx_layer_every_element (conditioned on the GPU's codes).
LAYER_CASES = [
    dict(T=512, d=256, f=256, E=8, k=2, zipf=1.2, forced_empty=1, seed=21),
]


@pytest.mark.parametrize("gate_in_act", [False, True], ids=["gates_in_combine", "gate_in_act"])
@pytest.mark.parametrize("case", LAYER_CASES, ids=lambda c: f"T{c['T']}d{c['d']}f{c['f']}E{c['E']}")
def test_mx_layer_vs_oracle(case, gate_in_act):
    note(f"mx layer {case} gate_in_act={gate_in_act}")
    from ragged_grouped_gemm_amd.layer import MoEFFN
    ops = ops_()
    cfg = synth.MoEConfig("mx_layer", gemm="mxfp8", score="sigmoid", backward=True, **case)
    inp = synth.make_inputs(cfg)
    t = lambda a: synth.to_torch(a, "cuda")
    x, lg, W1, W2, dout = t(inp["x"]), t(inp["logits"]), t(inp["W1"]), t(inp["W2"]), t(inp["dOut"])
    W1p, _ = ops.moe_repack_glu_weights(W1)
    L = MoEFFN(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, score="sigmoid", gemm="mxfp8",
               gate_in_act=gate_in_act)
    Wmx = MoEFFN.mx_weights(W1p, W2)
    L.forward(x, lg, Wmx, None)
    L.backward(dout, lg, Wmx, None)
    torch.cuda.synchronize()

    f64 = lambda a: synth.bf16_bits_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a
    spec = om.LayerSpec(cfg.k, "sigmoid", True, "swiglu", store="bf16", gemm="mxfp8",
                        gate_in_act=gate_in_act)
    fwd = om.layer_forward(f64(inp["x"]), inp["logits"], f64(inp["W1"]), f64(inp["W2"]), spec=spec)
    bwd = om.layer_backward(fwd, f64(inp["dOut"]), inp["logits"], f64(inp["W1"]), f64(inp["W2"]),
                            spec=spec)
    np.testing.assert_array_equal(host(L.topk_idx), fwd["topk_idx"])
    np.testing.assert_array_equal(host(L.offsets), fwd["offsets"])
    np.testing.assert_array_equal(host(L.pad_offsets), fwd["pad_offsets"])
    dW1 = om.unpack_glu(host(L.dW1p), None, G)
    rep = {"out": mx_errors(host(L.out), fwd["out_exact"], bf16=True),
           "dX": mx_errors(host(L.dX), bwd["dX_exact"], bf16=True),
           "dW1": mx_errors(dW1, bwd["dW1"]), "dW2": mx_errors(host(L.dW2), bwd["dW2"]),
           "dgate": mx_errors(host(L.dgate), bwd["dgate"]),
           "dlogits": mx_errors(host(L.dlogits), bwd["dlogits"])}
    print("mx layer", case, {k_: f"rms {a:.2e} max {b:.2e}" for k_, (a, b) in rep.items()},
          flush=True)
    for name, (r_, mx) in rep.items():
        assert r_ <= 5e-3 and mx <= 0.25, (name, rep)


# Mid-width layers held to the stated bound over every element: the oracle
# chain conditioned on the GPU's own A / dH codes (each checked to be a valid
# rounding of the exact value first), so a code that may round either way no
# longer decides the comparison (tests/mx_chain.py).  The unconditioned
# oracle chain is printed beside it.
MID_CASES = [
    dict(T=2048, d=2048, f=1024, E=8, k=4, zipf=1.2, forced_empty=1, seed=23),
    dict(T=512, d=256, f=256, E=8, k=2, zipf=1.2, forced_empty=1, seed=21),
]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
@pytest.mark.parametrize("case", MID_CASES, ids=lambda c: f"T{c['T']}d{c['d']}f{c['f']}E{c['E']}")
def test_mx_layer_every_element(case, fmt):
    import mx_chain
    gemm = "mxfp4" if fmt == "e2m1" else "mxfp8"
    note(f"mx layer every element {gemm} {case}")
    from ragged_grouped_gemm_amd.layer import MoEFFN
    ops = ops_()
    cfg = synth.MoEConfig("mx_mid", gemm=gemm, score="sigmoid", backward=True, **case)
    inp = synth.make_inputs(cfg)
    t = lambda a: synth.to_torch(a, "cuda")
    x, lg, W1, W2, dout = t(inp["x"]), t(inp["logits"]), t(inp["W1"]), t(inp["W2"]), t(inp["dOut"])
    W1p, _ = ops.moe_repack_glu_weights(W1)
    L = MoEFFN(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, score="sigmoid", gemm=gemm)
    Wmx = MoEFFN.mx_weights(W1p, W2, gemm)
    L.forward(x, lg, Wmx, None)
    L.backward(dout, lg, Wmx, None)
    torch.cuda.synchronize()
    got, cond, plain, dec = mx_chain.conditioned_layer(inp, L, fmt, cfg.k, "sigmoid", True)
    rep, rep_plain = {}, {}
    for name in got:
        bf16 = name in ("out", "dX")
        rep[name] = mx_errors(got[name], cond[name], bf16=bf16)
        rep_plain[name] = mx_errors(got[name], plain[name], bf16=bf16)
    fmt_dec = lambda v: f"{v[0]:.1e}/{v[1]:.1e}" if isinstance(v, tuple) else f"{v:.2f} ulp"
    print(f"{gemm} layer {case}: decisions (scale/element flips, bf16 ulps)",
          {k_: fmt_dec(v) for k_, v in dec.items()},
          "conditioned", {k_: f"rms {a:.2e} max {b:.2e}" for k_, (a, b) in rep.items()},
          "unconditioned", {k_: f"rms {a:.2e} max {b:.2e}" for k_, (a, b) in rep_plain.items()},
          flush=True)
    for name, (r_, mx) in rep.items():
        assert mx <= 2e-2 and r_ <= 1e-3, (name, rep)
