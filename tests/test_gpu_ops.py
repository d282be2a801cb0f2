"""Per-entry-point parity of the HIP library against the CPU oracle.

Each test feeds the same seeded inputs to a library call (through the C ABI)
and to the oracle, then compares: integer and index outputs bit for bit;
float32 outputs by relative L2 error <= 1e-5 (max |err| / rms <= 1e-4 too);
bf16 outputs by their max error beyond their own bf16 rounding, / rms
(<= 5e-3 here, a quarter of the layer tolerance).
Expert segment sizes include empty experts and tails around the tile sizes."""
import numpy as np
import pytest
import torch

import synth
from oracle import moe as om
from gpu_util import (bf16_excess, dev, host, norm_err, note, offsets_of, rand_bf16, rand_f32,
                      rel_l2)

pytestmark = pytest.mark.gpu

ops = None


@pytest.fixture(scope="module", autouse=True)
def _lib():
    global ops
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from ragged_grouped_gemm_amd import ops as _ops
    ops = _ops
    ops.moe_version()


TOL_BF16 = 2e-2
TOL_F32 = 1e-5
TOL_F32_MAX = 1e-4


G = 32


def f32_ok(got, ref):
    return rel_l2(got, ref) <= TOL_F32 and norm_err(got, ref) <= TOL_F32_MAX


# ragged segment sizes around the 128 / 256 tile heights, with empty experts
COUNTS_SMALL = [0, 1, 31, 32, 33, 255, 256, 257, 0, 130]
COUNTS_BIG = [0, 700, 1300, 300, 513]


# ------------------------------------------------------------------ routing

@pytest.mark.parametrize("score", ["softmax", "sigmoid"])
@pytest.mark.parametrize("normalize", [True, False])
@pytest.mark.parametrize("E,k", [(8, 2), (32, 8), (5, 5), (64, 1), (40, 12)])
def test_route_topk(score, normalize, E, k):
    note(f"route_topk {score} norm={normalize} E={E} k={k}")
    rng = np.random.default_rng(E * 100 + k)
    T = 1000
    lg = rng.standard_normal((T, E)).astype(np.float32)
    lg[::3] = np.round(lg[::3] * 2) / 2          # many exact ties
    lg[5, :] = 0.25                              # a row of all-equal logits
    idx_o, w_o, _ = om.route_topk(lg, k, score, normalize)
    idx, w = ops.moe_route_topk(dev(lg), k, score, normalize)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(idx), idx_o)
    assert f32_ok(host(w), w_o)
    np.testing.assert_allclose(host(w), w_o, rtol=2e-6, atol=1e-7)


def test_route_nan_sets_error_bit():
    note("route_topk NaN")
    lg = np.zeros((4, 6), np.float32)
    lg[1, 2] = np.nan
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    idx, _ = ops.moe_route_topk(dev(lg), 2, err_word=err)
    torch.cuda.synchronize()
    assert int(err.item()) & 1
    idx_o, _, nan = om.route_topk(lg, 2)
    assert nan
    np.testing.assert_array_equal(host(idx), idx_o)


@pytest.mark.parametrize("score", ["softmax", "sigmoid"])
@pytest.mark.parametrize("normalize", [True, False])
def test_route_topk_bwd(score, normalize):
    note(f"route_topk_bwd {score} norm={normalize}")
    rng = np.random.default_rng(7)
    T, E, k = 777, 16, 4
    lg = rng.standard_normal((T, E)).astype(np.float32)
    dw = rng.standard_normal((T, k)).astype(np.float32)
    idx_o, _, _ = om.route_topk(lg, k, score, normalize)
    ref = om.route_topk_bwd(lg, idx_o, dw, score, normalize)
    got = ops.moe_route_topk_bwd(dev(lg), dev(idx_o.astype(np.int32)), dev(dw), score, normalize)
    torch.cuda.synchronize()
    assert f32_ok(host(got), ref)


# ------------------------------------------------------------------ permute

@pytest.mark.parametrize("T,E,k,skew", [(1000, 8, 2, 1.0), (4096, 32, 8, 1.5), (333, 1, 1, 0.0),
                                        (257, 7, 7, 0.0), (5000, 64, 3, 2.0), (1, 4, 2, 0.0)])
def test_permute_bitexact(T, E, k, skew):
    note(f"permute T={T} E={E} k={k}")
    cfg = synth.MoEConfig("t", T=T, d=64, f=32, E=E, k=k, zipf=skew, seed=T + E,
                          forced_empty=1 if E > k else 0, forced_mode="top")
    inp = synth.make_inputs(cfg, parts=("x", "logits"))
    idx_o, _, _ = om.route_topk(inp["logits"], k)
    counts, off, row_map, src_row = om.permute_indices(idx_o, E)
    xp_o = inp["x"][src_row]                           # bf16 bit patterns, a pure copy
    c, o, po, rm, sr, xp = ops.moe_permute(synth.to_torch(inp["x"], "cuda"),
                                           dev(idx_o.astype(np.int32)), E, want_pad=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(c), counts)
    np.testing.assert_array_equal(host(o), off)
    np.testing.assert_array_equal(host(po), om.pad_offsets(counts))
    np.testing.assert_array_equal(host(rm), row_map)
    np.testing.assert_array_equal(host(sr), src_row)
    np.testing.assert_array_equal(xp.view(torch.int16).cpu().numpy().view(np.uint16), xp_o)


def test_permute_bad_expert_flagged():
    note("permute bad expert id")
    idx = np.array([[0, 1], [5, 1], [-1, 0]], np.int32)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    x = torch.zeros((3, 64), dtype=torch.bfloat16, device="cuda")
    c, o, _, rm, sr, _ = ops.moe_permute(x, dev(idx), 4, err_word=err)
    torch.cuda.synchronize()
    assert int(err.item()) & 2
    assert host(o)[-1] == 6 and sorted(host(rm).ravel().tolist()) == list(range(6))


# ------------------------------------------------------------------ repack

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_repack_roundtrip(dtype):
    note(f"repack {dtype}")
    rng = np.random.default_rng(3)
    E, f, d = 3, 96, 64
    Wh, Wd = (rand_bf16 if dtype == "bf16" else rand_f32)(rng, (E, 2 * f, d))
    bh, bd = rand_f32(rng, (E, 2 * f))
    Wp, bp = ops.moe_repack_glu_weights(Wd, bd)
    Wb, bb = ops.moe_repack_glu_weights(Wp, bp, inverse=True)
    torch.cuda.synchronize()
    ref_w, ref_b = om.repack_glu(Wh, bh, G=G)
    np.testing.assert_array_equal(host(Wp), ref_w)
    np.testing.assert_array_equal(host(bp), ref_b)
    np.testing.assert_array_equal(host(Wb), Wh)
    np.testing.assert_array_equal(host(bb), bh)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("E,rows,cols", [(3, 72, 200), (2, 64, 64), (5, 2880, 136)])
def test_transpose_weights(dtype, E, rows, cols):
    note(f"transpose_weights {dtype} E={E} {rows}x{cols}")
    rng = np.random.default_rng(rows + cols)
    mk = rand_bf16 if dtype == "bf16" else rand_f32
    wh, wd = mk(rng, (E, rows, cols))
    wt = ops.moe_transpose_weights(wd)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(wt), wh.transpose(0, 2, 1))   # a bit-exact copy


# ------------------------------------------------------------------ grouped GEMMs

def _setup(counts, seed):
    rng = np.random.default_rng(seed)
    off = offsets_of(counts)
    return rng, off, dev(off)


@pytest.mark.parametrize("counts,d,f", [(COUNTS_SMALL, 256, 256), (COUNTS_BIG, 1024, 512)])
@pytest.mark.parametrize("act,clamp,alpha,gtanh,bias", [
    ("swiglu", 0.0, 1.0, False, False), ("swiglu", 1.5, 1.0, False, True),
    ("swiglu", 0.0, 1.702, False, False), ("geglu", 0.0, 1.0, False, True),
    ("geglu", 0.0, 1.0, True, False), ("srelu", 0.0, 1.0, False, True),
    ("srelu", 0.5, 1.0, False, False)])
def test_glu_fwd_bf16(counts, d, f, act, clamp, alpha, gtanh, bias):
    note(f"glu_fwd bf16 R={sum(counts)} d={d} f={f} {act} clamp={clamp} a={alpha} tanh={gtanh}")
    rng, off, offd = _setup(counts, d + f)
    E, R = len(counts), int(off[-1])
    n1 = f if act == "srelu" else 2 * f
    xh, xd = rand_bf16(rng, (R, d))
    Wh, Wd = rand_bf16(rng, (E, n1, d), d ** -0.5)
    bh, bd = rand_f32(rng, (E, n1)) if bias else (None, None)
    if act == "srelu":
        Wpd, bpd = Wd, bd
    else:
        Wpd, bpd = ops.moe_repack_glu_weights(Wd, bd)
    A, H = ops.moe_grouped_gemm_glu_fwd(xd, Wpd, offd, b1p=bpd, act=act, clamp=clamp,
                                        alpha=alpha, gelu_tanh=gtanh)
    torch.cuda.synchronize()
    Hc = om.grouped_linear(xh, Wh, off, bh)
    if act == "srelu":
        Ao = om.srelu_forward(Hc, clamp)
        Hp = Hc
    else:
        Ao = om.glu_forward(Hc[:, :f], Hc[:, f:], act, clamp, alpha, gtanh)
        Hp = om.repack_glu(Hc[None], G=G, axis=2)[0]
    assert bf16_excess(host(H), Hp) <= TOL_BF16 / 4
    assert bf16_excess(host(A), Ao) <= TOL_BF16 / 4


@pytest.mark.parametrize("counts", [COUNTS_BIG, COUNTS_SMALL])
@pytest.mark.parametrize("act,clamp,gtanh,bias,scaled", [
    ("swiglu", 1.5, False, True, False), ("geglu", 0.0, True, False, True),
    ("swiglu", 0.0, False, False, True)])
def test_glu_fwd_h_saved_and_forward_only_agree(counts, act, clamp, gtanh, bias, scaled):
    """A with H saved equals, bit for bit, A of a forward-only call (which
    stages and writes A alone), at f = 352: 2f = 704 packed columns, so the
    last 256-column tile holds three live wave columns and one dead one;
    also against the oracle."""
    d, f = 512, 352
    note(f"glu_fwd staged vs direct R={sum(counts)} d={d} f={f} {act} scaled={scaled}")
    rng, off, offd = _setup(counts, 3 * d + f)
    E, R = len(counts), int(off[-1])
    xh, xd = rand_bf16(rng, (R, d))
    Wh, Wd = rand_bf16(rng, (E, 2 * f, d), d ** -0.5)
    bh, bd = rand_f32(rng, (E, 2 * f)) if bias else (None, None)
    sh = rng.uniform(0.1, 1.0, R) if scaled else None
    sd = torch.tensor(sh, dtype=torch.float32, device="cuda") if scaled else None
    Wpd, bpd = ops.moe_repack_glu_weights(Wd, bd)
    A1, H = ops.moe_grouped_gemm_glu_fwd(xd, Wpd, offd, b1p=bpd, act=act, clamp=clamp,
                                         gelu_tanh=gtanh, row_scale=sd)
    A0, none = ops.moe_grouped_gemm_glu_fwd(xd, Wpd, offd, b1p=bpd, act=act, clamp=clamp,
                                            gelu_tanh=gtanh, save_h=False, row_scale=sd)
    torch.cuda.synchronize()
    assert none is None
    assert torch.equal(A1.view(torch.int16), A0.view(torch.int16))
    Hc = om.grouped_linear(xh, Wh, off, bh)
    Ao = om.glu_forward(Hc[:, :f], Hc[:, f:], act, clamp, 1.0, gtanh)
    if scaled:
        Ao = om.row_scale_forward(Ao, sh.astype(np.float32).astype(np.float64))
    assert bf16_excess(host(H), om.repack_glu(Hc[None], G=G, axis=2)[0]) <= TOL_BF16 / 4
    assert bf16_excess(host(A1), Ao) <= TOL_BF16 / 4


@pytest.mark.parametrize("counts", [COUNTS_BIG, COUNTS_SMALL])
@pytest.mark.parametrize("act,clamp,gtanh", [("swiglu", 1.5, False), ("geglu", 0.0, True)])
def test_glu_bwd_staged_equals_direct(counts, act, clamp, gtanh):
    """dH without a feature scale (bf16: stored through LDS as whole rows)
    equals, bit for bit, dH with a unit feature scale (the kernel variant
    that also sums the scale's gradient, which stores dH directly), at f =
    352: the last 256-column tile holds three live wave columns and one dead
    one; also against the oracle."""
    d, f = 512, 352
    note(f"glu_bwd staged vs direct R={sum(counts)} d={d} f={f} {act} clamp={clamp}")
    rng, off, offd = _setup(counts, 7 * d + f)
    E, R = len(counts), int(off[-1])
    dyh, dyd = rand_bf16(rng, (R, d))
    w2h, w2d = rand_bf16(rng, (E, d, f), d ** -0.5)
    hh, hd = rand_bf16(rng, (R, 2 * f))
    dh0 = ops.moe_grouped_gemm_glu_bwd(dyd, w2d, hd, offd, act=act, clamp=clamp, gelu_tanh=gtanh)
    ones = torch.ones(R, dtype=torch.float32, device="cuda")
    ds = torch.empty(R, dtype=torch.float32, device="cuda")
    dh1 = ops.moe_grouped_gemm_glu_bwd(dyd, w2d, hd, offd, act=act, clamp=clamp, gelu_tanh=gtanh,
                                       row_scale=ones, d_row_scale=ds)
    torch.cuda.synchronize()
    assert torch.equal(dh0.view(torch.int16), dh1.view(torch.int16))
    dA = om.grouped_dgrad(dyh, w2h, off)
    hc = om.unpack_glu(hh[None], G=G, axis=2)[0]
    dg, dl = om.glu_backward(dA, hc[:, :f], hc[:, f:], act, clamp, 1.0, gtanh)
    ref = om.repack_glu(np.concatenate([dg, dl], 1)[None], G=G, axis=2)[0]
    assert bf16_excess(host(dh0), ref) <= TOL_BF16 / 4


@pytest.mark.parametrize("counts,d,f", [(COUNTS_SMALL, 128, 256), (COUNTS_BIG, 256, 512)])
@pytest.mark.parametrize("act,clamp", [("swiglu", 0.0), ("swiglu", 7.0), ("srelu", 0.0)])
def test_glu_fwd_f32(counts, d, f, act, clamp):
    note(f"glu_fwd f32 R={sum(counts)} {act} clamp={clamp}")
    rng, off, offd = _setup(counts, 11 + d)
    E, R = len(counts), int(off[-1])
    n1 = f if act == "srelu" else 2 * f
    xh, xd = rand_f32(rng, (R, d))
    Wh, Wd = rand_f32(rng, (E, n1, d), d ** -0.5)
    Wpd = Wd if act == "srelu" else ops.moe_repack_glu_weights(Wd)[0]
    A, H = ops.moe_grouped_gemm_glu_fwd(xd, Wpd, offd, act=act, clamp=clamp)
    torch.cuda.synchronize()
    Hc = om.grouped_linear(xh, Wh, off)
    if act == "srelu":
        Ao, Hp = om.srelu_forward(Hc, clamp), Hc
    else:
        Ao = om.glu_forward(Hc[:, :f], Hc[:, f:], act, clamp)
        Hp = om.repack_glu(Hc[None], G=G, axis=2)[0]
    assert f32_ok(host(H), Hp)
    assert f32_ok(host(A), Ao)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("counts,N,K,bias", [(COUNTS_SMALL, 256, 256, True),
                                             (COUNTS_SMALL, 200, 96, False),
                                             (COUNTS_BIG, 1024, 512, True),
                                             (COUNTS_BIG, 2880, 256, False)])
def test_gemm_fwd(dtype, counts, N, K, bias):
    note(f"gemm_fwd {dtype} R={sum(counts)} N={N} K={K}")
    rng, off, offd = _setup(counts, N + K)
    E, R = len(counts), int(off[-1])
    mk = rand_bf16 if dtype == "bf16" else rand_f32
    ah, ad = mk(rng, (R, K))
    wh, wd = mk(rng, (E, N, K), K ** -0.5)
    bh, bd = rand_f32(rng, (E, N)) if bias else (None, None)
    y = ops.moe_grouped_gemm_fwd(ad, wd, offd, b=bd)
    torch.cuda.synchronize()
    ref = om.grouped_linear(ah, wh, off, bh)
    if dtype == "bf16":
        assert bf16_excess(host(y), ref) <= TOL_BF16 / 4
    else:
        assert f32_ok(host(y), ref)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("counts,d,f", [(COUNTS_SMALL, 256, 256), (COUNTS_BIG, 1024, 512)])
@pytest.mark.parametrize("act,clamp", [("swiglu", 0.0), ("swiglu", 1.0), ("geglu", 0.0),
                                       ("srelu", 0.0)])
def test_glu_bwd(dtype, counts, d, f, act, clamp):
    note(f"glu_bwd {dtype} R={sum(counts)} d={d} f={f} {act} clamp={clamp}")
    rng, off, offd = _setup(counts, 5 * d + f)
    E, R = len(counts), int(off[-1])
    n1 = f if act == "srelu" else 2 * f
    mk = rand_bf16 if dtype == "bf16" else rand_f32
    dyh, dyd = mk(rng, (R, d))
    w2h, w2d = mk(rng, (E, d, f), d ** -0.5)
    hh, hd = mk(rng, (R, n1))          # saved pre-activation, packed layout
    dh = ops.moe_grouped_gemm_glu_bwd(dyd, w2d, hd, offd, act=act, clamp=clamp)
    # W2 transposed (both operands K-contiguous): the same products in the same order
    dh_t = ops.moe_grouped_gemm_glu_bwd(dyd, None, hd, offd, act=act, clamp=clamp,
                                        w2t=ops.moe_transpose_weights(w2d))
    torch.cuda.synchronize()
    assert torch.equal(dh, dh_t)
    dA = om.grouped_dgrad(dyh, w2h, off)
    if act == "srelu":
        ref = om.srelu_backward(dA, hh, clamp)
    else:
        hc = om.unpack_glu(hh[None], G=G, axis=2)[0]
        dg, dl = om.glu_backward(dA, hc[:, :f], hc[:, f:], act, clamp)
        ref = om.repack_glu(np.concatenate([dg, dl], 1)[None], G=G, axis=2)[0]
    if dtype == "bf16":
        assert bf16_excess(host(dh), ref) <= TOL_BF16 / 4
    else:
        assert f32_ok(host(dh), ref)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("counts,N,K", [(COUNTS_SMALL, 512, 256), (COUNTS_BIG, 1024, 1024),
                                        (COUNTS_SMALL, 96, 2880)])
def test_gemm_dgrad(dtype, counts, N, K):
    note(f"gemm dgrad {dtype} R={sum(counts)} N={N} K={K}")
    rng, off, offd = _setup(counts, 3 * N + K)
    E, R = len(counts), int(off[-1])
    mk = rand_bf16 if dtype == "bf16" else rand_f32
    gh, gd = mk(rng, (R, N))
    wh, wd = mk(rng, (E, N, K), N ** -0.5)
    da = ops.moe_grouped_gemm_bwd(gd, offd, mode="dgrad", w=wd)
    da_t = ops.moe_grouped_gemm_bwd(gd, offd, mode="dgrad", wt=ops.moe_transpose_weights(wd))
    torch.cuda.synchronize()
    assert torch.equal(da, da_t)
    ref = om.grouped_dgrad(gh, wh, off)
    if dtype == "bf16":
        assert bf16_excess(host(da), ref) <= TOL_BF16 / 4
    else:
        assert f32_ok(host(da), ref)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("counts,N,K", [(COUNTS_SMALL, 512, 256), (COUNTS_BIG, 1024, 1024),
                                        (COUNTS_SMALL, 2880, 96),
                                        ([0, 16352, 5, 129, 0, 1], 200, 64)])
def test_gemm_wgrad(dtype, counts, N, K):
    note(f"gemm wgrad {dtype} R={sum(counts)} N={N} K={K}")
    rng, off, offd = _setup(counts, N + 7 * K)
    E, R = len(counts), int(off[-1])
    mk = rand_bf16 if dtype == "bf16" else rand_f32
    gh, gd = mk(rng, (R, N))
    ah, ad = mk(rng, (R, K))
    dw, db = ops.moe_grouped_gemm_bwd(gd, offd, mode="wgrad", a=ad, want_db=True)
    # accumulate: a second call adds to the first result, bias gradient included
    dw2, db2 = dw.clone(), db.clone()
    ops.moe_grouped_gemm_bwd(gd, offd, mode="wgrad", a=ad, out=dw2, db=db2, accumulate=True)
    # accumulating onto zeros takes the direct float32 stores; the first call
    # (big bf16 tiles) stores whole rows through LDS: the same values
    dw3 = torch.zeros_like(dw)
    ops.moe_grouped_gemm_bwd(gd, offd, mode="wgrad", a=ad, out=dw3, accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(dw, dw3)
    ref, refb = om.grouped_wgrad(gh, ah, off, with_bias=True)
    got = host(dw)
    assert f32_ok(got, ref)
    assert f32_ok(host(db), refb)
    for e, c in enumerate(counts):
        if c == 0:
            assert not got[e].any() and not host(db)[e].any()     # exact zeros
    assert f32_ok(host(dw2), 2 * ref)
    assert f32_ok(host(db2), 2 * refb)


# ------------------------------------------------------------------ combine

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("T,E,k,d", [(1000, 8, 2, 256), (513, 32, 8, 2880), (64, 4, 4, 64)])
def test_combine_and_backward(dtype, T, E, k, d):
    note(f"combine {dtype} T={T} k={k} d={d}")
    rng = np.random.default_rng(T + d)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    idx, w, _ = om.route_topk(lg, k)
    _, _, row_map, _ = om.permute_indices(idx, E)
    w32 = w.astype(np.float32)
    mk = rand_bf16 if dtype == "bf16" else rand_f32
    yh, yd = mk(rng, (T * k, d))
    doh, dod = mk(rng, (T, d))
    rmd, wd = dev(row_map), dev(w32)
    out = ops.moe_unpermute_combine(yd, rmd, wd)
    unit = ops.moe_unpermute_combine(yd, rmd, None)
    dy, dgate = ops.moe_unpermute_combine_bwd(dod, yd, rmd, wd)
    torch.cuda.synchronize()
    ref = om.combine(yh, row_map, w32.astype(np.float64))
    ref_unit = om.combine(yh, row_map, None)
    rdy, rdg = om.combine_bwd(doh, yh, row_map, w32.astype(np.float64))
    if dtype == "bf16":
        assert bf16_excess(host(out), ref) <= 1e-3
        assert bf16_excess(host(unit), ref_unit) <= 1e-3
        assert bf16_excess(host(dy), rdy) <= 1e-3
    else:
        assert f32_ok(host(out), ref)
        assert f32_ok(host(unit), ref_unit)
        assert f32_ok(host(dy), rdy)
    assert f32_ok(host(dgate), rdg)


@pytest.mark.parametrize("k", [2, 4, 8])
def test_unpermute_of_permute_is_exact_multiple(k):
    """Unit-weight unpermute of the permuted rows gives k * x exactly (bf16)."""
    note(f"permute/unpermute round trip k={k}")
    cfg = synth.MoEConfig("t", T=700, d=256, f=32, E=16, k=k, zipf=1.0, seed=k)
    inp = synth.make_inputs(cfg, parts=("x", "logits"))
    xd = synth.to_torch(inp["x"], "cuda")
    idx, _ = ops.moe_route_topk(dev(inp["logits"]), k)
    _, _, _, rm, _, xp = ops.moe_permute(xd, idx, cfg.E)
    s = ops.moe_unpermute_combine(xp, rm, None)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(s), k * host(xd))


# ------------------------------------------------------------------ maximum sizes

@pytest.mark.parametrize("T,E,k", [(300, 1024, 32), (200, 32, 32), (500, 1024, 1)])
def test_route_and_permute_max_sizes(T, E, k):
    """E = MOE_MAX_EXPERTS and k = MOE_MAX_TOPK (and k = E): routing and the
    permutation bit-exact."""
    note(f"route+permute max sizes T={T} E={E} k={k}")
    rng = np.random.default_rng(T + E + k)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    lg[::4] = np.round(lg[::4] * 2) / 2          # ties
    for score in ("softmax", "sigmoid"):
        idx_o, w_o, _ = om.route_topk(lg, k, score, True)
        idx, w = ops.moe_route_topk(dev(lg), k, score, True)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(idx), idx_o)
        assert f32_ok(host(w), w_o)
    counts, off, row_map, src_row = om.permute_indices(idx_o, E)
    c, o, po, rm, sr, _ = ops.moe_permute(None, dev(idx_o.astype(np.int32)), E, gather=False,
                                          want_pad=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(c), counts)
    np.testing.assert_array_equal(host(o), off)
    np.testing.assert_array_equal(host(po), om.pad_offsets(counts))
    np.testing.assert_array_equal(host(rm), row_map)
    np.testing.assert_array_equal(host(sr), src_row)


def test_gemms_with_max_experts():
    """1024 experts, most of them empty, the rest with 1-40 rows: FC1 + GLU, the
    dgrad and the weight gradient against the oracle (empty experts exact zeros)."""
    note("gemms with E = 1024")
    rng = np.random.default_rng(1024)
    E, d, f = 1024, 128, 64
    counts = np.where(rng.random(E) < 0.7, 0, rng.integers(1, 41, E)).astype(np.int64)
    counts[-1] = 33
    rng, off, doff = _setup(list(counts), 9)
    R = int(off[-1])
    x64, xd = rand_bf16(rng, (R, d))
    w64, wd = rand_bf16(rng, (E, 2 * f, d), d ** -0.5)
    a, h = ops.moe_grouped_gemm_glu_fwd(xd, wd, doff)
    g64, gd = rand_bf16(rng, (R, 2 * f))
    da = ops.moe_grouped_gemm_bwd(gd, doff, mode="dgrad", w=wd)
    dw, _ = ops.moe_grouped_gemm_bwd(gd, doff, mode="wgrad", a=xd)
    torch.cuda.synchronize()
    H = om.grouped_linear(x64, w64, off)
    assert bf16_excess(host(h), H) <= 5e-3
    pos = om.glu_pack_rows(f, G)
    A = om.glu_forward(H[:, pos[:f]], H[:, pos[f:]], "swiglu")
    assert bf16_excess(host(a), A) <= 5e-3
    assert bf16_excess(host(da), om.grouped_dgrad(g64, w64, off)) <= 5e-3
    ref_dw = om.grouped_wgrad(g64, x64, off)
    got = host(dw)
    assert f32_ok(got, ref_dw)
    assert not np.any(got[counts == 0])
