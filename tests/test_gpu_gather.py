"""Gather-fused permute: FC1 + GLU and FC1's weight gradient reading the rows
of the unpermuted x through src_row, so the permuted copy Xp is never written.

Each case is checked two ways on the same seeded inputs:
  * against the oracle evaluated on the gathered rows x[src_row] (rows whose
    index lies outside [0, T) read as zeros), with the tolerances of the
    per-entry-point tests;
  * bit for bit against the same library call on a materialized Xp: the
    gather changes only where the DMA reads a row from, never the arithmetic.
Segment sizes include empty experts and tails around the 128 / 256 tiles; the
larger shapes take the 256 x 256 tiles (gated epilogue, ping-pong weight
gradient), the smaller ones the 128 x 128 tiles, float32 its own tile."""
import numpy as np
import pytest
import torch

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


G = 32
COUNTS_SMALL = [0, 1, 31, 32, 33, 255, 256, 257, 0, 130]
COUNTS_BIG = [0, 700, 1300, 300, 513]


def _f32_ok(got, ref):
    return rel_l2(got, ref) <= 1e-5 and norm_err(got, ref) <= 1e-4


def _src_rows(rng, R, T, bad):
    """A row -> token map with repeats (k > 1 picks a token several times) and,
    when `bad`, a few indices outside [0, T)."""
    src = rng.integers(0, T, size=R).astype(np.int32)
    if bad and R > 8:
        pos = rng.choice(R, size=4, replace=False)
        src[pos] = np.array([-1, T, T + 77, -(2 ** 31)], dtype=np.int32)
    return src


def _gathered(xh, src):
    ok = (src >= 0) & (src < xh.shape[0])
    g = np.zeros((src.shape[0], xh.shape[1]))
    g[ok] = xh[src[ok]]
    return g


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("counts,d,f,T", [(COUNTS_SMALL, 256, 256, 700),
                                          (COUNTS_BIG, 1024, 512, 1400)])
@pytest.mark.parametrize("act", ["swiglu", "srelu"])
@pytest.mark.parametrize("bad", [False, True])
def test_glu_fwd_gather(dtype, counts, d, f, T, act, bad):
    note(f"glu_fwd gather {dtype} R={sum(counts)} T={T} d={d} f={f} {act} bad={bad}")
    rng = np.random.default_rng(sum(counts) + d + f + T + (act == "srelu") + bad)
    off = offsets_of(counts)
    offd = dev(off)
    E, R = len(counts), int(off[-1])
    n1 = f if act == "srelu" else 2 * f
    mk = rand_bf16 if dtype == "bf16" else rand_f32
    xh, xd = mk(rng, (T, d))
    Wh, Wd = mk(rng, (E, n1, d), d ** -0.5)
    bh, bd = rand_f32(rng, (E, n1))
    Wpd, bpd = (Wd, bd) if act == "srelu" else ops.moe_repack_glu_weights(Wd, bd)
    src = _src_rows(rng, R, T, bad)
    srcd = dev(src)
    A, H = ops.moe_grouped_gemm_glu_fwd(xd, Wpd, offd, b1p=bpd, act=act, src_row=srcd)
    # the same call on a materialized copy of the gathered rows
    xpd = xd.new_zeros((R, d))
    okd = (srcd >= 0) & (srcd < T)
    xpd[okd] = xd[srcd[okd].long()]
    A0, H0 = ops.moe_grouped_gemm_glu_fwd(xpd, Wpd, offd, b1p=bpd, act=act)
    torch.cuda.synchronize()
    assert torch.equal(A, A0) and torch.equal(H, H0)
    Hc = om.grouped_linear(_gathered(xh, src), Wh, off, bh)
    if act == "srelu":
        Ao, Hp = om.srelu_forward(Hc, 0.0), Hc
    else:
        Ao = om.glu_forward(Hc[:, :f], Hc[:, f:], act)
        Hp = om.repack_glu(Hc[None], G=G, axis=2)[0]
    if dtype == "bf16":
        assert bf16_excess(host(H), Hp) <= 5e-3
        assert bf16_excess(host(A), Ao) <= 5e-3
    else:
        assert _f32_ok(host(H), Hp) and _f32_ok(host(A), Ao)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("counts,N,K,T", [(COUNTS_SMALL, 512, 256, 900),
                                          (COUNTS_BIG, 1024, 1024, 1500),
                                          (COUNTS_SMALL, 2880, 96, 300)])
@pytest.mark.parametrize("bad", [False, True])
def test_wgrad_gather(dtype, counts, N, K, T, bad):
    note(f"wgrad gather {dtype} R={sum(counts)} T={T} N={N} K={K} bad={bad}")
    rng = np.random.default_rng(3 * sum(counts) + N + K + T + bad)
    off = offsets_of(counts)
    offd = dev(off)
    R = int(off[-1])
    mk = rand_bf16 if dtype == "bf16" else rand_f32
    gh, gd = mk(rng, (R, N))
    xh, xd = mk(rng, (T, K))
    src = _src_rows(rng, R, T, bad)
    srcd = dev(src)
    dw, db = ops.moe_grouped_gemm_bwd(gd, offd, mode="wgrad", a=xd, a_src_row=srcd,
                                      want_db=True)
    xpd = xd.new_zeros((R, K))
    okd = (srcd >= 0) & (srcd < T)
    xpd[okd] = xd[srcd[okd].long()]
    dw0, db0 = ops.moe_grouped_gemm_bwd(gd, offd, mode="wgrad", a=xpd, want_db=True)
    torch.cuda.synchronize()
    assert torch.equal(dw, dw0) and torch.equal(db, db0)
    ref, refb = om.grouped_wgrad(gh, _gathered(xh, src), off, with_bias=True)
    got = host(dw)
    assert _f32_ok(got, ref)
    assert _f32_ok(host(db), refb)
    for e, c in enumerate(counts):
        if c == 0:
            assert not got[e].any()


def test_gather_rejected_where_not_built():
    """The fused gather exists for FC1 (+GLU) and the weight gradient only."""
    rng = np.random.default_rng(5)
    counts = [3, 0, 5]
    offd = dev(offsets_of(counts))
    _, gd = rand_bf16(rng, (8, 64))
    _, wd = rand_bf16(rng, (3, 64, 32))
    srcd = dev(np.arange(8, dtype=np.int32))
    with pytest.raises(RuntimeError):
        ops.moe_grouped_gemm_bwd(gd, offd, mode="dgrad", w=wd, a_src_row=srcd, a=gd)
