"""Pins of the oracle's E2M1 (MXFP4) element and block rules, against the
values the OCP Microscaling Formats specification v1.0 tabulates and against
a brute-force nearest-value search that shares no code with ``oracle.mx``."""
import numpy as np
import pytest

from oracle import mx

# E2M1 magnitudes by code 0..7 as tabulated in the specification
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def brute_round(v):
    """Nearest E2M1 value by exhaustive search; ties go to the even code
    (mantissa bit 0); magnitudes beyond 6 saturate."""
    out = []
    for x in np.asarray(v, dtype=np.float64).ravel():
        a = abs(x)
        best = None
        for code, m in enumerate(E2M1_TABLE):
            d = abs(a - m)
            key = (d, code & 1)              # smaller distance, then the even code
            if best is None or key < best[0]:
                best = (key, m)
        r = best[1] if a <= 6.0 else 6.0
        out.append(-r if np.signbit(x) else r)
    return np.array(out).reshape(np.shape(v))


def test_decode_matches_table():
    vals = mx.e2m1_decode(np.arange(16))
    np.testing.assert_array_equal(vals[:8], E2M1_TABLE)
    np.testing.assert_array_equal(vals[8:], [-m for m in E2M1_TABLE])
    assert np.signbit(vals[8])               # code 8 is -0


def test_encode_decode_roundtrip():
    for c in range(16):
        assert int(mx.e2m1_encode(mx.e2m1_decode(c))) == c


def test_rounding_matches_brute_force():
    rng = np.random.default_rng(0)
    grid = np.concatenate([
        np.arange(-7.0, 7.0, 1 / 64),                      # every midpoint is on this grid
        rng.uniform(-8, 8, 4000), rng.uniform(-1, 1, 2000) * 2.0 ** -rng.integers(0, 12, 2000),
        [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 1e9, -1e9, 6.0, 6.5, -0.0]])
    np.testing.assert_array_equal(mx.e2m1_round(grid), brute_round(grid))
    np.testing.assert_array_equal(np.signbit(mx.e2m1_round(grid)), np.signbit(grid))


def test_ties_go_to_even_codes():
    # midpoints between neighbours: the result is the neighbour with an even code
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    want = [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]
    np.testing.assert_array_equal(mx.e2m1_round(mids), want)
    np.testing.assert_array_equal(mx.e2m1_round(np.negative(mids)), np.negative(want))


def test_scale_rule_examples():
    # e = floor(log2 amax) - 2: amax 6 -> 0 (code 127), 1 -> -2, 0.75 -> -3, 7 -> 0
    assert list(mx.e8m0_exponent([6.0, 1.0, 0.75, 7.0, 4.0], fmt="e2m1")) == [0, -2, -3, 0, 0]
    assert int(mx.e8m0_exponent(0.0, fmt="e2m1")) == -127
    # clamping at both ends
    assert int(mx.e8m0_exponent(2.0 ** 200, fmt="e2m1")) == 127
    assert int(mx.e8m0_exponent(2.0 ** -140, fmt="e2m1")) == -127
    # a block whose largest magnitude is 7 saturates that element to 6
    v = np.zeros(32)
    v[3], v[5] = 7.0, -0.6
    c, s = mx.mx_quantize_blocks(v, fmt="e2m1")
    assert int(s[0]) == 127
    deq = mx.mx_dequantize_blocks(c, s, fmt="e2m1")
    assert deq[3] == 6.0 and deq[5] == -0.5


def test_qdq_error_bound():
    """Without saturation (amax mantissa <= 1.5), every element is within half
    an E2M1 quantum of its own binade, times the block scale."""
    rng = np.random.default_rng(1)
    v = rng.standard_normal((200, 64)) * 2.0 ** rng.integers(-20, 20, (200, 1))
    blocks = v.reshape(200, 2, 32)
    amax = np.abs(blocks).max(-1)
    m, _ = np.frexp(amax)
    keep = (m <= 0.75).all(1)                    # mantissa 2m <= 1.5: no saturation
    q = mx.mx_qdq(v, 1, fmt="e2m1")
    x = mx.e8m0_exponent(amax, fmt="e2m1")
    scaled = np.abs(blocks) / np.ldexp(1.0, x)[..., None]
    _, eb = np.frexp(np.where(scaled > 0, scaled, 1.0))
    half_q = np.ldexp(1.0, np.maximum(eb - 2, -1) - 1) * np.ldexp(1.0, x)[..., None]
    err = np.abs(q - v).reshape(200, 2, 32)
    assert (err[keep] <= half_q[keep] * (1 + 1e-15)).all()
    assert keep.sum() > 50


def test_pack_unpack():
    rng = np.random.default_rng(2)
    c = rng.integers(0, 16, (5, 64)).astype(np.uint8)
    p = mx.pack_fp4(c)
    assert p.shape == (5, 32)
    assert p[0, 0] == (c[0, 0] | (c[0, 1] << 4))
    np.testing.assert_array_equal(mx.unpack_fp4(p), c)


def test_column_copy_equals_row_quantize_of_transposed_segments():
    rng = np.random.default_rng(3)
    counts = [5, 0, 40, 33]
    off = np.concatenate([[0], np.cumsum(counts)])
    pad = np.concatenate([[0], np.cumsum([(c + 31) // 32 * 32 for c in counts])])
    v = rng.standard_normal((off[-1], 64))
    c, s = mx.mx_quantize_segments_colwise(v, off, pad, fmt="e2m1")
    for e in range(4):
        seg = np.zeros((64, pad[e + 1] - pad[e]))
        seg[:, :counts[e]] = v[off[e]:off[e + 1]].T
        if seg.shape[1] == 0:
            continue
        c2, s2 = mx.mx_quantize_blocks(seg, fmt="e2m1")
        np.testing.assert_array_equal(c[:, pad[e]:pad[e + 1]], c2)
        np.testing.assert_array_equal(s[:, pad[e] // 32:pad[e + 1] // 32], s2)
