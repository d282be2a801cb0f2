"""Pins of the oracle's MXFP8 codec (OCP MX v1.0: E4M3 elements, E8M0 scales).

The decode of every code is checked against torch's float8_e4m3fn (an
independent implementation of the same OCP E4M3 format); the round-to-nearest
rule against torch's float32 -> float8_e4m3fn cast inside the finite range;
saturation, the shared-exponent rule and the segment-anchored column copy
against values worked out by hand from the specification."""
import numpy as np
import pytest
import torch

from oracle import moe as om
from oracle import mx


def test_decode_all_codes_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = mx.e4m3_decode(codes)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(got[ok], ref[ok])
    assert np.sum(np.isnan(got)) == 2          # only S.1111.111
    assert mx.e4m3_decode(0x7E) == 448.0 and mx.e4m3_decode(0x01) == 2.0 ** -9
    assert mx.e4m3_decode(0x08) == 2.0 ** -6


def test_encode_decode_roundtrip():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    np.testing.assert_array_equal(mx.e4m3_encode(mx.e4m3_decode(codes)), codes)


def test_round_vs_torch_in_range():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.uniform(-448, 448, 20000), rng.standard_normal(20000),
                        rng.standard_normal(5000) * 2.0 ** -8]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(mx.e4m3_round(v.astype(np.float64)), ref)
    codes_ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(mx.e4m3_encode(v.astype(np.float64)), codes_ref)


def test_round_examples_and_saturation():
    cases = {1.0625: 1.0, 1.1875: 1.25, 248.0: 256.0, 464.0: 448.0, 2.0 ** -10: 0.0,
             3 * 2.0 ** -11: 2.0 ** -9, 500.0: 448.0, 1e6: 448.0, -1e6: -448.0, 449.0: 448.0}
    for v, r in cases.items():
        assert mx.e4m3_round(v) == r, v


def test_shared_exponent_rule():
    # amax = 1 -> 2^(0 - 8): code 119; amax = 448 -> 2^0: code 127; all-zero block -> code 0
    assert mx.e8m0_exponent(1.0) == -8
    assert mx.e8m0_exponent(448.0) == 0
    assert mx.e8m0_exponent(500.0) == 0
    assert mx.e8m0_exponent(0.0) == -127
    assert mx.e8m0_exponent(2.0 ** -200) == -127          # clamped
    assert mx.e8m0_exponent(1.0, "ceil") == -8
    assert mx.e8m0_exponent(500.0, "ceil") == 1
    blk = np.zeros((1, 32)); blk[0, 3] = 500.0; blk[0, 4] = -1.0
    c, s = mx.mx_quantize_blocks(blk)
    assert s.tolist() == [[127]]
    assert mx.e4m3_decode(c[0, 3]) == 448.0              # 500 saturates
    assert mx.e4m3_decode(c[0, 4]) == -1.0
    c0, s0 = mx.mx_quantize_blocks(np.zeros((2, 64)))
    assert s0.tolist() == [[0, 0], [0, 0]] and not c0.any()


def test_block_max_maps_to_top_binade():
    rng = np.random.default_rng(1)
    v = rng.standard_normal((50, 64)) * np.exp(rng.uniform(-20, 20, (50, 1)))
    c, s = mx.mx_quantize_blocks(v)
    deq = mx.e4m3_decode(c).reshape(50, 2, 32)
    amax_codes = np.max(np.abs(deq), axis=-1)
    assert np.all(amax_codes >= 256.0) and np.all(amax_codes <= 448.0)
    q = mx.mx_dequantize_blocks(c, s)
    scale = np.repeat(np.ldexp(1.0, s.astype(np.int64) - 127), 32, axis=1)
    scaled = np.abs(v) / scale
    inside = scaled <= 448.0
    # in range: at most half an E4M3 step (step 32 in the top binade [256, 512))
    assert np.all(np.abs(q - v)[inside] <= 16.0 * scale[inside])
    # beyond 448 (possible since the scaled block max lies in [256, 512)) the value saturates
    np.testing.assert_array_equal(np.abs(q)[~inside], 448.0 * scale[~inside])


def test_qdq_commutes_with_row_permutation_and_repack():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((40, 64))
    perm = rng.permutation(40)
    np.testing.assert_array_equal(mx.mx_qdq(x[perm]), mx.mx_qdq(x)[perm])
    W = rng.standard_normal((2, 256, 64))
    # quantizing along d commutes with the row repack; along the packed 2f axis it
    # does too when G is a multiple of 32 (each 32-block stays within one chunk)
    np.testing.assert_array_equal(mx.mx_qdq(om.repack_glu(W, G=64), axis=2),
                                  om.repack_glu(mx.mx_qdq(W, axis=2), G=64))
    Wt = np.swapaxes(W, 1, 2)
    np.testing.assert_array_equal(mx.mx_qdq(om.repack_glu(W, G=64), axis=1),
                                  np.swapaxes(mx.mx_qdq(np.swapaxes(om.repack_glu(W, G=64), 1, 2)), 1, 2))
    _ = Wt


def test_segment_colwise_copy():
    rng = np.random.default_rng(3)
    counts = [5, 0, 33, 32, 1]
    off = np.concatenate([[0], np.cumsum(counts)])
    pad = om.pad_offsets(counts)
    v = rng.standard_normal((off[-1], 64))
    c, s = mx.mx_quantize_segments_colwise(v, off, pad)
    assert c.shape == (64, pad[-1]) and s.shape == (64, pad[-1] // 32)
    for e in range(len(counts)):
        seg = v[off[e]:off[e + 1]].T
        n = counts[e]
        padded = np.zeros((64, pad[e + 1] - pad[e]))
        padded[:, :n] = seg
        ce, se = mx.mx_quantize_blocks(padded)
        np.testing.assert_array_equal(c[:, pad[e]:pad[e + 1]], ce)
        np.testing.assert_array_equal(s[:, pad[e] // 32:pad[e + 1] // 32], se)
        assert not c[:, pad[e] + n:pad[e + 1]].any()      # zero padding
    q = mx.mx_qdq_segments_colwise(v, off, pad)
    assert np.max(np.abs(q - v)) <= 2.0 ** -3 * np.max(np.abs(v))
