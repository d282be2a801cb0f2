"""CPU oracle of MXFP8 quantization (E4M3 elements, one E8M0 scale per 32).

TEST INFRASTRUCTURE ONLY (see ``oracle/moe.py``).

[P1 Quant] "MXFP8 および NVFP4 量子化の融合による露出メモリオーバーヘッドの削減"
(page "高度な融合カーネルによる MoE 学習スループットの向上"): after the activation
the output is quantized to MXFP8, and a transposed copy is written for the
backward pass.  The page names the format only; the format itself is the one
of the OCP Microscaling Formats (MX) Specification v1.0:

* E4M3 ("FN") element: 1 sign, 4 exponent bits (bias 7), 3 mantissa bits; no
  infinities; S.1111.111 is NaN; largest finite magnitude 448; smallest
  normal 2^-6; subnormals are multiples of 2^-9.
* E8M0 scale: the value 2^(code - 127); code 255 is NaN.
* Block of 32 values V with amax = max |V|: shared exponent
  e = floor(log2(amax)) - 8 (8 = exponent of E4M3's largest normal), clamped
  to [-127, 127]; amax = 0 gives the smallest scale (code 0).  Each element is
  V / 2^e rounded to nearest-even E4M3, saturated to +-448.

Readings (listed in DESIGN.md): the "round-up" scale rule
e = ceil(log2(amax / 448)), which never saturates, is kept as an alternative
(``rule="ceil"``); blocks run along the reduction axis of the GEMM that
consumes the tensor; token-axis blocks start at each expert's segment start
and the last block of a segment is zero-padded.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E4M3_EMAX = 8          # exponent of the largest normal, 448 = 1.75 * 2^8
BLOCK = 32


def e4m3_decode(codes) -> np.ndarray:
    """float64 value of each E4M3 code (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes, dtype=np.int64) & 0xFF
    s = np.where(c & 0x80, -1.0, 1.0)
    ex = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(ex == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.ldexp(1.0, ex - 7))
    val = s * val
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


def e4m3_round(v) -> np.ndarray:
    """Round float64 values to the nearest E4M3 value (ties to even), saturating at +-448."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, e = np.frexp(a)                   # a = m 2^e, 0.5 <= m < 1
    # E4M3 keeps 4 significant bits; the quantum of [2^(e-1), 2^e) is 2^(e-4),
    # and never below the subnormal quantum 2^-9.
    q = np.maximum(e - 4, -9)
    r = np.ldexp(np.rint(np.ldexp(a, -q)), q)
    r = np.minimum(r, E4M3_MAX)
    out = np.copysign(r, v)
    return np.where(np.isnan(v), np.nan, out)


def e4m3_encode(v) -> np.ndarray:
    """E4M3 code of each float64 value (rounded and saturated first)."""
    r = e4m3_round(v)
    sign = np.signbit(r).astype(np.int64) << 7
    a = np.abs(r)
    _, e = np.frexp(a)
    ex = np.where(a >= 2.0 ** -6, e - 1 + 7, 0)              # biased exponent
    man = np.where(ex == 0, np.rint(a / 2.0 ** -9),
                   np.rint((a / np.ldexp(1.0, np.maximum(ex, 1) - 7) - 1.0) * 8.0))
    code = sign | (ex.astype(np.int64) << 3) | man.astype(np.int64)
    code = np.where(np.isnan(r), 0x7F, code)
    return code.astype(np.uint8)


def e8m0_exponent(amax, rule: str = "ocp") -> np.ndarray:
    """Unbiased shared exponent of blocks with maximum magnitude ``amax``."""
    amax = np.asarray(amax, dtype=np.float64)
    safe = np.where(amax > 0, amax, 1.0)
    if rule == "ocp":
        _, e = np.frexp(safe)            # amax in [2^(e-1), 2^e)
        x = (e - 1) - E4M3_EMAX
    elif rule == "ceil":
        x = np.ceil(np.log2(safe / E4M3_MAX)).astype(np.int64)
    else:
        raise ValueError(rule)
    x = np.clip(x, -127, 127)
    return np.where(amax > 0, x, -127).astype(np.int64)


def mx_quantize_blocks(v, rule: str = "ocp"):
    """Quantize the last axis of ``v`` (length a multiple of 32) in blocks of 32.

    Returns ``(codes uint8, same shape as v; scale codes uint8, [..., n/32])``.
    """
    v = np.asarray(v, dtype=np.float64)
    n = v.shape[-1]
    if n % BLOCK:
        raise ValueError("length must be a multiple of 32")
    b = v.reshape(v.shape[:-1] + (n // BLOCK, BLOCK))
    amax = np.max(np.abs(b), axis=-1)
    x = e8m0_exponent(amax, rule)
    scaled = b / np.ldexp(1.0, x)[..., None]
    codes = e4m3_encode(scaled).reshape(v.shape)
    return codes, (x + 127).astype(np.uint8)


def mx_dequantize_blocks(codes, scales) -> np.ndarray:
    codes = np.asarray(codes)
    n = codes.shape[-1]
    vals = e4m3_decode(codes).reshape(codes.shape[:-1] + (n // BLOCK, BLOCK))
    sc = np.ldexp(1.0, np.asarray(scales, dtype=np.int64) - 127)
    return (vals * sc[..., None]).reshape(codes.shape)


def mx_qdq(v, axis: int = -1, rule: str = "ocp") -> np.ndarray:
    """Quantize-dequantize along ``axis`` (its length a multiple of 32)."""
    v = np.moveaxis(np.asarray(v, dtype=np.float64), axis, -1)
    c, s = mx_quantize_blocks(v, rule)
    return np.moveaxis(mx_dequantize_blocks(c, s), -1, axis)


def mx_quantize_segments_colwise(v, offsets, pad_offsets):
    """Column-wise MX copy of a row-major [R, N] tensor split into expert segments.

    Segment e (rows [offsets[e], offsets[e+1])) is transposed, zero-padded to
    the padded length pad_offsets[e+1] - pad_offsets[e] and quantized along the
    token axis.  Returns ``(codes [N, Rpad], scales [N, Rpad/32])``: column n of
    expert e lives in codes[n, pad_offsets[e]:pad_offsets[e+1]].
    """
    v = np.asarray(v, dtype=np.float64)
    N = v.shape[1]
    Rpad = int(pad_offsets[-1])
    buf = np.zeros((N, Rpad))
    for e in range(len(offsets) - 1):
        s, t = int(offsets[e]), int(offsets[e + 1])
        p = int(pad_offsets[e])
        buf[:, p:p + (t - s)] = v[s:t].T
    return mx_quantize_blocks(buf)


def mx_qdq_segments_colwise(v, offsets, pad_offsets) -> np.ndarray:
    """Quantize-dequantize of :func:`mx_quantize_segments_colwise`, returned in [R, N] layout."""
    v = np.asarray(v, dtype=np.float64)
    c, s = mx_quantize_segments_colwise(v, offsets, pad_offsets)
    deq = mx_dequantize_blocks(c, s)
    out = np.zeros_like(v)
    for e in range(len(offsets) - 1):
        st, t = int(offsets[e]), int(offsets[e + 1])
        p = int(pad_offsets[e])
        out[st:t] = deq[:, p:p + (t - st)].T
    return out
