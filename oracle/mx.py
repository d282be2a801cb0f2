"""CPU oracle of MXFP8 and MXFP4 quantization (E4M3 or E2M1 elements, one E8M0
scale per 32).

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

* E2M1 (MXFP4) element, same specification: 1 sign, 2 exponent bits (bias
  1), 1 mantissa bit; no infinities or NaN; magnitudes 0, 0.5, 1, 1.5, 2, 3,
  4, 6 (0.5 is the one subnormal); the block exponent uses E2M1's largest
  normal exponent, 2 (6 = 1.5 * 2^2): e = floor(log2(amax)) - 2, and elements
  round to nearest even and saturate to +-6.  The [P1 Quant] section's 4-bit
  format is NVFP4 (E2M1 elements too, with finer scales); the CDNA4 matrix
  cores take E2M1 with E8M0 scales per 32, so the 4-bit variant here is the
  OCP MXFP4 one.  A NaN input (which E2M1 cannot hold) is taken as the
  largest magnitude, keeping its sign.  Codes are unpacked here (one per
  element, sign in bit 3); storage packs two per byte, element 2 i in the low
  nibble of byte i (``pack_fp4``).

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
E2M1_MAX = 6.0
E2M1_EMAX = 2          # 6 = 1.5 * 2^2
BLOCK = 32
FORMATS = ("e4m3", "e2m1")


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


def e2m1_decode(codes) -> np.ndarray:
    """float64 value of each E2M1 code (low 4 bits; bit 3 is the sign)."""
    c = np.asarray(codes, dtype=np.int64) & 0xF
    s = np.where(c & 0x8, -1.0, 1.0)
    ex = (c >> 1) & 0x3
    m = c & 0x1
    val = np.where(ex == 0, m * 0.5, (1.0 + m / 2.0) * np.ldexp(1.0, ex - 1))
    return s * val


def e2m1_round(v) -> np.ndarray:
    """Round float64 values to the nearest E2M1 value (ties to even), saturating
    at +-6; NaN becomes +-6."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, e = np.frexp(a)                   # a = m 2^e, 0.5 <= m < 1
    # two significant bits: the quantum of [2^(e-1), 2^e) is 2^(e-2), never
    # below the subnormal quantum 2^-1
    q = np.maximum(e - 2, -1)
    r = np.ldexp(np.rint(np.ldexp(a, -q)), q)
    r = np.minimum(r, E2M1_MAX)
    r = np.where(np.isnan(v), E2M1_MAX, r)
    return np.copysign(r, v)


def e2m1_encode(v) -> np.ndarray:
    """E2M1 code of each float64 value (rounded and saturated first)."""
    r = e2m1_round(v)
    sign = np.signbit(r).astype(np.int64) << 3
    a = np.abs(r)
    _, e = np.frexp(a)
    ex = np.where(a >= 1.0, e - 1 + 1, 0)                    # biased exponent
    man = np.where(ex == 0, np.rint(a / 0.5),
                   np.rint((a / np.ldexp(1.0, np.maximum(ex, 1) - 1) - 1.0) * 2.0))
    return (sign | (ex.astype(np.int64) << 1) | man.astype(np.int64)).astype(np.uint8)


def pack_fp4(codes) -> np.ndarray:
    """Two E2M1 codes per byte along the last axis: element 2 i in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8) & 0xF
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_fp4(packed) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def _fmt(fmt):
    if fmt == "e4m3":
        return E4M3_EMAX, E4M3_MAX, e4m3_encode, e4m3_decode
    if fmt == "e2m1":
        return E2M1_EMAX, E2M1_MAX, e2m1_encode, e2m1_decode
    raise ValueError(fmt)


def e8m0_exponent(amax, rule: str = "ocp", fmt: str = "e4m3") -> np.ndarray:
    """Unbiased shared exponent of blocks with maximum magnitude ``amax``."""
    emax, vmax, _, _ = _fmt(fmt)
    amax = np.asarray(amax, dtype=np.float64)
    safe = np.where(amax > 0, amax, 1.0)
    if rule == "ocp":
        _, e = np.frexp(safe)            # amax in [2^(e-1), 2^e)
        x = (e - 1) - emax
    elif rule == "ceil":
        x = np.ceil(np.log2(safe / vmax)).astype(np.int64)
    else:
        raise ValueError(rule)
    x = np.clip(x, -127, 127)
    return np.where(amax > 0, x, -127).astype(np.int64)


def mx_quantize_blocks(v, rule: str = "ocp", fmt: str = "e4m3"):
    """Quantize the last axis of ``v`` (length a multiple of 32) in blocks of 32.

    Returns ``(codes uint8, same shape as v, unpacked; scale codes uint8,
    [..., n/32])``.
    """
    _, _, encode, _ = _fmt(fmt)
    v = np.asarray(v, dtype=np.float64)
    n = v.shape[-1]
    if n % BLOCK:
        raise ValueError("length must be a multiple of 32")
    b = v.reshape(v.shape[:-1] + (n // BLOCK, BLOCK))
    amax = np.max(np.abs(b), axis=-1)
    x = e8m0_exponent(amax, rule, fmt)
    scaled = b / np.ldexp(1.0, x)[..., None]
    codes = encode(scaled).reshape(v.shape)
    return codes, (x + 127).astype(np.uint8)


def mx_dequantize_blocks(codes, scales, fmt: str = "e4m3") -> np.ndarray:
    _, _, _, decode = _fmt(fmt)
    codes = np.asarray(codes)
    n = codes.shape[-1]
    vals = decode(codes).reshape(codes.shape[:-1] + (n // BLOCK, BLOCK))
    sc = np.ldexp(1.0, np.asarray(scales, dtype=np.int64) - 127)
    return (vals * sc[..., None]).reshape(codes.shape)


def mx_qdq(v, axis: int = -1, rule: str = "ocp", fmt: str = "e4m3") -> np.ndarray:
    """Quantize-dequantize along ``axis`` (its length a multiple of 32)."""
    v = np.moveaxis(np.asarray(v, dtype=np.float64), axis, -1)
    c, s = mx_quantize_blocks(v, rule, fmt)
    return np.moveaxis(mx_dequantize_blocks(c, s, fmt), -1, axis)


def mx_quantize_segments_colwise(v, offsets, pad_offsets, fmt: str = "e4m3"):
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
    return mx_quantize_blocks(buf, fmt=fmt)


def mx_qdq_segments_colwise(v, offsets, pad_offsets, fmt: str = "e4m3") -> np.ndarray:
    """Quantize-dequantize of :func:`mx_quantize_segments_colwise`, returned in [R, N] layout."""
    v = np.asarray(v, dtype=np.float64)
    c, s = mx_quantize_segments_colwise(v, offsets, pad_offsets, fmt)
    deq = mx_dequantize_blocks(c, s, fmt)
    out = np.zeros_like(v)
    for e in range(len(offsets) - 1):
        st, t = int(offsets[e]), int(offsets[e + 1])
        p = int(pad_offsets[e])
        out[st:t] = deq[:, p:p + (t - st)].T
    return out
