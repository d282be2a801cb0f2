"""Helpers of the GPU parity tests: host <-> device transfer and error metrics."""
import math
import sys

import numpy as np
import torch

import synth


def note(msg):
    """Name the case about to run on the GPU (flushed, so a crash still shows it)."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def dev(a, dtype=None):
    """numpy -> cuda tensor.  uint16 arrays are bf16 bit patterns."""
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        a = synth.f32_to_bf16_bits(a.astype(np.float32))
    return synth.to_torch(a, "cuda")


def host(t):
    """cuda tensor -> numpy (floats as float64, ints as int64)."""
    t = t.detach().cpu()
    if t.dtype in (torch.bfloat16, torch.float16, torch.float32, torch.float64):
        return t.to(torch.float64).numpy()
    return t.to(torch.int64).numpy()


def stored(t):
    """The stored values of a tensor as float64 (what the oracle is fed)."""
    return host(t)


def rand_bf16(rng, shape, scale=1.0):
    """Random values already on the bf16 grid, as float64 (host) and bf16 (device)."""
    v = (rng.standard_normal(shape, dtype=np.float32) * np.float32(scale))
    bits = synth.f32_to_bf16_bits(v)
    return synth.bf16_bits_to_f32(bits).astype(np.float64), synth.to_torch(bits, "cuda")


def rand_f32(rng, shape, scale=1.0):
    v = rng.standard_normal(shape, dtype=np.float32) * np.float32(scale)
    return v.astype(np.float64), synth.to_torch(v, "cuda")


def rms(o):
    o = np.asarray(o, dtype=np.float64)
    return math.sqrt(float(np.mean(o * o))) if o.size else 0.0


def norm_err(g, o):
    """max |g - o| / rms(o): the tolerance metric of the layer outputs."""
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    assert g.shape == o.shape, (g.shape, o.shape)
    r = rms(o)
    d = float(np.max(np.abs(g - o))) if o.size else 0.0
    return d / r if r > 0 else (0.0 if d == 0 else math.inf)


def half_ulp_bf16(o):
    """Half a bf16 unit in the last place at each value (the storage rounding bound)."""
    a = np.abs(np.asarray(o, dtype=np.float64))
    _, e = np.frexp(np.where(a > 0, a, 1.0))
    return np.where(a > 0, np.ldexp(1.0, np.maximum(e - 9, -134)), 2.0 ** -134)


def bf16_floor(o):
    """The normalised error a perfect bf16 store of o can show: max half-ulp / rms."""
    r = rms(o)
    return float(np.max(half_ulp_bf16(o))) / r if r > 0 else 0.0


def bf16_excess(g, o):
    """Error of a bf16-stored result g beyond its own rounding, normalised by rms(o):
    max(|g - o| - half_ulp(o), 0) / rms(o), against the unrounded reference o."""
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    assert g.shape == o.shape, (g.shape, o.shape)
    r = rms(o)
    ex = np.maximum(np.abs(g - o) - half_ulp_bf16(o), 0.0)
    d = float(np.max(ex)) if o.size else 0.0
    return d / r if r > 0 else (0.0 if d == 0 else math.inf)


def offsets_of(counts):
    off = np.zeros(len(counts) + 1, dtype=np.int32)
    off[1:] = np.cumsum(counts)
    return off


def rel_l2(g, o):
    """||g - o||_2 / ||o||_2: the relative error of a float32 result."""
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    assert g.shape == o.shape, (g.shape, o.shape)
    n = float(np.linalg.norm(o))
    d = float(np.linalg.norm(g - o))
    return d / n if n > 0 else (0.0 if d == 0 else math.inf)


def ulp_err(g, o):
    """max |g - o| / (one bf16 ulp at o + 1e-3 rms(o)): elementwise distance in bf16 ulps."""
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    assert g.shape == o.shape, (g.shape, o.shape)
    if o.size == 0:
        return 0.0
    den = 2.0 * half_ulp_bf16(o) + 1e-3 * rms(o)
    return float(np.max(np.abs(g - o) / den))
