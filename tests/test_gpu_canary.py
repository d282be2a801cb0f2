"""Guard bands and poisoned buffers around a whole layer step.

Every buffer the layer holds is allocated (through ``MoEFFN(alloc=...)``)
inside a larger block whose bytes -- the buffer's own included -- are all set
to a poison byte first.  After a forward + backward with one routing and then
a second one with another routing (different counts, so other rows are
padding and other tiles are ragged):
  * the guard bands before and after every buffer still hold the poison: no
    kernel wrote outside the tensors it was given;
  * the entries of the MX column copies past pad_offsets[E] (which no kernel
    owns) still hold the poison;
  * every output equals, bit for bit, that of a layer allocated with zeros
    that ran only the second step: nothing depends on the initial contents
    of a buffer or on what the first step left behind.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_util import note

pytestmark = pytest.mark.gpu

POISON = 0xA5
GUARD = 4096            # bytes on each side (keeps every buffer 256-byte aligned)


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from ragged_grouped_gemm_amd import ops
    ops.moe_version()


class GuardedAlloc:
    """alloc(shape, dtype, device) for MoEFFN: each buffer sits in the middle of
    a poisoned block of GUARD + nbytes + GUARD bytes."""

    def __init__(self):
        self.blocks = []

    def __call__(self, shape, dt, dev):
        n = int(np.prod(shape)) * torch.empty((), dtype=dt).element_size()
        raw = torch.full((GUARD + n + GUARD,), POISON, dtype=torch.uint8, device=dev)
        self.blocks.append((raw, n, tuple(shape), dt))
        return raw[GUARD:GUARD + n].view(dt).view(shape)

    def check_guards(self):
        bad = []
        for raw, n, shape, dt in self.blocks:
            for side, band in (("before", raw[:GUARD]), ("after", raw[GUARD + n:])):
                hit = (band != POISON).nonzero()
                if hit.numel():
                    bad.append((shape, dt, side, int(hit.numel())))
        assert not bad, f"writes outside a buffer: {bad}"


def _layer(cfg, gemm, router, mx_dxp, gia, alloc):
    from ragged_grouped_gemm_amd.layer import MoEFFN
    return MoEFFN(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, act=cfg.act, score=cfg.score,
                  normalize=cfg.normalize, clamp=cfg.clamp, alpha=cfg.alpha, bias=cfg.bias,
                  gemm=gemm, router=router, mx_dxp=mx_dxp, gate_in_act=gia, alloc=alloc)


def _step(L, cfg, inp, gemm, router, weights):
    t = lambda a: synth.to_torch(a, "cuda")
    x, dout = t(inp["x"]), t(inp["dOut"])
    lg = weights["Wr"] if router else t(inp["logits"])
    W1l, W2l, b1p, b2 = weights["W1"], weights["W2"], weights["b1p"], weights["b2"]
    L.forward(x, lg, W1l, W2l, b1p, b2)
    L.backward(dout, lg, W1l, W2l)


def _weights(cfg, inp, gemm, router):
    from ragged_grouped_gemm_amd import ops
    from ragged_grouped_gemm_amd.layer import MoEFFN
    t = lambda a: synth.to_torch(a, "cuda")
    W1, W2 = t(inp["W1"]), t(inp["W2"])
    b1 = t(inp["b1"]) if cfg.bias else None
    W1p, b1p = ops.moe_repack_glu_weights(W1, b1)
    w = {"b1p": b1p, "b2": t(inp["b2"]) if cfg.bias else None,
         "Wr": t(synth.draw_router_weights(cfg)) if router else None}
    if gemm == "bf16":
        w["W1"], w["W2"] = W1p, W2
    else:
        w["W1"], w["W2"] = MoEFFN.mx_weights(W1p, W2, gemm), None
    return w


def _buffers(L):
    """The layer's buffers by name: tensors and MX copies (data, scale)."""
    from ragged_grouped_gemm_amd import ops
    out = {}
    for name, v in vars(L).items():
        if isinstance(v, torch.Tensor) and v.is_cuda:
            out[name] = v
        elif isinstance(v, ops.MXTensor):
            out[name + ".data"] = v.data
            out[name + ".scale"] = v.scale
    return out


_DSV3 = synth.workload("dsv3_fwdbwd", T=300, d=256, f=256, E=8, k=4, forced_empty=1)
CASES = [
    # (workload, gemm, router, mx_dxp, gates in the activation)
    (synth.workload("gptoss_fwdbwd", T=333, d=256, f=160, E=8, k=4), "bf16", False, False, False),
    (_DSV3, "bf16", True, False, False),
    (_DSV3, "bf16", False, False, True),
    (_DSV3, "mxfp8", False, True, False),
    (_DSV3, "mxfp4", False, False, True),
]


@pytest.mark.parametrize("cfg,gemm,router,mx_dxp,gia", CASES,
                         ids=["gptoss_bf16_bias", "dsv3_bf16_router", "dsv3_bf16_gate_in_act",
                              "dsv3_mxfp8_dxp", "dsv3_mxfp4_gate_in_act"])
def test_guards_and_poisoned_buffers(cfg, gemm, router, mx_dxp, gia):
    note(f"canary {cfg.name} {gemm} router={router} mx_dxp={mx_dxp} gate_in_act={gia}")
    inp1 = synth.make_inputs(cfg)
    inp2 = synth.make_inputs(cfg.replace(seed=cfg.seed + 101))
    w = _weights(cfg, inp1, gemm, router)
    ga = GuardedAlloc()
    L = _layer(cfg, gemm, router, mx_dxp, gia, ga)
    _step(L, cfg, inp1, gemm, router, w)
    _step(L, cfg, inp2, gemm, router, w)
    R = _layer(cfg, gemm, router, mx_dxp, gia, None)
    _step(R, cfg, inp2, gemm, router, w)
    torch.cuda.synchronize()
    ga.check_guards()
    assert int(L.err.item()) == 0 and int(R.err.item()) == 0

    got, ref = _buffers(L), _buffers(R)
    assert got.keys() == ref.keys()
    pad_end = int(R.pad_offsets[-1].item()) if L.mx else None
    e2m1 = gemm == "mxfp4"
    checked = []
    for name in sorted(got):
        if name in ("ws", "ds_ws"):     # scratch: no defined contents
            continue
        a, b = got[name], ref[name]
        if name.endswith("_col.data") or name.endswith("_col.scale"):
            # entries past pad_offsets[E] belong to no expert: never written
            cut = pad_end // 32 if name.endswith("scale") else (pad_end // 2 if e2m1 else pad_end)
            tail = a[:, cut:]
            assert bool((tail == POISON).all()), f"{name}: written past pad_offsets[E]"
            a, b = a[:, :cut], b[:, :cut]
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), \
            f"{name} differs from the zero-allocated layer"
        checked.append(name)
    print(gemm, f"{len(ga.blocks)} guarded buffers; compared:", " ".join(checked), flush=True)
