"""The allocation-free permute (moe_permute_noalloc) against moe_permute.

moe_permute_noalloc keeps the per-chunk counts in a static device array
instead of the caller's workspace; otherwise it runs the same kernels, so its
outputs must equal moe_permute's bit for bit.  Two calls in a row on one GPU
(the second with a smaller input) check that the shared array's leftover
contents from the first call do not leak into the second.  Sizes beyond the
array are refused with MOE_ERR_WORKSPACE before anything reaches the device.
"""
import ctypes

import numpy as np
import pytest
import torch

import synth
from oracle import moe as om
from ragged_grouped_gemm_amd import _lib


def test_noalloc_rejects_sizes_beyond_the_static_scratch():
    lib = _lib.load()
    limit = 1 << 20
    fake = ctypes.c_void_p(256)
    # ceil(T*k / 1024) * E * 4 bytes of counters: 1025 chunks x 256 experts > 1 MiB
    T, k, E = 1025 * 1024 // 8, 8, 256
    assert lib.moe_permute_workspace_size(T, E, k) > limit
    st = lib.moe_permute_noalloc(None, 1, T, 0, fake, k, E, fake, fake, None, fake, fake, None,
                                 None, None)
    assert st == _lib.MOE_ERR_WORKSPACE
    # argument errors are still argument errors
    assert lib.moe_permute_noalloc(None, 1, T, 0, fake, k, 2000, fake, fake, None, fake, fake,
                                   None, None, None) == _lib.MOE_ERR_INVALID_ARG


def _outputs(T, k, E, d, dev):
    z = lambda shape: torch.full(shape, -7, dtype=torch.int32, device=dev)
    return dict(counts=z((E,)), offsets=z((E + 1,)), pad_offsets=z((E + 1,)), row_map=z((T, k)),
                src_row=z((T * k,)), xp=torch.zeros((T * k, d), dtype=torch.bfloat16, device=dev),
                err=torch.zeros((1,), dtype=torch.int32, device=dev))


@pytest.mark.gpu
def test_noalloc_permute_matches_workspace_permute_on_consecutive_calls():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from ragged_grouped_gemm_amd import ops
    # a large routing first, then a smaller one: the second call's chunk
    # counters must not see the first call's leftovers
    cases = [synth.workload("dsv3_fwdbwd", T=4096, d=256, f=64, E=32, k=8),
             synth.workload("gptoss_fwdbwd", T=300, d=128, f=64, E=8, k=2, seed=9)]
    for cfg in cases:
        print(f"[gpu] permute_noalloc T={cfg.T} E={cfg.E} k={cfg.k} d={cfg.d}", flush=True)
        inp = synth.make_inputs(cfg, parts=("x", "logits"))
        x = synth.to_torch(inp["x"], "cuda")
        idx, _, _ = om.route_topk(inp["logits"], cfg.k, cfg.score, cfg.normalize)
        idx_d = torch.from_numpy(np.ascontiguousarray(idx.astype(np.int32))).cuda()
        a = _outputs(cfg.T, cfg.k, cfg.E, cfg.d, "cuda")
        b = _outputs(cfg.T, cfg.k, cfg.E, cfg.d, "cuda")
        ops.moe_permute(x, idx_d, cfg.E, counts=a["counts"], offsets=a["offsets"],
                        pad_offsets=a["pad_offsets"], row_map=a["row_map"], src_row=a["src_row"],
                        xp=a["xp"], err_word=a["err"], gather=True)
        ops.moe_permute_noalloc(x, idx_d, cfg.E, counts=b["counts"], offsets=b["offsets"],
                                pad_offsets=b["pad_offsets"], row_map=b["row_map"],
                                src_row=b["src_row"], xp=b["xp"], err_word=b["err"])
        torch.cuda.synchronize()
        for name in a:
            assert torch.equal(a[name], b[name]), (cfg.T, name)
        # and both are the oracle's layout
        counts, offsets, row_map, src_row = om.permute_indices(idx, cfg.E)
        np.testing.assert_array_equal(b["counts"].cpu().numpy(), counts)
        np.testing.assert_array_equal(b["offsets"].cpu().numpy(), offsets)
        np.testing.assert_array_equal(b["row_map"].cpu().numpy(), row_map)
        np.testing.assert_array_equal(b["src_row"].cpu().numpy(), src_row)
        assert int(b["err"].item()) == 0
