"""MI355X (gfx950) dropless MoE expert-FFN layer: C-ABI HIP library + thin binding.

``ragged_grouped_gemm_amd.ops``   one Python function per C entry point
``ragged_grouped_gemm_amd.layer`` the whole layer (forward + backward) as a
                                  sequence of library calls, graph-capturable
The compute runs only in ``libmoe_mi355x.so`` (built in-tree with
``python -m ragged_grouped_gemm_amd.build``); there is no fallback path.
"""
__all__ = ["ops", "layer"]


def __getattr__(name):
    if name in ("ops", "layer"):
        import importlib
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
