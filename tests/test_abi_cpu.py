"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function the header declares, and rejects bad arguments with status
codes before touching the device."""
import ctypes

import pytest

from ragged_grouped_gemm_amd import _lib


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_exports_every_header_function(lib):
    names = _lib.header_functions()
    assert len(names) >= 14
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    # the binding declares a signature for each of them
    assert sorted(_lib._SIGS) == names


def test_host_only_queries(lib):
    assert b"gfx950" in lib.moe_version()
    assert lib.moe_status_string(0) == b"MOE_OK"
    assert lib.moe_status_string(4) == b"MOE_ERR_HIP"
    assert lib.moe_glu_granularity() == 32
    assert lib.moe_permute_workspace_size(16384, 32, 8) >= 128 * 32 * 4
    assert lib.moe_permute_workspace_size(16384, 32, 8) % 256 == 0


def test_bad_arguments_rejected(lib):
    INV = _lib.MOE_ERR_INVALID_ARG
    # k > E, E out of range, null pointers, bad score
    assert lib.moe_route_topk(None, 4, 2, 3, 0, 1, None, None, None, None) == INV
    assert lib.moe_route_topk(None, 4, 0, 1, 0, 1, None, None, None, None) == INV
    assert lib.moe_route_topk(None, 4, 8, 2, 0, 1, None, None, None, None) == INV
    assert lib.moe_route_topk(None, 4, 8, 2, 7, 1, None, None, None, None) == INV
    assert lib.moe_route_topk(None, 0, 8, 2, 0, 1, None, None, None, None) == _lib.MOE_OK
    assert lib.moe_unpermute_combine(None, 1, None, None, 4, 2, 64, None, None) == INV
    assert lib.moe_unpermute_combine(None, 9, None, None, 4, 2, 64, None, None) == INV
    # f not a multiple of the repack granularity
    assert lib.moe_repack_glu_weights(None, None, 1, 2, 48, 64, 0, None, None, None) == INV
    # too-small permute workspace
    fake = ctypes.c_void_p(256)
    st = lib.moe_permute(None, 1, 1000, 0, fake, 2, 8, fake, fake, None, fake, fake, None,
                         fake, 4, None, None)
    assert st == _lib.MOE_ERR_WORKSPACE
    # misaligned pointer
    a = _lib.GemmFwdArgs(ctypes.sizeof(_lib.GemmFwdArgs), 1, 258, 256, None, 256, 4, 64, 64, 64,
                         256, 0)
    assert lib.moe_grouped_gemm_fwd(ctypes.byref(a), None) == INV
    # struct_size too small (ABI versioning)
    a = _lib.GemmFwdArgs(8, 1, 256, 256, None, 256, 4, 64, 64, 64, 256, 0)
    assert lib.moe_grouped_gemm_fwd(ctypes.byref(a), None) == INV
    # d not a multiple of 32
    g = _lib.GluFwdArgs(ctypes.sizeof(_lib.GluFwdArgs), 1, 256, 256, None, 256, 4, 64, 48, 64, 0,
                        0.0, 1.0, 0, None, 256, 0)
    assert lib.moe_grouped_gemm_glu_fwd(ctypes.byref(g), None) == INV
    b = _lib.GemmBwdArgs(ctypes.sizeof(_lib.GemmBwdArgs), 1, 5, 256, 256, 256, 256, 4, 64, 64, 64,
                         256, None, 0, 0)
    assert lib.moe_grouped_gemm_bwd(ctypes.byref(b), None) == INV


def test_transpose_weights_host_checks(lib):
    """moe_transpose_weights: sizes, pointers and aliasing are checked before
    anything is launched."""
    INV = _lib.MOE_ERR_INVALID_ARG
    a, b = ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 24)
    assert lib.moe_transpose_weights(a, 1, 2, 12, 64, b, None) == INV       # rows % 8
    assert lib.moe_transpose_weights(a, 1, 2, 64, 12, b, None) == INV       # cols % 8
    assert lib.moe_transpose_weights(a, 1, 0, 64, 64, b, None) == INV       # E
    assert lib.moe_transpose_weights(a, 5, 2, 64, 64, b, None) == INV       # dtype
    assert lib.moe_transpose_weights(None, 1, 2, 64, 64, b, None) == INV
    assert lib.moe_transpose_weights(a, 1, 2, 64, 64, a, None) == INV       # in place
    # overlapping source and destination
    assert lib.moe_transpose_weights(a, 1, 2, 64, 64, ctypes.c_void_p((1 << 20) + 4096),
                                     None) == INV
    assert lib.moe_transpose_weights(ctypes.c_void_p((1 << 20) + 2), 1, 2, 64, 64, b,
                                     None) == INV                           # misaligned
    # the dgrads' transposed operands must be 16-byte aligned too
    g = _lib.GluBwdArgs(ctypes.sizeof(_lib.GluBwdArgs), 1, 256, None, 256, 256, 4, 64, 64, 64,
                        0, 0.0, 1.0, 0, 256, 0)
    g.w2t = 258
    assert lib.moe_grouped_gemm_glu_bwd(ctypes.byref(g), None) == INV
    g.w2t = None                                                            # neither w2 nor w2t
    assert lib.moe_grouped_gemm_glu_bwd(ctypes.byref(g), None) == INV
    d = _lib.GemmBwdArgs(ctypes.sizeof(_lib.GemmBwdArgs), 1, _lib.MOE_BWD_DGRAD, 256, None,
                         None, 256, 4, 64, 64, 64, 256, None, 0, 0)
    assert lib.moe_grouped_gemm_bwd(ctypes.byref(d), None) == INV          # neither w nor wt
    d.wt = 264
    assert lib.moe_grouped_gemm_bwd(ctypes.byref(d), None) == INV


def test_mx_host_checks():
    """MXFP8 entry points: host-side sizes and argument errors (nothing is launched)."""
    lib = _lib.load()
    INV = _lib.MOE_ERR_INVALID_ARG
    # token axis of a column copy: R + 31 E rounded up to 128
    assert lib.moe_mx_col_len(100, 2) == 256
    assert lib.moe_mx_col_len(131072, 32) == 132096
    # allocation stride: the smallest ld >= that length whose rows are an odd
    # number of 128-byte lines (E4M3: 1 byte per element, E2M1: 2 per byte)
    assert lib.moe_mx_col_ld(131072, 32, _lib.MOE_E4M3) == 1033 * 128
    assert lib.moe_mx_col_ld(131072, 32, _lib.MOE_E2M1) == 517 * 256
    assert lib.moe_mx_col_ld(100, 2, _lib.MOE_E4M3) == 384
    assert lib.moe_mx_col_ld(100, 2, _lib.MOE_E2M1) == 256
    assert lib.moe_mx_col_ld(100, 2, _lib.MOE_BF16) == 0
    fake = ctypes.c_void_p(256)
    good = _lib.MxT(256, 256, 64)
    # n not a multiple of 32; ld smaller than n; misaligned codes
    assert lib.moe_mx_quantize(fake, 1, 4, 48, ctypes.byref(good), None) == INV
    assert lib.moe_mx_quantize(fake, 1, 4, 96, ctypes.byref(good), None) == INV
    assert lib.moe_mx_quantize(fake, 1, 4, 64, ctypes.byref(_lib.MxT(258, 256, 64)), None) == INV
    # transposed copy needs rows a multiple of 32
    assert lib.moe_mx_quantize_transpose(fake, 1, 2, 48, 64, ctypes.byref(good), None) == INV
    # gates without the row map / source rows
    assert lib.moe_mx_quantize_experts(fake, 1, None, None, fake, 2, fake, fake, 4, 64, 64,
                                       ctypes.byref(good), None, None) == INV
    assert lib.moe_mx_quantize_experts(fake, 1, None, fake, fake, 2, fake, fake, 4, 64, 64,
                                       ctypes.byref(good), None, None) == INV
    # MXFP8 GEMM: K must be a multiple of 128; no bias
    mx = _lib.MxT(256, 256, 96)
    a = _lib.GemmFwdArgs(ctypes.sizeof(_lib.GemmFwdArgs), _lib.MOE_E4M3, None, None, None, 256, 4,
                         64, 64, 96, 256, 0, ctypes.pointer(mx), ctypes.pointer(mx))
    assert lib.moe_grouped_gemm_fwd(ctypes.byref(a), None) == INV
    a = _lib.GemmFwdArgs(ctypes.sizeof(_lib.GemmFwdArgs), _lib.MOE_E4M3, None, None, fake, 256, 4,
                         64, 64, 128, 256, 0, ctypes.pointer(good), ctypes.pointer(good))
    assert lib.moe_grouped_gemm_fwd(ctypes.byref(a), None) == INV
    # MXFP8 FC1: squared ReLU is not part of the MXFP8 variant
    g = _lib.GluFwdArgs(ctypes.sizeof(_lib.GluFwdArgs), _lib.MOE_E4M3, None, None, None, 256, 4, 64,
                        128, 64, _lib.ACT["srelu"], 0.0, 1.0, 0, None, None, 0,
                        ctypes.pointer(good), ctypes.pointer(good), None, None, None)
    assert lib.moe_grouped_gemm_glu_fwd(ctypes.byref(g), None) == INV
    # MXFP8 weight gradient without pad_offsets, or with a bias gradient
    b = _lib.GemmBwdArgs(ctypes.sizeof(_lib.GemmBwdArgs), _lib.MOE_E4M3, _lib.MOE_BWD_WGRAD, None,
                         None, None, 256, 4, 64, 64, 64, 256, None, 0, 0, ctypes.pointer(good),
                         ctypes.pointer(good), None, None)
    assert lib.moe_grouped_gemm_bwd(ctypes.byref(b), None) == INV


def test_gather_host_checks():
    """Gather-fused permute arguments: where it is not built, and a source over
    2 GiB, are refused before anything is launched."""
    lib = _lib.load()
    INV = _lib.MOE_ERR_INVALID_ARG
    fake = 256
    good = _lib.MxT(256, 256, 128)
    # MXFP8 FC1 takes its rows from the quantizer: no src_row
    g = _lib.GluFwdArgs(ctypes.sizeof(_lib.GluFwdArgs), _lib.MOE_E4M3, None, None, None, fake, 4,
                        64, 128, 64, _lib.ACT["swiglu"], 0.0, 1.0, 0, None, None, 0,
                        ctypes.pointer(good), ctypes.pointer(good), None, None, None, fake, 64)
    assert lib.moe_grouped_gemm_glu_fwd(ctypes.byref(g), None) == INV
    # bf16 FC1 whose gathered source spans more than 2 GiB (2^20 rows x 1024 x 2 B)
    g = _lib.GluFwdArgs(ctypes.sizeof(_lib.GluFwdArgs), _lib.MOE_BF16, fake, fake, None, fake, 4,
                        64, 1024, 64, _lib.ACT["swiglu"], 0.0, 1.0, 0, fake, fake, 0,
                        None, None, None, None, None, fake, 1 << 20)
    assert lib.moe_grouped_gemm_glu_fwd(ctypes.byref(g), None) == INV
    # ... or no source rows at all
    g.src_rows = 0
    assert lib.moe_grouped_gemm_glu_fwd(ctypes.byref(g), None) == INV
    # DGRAD has no gathered operand
    b = _lib.GemmBwdArgs(ctypes.sizeof(_lib.GemmBwdArgs), _lib.MOE_BF16, _lib.MOE_BWD_DGRAD, fake,
                         fake, fake, fake, 4, 64, 64, 64, fake, None, 0, 0, None, None, None,
                         None, fake, 64)
    assert lib.moe_grouped_gemm_bwd(ctypes.byref(b), None) == INV
    # WGRAD source over 2 GiB
    b.mode = _lib.MOE_BWD_WGRAD
    b.a_src_rows = 1 << 24
    assert lib.moe_grouped_gemm_bwd(ctypes.byref(b), None) == INV
    # MXFP8 WGRAD: no gathered operand
    b = _lib.GemmBwdArgs(ctypes.sizeof(_lib.GemmBwdArgs), _lib.MOE_E4M3, _lib.MOE_BWD_WGRAD, None,
                         None, None, fake, 4, 64, 64, 128, fake, None, 0, 0, ctypes.pointer(good),
                         ctypes.pointer(good), None, fake, fake, 64)
    assert lib.moe_grouped_gemm_bwd(ctypes.byref(b), None) == INV


def test_struct_layouts_match_header(tmp_path):
    """Field offsets and sizes of the ctypes structures equal the C compiler's."""
    import os
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    structs = {"moe_glu_fwd_args_t": _lib.GluFwdArgs, "moe_gemm_fwd_args_t": _lib.GemmFwdArgs,
               "moe_glu_bwd_args_t": _lib.GluBwdArgs, "moe_gemm_bwd_args_t": _lib.GemmBwdArgs,
               "moe_mx_t": _lib.MxT}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "moe.h"', "int main(void){"]
    for cname, py in structs.items():
        lines.append(f'printf("{cname} size %zu\\n", sizeof({cname}));')
        for fname, _ in py._fields_:
            lines.append(f'printf("{cname} {fname} %zu\\n", offsetof({cname}, {fname}));')
    lines.append("return 0;}")
    src = tmp_path / "probe.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "probe"
    inc = os.path.dirname(_lib.HEADER)
    subprocess.run([cc, "-I", inc, str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout
    got = {}
    for line in out.splitlines():
        c, f, v = line.split()
        got[(c, f)] = int(v)
    for cname, py in structs.items():
        assert got[(cname, "size")] == ctypes.sizeof(py), cname
        for fname, _ in py._fields_:
            assert got[(cname, fname)] == getattr(py, fname).offset, (cname, fname)


def test_layer_materializes_xp_when_x_is_too_large_to_gather():
    """The gather-fused loaders address x with 31-bit offsets: a layer whose x
    spans 2 GiB or more takes the materialized-Xp path (built on the meta
    device, so nothing is allocated or run)."""
    import torch
    from ragged_grouped_gemm_amd.layer import MoEFFN
    small = MoEFFN(16384, 7168, 2048, 32, 8, device="meta")
    assert small.fuse_permute and small.xp is None
    T = 160_000                      # 160000 * 7168 * 2 bytes > 2 GiB
    assert not MoEFFN.gather_fits(T, 7168, torch.bfloat16)
    big = MoEFFN(T, 7168, 2048, 32, 1, device="meta")
    assert not big.fuse_permute
    assert big.xp is not None and tuple(big.xp.shape) == (T, 7168)
    # a float32 x reaches the limit at half the tokens
    assert MoEFFN.gather_fits(80_000, 7168, torch.bfloat16)
    assert not MoEFFN.gather_fits(80_000, 7168, torch.float32)


def test_layer_makes_transposed_weight_copies_where_they_pay():
    """By default the dgrads' transposed weight copies are made from 2048
    routed rows per expert on (built on the meta device: nothing runs)."""
    from ragged_grouped_gemm_amd.layer import MoEFFN
    dsv3 = MoEFFN(16384, 7168, 2048, 32, 8, device="meta")            # 4096 rows / expert
    assert dsv3.W2t is not None and dsv3.W1pt is not None
    gptoss = MoEFFN(8192, 2880, 2880, 32, 4, device="meta", bias=True)  # 1024 rows / expert
    assert gptoss.W2t is None and gptoss.W1pt is None
    forced = MoEFFN(8192, 2880, 2880, 32, 4, device="meta", transpose_w2=True,
                    transpose_w1=False)
    assert forced.W2t is not None and forced.W1pt is None
    edge = MoEFFN(2048 * 32 // 8, 256, 256, 32, 8, device="meta")     # exactly 2048 rows / expert
    assert edge.W2t is not None
