"""The C ABI's host-side argument handling under AddressSanitizer, on the CPU.

The library sources are compiled for the host only (no device code: the
checks under test return before any kernel launch) with -fsanitize=address
applied to host code, linked with tests/abi_asan_driver.cpp, and run.  The
driver passes every argument struct at every size from 8 bytes up, allocated
at exactly that size, so a read past struct_size aborts the run; and it
checks the status codes of bad arguments of every entry point."""
import concurrent.futures as cf
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "ragged_grouped_gemm_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# sanitizer flags apply to host code only (-Xarch_host before each -fsanitize)
HOST_ASAN = ["-Xarch_host", "-fsanitize=address", "-fno-omit-frame-pointer", "-g", "-O1"]


CLANG = os.environ.get("MOE_CLANG", "/opt/rocm/llvm/bin/clang++")
ASAN = ["-fsanitize=address", "-fno-omit-frame-pointer", "-g", "-O1"]


def _fatbin_stubs(objs, path):
    """Each host-only object refers to its own device code bundle
    (__hip_fatbin_<hash>); define each as a well-formed offload bundle with
    no entries.  HIP registers them without reading code objects, and no
    kernel is ever launched here."""
    syms = set()
    for o in objs:
        out = subprocess.run(["nm", "-u", o], capture_output=True, text=True, check=True).stdout
        syms.update(l.split()[-1] for l in out.splitlines() if "__hip_fatbin_" in l)
    lines = ['\t.section .rodata.moe_asan_fatbin,"a",@progbits']
    for s_ in sorted(syms):
        lines += ["\t.p2align 4", f"\t.globl {s_}", f"{s_}:", '\t.ascii "__CLANG_OFFLOAD_BUNDLE__"',
                  "\t.quad 0"]
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    return len(syms)


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)),
                    reason="needs the ROCm compilers")
def test_abi_host_checks_under_asan(tmp_path):
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))

    def compile_one(name):
        obj = str(tmp_path / (name + ".o"))
        cmd = [HIPCC, "--offload-arch=gfx950", "--offload-host-only", "-std=c++17", "-fPIC",
               *HOST_ASAN, "-c", os.path.join(CSRC, name), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return obj

    with cf.ThreadPoolExecutor(max_workers=6) as ex:
        objs = list(ex.map(compile_one, srcs))
    stubs = str(tmp_path / "fatbin_stubs.s")
    assert _fatbin_stubs(objs, stubs) == len(srcs)
    drv = str(tmp_path / "driver.o")
    stub_o = str(tmp_path / "fatbin_stubs.o")
    exe = str(tmp_path / "abi_asan_driver")
    for cmd in ([CLANG, "-std=c++17", *ASAN, "-I", os.path.join(ROOT, "include"), "-c",
                 os.path.join(HERE, "abi_asan_driver.cpp"), "-o", drv],
                [CLANG, "-c", stubs, "-o", stub_o],
                [CLANG, *ASAN, drv, stub_o, *objs, "-L/opt/rocm/lib", "-lamdhip64",
                 "-Wl,-rpath,/opt/rocm/lib", "-o", exe]):
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    print(r.stdout[-2000:])
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-6000:])
    assert "abi host checks passed" in r.stdout
    # and the harness catches an over-read: a struct shorter than it claims
    r = subprocess.run([exe, "--overread"], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, (r.stdout, r.stderr[-3000:])
