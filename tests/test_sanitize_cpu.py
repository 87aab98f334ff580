"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU):

  * the CPU oracle (oracle/flo_oracle.c), driven through every function on
    small and edge-case inputs by tests/sanitize/oracle_drive.c, built with
    gcc -fsanitize=address,undefined;
  * the C ABI's host code (argument validation, error paths, workspace
    sizing, the timing and check switches, the host validators): abi.hip
    recompiled with the sanitizers on its host side only, linked with the
    library's other objects, and driven by tests/sanitize/abi_drive.c.

Sanitizer reports abort the drivers (-fno-sanitize-recover); a test fails on
a non-zero exit or any report in the output."""
import glob
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
BUILD = os.path.join(ROOT, "sparse_attention_kv_amd", "_build")
CLANG = "/opt/rocm/lib/llvm/bin/clang"
HIPCC = "/opt/rocm/bin/hipcc"


def _run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    return r.returncode, r.stdout + r.stderr


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_drive")
    rc, out = _run(["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                    os.path.join(SAN, "oracle_drive.c"), os.path.join(ROOT, "oracle", "flo_oracle.c"),
                    "-lm", "-o", exe])
    assert rc == 0, out
    rc, out = _run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0"))
    assert rc == 0 and "ERROR" not in out and "runtime error" not in out, out
    assert "ok" in out


@pytest.mark.slow
def test_abi_host_under_asan_ubsan(tmp_path):
    objs = [os.path.join(BUILD, f"{s}.o") for s in ("select", "quant", "attn", "adaptive", "block", "decode", "calib")]
    if not all(os.path.exists(o) for o in objs):
        from sparse_attention_kv_amd import build
        build.build()
    rt = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not (os.path.exists(CLANG) and os.path.exists(HIPCC) and rt):
        pytest.skip("ROCm clang / hipcc / sanitizer runtime not found")
    abi_o = str(tmp_path / "abi_san.o")
    # the sanitizers instrument the host side of abi.hip only
    rc, out = _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-std=c++17",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                    "-fhip-fp32-correctly-rounded-divide-sqrt",
                    "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(ROOT, "sparse_attention_kv_amd", "csrc"),
                    "-Wno-unused-command-line-argument",
                    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                    "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
                    "-c", os.path.join(ROOT, "sparse_attention_kv_amd", "csrc", "abi.hip"), "-o", abi_o])
    assert rc == 0, out
    lib = str(tmp_path / "libflashloop_san.so")
    rc, out = _run([CLANG + "++", "-shared", "-fPIC", "-fsanitize=address,undefined", "-shared-libsan",
                    "-o", lib, abi_o, *objs, "-L/opt/rocm/lib", "-lamdhip64"])
    assert rc == 0, out
    exe = str(tmp_path / "abi_drive")
    rc, out = _run([CLANG, "-O1", "-g", "-fsanitize=address,undefined", "-shared-libsan",
                    "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"),
                    os.path.join(SAN, "abi_drive.c"), lib, f"-Wl,-rpath,{tmp_path}", "-o", exe])
    assert rc == 0, out
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0",   # the HIP runtime keeps its allocations
               LD_LIBRARY_PATH=os.path.dirname(rt[-1]) + ":/opt/rocm/lib")
    rc, out = _run([exe], env=env)
    assert rc == 0 and "ERROR" not in out and "runtime error" not in out, out
    assert "ok" in out
