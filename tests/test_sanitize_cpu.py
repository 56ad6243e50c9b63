"""The host code of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

pa_api.cpp (argument checks, plan building, suggestions, table checks) is compiled with both
sanitizers on its host side (the device code is untouched), linked with the in-tree objects of
the other sources into a separate library, and tests/test_abi_cpu.py is run against that library
in a child process that loads the ASan runtime first.  Any sanitizer report fails the run."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_attention_attn_amd", "csrc")
BUILD = os.path.join(ROOT, "_build")
OTHERS = ["pa_decode", "pa_balanced", "pa_qblock", "pa_reduce", "pa_aux"]
CLANG = "/opt/rocm/llvm/bin/clang++"
HIPCC = "/opt/rocm/bin/hipcc"


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)),
                    reason="the ROCm toolchain is needed to build the library")
def test_abi_host_code_under_address_and_undefined_sanitizers(tmp_path):
    # the other sources' objects: the in-tree build's, or built here the same way
    spec = __import__("importlib.util").util.spec_from_file_location(
        "_pa_build", os.path.join(ROOT, "paged_kv_attention_attn_amd", "build.py"))
    build = __import__("importlib.util").util.module_from_spec(spec)
    spec.loader.exec_module(build)
    objs = []
    for name in OTHERS:
        obj = os.path.join(BUILD, name + ".o")
        if not os.path.exists(obj):
            os.makedirs(BUILD, exist_ok=True)
            obj = build._compile(name + ".hip", False)
        objs.append(obj)
    api = str(tmp_path / "pa_api_san.o")
    host_san = []
    for flag in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
                 "-fno-omit-frame-pointer"):
        host_san += ["-Xarch_host", flag]
    _run([HIPCC, "-x", "hip", "-O1", "-g", "-fPIC", "-std=c++17", f"--offload-arch={build.ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          f"-I{os.path.join(ROOT, 'include')}"] + host_san +
         ["-c", os.path.join(CSRC, "pa_api.cpp"), "-o", api])
    lib = str(tmp_path / "libpaged_attn_san.so")
    link_san = ["-f" + "sanitize=address", "-f" + "sanitize=undefined", "-shared-libsan"]
    _run([CLANG, "-shared", "-fPIC"] + link_san + ["-o", lib, api] + objs +
         ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"])
    # instrumented: the library calls into both runtimes
    undef = _run(["nm", "-D", "--undefined-only", lib]).stdout
    assert "__asan_report_load" in undef and "__ubsan_handle_" in undef
    runtime = _run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"]).stdout.strip()
    assert os.path.exists(runtime), runtime
    env = dict(os.environ)
    env["PA_LIBRARY"] = lib
    env["LD_PRELOAD"] = runtime + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    code = ("import sys, pytest, paged_kv_attention_attn_amd as pa\n"
            f"assert pa.LIB_PATH == {lib!r}, pa.LIB_PATH\n"
            "sys.exit(pytest.main(['-q', '-x', '-s', '-p', 'no:cacheprovider', "
            f"{os.path.join(ROOT, 'tests', 'test_abi_cpu.py')!r}]))\n")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                       cwd=ROOT, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-6000:]
    assert r.returncode == 0 and " passed" in r.stdout, out[-6000:]
