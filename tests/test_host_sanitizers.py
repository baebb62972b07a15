"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two builds, each loaded by the existing tests in a child process with the
sanitizer runtime preloaded (Python itself is not instrumented):
- the oracle (oracle.c, gcc) with -fsanitize=address,undefined, through
  ORACLE_LIB, running the oracle's own test files;
- the library's C-ABI layer (api.hip: argument validation, sizes, status
  strings) with its host half instrumented (clang via hipcc; device code is
  untouched), linked with the other objects of the normal build, through
  MOE_EP_LIB, running the host ABI tests, which never launch a kernel.

A sanitizer report ends the child with an error, and the report is shown.
"""

import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "combine_route_topk_amd")
ORACLE_TESTS = ["test_oracle_route.py", "test_oracle_layout.py", "test_oracle_combine.py",
                "test_oracle_fp8.py", "test_oracle_regroup.py", "test_oracle_expert.py"]


def _run_child(env_extra, tests, tmp_path):
    env = dict(os.environ)
    env.update(env_extra)
    logs = tmp_path / "reports"
    logs.mkdir()
    env["ASAN_OPTIONS"] = f"detect_leaks=0:halt_on_error=1:log_path={logs}/asan"
    env["UBSAN_OPTIONS"] = f"halt_on_error=1:print_stacktrace=1:log_path={logs}/ubsan"
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
           *[os.path.join(ROOT, "tests", t) for t in tests]]
    r = subprocess.run(cmd, env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    reports = "".join(open(p, errors="replace").read() for p in sorted(glob.glob(f"{logs}/*")))
    assert r.returncode == 0 and not reports, (reports or "") + r.stdout[-3000:] + r.stderr[-3000:]


def test_oracle_under_asan_ubsan(tmp_path):
    libasan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                             text=True).stdout.strip()
    if not os.path.isabs(libasan):
        pytest.skip("gcc has no AddressSanitizer runtime")
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
                    "-fno-fast-math", "-fno-builtin", "-shared", "-fPIC",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    os.path.join(ROOT, "oracle", "oracle.c"), "-o", lib, "-lm"], check=True)
    _run_child({"LD_PRELOAD": libasan, "ORACLE_LIB": lib}, ORACLE_TESTS, tmp_path)


def _moe_build():
    """The library's build script (combine_route_topk_amd/build.py) as a module."""
    import importlib.util
    spec = importlib.util.spec_from_file_location("moe_ep_build", os.path.join(PKG, "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_abi_layer_under_asan_ubsan(tmp_path):
    moe_build = _moe_build()
    runtimes = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    normal = [os.path.join(moe_build.BUILD_DIR, s.replace(".hip", ".o"))
              for s in moe_build.SOURCES if s != "api.hip"]
    if not runtimes or not all(os.path.exists(o) for o in normal):
        pytest.skip("needs the ROCm clang sanitizer runtime and a normal build's objects")
    api_o = str(tmp_path / "api_san.o")
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]
    flags = [f for f in moe_build.FLAGS if f != "-O3"] + ["-O1", "-g"] + host_san
    subprocess.run([moe_build.HIPCC, *flags, "-c", os.path.join(PKG, "csrc", "api.hip"), "-o", api_o],
                   check=True, capture_output=True)
    lib = str(tmp_path / "libmoe_ep_san.so")
    subprocess.run([moe_build.HIPCC, f"--offload-arch={moe_build.ARCH}", "-shared", "-fPIC", api_o, *normal,
                    "-o", lib], check=True, capture_output=True)
    _run_child({"LD_PRELOAD": runtimes[-1], "MOE_EP_LIB": lib}, ["test_abi_host.py"], tmp_path)
