"""The CPU oracle and the C ABI's host-side code under AddressSanitizer (CPU
only, no GPU work).

* oracle/qmm_oracle.c built with gcc -fsanitize=address,undefined (UB
  aborts), then the oracle's own pin tests run against that build;
* the exported C ABI (qmm_api.hip: argument checks, error strings, the
  geometry and name calls, the workspace-size functions) compiled with
  host-side ASan and linked with the library's other objects, then the ABI
  tests (refusals in the documented order, sizes, names) run against it.

Each run is a child Python process with the sanitizer runtime preloaded; a
sanitizer report ends it with a non-zero status.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gguf_block_quantized_kind_amd", "csrc")
OBJDIR = os.path.join(ROOT, "_build")
HIPCC = "/opt/rocm/bin/hipcc"


def _gcc_asan():
    if not shutil.which("gcc"):
        return None
    p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def _clang_asan():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def _run_child(code, preload):
    env = dict(os.environ, LD_PRELOAD=preload, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    assert r.returncode == 0, f"status {r.returncode}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r.stdout


CHILD = """
import sys
{setup}
import pytest
status = pytest.main(["-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu", {files}])
maps = open("/proc/self/maps").read()
if {lib!r} not in maps or "asan" not in maps:
    print("the sanitized library was not the one loaded")
    sys.exit(3)
sys.exit(int(status))
"""


def test_oracle_under_asan(tmp_path):
    rt = _gcc_asan()
    if rt is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = str(tmp_path / "liboracle_asan.so")
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-ffp-contract=off",
                    os.path.join(ROOT, "oracle", "qmm_oracle.c"), "-o", lib, "-lm"], check=True)
    files = ", ".join(repr(f"tests/{f}") for f in ("test_oracle_pins.py", "test_oracle_ffn.py",
                                                    "test_oracle_int8.py", "test_oracle_repack.py"))
    out = _run_child(CHILD.format(setup=f"import oracle\noracle._default = oracle.Oracle({lib!r})",
                                  files=files, lib=lib), rt)
    assert "passed" in out


def _library_objects():
    """The library's objects from the in-tree build, rebuilt when a source
    is newer than its object."""
    srcs = glob.glob(os.path.join(CSRC, "*.hip"))
    newest = max(os.path.getmtime(p) for p in glob.glob(os.path.join(CSRC, "*")))
    objs = [os.path.join(OBJDIR, os.path.basename(s) + ".o") for s in srcs]
    if any(not os.path.exists(o) or os.path.getmtime(o) < newest for o in objs):
        from gguf_block_quantized_kind_amd import _build
        _build.build()
    return [o for o in objs if not o.endswith("qmm_api.hip.o")]


def test_c_abi_host_code_under_asan(tmp_path):
    rt = _clang_asan()
    if rt is None or not os.path.exists(HIPCC):
        pytest.skip("hipcc or clang's AddressSanitizer runtime is not installed")
    others = _library_objects()
    api = str(tmp_path / "qmm_api_asan.o")
    lib = str(tmp_path / "libqmm_asan.so")
    # Host code only is sanitized; the file has no device code.
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-fno-omit-frame-pointer",
                    "-Xarch_host", "-fsanitize=address", "-I", os.path.join(ROOT, "include"), "-c",
                    os.path.join(CSRC, "qmm_api.hip"), "-o", api], check=True, capture_output=True)
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address", api,
                    *others, "-o", lib], check=True, capture_output=True)
    out = _run_child(CHILD.format(setup=f"import gguf_block_quantized_kind_amd as q\nq.load_library({lib!r})",
                                  files="'tests/test_abi.py'", lib=lib), rt)
    assert "passed" in out
