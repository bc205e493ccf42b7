"""The C ABI's host code under the undefined-behaviour sanitizer (CPU only): libcce is rebuilt
with UBSan on its host pass (the device code is compiled as usual, unsanitised) and the ABI
tests, which drive every argument check, workspace query and plan query with valid and invalid
values (out-of-range enums, sizes at and past the limits, null and misaligned pointers), run
against it in a child process, where any undefined behaviour aborts with a report."""
import glob
import os
import subprocess
import sys

import pytest

from linear_cross_entropy_cce_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _ubsan_runtime():
    pats = ["/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.ubsan_standalone-x86_64.so",
            "/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.ubsan_standalone-x86_64.so"]
    for p in pats:
        hits = sorted(glob.glob(p))
        if hits:
            return hits[-1]
    return None


def test_abi_host_code_is_free_of_undefined_behaviour(tmp_path):
    try:
        cmd = build.compile_command(str(tmp_path / "libcce.so"))
    except RuntimeError:
        pytest.skip("hipcc is not available")
    rt = _ubsan_runtime()
    if rt is None:
        pytest.skip("no UBSan runtime next to the ROCm compiler")
    cmd = [("-O1" if a == "-O3" else a) for a in cmd]
    cmd[1:1] = ["-g", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all"]
    cmd += [f"-Wl,{rt}", f"-Wl,-rpath,{os.path.dirname(rt)}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    code = (
        "import sys\n"
        f"sys.path[:0] = [{ROOT!r}, {os.path.join(ROOT, 'tests')!r}]\n"
        "import linear_cross_entropy_cce_amd._lib as L\n"
        f"L.LIB_PATH = {str(tmp_path / 'libcce.so')!r}\n"
        "import pytest\n"
        f"sys.exit(pytest.main(['-q', '-s', '-m', 'not gpu', '-p', 'no:cacheprovider', "
        f"{os.path.join(ROOT, 'tests', 'test_abi.py')!r}]))\n")
    env = dict(os.environ, UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                       cwd=ROOT, timeout=600)
    out = r.stdout + r.stderr
    assert "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
