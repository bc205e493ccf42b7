"""libcce from plain C: tests/c/cce_c_client.c uses only include/cce.h and HIP's C runtime API
(no Python, no PyTorch).  On the CPU it must compile as strict C99 (-Wall -Wextra -Werror
-pedantic for its own code and for cce.h) and link against libcce.so; on the GPU it runs a
forward and backward end to end, whose results are compared with the oracle."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import cce_synth as S
import oracle
from gpu_helpers import EPS, GRAD_TOL, II, LOSS_TOL, borderline_blocks, log, rel

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "linear_cross_entropy_cce_amd")
SRC = os.path.join(ROOT, "tests", "c", "cce_c_client.c")
ROCM = "/opt/rocm"


def compile_client(out_dir):
    gcc = shutil.which("gcc")
    if gcc is None or not os.path.exists(os.path.join(ROCM, "include", "hip")):
        pytest.skip("gcc or the HIP headers are not available")
    if not os.path.exists(os.path.join(PKG, "libcce.so")):
        pytest.skip("libcce.so is not built")
    exe = os.path.join(out_dir, "cce_c_client")
    cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-isystem", os.path.join(ROCM, "include"), SRC,
           "-o", exe, "-L", PKG, "-lcce", f"-Wl,-rpath,{PKG}",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    return exe


def test_c_client_compiles_as_c99(tmp_path):
    exe = compile_client(str(tmp_path))
    assert os.access(exe, os.X_OK)


def bf16_bits(x):
    """bf16 bit patterns of float32 values that are exact in bf16."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32)
    assert np.all(u & 0xFFFF == 0)
    return (u >> 16).astype(np.uint16)


@pytest.mark.gpu
def test_c_client_matches_the_oracle(tmp_path):
    exe = compile_client(str(tmp_path))
    N, D, V = 300, 136, 20000          # three vocabulary chunks, a K tail
    d = S.small_case(N, D, V, "bf16", 141, 3.0, 1.1, 0.1)
    w = S.dloss_weights(141, N)
    src, dst = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(src, "wb") as f:
        f.write(np.array([N, V, D, II], np.int64).tobytes())
        f.write(np.array([EPS], np.float32).tobytes())
        f.write(bf16_bits(d["E"]).tobytes())
        f.write(bf16_bits(d["C"]).tobytes())
        f.write(np.ascontiguousarray(d["targets"], np.int64).tobytes())
        f.write(np.asarray(w, np.float32).tobytes())
    r = subprocess.run([exe, str(src), str(dst)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    log(r.stdout.strip())
    raw = np.fromfile(dst, dtype=np.uint8)
    off = 0

    def take(n, dt):
        nonlocal off
        a = raw[off:off + n * np.dtype(dt).itemsize].view(dt)
        off += n * np.dtype(dt).itemsize
        return a

    loss, lse = take(N, np.float32), take(N, np.float32)
    dE, dC = take(N * D, np.float32).reshape(N, D), take(V * D, np.float32).reshape(V, D)
    skipped, total = take(2, np.int64)
    assert off == raw.size
    rl, rs = oracle.forward(d["E"], d["C"], d["targets"], II)
    rE, rC, (sk, tot) = oracle.backward(d["E"], d["C"], d["targets"], w, II, filter_eps=EPS)
    uE, uC, _ = oracle.backward(d["E"], d["C"], d["targets"], w, II)
    log(f"[C client] loss {np.abs(loss - rl).max():.2e} dE {rel(dE, rE):.2e} dC {rel(dC, rC):.2e} "
        f"skipped {skipped}/{total} (oracle {sk}/{tot})")
    assert np.abs(loss - rl).max() <= LOSS_TOL and np.abs(lse - rs).max() <= LOSS_TOL
    assert rel(dE, rE) <= GRAD_TOL and rel(dC, rC) <= GRAD_TOL
    assert rel(dE, uE) <= GRAD_TOL and rel(dC, uC) <= GRAD_TOL
    assert total == tot
    assert skipped == sk or abs(int(skipped) - sk) <= borderline_blocks(d["E"], d["C"],
                                                                        d["targets"], EPS)
