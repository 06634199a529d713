"""libhc from a C99 program (tests/c_client/hc_client.c): the header serves a
C caller, the library links with the HIP runtime alone, and the entry points
work through plain pointers.  Built with gcc into the test's temporary folder."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_client", "hc_client.c")
LIBDIR = os.path.join(ROOT, "transformer_hyper_connection_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _build(tmp_path):
    if not os.path.exists(os.path.join(LIBDIR, "libhc.so")):
        pytest.skip("libhc.so is not built")
    if shutil.which("gcc") is None:
        pytest.skip("no gcc")
    exe = str(tmp_path / "hc_client")
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROCM, "include"), SRC, "-o", exe, "-L", LIBDIR, "-lhc", "-L", os.path.join(ROCM, "lib"),
           "-lamdhip64", f"-Wl,-rpath,{LIBDIR}", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return exe


def test_c_client_abi(tmp_path):
    exe = _build(tmp_path)
    r = subprocess.run([exe, "abi"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "hc_client abi: ok" in r.stdout


@pytest.mark.gpu
def test_c_client_gpu(tmp_path):
    exe = _build(tmp_path)
    r = subprocess.run([exe, "gpu"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "hc_client gpu: ok" in r.stdout
