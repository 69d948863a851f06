"""The host layer of libi4s built for the CPU with AddressSanitizer and
UndefinedBehaviorSanitizer (no GPU needed).

``i4s_api.cpp`` (argument checks, device check, adaptive group choice,
dispatch) and ``i4s_plan.cpp`` (the K-split workspace plan) are compiled with
g++ against a stand-in for the HIP runtime and the kernel launchers
(``host/i4s_hip_stub.cpp``), and ``host/host_driver.cpp`` calls every entry
point of ``include/i4s.h`` through the C ABI.  Any sanitizer report aborts the
driver (``-fno-sanitize-recover=all``), so the test passes only when every
check holds and nothing out of bounds, uninitialized-size or undefined was
touched.  A second run makes the stand-in device report another
architecture and expects I4S_ERR_UNSUPPORTED from every call that would use
the device.
"""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "int4_sparse_gemv_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=99",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def gxx():
    cc = shutil.which("g++")
    if cc is None or not os.path.isdir("/opt/rocm/include/hip"):
        pytest.skip("g++ or the HIP headers are missing")
    return cc


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("host") / "host_driver")
    cmd = [gxx(), "-std=c++17", "-g", "-O1", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", os.path.join(HERE, "host"),
           os.path.join(CSRC, "i4s_api.cpp"), os.path.join(CSRC, "i4s_plan.cpp"),
           os.path.join(HERE, "host", "i4s_hip_stub.cpp"), os.path.join(HERE, "host", "host_driver.cpp"),
           "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    return out


def test_sanitizers_are_active(tmp_path):
    """The same flags catch a planted heap overflow (the toolchain's
    sanitizer runtime is really in the build)."""
    src = tmp_path / "overflow.cpp"
    src.write_text("#include <cstdlib>\nint main(int c, char**) { int *p = (int*)std::malloc(16);"
                   " int v = p[c + 3]; std::free(p); return v == 12345; }\n")
    exe = str(tmp_path / "overflow")
    r = subprocess.run([gxx(), "-g", "-O0", *SAN, str(src), "-o", exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=60)
    assert r.returncode != 0 and "AddressSanitizer" in r.stderr


def test_host_layer_every_entry_point(driver):
    r = subprocess.run([driver], capture_output=True, text=True, env=ENV, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr[-4000:]
    assert r.stdout.startswith("ok "), r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr


@pytest.mark.parametrize("arch", ["gfx942", "gfx90a", "gfx1100"])
def test_other_architecture_is_unsupported(driver, arch):
    r = subprocess.run([driver, "--arch", arch], capture_output=True, text=True, env=ENV, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr[-4000:]
    assert r.stdout.startswith("ok "), r.stdout
