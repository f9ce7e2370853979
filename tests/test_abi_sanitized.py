"""The C-ABI boundary code (csrc/qmoe_api.cpp, csrc/expert_cache.cpp) built with AddressSanitizer and
UndefinedBehaviorSanitizer on the host, driven by tests/native/abi_sanitize.cpp
through every entry point's validation and the workspace sizing.  CPU only:
none of these calls reaches the device.  The kernels' objects come from the
regular build (_build/), unsanitised; only the boundary is instrumented."""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang++"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


@pytest.mark.slow
def test_abi_under_host_sanitizers(tmp_path):
    boundary = ("qmoe_api", "expert_cache")   # host-only sources of the boundary
    objs = [o for o in glob.glob(os.path.join(ROOT, "_build", "*.o"))
            if os.path.splitext(os.path.basename(o))[0] not in boundary]
    if not shutil.which(CLANG) or len(objs) < 5:
        pytest.skip("needs the regular build (_build/*.o) and the ROCm clang")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "quantized_moe_02_amd", "csrc"),
           "-I", "/opt/rocm/include", "-D__HIP_PLATFORM_AMD__"]
    drv = str(tmp_path / "abi_sanitize.o")
    exe = str(tmp_path / "abi_sanitize")
    # host-only C++ (the boundary holds no device code)
    san_objs = []
    for name in boundary:
        o = str(tmp_path / f"{name}_san.o")
        subprocess.run([CLANG, "-x", "c++", "-std=c++17", "-O1", "-g", *SAN, *inc, "-c",
                        os.path.join(ROOT, "quantized_moe_02_amd", "csrc", f"{name}.cpp"), "-o", o],
                       check=True)
        san_objs.append(o)
    subprocess.run([CLANG, "-std=c++17", "-O1", "-g", *SAN, *inc, "-c",
                    os.path.join(ROOT, "tests", "native", "abi_sanitize.cpp"), "-o", drv], check=True)
    subprocess.run([CLANG, *SAN, drv, *san_objs, *objs, "-L/opt/rocm/lib", "-lamdhip64",
                    "-Wl,-rpath,/opt/rocm/lib", "-o", exe], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failure(s)" in r.stdout
