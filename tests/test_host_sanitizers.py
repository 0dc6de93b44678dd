"""The library's host code (argument validation, size arithmetic, the device
set-up) built with AddressSanitizer and UndefinedBehaviorSanitizer on the CPU
and driven through every entry point of include/mapl.h by
tests/sanitize/abi_driver.cpp: invalid arguments, extreme sizes and valid
shapes (which stop at the device set-up without a device).  Only host code is
instrumented; no kernel is launched."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "learned_activation_compression_amd", "csrc")
SAN = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -fno-sanitize-recover=all"


def _hipcc():
    for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


@pytest.mark.timeout(900)
def test_host_abi_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    cc = _hipcc()
    if cc is None:
        pytest.skip("hipcc not available")
    import torch
    if torch.cuda.is_available():
        pytest.skip("a device is present: the driver's valid calls would launch kernels")
    from learned_activation_compression_amd.build import SOURCES
    common = ["-O1", "-g", "-std=c++17", "-fPIC", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]
    # the device code is compiled as usual (and never run here); only the host side is instrumented
    import concurrent.futures as cf
    objs, cmds = [], []
    for src in SOURCES:
        obj = str(tmp_path / src.replace(".hip", ".o"))
        cmds.append([cc, "--offload-arch=gfx950", *SAN.split(), *common, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(cmds))) as ex:
        for f in [ex.submit(subprocess.run, c, check=True, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
                  for c in cmds]:
            f.result()
    drv = str(tmp_path / "abi_driver.o")
    subprocess.run([cc, "-x", "c++", *SAN.split(), *common, "-I/opt/rocm/include", "-D__HIP_PLATFORM_AMD__", "-c",
                    os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp"), "-o", drv],
                   check=True, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    exe = str(tmp_path / "abi_driver")
    subprocess.run([cc, "--offload-arch=gfx950", *SAN.split(), *objs, drv, "-o", exe], check=True,
                   stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    p = subprocess.run([exe], env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=300)
    assert p.returncode == 0, p.stdout[-4000:]
    assert "runtime error" not in p.stdout and "AddressSanitizer" not in p.stdout, p.stdout[-4000:]
    assert "all expectations held" in p.stdout
