"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

mq_api.hip (validation, kernel choice, the mixed-call planner) is compiled
with the sanitizers on its host side, linked with the kernel objects of the
ordinary build, and driven by tests/abi_sanitizer_driver.c, which calls every
entry point with arguments that fail validation and the pure queries with
shapes up to the int32 limits.  Nothing reaches a GPU, so this runs on the
CPU."""
import os
import shutil
import subprocess

import pytest

from nested_integer_weight_amd import build as B

HERE = os.path.dirname(os.path.abspath(__file__))
DRIVER = os.path.join(HERE, "abi_sanitizer_driver.c")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-fno-sanitize-recover=all"]


def _run(cmd, **kw):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, **kw)
    return p.returncode, p.stdout


def _kernel_objects(tmp):
    """The ordinary build's objects of every source but mq_api.hip, rebuilt
    into `tmp` when missing or older than a source."""
    hipcc = B._hipcc()
    headers = [os.path.join(B.CSRC, f) for f in os.listdir(B.CSRC) if f.endswith(".h")]
    newest_header = max(os.path.getmtime(h) for h in headers)
    objs = []
    for src in B.SOURCES:
        if src == "mq_api.hip":
            continue
        path = os.path.join(B.CSRC, src)
        obj = os.path.join(B.BUILD, src.replace(".hip", ".o"))
        if not os.path.exists(obj) or os.path.getmtime(obj) < max(os.path.getmtime(path), newest_header):
            obj = os.path.join(tmp, src.replace(".hip", ".o"))
            rc, out = _run([hipcc, *B.COMMON, *B.EXTRA.get(src, []), "-c", path, "-o", obj])
            assert rc == 0, out
        objs.append(obj)
    return objs


@pytest.mark.timeout(900)
def test_abi_validation_under_asan_and_ubsan(tmp_path):
    try:
        hipcc = B._hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    if shutil.which("ld.lld") is None and not os.path.exists("/opt/rocm/llvm/bin/ld.lld"):
        pytest.skip("no linker")
    tmp = str(tmp_path)
    api = os.path.join(tmp, "mq_api_san.o")
    rc, out = _run([hipcc, *B.COMMON, "-O1", "-g", *SAN, "-c", os.path.join(B.CSRC, "mq_api.hip"), "-o", api])
    assert rc == 0, out
    drv = os.path.join(tmp, "driver.o")
    rc, out = _run([hipcc, "-O1", "-g", *SAN, "-x", "c", f"-I{os.path.join(B.ROOT, 'include')}", "-c", DRIVER,
                    "-o", drv])
    assert rc == 0, out
    exe = os.path.join(tmp, "abi_driver")
    rc, out = _run([hipcc, f"--offload-arch={B.ARCH}", *SAN, drv, api, *_kernel_objects(tmp), "-o", exe])
    assert rc == 0, out
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    rc, out = _run([exe], env=env, timeout=300)
    assert rc == 0 and "all checks passed" in out, out
    assert "runtime error" not in out and "AddressSanitizer" not in out, out
