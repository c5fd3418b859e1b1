"""The runtime's host code and the CPU comparator under AddressSanitizer and
UndefinedBehaviorSanitizer, without a GPU.

Builds tests/host_asan/driver.cpp against every library source with the
sanitizers on the host code only (device code is compiled as usual and never
runs), and runs it: pure host functions over their input ranges, the argument
checks of the entry points, the host-CPU attention on ragged pages and the
host-DRAM probe. Any sanitizer report fails the test."""
import os
import subprocess

import pytest

from decode_attention_zero_amd import _build

HOST_SAN = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, " ".join(cmd) + "\n" + res.stdout[-3000:] + res.stderr[-3000:]
    return res


@pytest.mark.skipif(not os.path.exists(_build.HIPCC), reason="needs hipcc")
def test_host_code_is_clean_under_sanitizers(tmp_path):
    clang = os.path.join(os.path.dirname(os.path.realpath(_build.HIPCC)), "..", "lib", "llvm", "bin", "clang++")
    clang = clang if os.path.exists(clang) else "/opt/rocm/lib/llvm/bin/clang++"
    inc = ["-I", _build.INCLUDE, "-I", _build.CSRC]
    objs = []
    for src in [os.path.join(_build.CSRC, s) for s in _build.HOST_SOURCES] + \
               [os.path.join(os.path.dirname(__file__), "host_asan", "driver.cpp")]:
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([clang, "-O1", "-g", "-std=c++17", "-c", src, "-o", obj] + HOST_SAN + inc)
        objs.append(obj)
    exe = str(tmp_path / "driver")
    host_flags = []
    for flag in HOST_SAN:
        host_flags += ["-Xarch_host", flag]
    _run([_build.HIPCC, "-O1", "-g", "-std=c++17", "--offload-arch=" + _build.ARCH,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"] + host_flags + inc +
         _build.sources() + ["-x", "none"] + objs + ["-o", exe, "-pthread"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", HIP_VISIBLE_DEVICES="")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert "AddressSanitizer" not in res.stderr and "runtime error" not in res.stderr, res.stderr[-3000:]
    assert res.returncode == 0 and res.stdout.strip().endswith("OK"), res.stdout + res.stderr[-2000:]
