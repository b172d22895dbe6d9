"""The C ABI's host-side validation under AddressSanitizer.

The library's host code (argument validation, workspace arithmetic, slice
tables) is compiled with AddressSanitizer and linked with a driver
(tests/asan/abi_driver.cpp) that walks every entry point's checks.  Only host
code is sanitized (device code is built as usual and never run: no call in the
driver reaches a launch), so this runs on the CPU."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "top_sampling_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Every source of the library: host code only, sanitized.
SOURCES = ["api.hip", "lmhead_gemm.hip", "lmhead_fp8.hip", "sampler_fast.hip", "sampler_exact.hip",
           "assemble.hip", "clock_probe.hip", "noise_readout.hip", "noalloc.hip"]


def _compile(args):
    r = subprocess.run(args, capture_output=True, text=True, timeout=600)
    return r.returncode, r.stdout[-3000:] + r.stderr[-3000:]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_validation_layer_under_asan(tmp_path):
    import concurrent.futures

    # Device code is built as usual (unsanitized); only the host side of each
    # translation unit carries the sanitizer.
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer",
             "-Xarch_host", "-fsanitize=address", "-Wno-unused-command-line-argument",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    srcs = [os.path.join(CSRC, s) for s in SOURCES] + [
        os.path.join(ROOT, "tests", "asan", "abi_driver.cpp")]
    objs = [str(tmp_path / (os.path.basename(s) + ".o")) for s in srcs]
    jobs = [[HIPCC, *flags, "-x", "hip", "-c", s, "-o", o] for s, o in zip(srcs, objs)]
    with concurrent.futures.ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        for rc, log in ex.map(_compile, jobs):
            assert rc == 0, log
    exe = tmp_path / "abi_driver"
    rc, log = _compile([HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address",
                        *objs, "-o", str(exe)])
    assert rc == 0, log
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=23",
               HIP_VISIBLE_DEVICES="")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "abi_driver: 0 failures" in r.stdout
    assert "AddressSanitizer" not in r.stderr
