"""One HIP runtime per process.

PyTorch ships its own HIP and HSA runtimes.  The library links them by
soname, so it must bind to the copies torch already loaded: two copies of the
runtime in one process own the device independently (every launch through the
second copy fails, and the process later crashes).  Importing the package
imports torch first; these checks pin that, on the CPU, by reading the
process's own memory map (no GPU call is made)."""
import os
import subprocess
import sys
import textwrap

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROBE = textwrap.dedent("""
    import ctypes, sys
    sys.path.insert(0, {root!r})
    if {lib_first}:
        ctypes.CDLL({lib!r})
    import top_sampling_amd  # imports torch, then loads the library
    maps = open("/proc/self/maps").read().splitlines()
    for key in ("amdhip64", "hsa-runtime64"):
        paths = sorted({{ln.split()[-1] for ln in maps if key in ln and "/" in ln}})
        print(key, len(paths), *paths)
""")


def _mapped(lib_first: bool) -> dict:
    import top_sampling_amd as ts

    code = PROBE.format(root=ROOT, lib=ts.LIB_PATH, lib_first=lib_first)
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                         timeout=300, env={**os.environ, "HIP_VISIBLE_DEVICES": ""})
    assert out.returncode == 0, out.stderr[-2000:]
    res = {}
    for ln in out.stdout.splitlines():
        f = ln.split()
        if f and f[0] in ("amdhip64", "hsa-runtime64"):
            res[f[0]] = f[2:]
    return res


def test_import_maps_one_hip_runtime():
    import torch

    res = _mapped(lib_first=False)
    torch_lib = os.path.join(os.path.dirname(torch.__file__), "lib")
    for key in ("amdhip64", "hsa-runtime64"):
        assert len(res[key]) == 1, res
        assert os.path.dirname(os.path.realpath(res[key][0])) == os.path.realpath(torch_lib), res


def test_loading_the_library_before_torch_maps_two():
    """The failure this guards against, reproduced on the CPU: loading the
    library before torch maps a second HIP runtime (so the check above can
    tell the two orders apart)."""
    res = _mapped(lib_first=True)
    assert len(res["amdhip64"]) == 2, res
