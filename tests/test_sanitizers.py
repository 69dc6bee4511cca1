"""AddressSanitizer + UndefinedBehaviorSanitizer (+ LeakSanitizer) builds of
the CPU oracle and of the host side of libgear.so, each run by a C driver
(tests/native/).  Host code only: device code is built without sanitizers,
and no driver needs a GPU (device pointers there are fake and every call is
refused on the host, or fails to launch on a machine without a GPU)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")
CSRC = os.path.join(ROOT, "kv_cache_compression_gear_amd", "csrc")
OBJS = os.path.join(ROOT, "kv_cache_compression_gear_amd", "_build")
ROCM = "/opt/rocm"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, **kw)
    assert r.returncode == 0, " ".join(cmd) + "\n" + r.stdout[-4000:]
    return r.stdout


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", *SAN, "-std=c11", "-ffp-contract=off", os.path.join(ROOT, "oracle", "gear_oracle.c"),
          os.path.join(NATIVE, "oracle_san_driver.c"), "-lm", "-o", exe])
    out = _run([exe])
    assert "oracle sanitizer run: ok" in out


@pytest.mark.skipif(not os.path.exists(os.path.join(ROCM, "bin", "hipcc")), reason="needs ROCm")
def test_host_library_under_asan_ubsan(tmp_path):
    import torch
    objs = [os.path.join(OBJS, f"{n}.hip.o") for n in ("gear_attn", "gear_compress", "gear_decompress")]
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("kernel objects not built (python -m kv_cache_compression_gear_amd.build)")
    api = str(tmp_path / "gear_api_san.o")
    # the API's host pass instrumented (each sanitizer flag applies to the host
    # pass only), the kernel objects as built
    _run([os.path.join(ROCM, "bin", "hipcc"), "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-O1",
          "-g", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
          "-Xarch_host", "-fno-sanitize-recover=all",
          "-c", os.path.join(CSRC, "gear_api.hip"), "-o", api])
    clang = os.path.join(ROCM, "llvm", "bin", "clang")
    drv = str(tmp_path / "drv.o")
    _run([clang, *SAN, "-c", os.path.join(NATIVE, "abi_san_driver.c"), "-o", drv])
    exe = str(tmp_path / "abi_san")
    _run([clang + "++", *SAN, drv, api, *objs, f"-L{ROCM}/lib", "-lamdhip64",
          f"-Wl,-rpath,{ROCM}/lib", "-o", exe])
    args = [] if torch.cuda.is_available() else ["--no-gpu"]
    out = _run([exe, *args])
    assert "host library sanitizer run: ok" in out
