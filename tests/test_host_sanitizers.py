"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

Every source of the library is compiled for the host only (no device pass, no GPU needed) with
both sanitizers, and linked with a stand-in for the HIP runtime's launch interface
(host_check/hip_runtime_stub.cpp) and a mutation fuzz of the C entry points
(host_check/abi_fuzz.cpp). The fuzz runs the real validation and the real launch set-up; the
stand-in checks each launch against HIP's limits and records it instead of running it.
"""

import concurrent.futures as cf
import glob
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_chunk_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "host_check")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANGXX = os.path.join(ROCM, "llvm", "bin", "clang++")

# host-side sanitizer flags (each one host-only, and no device pass is compiled anyway)
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined"]


def _compile(src, obj):
    cmd = [HIPCC, "-x", "hip", "--offload-host-only", f"--offload-arch=gfx950", "-O1", "-g",
           "-std=c++17", "-fno-omit-frame-pointer", *SAN, "-Wno-unused-command-line-argument",
           f"-I{ROOT}/include", f"-I{CSRC}", f"-I{HERE}", "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, f"compiling {src}:\n{res.stderr[-4000:]}"
    return obj


@pytest.fixture(scope="module")
def fuzz_binary(tmp_path_factory):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)):
        pytest.skip("hipcc / clang++ not found")
    out = tmp_path_factory.mktemp("host_check")
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [
        os.path.join(HERE, "hip_runtime_stub.cpp"), os.path.join(HERE, "abi_fuzz.cpp")]
    with cf.ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(lambda s: _compile(s, str(out / (os.path.basename(s) + ".o"))), srcs))
    # the host-only objects still name the (absent) device images of their modules: give the
    # stand-in registration something to point at
    nm = shutil.which("nm") or os.path.join(ROCM, "llvm", "bin", "llvm-nm")
    names = set()
    for o in objs:
        res = subprocess.run([nm, "-u", o], capture_output=True, text=True, check=True)
        names.update(re.findall(r"\b(__hip_fatbin\w*)", res.stdout))
    images = out / "device_images.c"
    images.write_text("".join(f"char {n}[16];\n" for n in sorted(names)))
    img_obj = str(out / "device_images.o")
    subprocess.run([CLANGXX, "-x", "c", "-c", str(images), "-o", img_obj], check=True)
    exe = str(out / "abi_fuzz")
    res = subprocess.run([CLANGXX, "-fsanitize=address,undefined", *objs, img_obj, "-o", exe],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    return exe


def _run(exe, *args):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    return subprocess.run([exe, *map(str, args)], capture_output=True, text=True, env=env,
                          timeout=600)


@pytest.mark.parametrize("seed", [1, 2])
def test_entry_points_under_sanitizers(fuzz_binary, seed):
    res = _run(fuzz_binary, 20000, seed)
    assert res.returncode == 0, (res.stdout[-3000:] + "\n" + res.stderr[-6000:])
    assert res.stdout.strip().endswith("OK"), res.stdout
    # every entry point accepted some mutated calls, so the launch set-up ran under the sanitizers
    assert len(re.findall(r"accepted \d+ of", res.stdout)) == 10, res.stdout
