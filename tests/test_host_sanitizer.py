"""The C ABI layer (csrc/capi.cpp) built with host sanitizers and run on the
CPU against recording stand-ins for its kernel launchers
(tests/host_sanitize/): AddressSanitizer + UndefinedBehaviorSanitizer in one
build, ThreadSanitizer in another. The checks cover the kernel each entry
point dispatches to, the parameters its launcher receives (group size, RoPE
frequencies, the log2-scaled softmax scale, split counts and the split-KV
workspace layout), every argument error with its status and message, and the
per-thread error text under concurrent calls. Device code is compiled but
never run; the sanitizers instrument host code only (-Xarch_host).
"""

import os
import shutil
import subprocess
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
CSRC = ROOT / "attention_ragged_gqa_amd" / "csrc"
HERE = ROOT / "tests" / "host_sanitize"
CLANG = "/opt/rocm/llvm/bin/clang++"
ROCM_LIB = "/opt/rocm/lib"
SOURCES = (CSRC / "capi.cpp", HERE / "launch_stubs.cpp", HERE / "host_checks.cpp")
BUILDS = {"asan_ubsan": ("address", "undefined"), "tsan": ("thread",)}
RUN_ENV = {
    # the HIP runtime keeps process-lifetime allocations: leaks are not the point
    "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1",
    "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    "TSAN_OPTIONS": "halt_on_error=1",
}


def _build(out_dir: Path, name: str, sanitizers) -> Path:
    flags = ["-x", "hip", "--offload-arch=gfx950", "-std=c++17", "-O1", "-g"]
    for s in sanitizers:
        flags += ["-Xarch_host", "-fsanitize=" + s]
    flags += ["-Xarch_host", "-fno-omit-frame-pointer"]
    if "undefined" in sanitizers:
        flags += ["-Xarch_host", "-fno-sanitize-recover=undefined"]
    objs = []
    for src in SOURCES:
        obj = out_dir / ("%s_%s.o" % (name, src.stem))
        cmd = [CLANG, *flags, "-I", str(CSRC), "-I", str(ROOT / "include"), "-I", str(HERE), "-c", str(src),
               "-o", str(obj)]
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
        assert r.returncode == 0, "compile %s failed:\n%s" % (src.name, r.stderr[-4000:])
        objs.append(str(obj))
    exe = out_dir / name
    link = [CLANG, "-fsanitize=" + ",".join(sanitizers), *objs, "-L" + ROCM_LIB, "-lamdhip64",
            "-Wl,-rpath," + ROCM_LIB, "-o", str(exe)]
    r = subprocess.run(link, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, "link failed:\n%s" % r.stderr[-4000:]
    return exe


@pytest.fixture(scope="module")
def build_dir(tmp_path_factory):
    if not os.path.exists(CLANG) or not os.path.exists(os.path.join(ROCM_LIB, "libamdhip64.so")):
        pytest.skip("ROCm clang or the HIP runtime is not installed")
    return tmp_path_factory.mktemp("host_sanitize")


@pytest.mark.parametrize("name", sorted(BUILDS))
def test_capi_under_host_sanitizers(build_dir, name):
    exe = _build(build_dir, name, BUILDS[name])
    env = dict(os.environ, **RUN_ENV)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    report = (r.stdout + r.stderr)[-6000:]
    assert r.returncode == 0, "%s build: checks failed or a sanitizer reported\n%s" % (name, report)
    assert "0 failed" in r.stdout and "Sanitizer" not in r.stderr, report
