"""AddressSanitizer + UndefinedBehaviorSanitizer run of the host code, on the CPU only.

Test infrastructure.  Two builds, each checked by the CPU tests that exercise it:

1. the fp64 oracle (oracle/fwa_oracle.c) with gcc and the sanitizers, run through the oracle
   pins (tests/test_oracle_pins.py) with gcc's ASan runtime preloaded into Python;
2. the library with the sanitizers on the host pass only (argument and size validation,
   implementation choice, workspace layout, the C ABI; the device code is built as usual and
   carries no instrumentation), run through tests/test_abi_cpu.py with clang's ASan runtime
   preloaded.  No kernel is launched: those tests only call entry points that must reject their
   arguments before any launch, and the info queries.

Usage: python tests/sanitize_host.py [--out DIR].  Exit status 0 when both runs pass with no
sanitizer report (every report aborts the process: halt_on_error, no recovery from UB).
"""
import argparse
import concurrent.futures as cf
import glob
import os
import subprocess
import sys
import tempfile

TESTS = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(TESTS)
CSRC = os.path.join(ROOT, "weight_linear_attention_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"

HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer"]
ENV_SAN = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def clang_asan_runtime():
    """clang's shared ASan runtime (it carries the UBSan handlers too)."""
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
                  + glob.glob("/opt/rocm/llvm/lib/clang/*/lib/x86_64-unknown-linux-gnu/"
                              "libclang_rt.asan.so"))
    if not hits:
        raise FileNotFoundError("clang's libclang_rt.asan shared runtime not found under /opt/rocm/llvm")
    return hits[-1]


def gcc_asan_runtime():
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True, check=True).stdout.strip()
    if not os.path.isabs(path):
        raise FileNotFoundError("gcc's libasan.so not found")
    return path


def build_oracle(out_dir):
    sys.path.insert(0, ROOT)
    from oracle import build as obuild
    out = os.path.join(out_dir, "liboracle_fwa_san.so")
    return obuild.build(obuild.SRC, out, extra_flags=(
        "-g", "-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
        "-fno-omit-frame-pointer"))


def _compile(src, out_dir):
    obj = os.path.join(out_dir, os.path.basename(src) + ".san.o")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *HOST_SAN,
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"host compile failed for {src}:\n{r.stdout}{r.stderr}")
    return obj


def build_library(out_dir):
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, out_dir), srcs))
    out = os.path.join(out_dir, "libfwa_host_san.so")
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *HOST_SAN, "-shared-libsan",
           "-o", out, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    return out


# Each run is a fresh Python process: the runtime must be preloaded before anything else loads.
_RUN_PINS = """
import sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import oracle
oracle._DEFAULT = oracle.Oracle({lib!r})
import pytest
sys.exit(pytest.main(["-q", "-s", "-p", "no:cacheprovider", {tests!r} + "/test_oracle_pins.py"]))
"""
_RUN_ABI = """
import sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
from weight_linear_attention_amd import fwa
fwa.LIB_PATH = {lib!r}
import pytest
sys.exit(pytest.main(["-q", "-s", "-p", "no:cacheprovider", {tests!r} + "/test_abi_cpu.py"]))
"""


def run(script, lib, preload):
    env = dict(os.environ, **ENV_SAN, LD_PRELOAD=preload, HIP_VISIBLE_DEVICES="")
    code = script.format(root=ROOT, tests=TESTS, lib=lib)
    return subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env,
                          capture_output=True, text=True)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--out", default=None, help="build directory (default: a temporary one)")
    args = ap.parse_args(argv)
    out_dir = args.out or tempfile.mkdtemp(prefix="fwa_san_")
    os.makedirs(out_dir, exist_ok=True)
    status = 0
    for name, builder, script, preload in (
            ("oracle pins", build_oracle, _RUN_PINS, gcc_asan_runtime()),
            ("C ABI host checks", build_library, _RUN_ABI, clang_asan_runtime())):
        lib = builder(out_dir)
        r = run(script, lib, preload)
        tail = "\n".join((r.stdout + r.stderr).strip().splitlines()[-15:])
        print(f"[{name}] {lib}: exit {r.returncode}\n{tail}\n", flush=True)
        status = status or r.returncode
    return status


if __name__ == "__main__":
    sys.exit(main())
