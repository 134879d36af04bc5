"""Host sanitizer builds, on the CPU: the fp64 oracle (C) built with gcc's
AddressSanitizer and UndefinedBehaviorSanitizer runs its pins, and the C ABI's
host code (dp_api.hip: validation, planning, the pipeline handle's host side)
built with clang's host ASan/UBSan runs the CPU API tests.  Only host code is
instrumented (each -fsanitize= follows -Xarch_host); the GPU code objects are
the product build's.  A sanitizer report fails the run."""
import glob
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "linear_rnn_sequence_amd", "csrc")
RUNNER = os.path.join(HERE, "sanitize_runner.py")
ASAN_OPTS = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
UBSAN_OPTS = "halt_on_error=1:print_stacktrace=1"


def run(which, lib, preload, files):
    env = dict(os.environ, LD_PRELOAD=preload, ASAN_OPTIONS=ASAN_OPTS, UBSAN_OPTIONS=UBSAN_OPTS)
    r = subprocess.run([sys.executable, RUNNER, which, lib, *files], capture_output=True, text=True,
                       timeout=600, env=env, cwd=ROOT)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]


def test_oracle_under_asan_and_ubsan(tmp_path):
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-fno-omit-frame-pointer", os.path.join(ROOT, "oracle", "dp_oracle.c"), "-o", lib, "-lm"],
                   check=True)
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                          check=True).stdout.strip()
    run("oracle", lib, asan, [os.path.join(HERE, "test_oracle_pins.py"),
                              os.path.join(HERE, "test_oracle_bwd_pins.py")])


def test_c_abi_host_code_under_asan_and_ubsan(tmp_path):
    from linear_rnn_sequence_amd import build as b

    objs = sorted(glob.glob(os.path.join(b.OBJDIR, "*.o")))
    if not any(o.endswith("dp_inst_bf16_128.hip.o") or "dp_inst_bf16_128" in o for o in objs):
        b.build()
        objs = sorted(glob.glob(os.path.join(b.OBJDIR, "*.o")))
    objs = [o for o in objs if "dp_api" not in os.path.basename(o)]
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    api = str(tmp_path / "dp_api_san.o")
    subprocess.run([b.HIPCC, *b.CFLAGS, "-O1", "-g", *san, "-c", os.path.join(CSRC, "dp_api.hip"), "-o", api],
                   check=True, capture_output=True)
    lib = str(tmp_path / "libdp_san.so")
    subprocess.run([b.HIPCC, f"--offload-arch={b.ARCH}", "-shared", "-fPIC", api, *objs, "-o", lib,
                    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                    "-Xarch_host", "-shared-libasan"], check=True, capture_output=True)
    clang_rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not clang_rt:
        pytest.skip("clang's ASan runtime is not installed")
    run("abi", lib, clang_rt[-1], [os.path.join(HERE, "test_api_cpu.py")])
