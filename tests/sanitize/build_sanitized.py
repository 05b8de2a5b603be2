"""Host builds with AddressSanitizer and UndefinedBehaviorSanitizer for the
CPU test suite: the oracle (plain C) and the runtime's host code (C++, with
the kernel launcher stubbed out).  GCC only; no GPU code is built here."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SAN = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-g", "-O1"]


def runtime_libraries():
    """Paths of the sanitizer runtimes to preload into an uninstrumented
    interpreter."""
    out = []
    for name in ("libasan.so", "libubsan.so"):
        out.append(subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                                  text=True, check=True).stdout.strip())
    return out


def build_oracle(out_dir):
    out = os.path.join(out_dir, "liboracle_adam_san.so")
    subprocess.run(["gcc", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", *SAN,
                    os.path.join(ROOT, "oracle", "adam_oracle.c"), "-lm", "-o", out], check=True)
    return out


def build_host_runtime(out_dir):
    out = os.path.join(out_dir, "libadam_host_san.so")
    csrc = os.path.join(ROOT, "memory_efficient_adam_amd", "csrc")
    subprocess.run(["g++", "-std=c++17", "-fPIC", "-shared", "-D__HIP_PLATFORM_AMD__", *SAN,
                    "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
                    "-I", csrc, os.path.join(csrc, "adam_runtime.cpp"),
                    os.path.join(HERE, "launch_stub.cpp"), "-L", os.path.join(ROCM, "lib"),
                    "-lamdhip64", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", out], check=True)
    return out


def env_with_sanitizers():
    env = dict(os.environ)
    env["LD_PRELOAD"] = " ".join(runtime_libraries())
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    return env
