"""Host-sanitizer builds (AddressSanitizer + UndefinedBehaviorSanitizer) of the
CPU code: the oracle, and libvelox's host code (argument checks and entry
points) linked with launch stubs.  Host compilers only (gcc, g++); nothing
here builds GPU code."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
CSRC = os.path.join(ROOT, "geometry_routed_block_velox_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def build(out_dir: str) -> dict:
    """Build both libraries into out_dir; returns their paths and the ASan runtime to preload."""
    os.makedirs(out_dir, exist_ok=True)
    velox = os.path.join(out_dir, "libvelox_host_san.so")
    oracle = os.path.join(out_dir, "libvelox_oracle_san.so")
    subprocess.run(["g++", "-std=c++17", "-fPIC", "-shared", "-Wall", "-Wextra", *SAN, "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", os.path.join(ROCM, "include"),
                    os.path.join(CSRC, "velox_check.cpp"), os.path.join(CSRC, "velox_api.cpp"),
                    os.path.join(HERE, "launch_stubs.cpp"), "-o", velox], check=True)
    # the oracle's own flags, plus the sanitizers
    subprocess.run(["gcc", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-Wall",
                    "-Wextra", *SAN, os.path.join(ROOT, "oracle", "velox_oracle.c"), "-lm", "-o", oracle],
                   check=True)
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], check=True, capture_output=True,
                          text=True).stdout.strip()
    return {"velox": velox, "oracle": oracle, "asan": asan}
