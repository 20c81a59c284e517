"""Host-only AddressSanitizer + UndefinedBehaviorSanitizer build of libfattn's C ABI.

    python tests/sanitize/build_sanitized.py OUT_DIR     # prints the library path

api.cpp (argument checks, planning, workspaces, the exported calls) is compiled with g++ as plain
host C++ and linked with launch_stubs.cpp in place of the HIP kernels, with hidden visibility
like the real library. Nothing here runs on a GPU: the ABI tests loaded against this library
exercise only the paths that return before any kernel launch.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
CSRC = os.path.join(ROOT, "io_aware_tiled_amd", "csrc")


def build(out_dir: str) -> str:
    os.makedirs(out_dir, exist_ok=True)
    lib = os.path.join(out_dir, "libfattn_sanitized.so")
    # __HIP_PLATFORM_AMD__ only names the platform for the HIP runtime headers, which a plain host
    # compiler includes here without hipcc's driver defining it
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fvisibility=hidden",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-I", "/opt/rocm/include", os.path.join(CSRC, "api.cpp"),
           os.path.join(HERE, "launch_stubs.cpp"), "-L/opt/rocm/lib", "-lamdhip64",
           "-Wl,-rpath,/opt/rocm/lib", "-o", lib]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return lib


if __name__ == "__main__":
    print(build(sys.argv[1]))
