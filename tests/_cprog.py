"""Build commands of the C test programs (tests/abi_c_check.c,
tests/abi_c_decode.c).  build() in __graft_entry__ compiles them into
tests/_bin/ beside the library build; the tests take those binaries and
compile their own copy only when none is there or it is older than its
source or the library."""

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
BIN = os.path.join(HERE, "_bin")
LIB_DIR = os.path.join(ROOT, "mla_latent_kv_lat_amd")
ROCM = "/opt/rocm"

_FLAGS = {
    # the header alone, as pedantic C99, host-only calls
    "abi_c_check": ["-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror"],
    # a whole decode step: HIP's runtime header (C11, taken as a system header)
    "abi_c_decode": ["-std=c11", "-Wall", "-Wextra", "-pedantic", "-Werror", "-D__HIP_PLATFORM_AMD__",
                     "-isystem", os.path.join(ROCM, "include")],
}
_LIBS = {
    "abi_c_check": ["-L", LIB_DIR, "-lmla", f"-Wl,-rpath,{LIB_DIR}"],
    "abi_c_decode": ["-L", LIB_DIR, "-lmla", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
                     f"-Wl,-rpath,{LIB_DIR}", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"],
}


def compile_program(name: str, out_dir: str) -> str:
    os.makedirs(out_dir, exist_ok=True)
    exe = os.path.join(out_dir, name)
    subprocess.run(["gcc", *_FLAGS[name], "-I", os.path.join(ROOT, "include"),
                    os.path.join(HERE, name + ".c"), *_LIBS[name], "-o", exe], check=True)
    return exe


def build_all() -> None:
    for name in _FLAGS:
        compile_program(name, BIN)


def program(name: str, tmp_dir: str) -> str:
    """The prebuilt binary if it is current, else one compiled into tmp_dir
    (None when there is no C compiler)."""
    exe = os.path.join(BIN, name)
    deps = [os.path.join(HERE, name + ".c"), os.path.join(ROOT, "include", "mla.h"),
            os.path.join(LIB_DIR, "libmla.so")]
    if os.path.exists(exe) and all(os.path.getmtime(exe) >= os.path.getmtime(p) for p in deps
                                   if os.path.exists(p)):
        return exe
    if shutil.which("gcc") is None:
        return None
    return compile_program(name, tmp_dir)
