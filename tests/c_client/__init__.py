"""A plain C client of libtilepipe (tp_c_client.c): TEST CODE.

build() compiles it with gcc into a shared object linked against
libtilepipe.so, liboracle.so and the HIP runtime, using only
include/tilepipe.h; run(mode) calls its entry point in this process.
"""
import ctypes
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "tp_c_client.c")
LIB = os.path.join(HERE, "libtp_c_client.so")
PKG = os.path.join(ROOT, "software_pipelining_amd")
ORACLE = os.path.join(ROOT, "oracle")
ROCM = "/opt/rocm"


def build() -> str:
    """Compile the client; libtilepipe.so and liboracle.so must be built."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-fPIC", "-shared",
           "-D__HIP_PLATFORM_AMD__", f"-I{ROOT}/include", f"-I{ROCM}/include", SRC, "-o", tmp,
           f"-L{PKG}", "-ltilepipe", f"-L{ORACLE}", "-loracle", f"-L{ROCM}/lib", "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../software_pipelining_amd:$ORIGIN/../../oracle:"
           f"{ROCM}/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError("C client build failed:\n" + r.stderr[-4000:])
    os.replace(tmp, LIB)
    return LIB


def run(mode: str):
    """(status, message) of tp_c_client_run(mode): 0 and "" when every case passed."""
    if not os.path.exists(LIB):
        raise RuntimeError(f"{LIB} is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(LIB)
    lib.tp_c_client_run.argtypes = [ctypes.c_char_p, ctypes.c_char_p, ctypes.c_int]
    lib.tp_c_client_run.restype = ctypes.c_int
    msg = ctypes.create_string_buffer(1024)
    st = lib.tp_c_client_run(mode.encode(), msg, len(msg))
    return st, msg.value.decode()
