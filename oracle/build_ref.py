"""Build oracle/libkvs_ref.so, the plain C fp64 cross-check of the window score
(TEST INFRASTRUCTURE ONLY), with gcc."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "score_ref.c")
LIB = os.path.join(HERE, "libkvs_ref.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-o", LIB, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return LIB


def load():
    """The library (built first when missing or older than its source)."""
    import ctypes
    if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        build()
    lib = ctypes.CDLL(LIB)
    P = ctypes.c_void_p
    lib.kvs_ref_score.restype = ctypes.c_int
    lib.kvs_ref_score.argtypes = [P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_int, ctypes.c_longlong, ctypes.c_int, ctypes.c_double, P]
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
