"""Build the CPU oracle (test infrastructure only) into oracle/liboracle.so.

Plain gcc, no fused multiply-add, no fast-math: the encoder's fp32 steps are
the definition the GPU encoder is checked against bit for bit.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False, out: str = LIB, sanitize: bool = False) -> str:
    """sanitize: an AddressSanitizer + UndefinedBehaviorSanitizer build (for the
    sanitizer test; the process that loads it needs the two runtimes preloaded)."""
    src = os.path.join(HERE, "kvq_oracle.c")
    tmp = out + ".tmp"
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer", "-g"] if sanitize else []
    cmd = ["gcc", "-std=c11", "-D_GNU_SOURCE", "-O2" if not sanitize else "-O1", "-fPIC", "-shared",
           "-ffp-contract=off", "-fno-fast-math", "-fno-strict-aliasing", "-pthread",
           "-Wall", "-Wextra", "-Wno-unused-parameter", *san,
           src, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
