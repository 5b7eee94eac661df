"""Build liboracle.so (plain C, gcc). The oracle is test infrastructure."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))


def build(out: str | None = None, defines=()) -> str:
    """Compile lmoe_oracle.c into a shared library. No fast-math: the oracle's
    rounding (ties to even) and exponent extraction must follow IEEE semantics."""
    out = out or os.path.join(HERE, "liboracle.so")
    cmd = ["gcc", "-O2", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           *[f"-D{d}" for d in defines], os.path.join(HERE, "lmoe_oracle.c"), "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


if __name__ == "__main__":
    print(build(*sys.argv[1:2]))
