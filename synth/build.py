"""Build libsynth.so, the seeded input generator (gcc, OpenMP)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def build() -> str:
    out = os.path.join(HERE, "libsynth.so")
    # x86-64-v3 (AVX2/FMA) lets glibc's vector math library serve the Box-Muller
    # loops; values depend only on this binary, which both sides of a comparison share.
    cmd = ["gcc", "-O3", "-ffast-math", "-march=x86-64-v3", "-fopenmp", "-fPIC", "-shared",
           "-Wall", os.path.join(HERE, "synth.c"), "-o", out, "-lmvec", "-lm"]
    subprocess.run(cmd, check=True)
    return out


if __name__ == "__main__":
    print(build())
