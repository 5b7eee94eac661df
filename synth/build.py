"""Build libsynth.so, the seeded input generator (gcc, OpenMP)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def build() -> str:
    out = os.path.join(HERE, "libsynth.so")
    obj = os.path.join(HERE, "synth.o")
    # x86-64-v3 (AVX2/FMA) and fast-math at compile time let glibc's vector math
    # library serve the Box-Muller loops; values depend only on this binary, which
    # both sides of a comparison share. The link step has no fast-math flag: with
    # it gcc adds a start-up routine that switches the loading process to
    # flush-to-zero / denormals-are-zero, which would change every later FP32
    # computation in the process (the oracle's included).
    subprocess.run(["gcc", "-O3", "-ffast-math", "-march=x86-64-v3", "-fopenmp", "-fPIC", "-Wall", "-c",
                    os.path.join(HERE, "synth.c"), "-o", obj], check=True)
    subprocess.run(["gcc", "-shared", "-fopenmp", obj, "-o", out, "-lmvec", "-lm"], check=True)
    os.remove(obj)
    return out


if __name__ == "__main__":
    print(build())
