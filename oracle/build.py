"""Build the CPU oracle (test infrastructure): gcc -> oracle/libmoe_oracle.so."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libmoe_oracle.so")


def build():
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-Wall",
           "-o", LIB + ".tmp", "moe_oracle.c", "-lm"]
    r = subprocess.run(cmd, cwd=HERE, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("oracle build failed:\n%s\n%s" % (r.stdout, r.stderr))
    os.replace(LIB + ".tmp", LIB)


if __name__ == "__main__":
    build()
