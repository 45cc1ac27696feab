"""Build step for the fp64 CPU oracle (test infrastructure only).

Compiles ``ssm_oracle.c`` with the host C compiler into ``liboracle.so`` next
to it: plain ``-O2``, OpenMP for the loop over independent channels, and no
fast-math, so every ``exp`` is the C library's correctly behaved double one.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "ssm_oracle.c")
LIBRARY = os.path.join(HERE, "liboracle.so")


def compile_oracle(source=SOURCE, output=LIBRARY, cc="gcc"):
    """Compile ``source`` into the shared library ``output`` and return its path."""
    cmd = [cc, "-O2", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
           "-std=c11", "-Wall", "-Werror", source, "-o", output + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(output + ".tmp", output)
    return output


if __name__ == "__main__":
    print(compile_oracle())
