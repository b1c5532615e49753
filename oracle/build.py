"""Build the CPU oracle shared library (g++; test infrastructure only)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SO = os.path.join(HERE, "liboracle.so")


def build():
    cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
           os.path.join(HERE, "qwen3_oracle.cpp"), "-o", SO + ".tmp"]
    subprocess.run(cmd, check=True)
    os.replace(SO + ".tmp", SO)


if __name__ == "__main__":
    build()
