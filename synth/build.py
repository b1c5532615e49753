"""Build the seeded input generator libraries (host: gcc, device: hipcc for gfx950)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
HOST_SO = os.path.join(HERE, "libsynth_host.so")
DEVICE_SO = os.path.join(HERE, "libsynth_device.so")

HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def build_host():
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-ffp-contract=off", "-pthread",
           os.path.join(HERE, "synth_host.c"), "-o", HOST_SO + ".tmp"]
    subprocess.run(cmd, check=True)
    os.replace(HOST_SO + ".tmp", HOST_SO)


def build_device():
    cmd = ["hipcc", *HIP_FLAGS, os.path.join(HERE, "synth_device.hip"), "-o", DEVICE_SO + ".tmp"]
    subprocess.run(cmd, check=True)
    os.replace(DEVICE_SO + ".tmp", DEVICE_SO)


def build():
    build_host()
    build_device()


if __name__ == "__main__":
    build()
