"""Build the test-only probe libraries in-tree (hipcc, gfx950)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
PROBES = ("mfma_rounding",)


def build() -> None:
    for name in PROBES:
        src = os.path.join(HERE, name + ".hip")
        out = os.path.join(HERE, "lib" + name + ".so")
        tmp = out + ".tmp"
        subprocess.run(["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O3", "-fPIC", "-shared",
                        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", src, "-o",
                        tmp], check=True, capture_output=True)
        os.replace(tmp, out)


if __name__ == "__main__":
    build()
