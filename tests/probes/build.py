"""Build the test-only probes in-tree: the HIP probe libraries (hipcc, gfx950)
and the plain-C caller of libbeaconkv.so (gcc, host code only; it finds the
in-tree library and the ROCm runtime through its run path)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PROBES = ("mfma_rounding",)
ROCM = "/opt/rocm"


def build_c_driver() -> str:
    src = os.path.join(HERE, "c_abi_driver.c")
    out = os.path.join(HERE, "c_abi_driver")
    tmp = out + ".tmp"
    subprocess.run(["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
                    "-I", f"{ROCM}/include", "-I", os.path.join(ROOT, "include"), src,
                    "-L", os.path.join(ROOT, "decode_kv_cache_beacon_amd"), "-lbeaconkv",
                    "-L", f"{ROCM}/lib", "-lamdhip64",
                    "-Wl,-rpath,$ORIGIN/../../decode_kv_cache_beacon_amd",
                    f"-Wl,-rpath,{ROCM}/lib", "-o", tmp], check=True, capture_output=True)
    os.replace(tmp, out)
    return out


def build() -> None:
    for name in PROBES:
        src = os.path.join(HERE, name + ".hip")
        out = os.path.join(HERE, "lib" + name + ".so")
        tmp = out + ".tmp"
        subprocess.run(["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O3", "-fPIC", "-shared",
                        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", src, "-o",
                        tmp], check=True, capture_output=True)
        os.replace(tmp, out)
    build_c_driver()


if __name__ == "__main__":
    build()
