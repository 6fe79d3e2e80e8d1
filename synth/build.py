"""Build the generator libraries: the HIP fill kernel (libcsa2_synth.so,
hipcc for gfx950) and the host generator (libcsa2_synth_host.so, gcc)."""
import os
import subprocess

from . import build_host

HERE = os.path.dirname(os.path.abspath(__file__))


def build() -> None:
    out = os.path.join(HERE, "libcsa2_synth.so")
    tmp = out + f".tmp{os.getpid()}"
    subprocess.check_call([os.environ.get("HIPCC", "/opt/rocm/bin/hipcc"), "-x", "hip", "-O3", "-fPIC", "-shared",
                           "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                           "-o", tmp, os.path.join(HERE, "fill.hip")],
                          stderr=subprocess.DEVNULL)
    os.replace(tmp, out)
    build_host(force=True)


if __name__ == "__main__":
    build()
