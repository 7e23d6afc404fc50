"""Build and run the hardware probes (tests/hw/hw_probes.hip) on the GPU.

    python tests/hw/run_hw_probes.py

Prints one line per probe: the clocks a wave spends issuing vector-memory
loads (direct to LDS and into registers), the rate of three MFMA shapes, the
back-to-back launch interval and LDS read bandwidth per CU. The figures back
the design notes of the kernels; the build goes to _build/ at the repository
root.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build():
    out_dir = os.path.join(ROOT, "_build")
    os.makedirs(out_dir, exist_ok=True)
    exe = os.path.join(out_dir, "hw_probes")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", os.path.join(HERE, "hw_probes.hip"), "-o", exe]
    subprocess.run(cmd, check=True)
    return exe


if __name__ == "__main__":
    exe = build() if "--no-build" not in sys.argv else os.path.join(ROOT, "_build", "hw_probes")
    sys.exit(subprocess.run([exe]).returncode)
