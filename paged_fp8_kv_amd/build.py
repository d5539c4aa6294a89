"""Build libpkv.so (the C-ABI library with the gfx950 kernels) and
libpkv_probe.so (the HBM read-bandwidth probes) in place.

    python -m paged_fp8_kv_amd.build [--verbose]

Every HIP source is compiled for gfx950 only, with packed-fp32 instructions
disabled (``-packed-fp32-ops``; the host pass warns that it does not know
that feature, which is harmless) and MFMA accumulators kept in ordinary
VGPRs (``-amdgpu-mfma-vgpr-form``).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpkv.so")
SOURCES = ["abi.cpp", "control.hip", "decode_attn.hip"]
PROBE_LIB = os.path.join(HERE, "libpkv_probe.so")
PROBE_SOURCES = ["hbm_probe.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs: with AGPR accumulators the
    # compiler copied the 16 output accumulators between AGPR sets around the
    # online-softmax rescale branch in every sub-tile (about 36 of ~250
    # instructions); measured 1 us faster per full layer at batch 64 x 8192
    # and 1.9 us at the 256-sequence short-context batch, identical outputs
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function",
]


def build(verbose: bool = False, extra=()) -> str:
    _build_one(PROBE_LIB, PROBE_SOURCES, verbose, ())
    return _build_one(LIB, SOURCES, verbose, extra)


def _build_one(lib, sources, verbose, extra) -> str:
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, *extra, "-o", tmp] + [os.path.join(CSRC, s) for s in sources]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError("hipcc failed:\n" + msg)
    if verbose and msg.strip():
        print(msg)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
