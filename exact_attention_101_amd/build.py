"""Build libfa.so in-tree with hipcc for gfx950.

Usage: python -m exact_attention_101_amd.build [--verbose]
"""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfa.so")
# Race-check build of the same sources: every tile copy of the forward
# kernels serialised behind barriers (FA_SERIAL_COPIES, fa_common.h).
SERIAL_LIB = os.path.join(HERE, "libfa_serial.so")
# Issue-rate probes of the SIMD (measurement support, its own library).
PROBE_LIB = os.path.join(HERE, "libfa_probe.so")
PROBE_SOURCES = ["fa_probe_rates.hip"]
SOURCES = ["fa_api.hip", "fa_fwd_bf16.hip", "fa_fwd_fp8.hip", "fa_quant.hip",
           "fa_bwd_bf16.hip", "fa_splitkv_bf16.hip", "fa_varlen_bf16.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Code generation flags shared by the library build and the ISA checks.
CODEGEN = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    # Keep the compiler from forming packed fp32 VALU ops.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMAs the compiler emits write vector registers (the attention scores
    # are read by VALU code); accumulators meant for AGPRs are pinned there
    # explicitly in the kernels.
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
]
FLAGS = [
    *CODEGEN,
    "-fPIC",
    "-shared",
    "-fvisibility=hidden",
    "-Wall",
    "-Wno-unused-command-line-argument",
]
# gfx950 assembly of one source (device code only), for inspection and tests.
FLAGS_DEVICE_ASM = [*CODEGEN, "--cuda-device-only", "-S",
                    "-Wno-unused-command-line-argument"]


def _compile(out: str, sources, extra=(), verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in sources]
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *extra, "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so.
    noise = ("packed-fp32-ops", "is not a recognized feature")
    lines = [ln for ln in (res.stdout + res.stderr).splitlines()
             if ln.strip() and not any(n in ln for n in noise)]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(lines))
    if verbose and lines:
        print("\n".join(lines))
    os.replace(tmp, out)
    return out


ROOT = os.path.dirname(HERE)
# Host-side C-ABI driver under AddressSanitizer and UndefinedBehaviorSanitizer
# (CPU only: every call it makes is rejected before reaching the GPU).  The
# sanitizers instrument the host pass only.
SANITIZE_DRIVER = os.path.join(ROOT, "tests", "cabi_sanitize_driver.cpp")
SANITIZE_BIN = os.path.join(ROOT, "tests", "_build", "cabi_sanitize")
SANITIZE_FLAGS = [
    "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=all",
    "-Xarch_host", "-fno-omit-frame-pointer",
    "-Wno-unused-command-line-argument",
]


def build_sanitized(verbose: bool = False) -> str:
    """Compile the sanitised C-ABI driver with every library source."""
    os.makedirs(os.path.dirname(SANITIZE_BIN), exist_ok=True)
    srcs = [SANITIZE_DRIVER] + [os.path.join(CSRC, s) for s in SOURCES]
    cmd = [HIPCC, *SANITIZE_FLAGS, "-o", SANITIZE_BIN + ".tmp", *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    os.replace(SANITIZE_BIN + ".tmp", SANITIZE_BIN)
    return SANITIZE_BIN


def build(verbose: bool = False) -> str:
    """Compile every HIP source into libfa.so, the race-check build of the
    same sources, the probe library and the sanitised C-ABI driver (always
    rebuilds)."""
    from concurrent.futures import ThreadPoolExecutor
    jobs = [
        lambda: _compile(LIB, SOURCES, verbose=verbose),
        lambda: _compile(SERIAL_LIB, SOURCES, extra=["-DFA_SERIAL_COPIES=1"],
                         verbose=verbose),
        lambda: _compile(PROBE_LIB, PROBE_SOURCES, verbose=verbose),
        lambda: build_sanitized(verbose=verbose),
    ]
    with ThreadPoolExecutor(max_workers=len(jobs)) as pool:
        for f in [pool.submit(j) for j in jobs]:
            f.result()
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
