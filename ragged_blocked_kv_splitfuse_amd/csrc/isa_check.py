"""Build-time guard: the device code must contain no scalar-cache writes.

Disassembles the gfx950 device code of the kernels (compiled to assembly with
--cuda-device-only -S) and fails if any scalar memory store, scalar atomic or
scalar data-cache write-back / discard appears.  All device writes must go
through vector memory instructions.
"""
import os
import re
import subprocess
import sys

FORBIDDEN = re.compile(
    r"^\s*(s_store_\w+|s_buffer_store_\w+|s_scratch_store_\w+|s_atomic_\w+|"
    r"s_buffer_atomic_\w+|s_dcache_wb\w*|s_dcache_discard\w*)\b", re.M)


def device_asm(src, hipcc, flags):
    r = subprocess.run([hipcc, *flags, "--cuda-device-only", "-S", src, "-o", "-"],
                       stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
    if r.returncode != 0:
        raise RuntimeError(r.stderr)
    return r.stdout


def check(src, hipcc, flags):
    asm = device_asm(src, hipcc, flags)
    bad = sorted(set(m.group(1) for m in FORBIDDEN.finditer(asm)))
    if bad:
        raise RuntimeError(f"{os.path.basename(src)}: forbidden scalar-cache writes: {bad}")
    return len(asm)


if __name__ == "__main__":
    from ragged_blocked_kv_splitfuse_amd import build as b
    n = check(os.path.join(b.CSRC, "fg_kernels.hip"), b.HIPCC, b.HIP_FLAGS)
    print(f"ok ({n} bytes of device assembly scanned)")
    sys.exit(0)
