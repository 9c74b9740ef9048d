"""Build the gfx950 HIP library in-tree: mla_decode_amd/libmla_decode.so.

Run as ``python -m mla_decode_amd.build``.  Compiles every ``csrc/*.hip`` with
hipcc for gfx950 only.  Packed-fp32 instruction selection is disabled, and MFMA
accumulators are kept in VGPRs (the per-tile rescale of the output
accumulator then needs no AGPR copies).

Register spills are a build error: the compiler's per-kernel resource report
(``-Rpass-analysis=kernel-resource-usage``) is parsed and any kernel with
VGPR or SGPR spills or scratch memory fails the build (``SPILL_ALLOWANCE``
could exempt a kernel up to fixed figures; it is empty).
``MLA_ALLOW_SPILLS=1`` turns the failure into a warning.
"""

import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmla_decode.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wno-unused-command-line-argument",
    "-Rpass-analysis=kernel-resource-usage",
]

# Kernels allowed to spill, with the most they may spill: (scratch bytes per
# lane, VGPR spills, SGPR spills).  Empty: every kernel of the library builds
# without spills.
SPILL_ALLOWANCE = {}

_REMARK = re.compile(r"remark:\s+(?P<key>[^:]+?):\s+(?P<val>\S+)\s+\[-Rpass-analysis=kernel-resource-usage\]")

# resource report of the last build(): kernel name -> {field: value}
LAST_USAGE = {}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def parse_resource_usage(text):
    """Kernel name -> {report field: int or str} from hipcc's resource remarks."""
    usage, cur = {}, None
    for line in text.splitlines():
        m = _REMARK.search(line)
        if not m:
            continue
        key, val = m.group("key").strip(), m.group("val")
        if key == "Function Name":
            cur = usage.setdefault(val, {})
            continue
        if cur is not None:
            cur[key] = int(val) if re.fullmatch(r"-?\d+", val) else val
    return usage


def spill_problems(usage, allowance=None):
    """Messages for every kernel that spills more than it may."""
    allowance = SPILL_ALLOWANCE if allowance is None else allowance
    out = []
    for name, u in sorted(usage.items()):
        got = (u.get("ScratchSize [bytes/lane]", 0), u.get("VGPRs Spill", 0), u.get("SGPRs Spill", 0))
        lim = allowance.get(name, (0, 0, 0))
        if any(g > l for g, l in zip(got, lim)):
            out.append(f"{name}: scratch {got[0]} B/lane, {got[1]} VGPR and {got[2]} SGPR spills "
                       f"(allowed {lim[0]}, {lim[1]}, {lim[2]})")
    return out


def build(verbose=False, out=LIB):
    """Compile the library to ``out`` (default: in-tree) and return its path; raises on a compile error or on
    spills beyond the allowance."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = out + ".tmp"
    cmd = [hipcc] + HIPCC_FLAGS + sources() + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    lines = [l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed (%d):\n%s" % (r.returncode, "\n".join(l for l in lines if "remark:" not in l)))
    usage = parse_resource_usage(r.stdout)
    if not usage:
        raise RuntimeError("hipcc printed no kernel resource report")
    LAST_USAGE.clear()
    LAST_USAGE.update(usage)
    problems = spill_problems(usage)
    if problems:
        msg = "register spills beyond the allowance:\n  " + "\n  ".join(problems)
        if os.environ.get("MLA_ALLOW_SPILLS") != "1":
            os.remove(tmp)
            raise RuntimeError(msg + "\n(set MLA_ALLOW_SPILLS=1 to build anyway)")
        print("warning: " + msg, file=sys.stderr, flush=True)
    if verbose:
        for name, u in sorted(usage.items()):
            print(f"{name}: VGPRs {u.get('VGPRs')} AGPRs {u.get('AGPRs')} scratch {u.get('ScratchSize [bytes/lane]')}"
                  f" LDS {u.get('LDS Size [bytes/block]')}", flush=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
