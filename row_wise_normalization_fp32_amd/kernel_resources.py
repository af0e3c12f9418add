"""Per-kernel resource usage of the built librownorm.so, read from the metadata of its gfx950
code objects: VGPRs, SGPRs, register spills, LDS and scratch (private segment) bytes.

The library's HIP fat binary (ELF section .hip_fatbin) holds one offload bundle per HIP
translation unit. Each bundle starts with the bundler's magic string, then the number of
entries and, per entry, its offset (from the bundle start), size, and target-triple
length and text. The gfx950 entry is an AMDGPU ELF code object whose metadata note
(printed by llvm-readelf --notes) lists every kernel with its resource counts.

    python -m row_wise_normalization_fp32_amd.kernel_resources           # summary
    python -m row_wise_normalization_fp32_amd.kernel_resources --all     # every kernel
"""

from __future__ import annotations

import os
import re
import struct
import subprocess
import sys
import tempfile
from typing import Dict, List

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(_PKG, "librownorm.so")
LLVM_BIN = os.environ.get("ROCM_LLVM_BIN", "/opt/rocm/llvm/bin")
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
TARGET = "amdgcn-amd-amdhsa--gfx950"
FIELDS = (".vgpr_count", ".agpr_count", ".sgpr_count", ".vgpr_spill_count", ".sgpr_spill_count",
          ".group_segment_fixed_size", ".private_segment_fixed_size", ".max_flat_workgroup_size")


def _tool(name: str) -> str:
    return os.path.join(LLVM_BIN, name)


def code_objects(lib: str = LIB) -> List[bytes]:
    """The gfx950 code objects of every offload bundle in the library's fat binary."""
    with tempfile.TemporaryDirectory() as d:
        fb = os.path.join(d, "fatbin")
        subprocess.run([_tool("llvm-objcopy"), "--dump-section", f".hip_fatbin={fb}", lib, os.path.join(d, "x")],
                       check=True, capture_output=True)
        data = open(fb, "rb").read()
    out = []
    start = data.find(MAGIC)
    while start >= 0:
        pos = start + len(MAGIC)
        (n,) = struct.unpack_from("<Q", data, pos)
        pos += 8
        for _ in range(n):
            off, size, tlen = struct.unpack_from("<QQQ", data, pos)
            pos += 24
            triple = data[pos:pos + tlen].decode()
            pos += tlen
            if triple.endswith(TARGET):
                out.append(data[start + off:start + off + size])
        start = data.find(MAGIC, pos)
    return out


def kernels(lib: str = LIB) -> List[Dict[str, object]]:
    """One record per kernel: its name and the FIELDS counts from the code-object metadata."""
    recs: List[Dict[str, object]] = []
    with tempfile.TemporaryDirectory() as d:
        for i, co in enumerate(code_objects(lib)):
            path = os.path.join(d, f"co{i}.o")
            with open(path, "wb") as f:
                f.write(co)
            notes = subprocess.run([_tool("llvm-readelf"), "--notes", path], check=True, capture_output=True,
                                   text=True).stdout
            cur = None
            for line in notes.splitlines():
                if line.startswith("  - "):  # a new kernel map in amdhsa.kernels
                    cur = {}
                    recs.append(cur)
                    line = "    " + line[4:]
                if cur is None:
                    continue
                m = re.match(r"^    (\.[a-z_]+):\s+(\S+)$", line)  # the kernel's own scalar keys
                if m and m.group(1) == ".name":
                    cur["name"] = m.group(2)
                elif m and m.group(1) in FIELDS:
                    cur[m.group(1)[1:]] = int(m.group(2))
    return [r for r in recs if "name" in r]


def main(argv: List[str]) -> int:
    ks = kernels()
    if "--all" in argv:
        for k in sorted(ks, key=lambda k: k["name"]):
            print(f"{k['name']}: vgpr {k.get('vgpr_count')} sgpr {k.get('sgpr_count')} "
                  f"spill v/s {k.get('vgpr_spill_count')}/{k.get('sgpr_spill_count')} "
                  f"lds {k.get('group_segment_fixed_size')} scratch {k.get('private_segment_fixed_size')}")
        return 0
    fam: Dict[str, List[Dict[str, object]]] = {}
    for k in ks:
        m = re.match(r"_ZN2rn\d+(\w+?)I", str(k["name"]))
        fam.setdefault(m.group(1) if m else str(k["name"]), []).append(k)
    print(f"{len(ks)} kernels in {len(code_objects())} gfx950 code objects of {os.path.basename(LIB)}")
    print(f"{'kernel family':34s} {'instances':>9s} {'max VGPRs':>9s} {'max SGPRs':>9s} {'VGPR spills':>11s} "
          f"{'SGPR spills':>11s} {'max LDS B':>9s} {'scratch B':>9s}")
    for name in sorted(fam):
        g = fam[name]
        mx = lambda f: max(int(k.get(f, 0)) for k in g)  # noqa: E731
        print(f"{name:34s} {len(g):9d} {mx('vgpr_count'):9d} {mx('sgpr_count'):9d} {mx('vgpr_spill_count'):11d} "
              f"{mx('sgpr_spill_count'):11d} {mx('group_segment_fixed_size'):9d} "
              f"{mx('private_segment_fixed_size'):9d}")
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
