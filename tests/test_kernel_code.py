"""The built kernels' code (CPU: disassembles this repository's own libpkv.so).

Two properties the partition kernels' speed depends on:
- no flat (generic-address) memory instructions: a flat load's wait also
  covers the wave's outstanding global stores, which once held every run's
  first tile;
- no scratch memory in the MFMA partition kernels, except the one-head
  RoPE decode-step instantiations, whose register spills are known and
  which the library routes around when the workspace allows: a run-time
  indexed array in scratch cost 2-3 us at the end of every workgroup.  (The
  VALU kernel, kept for comparison, spills at G = 8 and is not checked.)
The merge kernels are held to the first property too.
"""
from __future__ import annotations

import os
import pathlib
import re
import shutil
import subprocess
from collections import Counter, defaultdict

import pytest

from paged_kv_decode_06_amd import ops

OBJDUMP = "/opt/rocm/llvm/bin/llvm-objdump"


@pytest.fixture(scope="module")
def disassembly():
    lib = ops.library_path()
    if not os.path.exists(lib):
        pytest.fail("libpkv.so is not built (run __graft_entry__.build())")
    if not os.path.exists(OBJDUMP):
        pytest.skip("llvm-objdump is not installed")
    from paged_kv_decode_06_amd import build as B
    work = pathlib.Path(B.BUILD) / "code_test"    # (the build folder: not tracked)
    shutil.rmtree(work, ignore_errors=True)
    work.mkdir(parents=True)
    copy = work / "libpkv.so"
    shutil.copyfile(lib, copy)
    # (the offload bundles are written next to the input file)
    subprocess.run([OBJDUMP, "--offloading", str(copy)], cwd=work, check=True,
                   capture_output=True, timeout=300)
    per_kernel = defaultdict(Counter)
    bundles = [p for p in work.iterdir() if "amdgcn" in p.name and "gfx950" in p.name]
    assert bundles, "no gfx950 code object in libpkv.so"
    for b in bundles:
        text = subprocess.run([OBJDUMP, "-d", "--no-show-raw-insn", str(b)], check=True,
                              capture_output=True, text=True, timeout=300).stdout
        name = None
        for line in text.splitlines():
            m = re.match(r"^[0-9a-f]+ <(.+)>:$", line)
            if m:
                name = m.group(1)
                continue
            if name is None:
                continue
            parts = line.split()
            if not parts or not re.match(r"^[a-z_0-9]+$", parts[0]):
                continue
            op = parts[0]
            if op.startswith("flat_"):
                per_kernel[name]["flat"] += 1
            elif op.startswith("scratch_"):
                per_kernel[name]["scratch"] += 1
            per_kernel[name]["all"] += 1
    return per_kernel


def demangled(names):
    out = subprocess.run(["c++filt"], input="\n".join(names), capture_output=True, text=True,
                         check=True).stdout.splitlines()
    return dict(zip(names, out))


def test_partition_and_merge_kernels_use_no_flat_memory_instructions(disassembly):
    kernels = [n for n in disassembly if "partition_kernel" in n or "merge_" in n]
    assert len(kernels) > 300
    bad = {n: c["flat"] for n, c in disassembly.items() if n in kernels and c["flat"]}
    assert not bad, demangled(list(bad))


def test_mfma_partition_kernels_use_no_scratch_but_the_one_head_rope_ones(disassembly):
    names = [n for n in disassembly if "mfma_partition_kernel" in n]
    assert len(names) > 300
    d = demangled(names)
    bad = []
    for n in names:
        if not disassembly[n]["scratch"]:
            continue
        m = re.search(r"MfmaShape<\d+, \d+, \d+, \d, (\d)>, (true|false), (true|false), \d>", d[n])
        if m and m.group(1) == "1" and m.group(3) == "true":
            continue          # one kv head per wave, RoPE inside the decode step
        bad.append(d[n])
    assert not bad, bad[:5]
