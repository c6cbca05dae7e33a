"""Generated-code checks of the ratio-128 kernels' waits and hand-written copies.

The ratio-128 backward copies each window into LDS with inline-asm
`s_mov_b32 m0, ...; buffer_load_dwordx4 ... lds` and waits for the copies
itself (see the kernel's comments).  Two assumptions of that code are
properties of the generated code, checked here on the gfx950 assembly of the
kernels (hipcc, device only, no GPU):

  * M0 is written only inside those asm blocks, so the asm's M0 clobber
    cannot break a value the compiler keeps in M0;
  * every LDS copy of the kernels is one of those asm blocks (the compiler
    emits none of its own, which its wait insertion would track).

The ratio-128 forward keeps the next half window's loads in flight in a
second register slot while it writes the current one to LDS; inside its row
loop every wait for vector memory must leave those four loads outstanding
(`s_waitcnt vmcnt(N)` with N >= 4, never a drain), for every segment-table
kind, including the workspace table, whose lookups go through the scalar
cache.
"""
from __future__ import annotations

import os
import re
import subprocess
import tempfile

import pytest

from gated_pooling_amd import build as B


@pytest.fixture(scope="module")
def asm():
    flags = [f for f in B.FLAGS if f not in ("-shared", "-fPIC")]
    with tempfile.TemporaryDirectory() as tmp:
        out = os.path.join(tmp, "k.s")
        res = subprocess.run([B.HIPCC, *flags, "--cuda-device-only", "-S", "-o", out, B.SOURCES[0]],
                             capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(res.stderr[-3000:])
        return open(out).read()


def kernel_bodies(text, pattern):
    names = re.findall(r"\n(" + pattern + r"\w*):", text)
    assert names, pattern
    for name in names:
        i = text.index("\n" + name + ":")
        yield name, text[i:text.index(".Lfunc_end", i)].split("\n")


def test_m0_and_lds_copies_only_in_the_copy_asm(asm):
    n = 0
    for name, body in kernel_bodies(asm, r"_ZN3csa12_GLOBAL__N_113bwd128_kernel"):
        in_asm = False
        copies = 0
        for line in body:
            if "ASMSTART" in line:
                in_asm = True
            elif "ASMEND" in line:
                in_asm = False
            elif re.search(r"\bm0\b", line) and not line.strip().startswith(";"):
                assert in_asm, f"{name}: M0 used outside the copy asm: {line.strip()}"
            elif re.search(r"buffer_load_dwordx4 .* lds", line):
                assert in_asm, f"{name}: an LDS copy outside the copy asm: {line.strip()}"
                copies += 1
        assert copies > 0, name
        n += 1
    assert n == 6  # coff 1, 2 x three segment-table kinds


def test_forward_row_loop_never_drains_the_prefetch(asm):
    n = 0
    for name, body in kernel_bodies(asm, r"_ZN3csa12_GLOBAL__N_113fwd128_kernel"):
        heads = [i for i, line in enumerate(body) if "This Loop Header: Depth=1" in line]
        assert len(heads) == 1, name
        waits = [int(m.group(1)) for line in body[heads[0]:]
                 for m in [re.search(r"s_waitcnt vmcnt\((\d+)\)", line)] if m]
        assert waits and min(waits) >= 4, f"{name}: row-loop vmcnt waits {sorted(set(waits))}"
        n += 1
    assert n == 6  # coff 1, 2 x three segment-table kinds
