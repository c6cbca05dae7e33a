"""Every tuning path of libcsa against the oracle.

The default configuration is covered by the main parity tests; this runs the
other kernel variants (prefetch depths, 4 columns per lane, 512/1024-thread
backward workgroups, small grids that make lanes walk many windows, other
column slices, the per-lane path instead of the wave-uniform one, ratio-128
grids from a few workgroups walking many rows to one workgroup per row), each
in a fresh process because the knobs are read once per process.
"""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

VARIANTS = [
    {"CSA_BWD_PREFETCH": "2"},
    {"CSA_BWD_PREFETCH": "4", "CSA_FWD_PREFETCH": "4"},
    {"CSA_FWD_PREFETCH": "3"},
    {"CSA_FWD_COLS": "4", "CSA_BWD_COLS": "4"},
    {"CSA_BWD_THREADS": "512", "CSA_BWD_MAX_WGS": "96"},
    {"CSA_BWD_THREADS": "1024"},
    {"CSA_UNIFORM": "0"},
    {"CSA_FWD_MAX_WGS": "37", "CSA_BWD_MAX_WGS": "6", "CSA_FWD_PREFETCH": "4"},
    {"CSA_BWD_SLICE_BYTES": "256", "CSA_BWD_MAX_WGS": "1000"},
    {"CSA_BWD_SLICE_BYTES": "2048"},
    {"CSA_BWD_SLICE_BYTES": "384"},   # not a power of two: rounded down to 256-byte slices
]

# ratio-128 grid caps: fewer workgroups than column slices (one per slice),
# a handful walking many rows unevenly, and one per (row, slice)
VARIANTS_R128 = [
    {"CSA_R128_FWD_WGS": "1", "CSA_R128_BWD_WGS": "1"},
    {"CSA_R128_FWD_WGS": "7", "CSA_R128_BWD_WGS": "5"},
    {"CSA_R128_FWD_WGS": "100000", "CSA_R128_BWD_WGS": "60000"},
]


@pytest.fixture(scope="module")
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("knobs", VARIANTS, ids=lambda k: ",".join(f"{a[4:]}={b}" for a, b in k.items()))
def test_tuning_variant_parity(gpu, knobs):
    env = dict(os.environ, **knobs)
    print("variant", knobs, flush=True)
    p = subprocess.run([sys.executable, "-u", "-m", "tests.tuning_parity"], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=240)
    assert p.returncode == 0, f"{knobs}: rc {p.returncode}\n{p.stdout[-2000:]}\n{p.stderr[-3000:]}"
    assert p.stdout.count("ok ") == 9, p.stdout


@pytest.mark.parametrize("knobs", VARIANTS_R128, ids=lambda k: ",".join(f"{a[4:]}={b}" for a, b in k.items()))
def test_ratio128_grid_variant_parity(gpu, knobs):
    env = dict(os.environ, **knobs)
    print("variant", knobs, flush=True)
    p = subprocess.run([sys.executable, "-u", "-m", "tests.tuning_parity", "r128"], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=240)
    assert p.returncode == 0, f"{knobs}: rc {p.returncode}\n{p.stdout[-2000:]}\n{p.stderr[-3000:]}"
    assert p.stdout.count("ok ") == 4, p.stdout
