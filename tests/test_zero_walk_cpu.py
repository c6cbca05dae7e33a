"""The zero-fill walk of the backward kernels, compiled for the host.

gated_pooling_amd/csrc/csa_walk.h holds the strided element walk that the
backward's zero workgroups use to write +0.0 into byte ranges of dkv/dscore
(rows past cu_seqlens[S], rows of segments shorter than ratio).  This test
builds that same header into a small host program with g++ and runs the walk
for every thread of the largest zero-fill launch (256 workgroups x 1024
threads) over ranges that end where the 32-bit offset envelope ends
(total_tokens * coff * head_dim * 2 = 2^32 - 4096 bytes, the largest buffer
the library accepts at coff 2, head_dim 512).  Every element of the range must
be visited exactly once and no offset outside it, for 16-, 4- and 2-byte
elements.  A walk that stepped the byte offset itself by step * 16 would pass
2^32 there and wrap onto the start of the buffer.
"""
from __future__ import annotations

import os
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_pooling_amd", "csrc")

DRIVER = r"""
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <vector>
#include "csa_walk.h"

// args: E begin end threads  -> "visits dup outside missing"
template <uint32_t E>
static int run(uint32_t begin, uint32_t end, uint32_t threads) {
  const uint64_t count = end > begin ? (uint64_t(end) - begin) / E : 0;
  std::vector<uint8_t> seen(count + 1, 0);
  uint64_t visits = 0, dup = 0, outside = 0;
  for (uint32_t t = 0; t < threads; ++t) {
    csa::walk_elements<E>(begin, end, t, threads, [&](uint32_t o) {
      ++visits;
      if (o < begin || uint64_t(o) + E > end || (o - begin) % E) { ++outside; return; }
      const uint64_t k = (o - begin) / E;
      if (seen[k]) ++dup;
      seen[k] = 1;
    });
  }
  uint64_t missing = 0;
  for (uint64_t k = 0; k < count; ++k) missing += !seen[k];
  printf("%llu %llu %llu %llu\n", (unsigned long long)visits, (unsigned long long)dup,
         (unsigned long long)outside, (unsigned long long)missing);
  return 0;
}

int main(int argc, char** argv) {
  const uint32_t E = strtoul(argv[1], 0, 0), b = strtoul(argv[2], 0, 0), e = strtoul(argv[3], 0, 0),
                 th = strtoul(argv[4], 0, 0);
  if (E == 16) return run<16>(b, e, th);
  if (E == 4) return run<4>(b, e, th);
  return run<2>(b, e, th);
}
"""

TOP = 2 ** 32 - 4096          # io_bytes of T = 2^21 - 2 rows of 1024 bf16 columns
THREADS = 256 * 1024          # 256 zero workgroups of up to 1024 threads


@pytest.fixture(scope="module")
def walker():
    tmp = tempfile.mkdtemp(prefix="csa_walk_")
    src, exe = os.path.join(tmp, "walk.cpp"), os.path.join(tmp, "walk")
    with open(src, "w") as f:
        f.write(DRIVER)
    subprocess.check_call(["g++", "-O2", "-std=c++17", "-I", CSRC, "-o", exe, src])
    return exe


def _walk(exe, E, begin, end, threads):
    out = subprocess.check_output([exe, str(E), str(begin), str(end), str(threads)], text=True, timeout=120)
    visits, dup, outside, missing = map(int, out.split())
    return visits, dup, outside, missing


@pytest.mark.parametrize("E,begin,end", [
    (16, TOP - 8 * 2 ** 20, TOP),          # padding rows at the top of the largest buffer
    (16, TOP - 2048 * 3, TOP),             # fewer elements than threads
    (16, 0, TOP),                          # the whole buffer (every row padding)
    (4, TOP - 8 * 2 ** 20 - 4, TOP - 4),   # 4-byte aligned ends (even coff * head_dim)
    (2, TOP - 8 * 2 ** 20 - 2, TOP - 2),   # 2-byte ends (odd coff * head_dim)
    (2, 2 ** 32 - 2 ** 24 - 2, 2 ** 32 - 2),  # the last 2-byte element below 2^32
    (16, 4096, 4096),                      # empty range
])
def test_walk_covers_range_once_near_2_32(walker, E, begin, end):
    # the byte offset reached by stepping it directly would pass 2^32 here
    if end - begin >= E * THREADS:
        assert end - E + THREADS * E >= 2 ** 32 or end < 2 ** 31
    visits, dup, outside, missing = _walk(walker, E, begin, end, THREADS)
    assert (dup, outside, missing) == (0, 0, 0)
    assert visits == (end - begin) // E
