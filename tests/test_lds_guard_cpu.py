"""The launch guard's LDS rule (csrc/cc_lds.h), compiled for the host with
g++: a kernel's static LDS plus the occupancy reservation must fit the
per-workgroup limit, with no wrap-around, and an unknown limit defers to the
runtime."""
import os
import shutil
import subprocess

import pytest

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "ring_allreduce_reduction_02_amd", "csrc")

PROGRAM = r"""
#include "cc_lds.h"
#include <cstdio>
#define CHECK(x) do { if (!(x)) { std::printf("FAIL %s\n", #x); ++bad; } } while (0)
int main() {
  int bad = 0;
  CHECK(lds_fits(0, 65536, 65536));            // the whole per-workgroup limit
  CHECK(!lds_fits(4, 65536, 65536));           // a static word on top of it
  CHECK(!lds_fits(0, 163840, 65536));          // a whole CU's LDS for one workgroup
  CHECK(lds_fits(8192, 20480, 65536));
  CHECK(lds_fits(65536, 0, 65536));
  CHECK(!lds_fits(65537, 0, 65536));
  CHECK(!lds_fits(0xffffffffu, 2, 65536));     // no wrap-around
  CHECK(lds_fits(0xffffffffu, 0xffffffffu, 0)); // limit unknown
  CHECK(lds_fits(1, 1, -1));
  return bad;
}
"""


def test_lds_rule_on_the_host(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ is not installed")
    src = tmp_path / "lds_rule.cpp"
    src.write_text(PROGRAM)
    exe = tmp_path / "lds_rule"
    subprocess.run([gxx, "-std=c++17", "-Wall", "-Werror", "-I", CSRC, "-o", str(exe), str(src)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout
