"""The boundary from C: include/ridgefill.h compiles as strict C99 and as C++17, and a C
program linked against libridgefill.so calls its host-only entry points (no GPU): the row
partition of the review's worked example (section "A small example: how one row lands in
the cache": a 12-row prompt, 3 tail rows, so 9 prefix rows), size queries and error
reporting."""

import os
import shutil
import subprocess

import pytest

from ridge_map_kv_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")
LIBDIR = os.path.dirname(B.LIB_PATH)

PROGRAM = r"""
#include "ridgefill.h"
#include <stdio.h>
#include <string.h>

int main(void) {
  /* 12 rows, the last 3 the tail; prefix rows 2 and 5 computed exactly */
  uint8_t mask[9] = {0, 0, 1, 0, 0, 1, 0, 0, 0};
  int32_t idx[9];
  int64_t n = -1;
  if (ridgefill_partition(12, 3, mask, idx, &n) != RF_OK) return 1;
  if (n != 7) return 2;
  {
    const int32_t want[7] = {0, 1, 3, 4, 6, 7, 8};
    int i;
    for (i = 0; i < 7; ++i)
      if (idx[i] != want[i]) return 3;
  }
  /* T > N is a shape error with a description */
  if (ridgefill_partition(3, 4, NULL, idx, &n) != RF_E_SHAPE) return 4;
  if (strlen(ridgefill_last_error()) == 0) return 5;
  if (strlen(ridgefill_status_string(RF_E_SHAPE)) == 0) return 6;
  {
    rf_shape s;
    memset(&s, 0, sizeof s);
    s.d = 4096;
    s.n_kv_heads = 8;
    s.head_dim = 128;
    s.rms_eps = 1e-5f;
    s.rope_theta = 500000.0;
    if (ridgefill_fold_bytes(&s) == 0) return 7;
    s.head_dim = 96;                       /* unsupported head size: no buffer */
    if (ridgefill_fold_bytes(&s) != 0) return 8;
  }
  if (ridgefill_calib_state_bytes(4096, 20) == 0) return 9;
  printf("ok %lld\n", (long long)n);
  return 0;
}
"""


def _compile_and_run(tmp_path, compiler, std, src_name):
    src = tmp_path / src_name
    src.write_text(PROGRAM)
    exe = tmp_path / (src_name + ".out")
    cmd = [compiler, f"-std={std}", "-Wall", "-Wextra", "-Werror", "-I", INCLUDE, str(src),
           "-L", LIBDIR, "-lridgefill", f"-Wl,-rpath,{LIBDIR}", "-o", str(exe)]
    if std == "c99":
        cmd.insert(2, "-pedantic")
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, f"exit {r.returncode}: {r.stdout}{r.stderr}"
    assert r.stdout.strip() == "ok 7"


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_header_compiles_as_c99_and_links(tmp_path):
    assert os.path.exists(B.LIB_PATH), "build the library first"
    _compile_and_run(tmp_path, "gcc", "c99", "abi.c")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not found")
def test_header_compiles_as_cpp17_and_links(tmp_path):
    assert os.path.exists(B.LIB_PATH), "build the library first"
    _compile_and_run(tmp_path, "g++", "c++17", "abi.cpp")
