"""The boundary's host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

ridgefill.cpp (argument checks, workspace carve-up, the row partition, status reporting) is
compiled by g++ with -fsanitize=address,undefined and linked with the library's other
objects as built; a C program then drives every entry point through its host-side checks:
the row partition of the review's worked example (section "A small example: how one row
lands in the cache": 12 rows, 3 of them the tail) and its error cases, every size query
with valid and invalid arguments, and every device entry point with arguments that must be
refused before anything is enqueued.  Any out-of-bounds access, use of freed memory,
signed overflow or misaligned access stops the program with a report."""

import os
import shutil
import subprocess

import pytest

from ridge_map_kv_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")
CSRC = os.path.join(ROOT, "ridge_map_kv_amd", "csrc")
BUILD = os.path.join(ROOT, "_build")
DEVICE_OBJS = ["rf_fill.o", "rf_calib.o", "rf_solve.o", "rf_select.o", "rf_fold.o", "rf_profile.o"]

PROGRAM = r"""
#include "ridgefill.h"
#include <stdio.h>
#include <string.h>

#define CHECK(cond, code) do { if (!(cond)) { printf("failed at %d\n", __LINE__); return code; } } while (0)

int main(void) {
  uint8_t mask[9] = {0, 0, 1, 0, 0, 1, 0, 0, 0};
  int32_t idx[9];
  int64_t n = -1;
  rf_shape s;
  rf_layer lay;
  rf_paged_kv kv;
  const uint16_t* xl[1] = {0};
  float fbuf[16];
  int k;
  CHECK(ridgefill_partition(12, 3, mask, idx, &n) == RF_OK && n == 7, 1);
  CHECK(ridgefill_partition(12, 3, NULL, idx, &n) == RF_OK && n == 9, 2);
  CHECK(ridgefill_partition(3, 4, NULL, idx, &n) == RF_E_SHAPE, 3);
  CHECK(strlen(ridgefill_last_error()) > 0, 4);
  CHECK(ridgefill_partition(12, 3, mask, idx, NULL) == RF_E_INVALID, 5);
  CHECK(ridgefill_partition(((int64_t)1 << 40), 0, NULL, idx, &n) == RF_E_SHAPE, 6);
  CHECK(ridgefill_partition(-1, 0, NULL, idx, &n) == RF_E_SHAPE, 7);
  CHECK(ridgefill_partition(0, 0, NULL, NULL, &n) == RF_OK && n == 0, 8);
  for (k = 0; k <= 8; ++k) CHECK(ridgefill_status_string((rf_status)k) != NULL, 9);

  memset(&s, 0, sizeof s);
  s.d = 4096; s.n_kv_heads = 8; s.head_dim = 128; s.rms_eps = 1e-5f; s.rope_theta = 500000.0;
  CHECK(ridgefill_fill_workspace_bytes(&s, 25805, 20) > 0, 10);
  CHECK(ridgefill_fill_workspace_bytes_ex(&s, 25805, 20, RF_MAPS_FOLDED) > 0, 11);
  CHECK(ridgefill_fill_workspace_bytes_ex(&s, 25805, 20, RF_MAPS_FOLDED | RF_MAPS_INT8) == 0, 12);
  CHECK(ridgefill_fill_workspace_bytes_ex(&s, 25805, 20, 1 << 20) == 0, 13);
  CHECK(ridgefill_fill_workspace_bytes(&s, -1, 20) == 0, 14);
  CHECK(ridgefill_fill_workspace_bytes(NULL, 10, 1) == 0, 15);
  CHECK(ridgefill_fill_workspace_bytes(&s, 10, 0) == 0, 16);
  CHECK(ridgefill_fold_bytes(&s) > 0 && ridgefill_fold_workspace_bytes(&s) > 0, 17);
  CHECK(ridgefill_fold_workspace_bytes_ex(&s, 0) == 0, 18);
  CHECK(ridgefill_value_scale_workspace_bytes(&s, 512, 48, 0) > 0, 19);
  CHECK(ridgefill_value_scale_workspace_bytes(&s, -5, 48, 0) == 0, 20);
  CHECK(ridgefill_select_workspace_bytes(28672) > 0, 21);
  CHECK(ridgefill_select_workspace_bytes(-1) == 0, 22);
  CHECK(ridgefill_calib_state_bytes(4096, 20) > 0 && ridgefill_solve_workspace_bytes(4096, 20) > 0, 23);
  CHECK(ridgefill_calib_state_bytes(300, 20) == 0 && ridgefill_calib_state_bytes(4096, 0) == 0, 24);
  CHECK(ridgefill_calib_state_bytes_ex(8192, 4096, 20) > ridgefill_calib_state_bytes(4096, 20), 25);
  CHECK(ridgefill_solve_workspace_bytes_ex(256, 300, 2) == 0, 26);

  /* shapes the library refuses */
  s.head_dim = 96;
  CHECK(ridgefill_fold_bytes(&s) == 0, 30);
  CHECK(ridgefill_fill_workspace_bytes(&s, 10, 1) == 0, 31);
  s.head_dim = 128; s.d = 300;
  CHECK(ridgefill_fill_workspace_bytes(&s, 10, 1) == 0, 32);
  s.d = 4096; s.d_in = 8192;                       /* wide maps cannot be folded */
  CHECK(ridgefill_fold_bytes(&s) == 0, 33);
  CHECK(ridgefill_fill_workspace_bytes(&s, 10, 1) > 0, 34);
  s.d_in = 0; s.reserved = 1;
  CHECK(ridgefill_fill_workspace_bytes(&s, 10, 1) == 0, 35);
  s.reserved = 0; s.rope_theta = 0.5;
  CHECK(ridgefill_fill_workspace_bytes(&s, 10, 1) == 0, 36);
  s.rope_theta = 500000.0;

  /* device entry points: every one of these is refused on the host */
  memset(&lay, 0, sizeof lay);
  memset(&kv, 0, sizeof kv);
  CHECK(ridgefill_fill(NULL, NULL, 10, 2, 4096, NULL, 1, NULL, 1, NULL, NULL, 0, NULL) == RF_E_INVALID, 40);
  CHECK(ridgefill_fill(&s, NULL, 10, 12, 4096, NULL, 1, &lay, 1, &kv, NULL, 0, NULL) == RF_E_SHAPE, 41);
  CHECK(ridgefill_fill(&s, NULL, 10, 2, 4096, NULL, 9, &lay, 1, &kv, NULL, 0, NULL) == RF_E_SHAPE, 42);
  CHECK(ridgefill_fill(&s, NULL, 10, 2, 4096, NULL, 1, &lay, 1, &kv, NULL, 0, NULL) == RF_E_INVALID, 43);
  CHECK(ridgefill_fill(&s, NULL, 10, 2, 4096, NULL, 1, &lay, -1, &kv, NULL, 0, NULL) == RF_E_INVALID, 44);
  CHECK(ridgefill_fill_streamed(&s, NULL, 10, 2, 4096, NULL, 1, &lay, 1, &kv, NULL, 0, NULL, NULL) != RF_OK, 45);
  CHECK(ridgefill_fill_noalloc(&s, NULL, 10, 2, 4096, NULL, 1, &lay, 1, &kv, NULL, NULL) == RF_E_INVALID, 46);
  CHECK(ridgefill_value_scale(&s, NULL, 4096, xl, 512, &lay, 1, NULL, NULL, 0, NULL) != RF_OK, 47);
  CHECK(ridgefill_fold_maps(&s, &lay, 1, NULL, NULL, 0, NULL) != RF_OK, 48);
  CHECK(ridgefill_quantize_map(NULL, 4, 4, NULL, NULL, NULL) == RF_E_INVALID, 49);
  CHECK(ridgefill_quantize_map(fbuf, -4, 4, NULL, NULL, NULL) != RF_OK, 50);
  CHECK(ridgefill_select_rows(NULL, 10, 1, NULL, NULL, NULL, 0, NULL) != RF_OK, 51);
  CHECK(ridgefill_select_rows(fbuf, 10, 11, NULL, NULL, NULL, 0, NULL) != RF_OK, 52);
  CHECK(ridgefill_calib_reset(NULL, 0, 4096, 20, NULL) == RF_E_INVALID, 53);
  CHECK(ridgefill_calibrate(NULL, 0, 4096, 20, NULL, xl, 10, NULL) == RF_E_INVALID, 54);
  CHECK(ridgefill_calibrate_ex((void*)256, 16, 256, 256, 1, NULL, xl, 10, NULL) == RF_E_WORKSPACE, 55);
  CHECK(ridgefill_solve((void*)256, 1u << 30, 4096, 20, -1.0, NULL, NULL, NULL, NULL, 0, NULL) != RF_OK, 56);
  CHECK(ridgefill_solve(NULL, 0, 4096, 20, 0.03, NULL, NULL, NULL, NULL, 0, NULL) == RF_E_INVALID, 57);
  CHECK(ridgefill_read_status(NULL, NULL) == RF_E_INVALID, 58);
  CHECK(ridgefill_solve_info(NULL, NULL, NULL, NULL) == RF_E_INVALID, 59);
  CHECK(ridgefill_profile_read(RF_KERNEL_COUNT, NULL, NULL) != RF_OK, 60);
  CHECK(strlen(ridgefill_last_error()) > 0, 61);
  CHECK(ridgefill_fold_workspace_bytes_maps(&s, 1, RF_MAPS_INT8) > ridgefill_fold_workspace_bytes(&s), 62);
  CHECK(ridgefill_fold_workspace_bytes_maps(&s, 1, RF_MAPS_FOLDED) == 0, 63);
  CHECK(ridgefill_fold_workspace_bytes_maps(NULL, 1, 0) == 0, 64);
  {                              /* int8 fold: checked on the host, nothing enqueued */
    rf_layer q;
    void* fold_out[1] = {(void*)256};
    memset(&q, 0, sizeof q);
    q.A_q = (const int8_t*)256; q.A_scale = (const float*)256; q.b = (const float*)256;
    q.norm_w = (const uint16_t*)256; q.W_K = (const uint16_t*)256; q.W_V = (const uint16_t*)256;
    CHECK(ridgefill_fold_maps(&s, &q, 1, fold_out, (void*)256, 4096, NULL) == RF_E_WORKSPACE, 65);
    q.A = (const uint16_t*)256;  /* both maps given */
    CHECK(ridgefill_fold_maps(&s, &q, 1, fold_out, (void*)256, 4096, NULL) == RF_E_INVALID, 66);
  }
  printf("ok\n");
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not found")
def test_host_entry_points_under_asan_and_ubsan(tmp_path):
    objs = [os.path.join(BUILD, o) for o in DEVICE_OBJS]
    if not all(os.path.exists(o) for o in objs) or not os.path.exists(B.LIB_PATH):
        pytest.fail("build the library first (python -m ridge_map_kv_amd.build)")
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
    host_obj = tmp_path / "ridgefill_san.o"
    r = subprocess.run(["g++", "-std=c++17", "-g", "-O1", *san, "-D__HIP_PLATFORM_AMD__",
                        "-I/opt/rocm/include", "-I", INCLUDE, "-I", CSRC, "-c",
                        os.path.join(CSRC, "ridgefill.cpp"), "-o", str(host_obj)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    src = tmp_path / "prog.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "prog"
    r = subprocess.run(["g++", "-std=c++17", "-g", *san, "-Wall", "-Werror", "-I", INCLUDE,
                        "-x", "c++", str(src), "-x", "none", str(host_obj), *objs,
                        "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0, f"exit {r.returncode}:\n{r.stdout}\n{r.stderr[-4000:]}"
    assert r.stdout.strip() == "ok"
