"""The C ABI used from C: a program compiled against include/tj2.h and linked with libtj2.so calls the
host-only entry points and the argument checks of the device entry points (no device work), so the header's
declarations and the library's exported functions are checked by a C compiler and linker, not only through
ctypes.  Expected values: the oracle's Philox (RHT sign masks) and the header's storage table."""
import os
import shutil
import subprocess

import pytest

from oracle import philox

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_DIR = os.path.join(ROOT, "bit_fully_quantized_amd")

PROGRAM = r"""
#include <stdio.h>
#include <inttypes.h>
#include "tj2.h"

int main(void) {
  printf("version %s\n", tj2_version());
  const uint64_t seeds[4][2] = {{0, 0}, {0, 2}, {1234, 8}, {9223372036854775813ull, 1099511627779ull}};
  for (int i = 0; i < 4; ++i) printf("signs %u\n", tj2_rht_signs(seeds[i][0], seeds[i][1]));
  size_t c = 0, s16 = 0, s128 = 0;
  tj2_status st = tj2_qtensor_bytes(TJ2_NVFP4, 3, 144, &c, &s16, &s128);
  printf("nvfp4 %d %zu %zu %zu\n", st, c, s16, s128);
  st = tj2_qtensor_bytes(TJ2_FP8, 2, 128, &c, &s16, &s128);
  printf("fp8 %d %zu %zu %zu\n", st, c, s16, s128);
  printf("bad_len %d\n", tj2_qtensor_bytes(TJ2_NVFP4, 2, 100, &c, &s16, &s128));
  /* argument checks happen before any device work */
  tj2_osci_tensor t = {0};
  printf("osci_multi_empty %d\n", osci_reset_step_multi(&t, 0, TJ2_OSCI_ACCUM, 4.0f, 0, NULL, NULL, NULL));
  tj2_adamw_params ap = {1e-3f, 0.9f, 0.95f, 1e-8f, 0.1f, 0.1f, 0.05f};
  tj2_master_tensor m = {0};
  printf("master_multi_null %d\n", master_update_step_multi(&m, 1, &ap, TJ2_OSCI_ACCUM, 4.0f, 0, NULL, NULL, NULL));
  printf("last_error %s\n", tj2_last_error());
  /* OutControl plan from host scores */
  double scores[32];
  for (int i = 0; i < 32; ++i) scores[i] = (double)((i * 7) % 32);
  int32_t outl[32], rest[32], n = 0;
  st = tj2_select_outliers(scores, 32, 0.25, outl, rest, &n);
  printf("plan %d %d", st, (int)n);
  for (int i = 0; i < n; ++i) printf(" %d", (int)outl[i]);
  printf("\n");
  printf("fwd_ws %zu %zu\n", nvfp4_linear_fwd_workspace_size(16384, 4096, 1024, 112),
         nvfp4_linear_fwd_workspace_size(128, 128, 16384, 0));
  printf("gemm_ws %zu\n", nvfp4_gemm_workspace_size(256, 128, 880, 112));
  printf("sumsq_ws %zu\n", tj2_channel_sumsq_workspace_size(1024, 256));
  /* the fused two-grouping quantizer refuses mismatched outputs before any device work */
  tj2_qtensor r = {0}, q = {0};
  r.rows = 32; r.len = 64; r.fmt = TJ2_NVFP4;
  q.rows = 64; q.len = 32; q.fmt = TJ2_NVFP6;
  printf("dual_fmt %d\n", nvfp4_quantize_dual((const void*)0x1000, 32, 64, 1, 0, 0, 2, &r, &q, NULL));
  printf("dual_shape %d\n", nvfp4_quantize_dual((const void*)0x1000, 32, 40, 1, 0, 0, 2, &r, &r, NULL));
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_c_program_against_header_and_library(tmp_path):
    if not os.path.exists(os.path.join(LIB_DIR, "libtj2.so")):
        pytest.fail("libtj2.so is not built (run __graft_entry__.build())")
    src = tmp_path / "abi.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "abi"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), str(src), "-L", LIB_DIR,
                    "-ltj2", "-Wl,-rpath," + LIB_DIR, "-o", str(exe)], check=True, capture_output=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.splitlines()
    kv = {}
    signs = []
    for line in out:
        key, _, rest = line.partition(" ")
        if key == "signs":
            signs.append(int(rest))
        else:
            kv[key] = rest
    assert "gfx950" in kv["version"]
    want = [philox.rht_signs(s, o) for s, o in [(0, 0), (0, 2), (1234, 8), (2 ** 63 + 5, 2 ** 40 + 3)]]
    assert signs == want
    assert kv["nvfp4"].split() == ["0", str(3 * 2 * 64), str(3 * 2 * 8), str(3 * 2 * 4)]
    assert kv["fp8"].split() == ["0", "256", "0", "8"]
    assert kv["bad_len"] == "2"                   # TJ2_ERR_SHAPE
    assert kv["osci_multi_empty"] == "1"          # TJ2_ERR_ARG
    assert kv["master_multi_null"] == "1"         # null arrays: TJ2_ERR_ARG, named by index
    assert "tensors[0]" in kv["last_error"]
    # (i * 7) % 32 is a permutation of 0..31: the 16 largest scores (16..31) sit at these channels
    plan = [int(x) for x in kv["plan"].split()]
    assert plan[:2] == [0, 16]
    assert plan[2:] == sorted(i for i in range(32) if (i * 7) % 32 >= 16)
    fwd = [int(x) for x in kv["fwd_ws"].split()]
    # many output tiles: no split, room for the B image (32 column tiles x 9 chunks, then the scales);
    # one tile over a long K: split
    assert fwd[0] == 32 * 9 * 128 * 272 + 9 * 4096 * 4 and fwd[1] > 0
    assert int(kv["gemm_ws"]) > 0
    assert kv["dual_fmt"] == "1"      # TJ2_ERR_ARG: NVFP4 rows, NVFP6 columns
    assert kv["dual_shape"] == "2"    # TJ2_ERR_SHAPE: cols not a multiple of 16
    assert int(kv["sumsq_ws"]) == 2 * 256 * 8
