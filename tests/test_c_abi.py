"""The boundary is a C ABI: a C11 program that includes include/invariant_matmul.h
and links the shared library plans products, reads plan information and gets
the documented errors -- all before any HIP call, so it runs without a GPU."""
import os
import subprocess

import pytest

import invariant_matmul_amd as imm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROGRAM = r"""
#include <stdio.h>
#include "invariant_matmul.h"

#define CHECK(cond) do { if (!(cond)) { printf("FAILED line %d: %s\n", __LINE__, #cond); return 1; } } while (0)

int main(void) {
  gemm_plan_t p = 0;
  gemm_plan_info_t info;
  CHECK(gemm_plan(4096, 4096, 14336, GEMM_BF16, &p) == GEMM_OK);
  CHECK(gemm_plan_info(p, &info) == GEMM_OK);
  CHECK(info.N == 4096 && info.K == 14336 && info.out_dtype == GEMM_F32);
  CHECK(info.split_k > 1 && gemm_workspace_size(p) == (size_t)info.split_k * 4096 * 4096 * 4);
  /* validation happens before any HIP call */
  CHECK(gemm_run(p, 0, (void*)16, (void*)16, 0) == GEMM_ERR_INVALID_VALUE);
  CHECK(gemm_splitk_run(p, (void*)16, (void*)16, (void*)16, 0, 0, 0) == GEMM_ERR_WORKSPACE);
  gemm_plan_destroy(p);
  CHECK(gemm_plan(8, 12, 8, GEMM_F16, &p) == GEMM_ERR_UNSUPPORTED);   /* N not a multiple of 8 */
  CHECK(gemm_plan(-1, 8, 8, GEMM_F16, &p) == GEMM_ERR_INVALID_VALUE);
  CHECK(gemm_plan_ex2(64, 64, 64, GEMM_F16, GEMM_F16, 0, 0, GEMM_TILE_DEFAULT, 1.0f, 1.0f,
                      GEMM_PLAN_B_TRANSPOSED | GEMM_PLAN_PERSISTENT | GEMM_PLAN_TILE_BY_M,
                      &p) == GEMM_OK);
  gemm_plan_destroy(p);

  ozaki_plan_t q = 0;
  ozaki_plan_info_t oi;
  CHECK(ozaki_plan(100, 300, 16384, GEMM_BF16, 0, 0, 0, &q) == GEMM_OK);
  CHECK(ozaki_plan_info(q, &oi) == GEMM_OK);
  CHECK(oi.slices == 7 && oi.d == 9 && oi.pairs == 39 && oi.chunk == 256);
  CHECK(ozaki_workspace_size(q) == oi.workspace_bytes);
  CHECK(ozaki_run(q, (const double*)8, (const double*)8, (double*)8, 0, 0, 0) == GEMM_ERR_WORKSPACE);
  ozaki_plan_destroy(q);
  CHECK(ozaki_plan(8, 8, 8, GEMM_I8, 0, 0, 0, &q) == GEMM_OK);
  CHECK(ozaki_plan_info(q, &oi) == GEMM_OK && oi.pairs == 60);
  ozaki_plan_destroy(q);
  CHECK(ozaki_plan(8, 8, 8, GEMM_F16, 0, 0, 0, &q) == GEMM_ERR_UNSUPPORTED);
  printf("%s %s\n", gemm_status_string(GEMM_OK), gemm_status_string(GEMM_ERR_HIP));
  return 0;
}
"""


def test_c_program_uses_the_abi(tmp_path):
    src = tmp_path / "abi.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "abi"
    libdir = os.path.dirname(imm.LIB_PATH)
    r = subprocess.run(["gcc", "-std=c11", "-Wall", "-Werror", "-pedantic", "-I",
                        os.path.join(ROOT, "include"), str(src), "-L", libdir,
                        "-linvariant_matmul", f"-Wl,-rpath,{libdir}", "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert run.stdout.strip() == "GEMM_OK GEMM_ERR_HIP"
