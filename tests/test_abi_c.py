"""The C ABI as a C program sees it (no GPU needed, no kernel is launched).

include/rfp2.h must compile as C99 and link against librfp2.so; every entry
point, called from C with a null data pointer, must return RFP2_E_NULL before
touching the GPU, and the size query must refuse bad arguments with 0.
"""
import os
import shutil
import subprocess

import pytest

import bit_gemv_amd as rf

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROGRAM = r"""
#include "rfp2.h"
#include <stdio.h>

#define N_ 4
#define K_ 256
static int fails = 0;
static void expect(const char* call, int got, int want) {
  if (got != want) { printf("%s: %d, expected %d\n", call, got, want); ++fails; }
}

int main(void) {
  char dummy[64];
  void* p = (void*)(((unsigned long)dummy + 15) & ~15ul);  /* never dereferenced */
  hipStream_t st = (hipStream_t)0;
  expect("abi_version", rfp2_abi_version(), 1);
  expect("status_string", rfp2_status_string(RFP2_E_NULL)[0] != 'u', 1);
  expect("quantize_acts", rfp2_quantize_acts(NULL, 1, K_, p, p, st), RFP2_E_NULL);
  expect("quantize_weights", rfp2_quantize_weights(p, N_, K_, NULL, st), RFP2_E_NULL);
  expect("quantize_weights_imatrix",
         rfp2_quantize_weights_imatrix(p, N_, K_, NULL, p, st), RFP2_E_NULL);
  expect("gemv", rfp2_gemv(NULL, N_, K_, p, p, 1, p, st), RFP2_E_NULL);
  expect("gemm", rfp2_gemm(p, N_, K_, p, p, 1, NULL, st), RFP2_E_NULL);
  expect("gemm_f16", rfp2_gemm_f16(p, N_, K_, NULL, p, 1, p, st), RFP2_E_NULL);
  expect("moe_gemv", rfp2_moe_gemv(p, 2, N_, K_, NULL, 1, p, p, p, NULL, st), RFP2_E_NULL);
  expect("moe_gemv_tokens",
         rfp2_moe_gemv_tokens(p, 2, N_, K_, p, 2, 1, p, p, NULL, NULL, st), RFP2_E_NULL);
  expect("moe_sort", rfp2_moe_sort(p, 8, 2, NULL, p, NULL, st), RFP2_E_NULL);
  expect("moe_gemm_workspace_bytes", rfp2_moe_gemm_workspace_bytes(0, 1, 1) == 0, 1);
  expect("moe_gemm_workspace_bytes", rfp2_moe_gemm_workspace_bytes(2, 4, 1) > 0, 1);
  expect("moe_gemm", rfp2_moe_gemm(p, 2, N_, K_, p, 4, 1, p, p, p, NULL, NULL, 0, st),
         RFP2_E_NULL);
  expect("moe_gemm_noalloc",
         rfp2_moe_gemm_noalloc(p, 2, N_, K_, p, 4, 1, p, p, NULL, NULL, st), RFP2_E_NULL);
  expect("moe_gemm_noalloc",
         rfp2_moe_gemm_noalloc(p, 128, N_, K_, p, 32736, 8, p, p, p, NULL, st), RFP2_E_SHAPE);
  expect("quant_gemv", rfp2_quant_gemv(p, N_, K_, NULL, p, p, p, st), RFP2_E_NULL);
  expect("quant_moe_gemv",
         rfp2_quant_moe_gemv(p, 2, N_, K_, p, 1, p, p, p, NULL, NULL, st), RFP2_E_NULL);
  expect("read_ceiling", rfp2_read_ceiling(NULL, 16, 0u, p, st), RFP2_E_NULL);
  expect("debug_decode", rfp2_debug_decode(p, N_, K_, NULL, p, st), RFP2_E_NULL);
  expect("debug_half_dots", rfp2_debug_half_dots(p, N_, K_, p, 1, NULL, st), RFP2_E_NULL);
  expect("debug_half_sums_mf", rfp2_debug_half_sums_mf(p, N_, K_, p, 1, NULL, st), RFP2_E_NULL);
  expect("debug_decode_i8", rfp2_debug_decode_i8(p, N_, K_, p, p, NULL, st), RFP2_E_NULL);
  expect("debug_decode_f16", rfp2_debug_decode_f16(p, N_, K_, 0, NULL, st), RFP2_E_NULL);
  expect("shape", rfp2_gemv(p, N_, 288, p, p, 1, p, st), RFP2_E_SHAPE);
  expect("align", rfp2_gemv((const uint8_t*)p + 2, N_, K_, p, p, 1, p, st), RFP2_E_ALIGN);
  printf("%s\n", fails ? "FAILED" : "ok");
  return fails != 0;
}
"""


def test_header_compiles_as_c_and_every_call_checks_its_arguments(tmp_path):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    lib = rf.LIB_PATH
    assert os.path.exists(lib), "librfp2.so is not built"
    src = tmp_path / "abi.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "abi"
    cmd = [cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"), str(src), "-o",
           str(exe), lib, "-Wl,-rpath," + os.path.dirname(lib)]
    built = subprocess.run(cmd, capture_output=True, text=True, timeout=120)
    assert built.returncode == 0, built.stderr[-2000:]
    ran = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert ran.returncode == 0 and ran.stdout.strip().endswith("ok"), ran.stdout + ran.stderr
