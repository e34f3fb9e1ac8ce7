"""The boundary from plain C: a C99 program that includes only include/qrw.h
compiles with gcc -std=c99 -Wall -Werror, links against libqrw.so and gets
the documented status codes back from argument validation (no device calls:
every call is invalid or empty)."""
import os
import subprocess
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "quant_row_workgroup_amd")

PROGRAM = textwrap.dedent(r"""
    #include <stdio.h>
    #include <string.h>
    #include "qrw.h"

    static int fails = 0;
    static void expect(const char* what, int got, int want) {
      if (got != want) {
        printf("%s: got %d (%s), want %d\n", what, got, qrw_status_string(got), want);
        ++fails;
      }
    }

    int main(void) {
      void* x = (void*)(uintptr_t)(1ull << 32);   /* never dereferenced */
      void* y = (void*)(uintptr_t)(2ull << 32);
      expect("rmsnorm empty", rmsnorm_fwd(NULL, NULL, NULL, 0, 64, 64, 64, QRW_BF16, 1e-6f, NULL), QRW_OK);
      expect("rmsnorm dtype", rmsnorm_fwd(x, NULL, y, 4, 64, 64, 64, QRW_F32, 1e-6f, NULL), QRW_ERR_DTYPE);
      expect("rmsnorm null", rmsnorm_fwd(NULL, NULL, y, 4, 64, 64, 64, QRW_BF16, 1e-6f, NULL), QRW_ERR_NULL);
      expect("layernorm stride", layernorm_fwd(x, NULL, NULL, y, 4, 64, 60, 64, QRW_F16, 1e-5f, NULL), QRW_ERR_STRIDE);
      expect("rope shape", rope_apply_neox(x, x, x, y, 4, 2, 64, 24, 128, 128, QRW_F16, QRW_F32, NULL), QRW_ERR_SHAPE);
      expect("fused eps", rmsnorm_rope_fp8_fwd(x, NULL, x, x, (uint8_t*)y, (float*)y, 4, 1, 64, 64, 64, 64,
                                               QRW_BF16, QRW_BF16, 1, -1.0f, NULL), QRW_ERR_VALUE);
      expect("act quant group", act_quant_fp8_fwd(x, (uint8_t*)y, (float*)y, 4, 256, 96, 256, 256, QRW_BF16, NULL),
             QRW_ERR_SHAPE);
      expect("qk head_dim", qk_norm_rope_fwd(x, NULL, NULL, x, x, 4, 2, 1, 96, 64, 384, QRW_BF16, QRW_BF16, 1,
                                             1e-6f, NULL), QRW_ERR_SHAPE);
      expect("ew alias", ew_add_fwd(x, y, (char*)x + 32, 64, QRW_F16, NULL), QRW_ERR_ALIAS);
      expect("status of OK", strcmp(qrw_status_string(QRW_OK), "unknown status") != 0, 1);
      printf("%d failures\n", fails);
      return fails != 0;
    }
""")


def test_header_compiles_as_c99_and_validates(tmp_path):
    import torch

    if torch.cuda.is_available():
        pytest.skip("the calls use fake device addresses: run without a GPU")
    lib = os.path.join(LIBDIR, "libqrw.so")
    if not os.path.exists(lib):
        pytest.skip("libqrw.so is not built")
    src = tmp_path / "abi.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "abi"
    torch_lib = os.path.join(os.path.dirname(torch.__file__), "lib")
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
                    "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe),
                    "-L", LIBDIR, "-lqrw", f"-Wl,-rpath,{LIBDIR}:{torch_lib}"], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failures" in r.stdout
