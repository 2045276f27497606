"""The C ABI from C: a program compiled with gcc against include/flashprefill.h
and linked to the built library makes the host-only size queries (no GPU
needed) and checks the documented values and the error path."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "block_sparse_long_kpool_amd", "lib")

PROGRAM = r"""
#include <stdio.h>
#include "flashprefill.h"
int main(void) {
  int32_t cu[5] = {0, 300, 429, 430, 1430};   /* 300, 129, 1, 1000 tokens */
  fp_problem p = {0};
  p.num_seqs = 4; p.cu_seqlens_host = cu; p.cu_seqlens_dev = (const int32_t*)16;
  p.num_q_heads = 8; p.num_kv_heads = 2; p.head_dim = 128; p.block_size = 128;
  p.page_size = 16; p.max_pages_per_seq = 63; p.num_pages = 1000;
  p.page_table_dev = (const int32_t*)16;       /* never dereferenced by size queries */
  p.qk_dtype = FP_BF16; p.v_dtype = FP_BF16; p.out_dtype = FP_BF16;
  printf("%lld %lld %d %lld %lld %lld\n", (long long)fp_num_blocks(&p),
         (long long)fp_num_query_blocks(&p), fp_max_blocks(&p), (long long)fp_num_rows(&p),
         (long long)fp_scores_elems(&p), (long long)fp_csr_capacity(&p));
  p.head_lists = 1;
  printf("%lld %lld\n", (long long)fp_num_rows(&p), (long long)fp_csr_capacity(&p));
  p.head_dim = 64;
  printf("%lld|%s|%s\n", (long long)fp_num_rows(&p), fp_last_error(),
         fp_status_string(FP_ERR_UNSUPPORTED));
  return 0;
}
"""


def test_c_program_uses_the_abi(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    if not os.path.exists(os.path.join(LIB, "libflashprefill.so")):
        pytest.fail("libflashprefill.so is not built")
    src = tmp_path / "t.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "t"
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    str(src), "-L", LIB, "-lflashprefill", f"-Wl,-rpath,{LIB}",
                    "-Wl,-rpath,/opt/rocm/lib", "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.splitlines()
    n = [3, 2, 1, 8]                       # key blocks per sequence
    causal = sum(x * (x + 1) // 2 for x in n)
    assert out[0].split() == [str(v) for v in (sum(n), sum(n), 8, 2 * sum(n), 2 * sum(n) * (8 + 1),
                                                 2 * causal)]
    assert out[1].split() == [str(8 * sum(n)), str(8 * causal)]
    rows, msg, status = out[2].split("|")
    assert rows == "-1" and "head_dim" in msg and status
