"""The boundary from C: include/pa.h compiles as C99 with every warning an
error, a C program links libpa.so and calls it (host-side paths only, no GPU)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "paged_kv_cache_321_amd")

PROGRAM = r"""
#include <stdio.h>
#include "pa.h"

int main(void) {
  /* The entry points keep these exact C types. */
  int (*reshape)(const void*, const void*, void*, void*, const int64_t*, int, int, int, int, int,
                 int, int, float, float, void*) = pa_reshape_and_cache;
  int (*copy)(void*, void*, const int64_t*, int, int, int, int, int, int, void*) = pa_copy_blocks;
  int (*decode)(void*, const void*, const void*, const void*, const int32_t*, int, const int32_t*,
                const int32_t*, int, int, int, int, int, int, int, float, int, int, float, float, int,
                int, void*, size_t, void*) = pa_decode;
  size_t (*ws)(int, int, int, int, int, int, int, int, int) = pa_decode_workspace_size;
  const char* (*name)(int) = pa_status_string;
  (void)reshape;
  (void)copy;
  printf("%s\n", name(PA_OK));
  /* LLaMA-13B shape at 2048 tokens: one partition per sequence, no workspace. */
  printf("%zu\n", ws(128, 40, 40, 128, 16, 2048, PA_BF16, PA_BF16, 0));
  /* GQA 70B shape at 32768 tokens: 4 partitions of 8192 tokens per sequence. */
  printf("%zu\n", ws(16, 64, 8, 128, 32, 32768, PA_BF16, PA_BF16, 0));
  /* Host validation: a null output pointer is refused before any GPU call. */
  printf("%d\n", decode(NULL, NULL, NULL, NULL, NULL, 128, NULL, NULL, 1, 8, 8, 128, 16, 64, 2048,
                        0.125f, PA_BF16, PA_BF16, 1.f, 1.f, 0, 0, NULL, 0, NULL));
  printf("%s\n", name(PA_ERR_NULL));
  return 0;
}
"""


@pytest.fixture(scope="module")
def program(tmp_path_factory):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    if not os.path.exists(os.path.join(LIBDIR, "libpa.so")):
        pytest.skip("libpa.so is not built")
    d = tmp_path_factory.mktemp("cabi")
    src = d / "use_pa.c"
    src.write_text(PROGRAM)
    exe = d / "use_pa"
    subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
                    str(src), "-L", LIBDIR, "-lpa", f"-Wl,-rpath,{LIBDIR}", "-o", str(exe)],
                   check=True, capture_output=True, text=True)
    return exe


def test_c_program_uses_the_library(program):
    r = subprocess.run([str(program)], capture_output=True, text=True, timeout=120, check=True)
    lines = r.stdout.splitlines()
    assert lines[0].startswith("PA_OK")
    assert int(lines[1]) == 0
    # (max, sum) pair and a D-float accumulator per (sequence, head, partition).
    assert int(lines[2]) == 16 * 64 * 4 * (128 + 2) * 4
    assert int(lines[3]) == -1 and lines[4].startswith("PA_ERR_NULL")
