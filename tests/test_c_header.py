"""The C ABI is usable from plain C: include/bsgm.h compiles as C99 and as C++,
and a C program linked against libbsgm.so calls it (host-only calls, no GPU)."""
import os
import shutil
import subprocess

import pytest

from block_sparse_global_mean_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "include", "bsgm.h")

C_PROGRAM = r"""
#include <stdio.h>
#include "bsgm.h"
int main(void) {
  bsgm_layout L = {1, 2, 64, 4, 256, 250, 128, BSGM_BF16, 0.125f};
  int32_t keep[2] = {3, 5};
  bsgm_select_params P = {BSGM_SEL_TOPK, keep, 0.9f, 0, 0, 0};
  long long cap = (long long)bsgm_col_capacity(&L, &P);
  size_t ws = bsgm_workspace_bytes(&L, BSGM_SEL_TOPK);
  int bad = bsgm_select_blocks(&L, &P, NULL, NULL, NULL, NULL, NULL, NULL, cap, NULL, NULL, NULL,
                               NULL, 0, NULL);
  printf("%d %lld %zu %d\n", (int)bsgm_version(), cap, ws, bad);
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
@pytest.mark.parametrize("lang,std", [("c", "-std=c99"), ("c++", "-std=c++11")])
def test_header_compiles(lang, std):
    compiler = "gcc" if lang == "c" else "g++"
    res = subprocess.run([compiler, std, "-Wall", "-Werror", "-fsyntax-only", "-x", lang, HDR],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_c_program_links_and_calls(tmp_path):
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libbsgm.so is not built")
    src = tmp_path / "use_bsgm.c"
    src.write_text(C_PROGRAM)
    exe = tmp_path / "use_bsgm"
    libdir = os.path.dirname(_lib.LIB_PATH)
    res = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", str(src), "-I",
                          os.path.join(ROOT, "include"), "-L", libdir, "-lbsgm",
                          "-Wl,-rpath," + libdir, "-o", str(exe)], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, run.stderr
    version, cap, ws, bad = run.stdout.split()
    assert int(version) == _lib.library().bsgm_version()
    assert int(cap) == 8 * 3 + 8 * 5                 # Nb = 8 blocks per row
    assert int(ws) == 2 * 16 * 64 * 4                # pooled Q and K, 16 rows
    assert int(bad) == -1                            # NULL q and k: BSGM_E_ARG
