"""The C ABI from C: include/mxfp8.h compiles as C99 (and as C++17) with warnings
as errors, and a C program links against the library and gets host-side results
from it (no GPU: only calls that return before any device access)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_DIR = os.path.join(ROOT, "mxfp8_block_scaled_amd")
LIB = os.path.join(LIB_DIR, "libmxfp8.so")

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "mxfp8.h"

int main(void) {
  int bad = 0;
  if (mx_scale_bytes(32, 256) != 256) bad |= 1;
  if (mx_scale_bytes(33, 288) != 1024) bad |= 2;
  if (mx_scale_bytes(32, 48) != -1) bad |= 4;
  if (mx_padded_rows(16384, 8) != 16640) bad |= 8;
  /* validation happens on the host, before any device call */
  if (mx_quantize_dim0(NULL, 32, 32, 32, NULL, NULL, NULL) != MX_E_NULL) bad |= 16;
  if (strstr(mx_last_error(), "NULL") == NULL) bad |= 32;
  if (strcmp(mx_status_string(MX_E_SHAPE), "MX_E_SHAPE") != 0) bad |= 64;
  if (mx_check_offs(NULL, 0, 0, 32, NULL, NULL) != MX_E_SHAPE) bad |= 128;
  printf("%d\n", bad);
  return bad;
}
"""


@pytest.fixture(scope="module")
def workdir(tmp_path_factory):
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} is missing: build it first (__graft_entry__.build())")
    return tmp_path_factory.mktemp("cabi")


@pytest.mark.parametrize("compiler,flags", [("gcc", ["-std=c99", "-x", "c"]), ("g++", ["-std=c++17", "-x", "c++"])])
def test_header_compiles(workdir, compiler, flags):
    if shutil.which(compiler) is None:
        pytest.skip(f"{compiler} not installed")
    src = workdir / "header_only.txt"
    src.write_text('#include "mxfp8.h"\nint mx_header_ok(void) { return MX_OK; }\n')
    subprocess.run([compiler, *flags, "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
                    "-c", str(src), "-o", str(workdir / f"h_{compiler}.o")], check=True)


def test_c_program_links_and_runs(workdir):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not installed")
    src = workdir / "prog.c"
    src.write_text(PROGRAM)
    exe = workdir / "prog"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), str(src), "-o",
                    str(exe), "-L", LIB_DIR, "-lmxfp8", f"-Wl,-rpath,{LIB_DIR}"], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, f"C program reported failures (bitmask {r.stdout.strip()}): {r.stderr}"
