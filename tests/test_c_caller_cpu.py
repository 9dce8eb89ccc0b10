"""The boundary from C: a C99 program including include/linattn.h, linked
against the built library, calls entry points that fail host validation
before any HIP call (no GPU needed) and reads their status strings."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "long_sequence_causal_amd", "liblinattn.so")

SRC = r'''
#include <stdio.h>
#include <string.h>
#include "linattn.h"
int main(void) {
  la_shape s;
  memset(&s, 0, sizeof(s));
  s.B = 1; s.H = 2; s.L = 128; s.dk = 96; s.dv = 96; s.nseg = 1; s.dtype = LA_BF16;
  if (la_version() != 1) return 1;
  la_status r = la_chunk_fwd(&s, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0);
  if (r != LA_ERR_UNSUPPORTED) return 2;
  if (strcmp(la_status_str(r), "LA_ERR_UNSUPPORTED") != 0) return 3;
  if (strlen(la_last_error()) == 0) return 4;
  s.dk = s.dv = 64;
  s.split = 1;
  if (la_fwd_workspace_bytes(&s) != 0) return 5;  /* one sub-segment: no workspace */
  s.split = 2;
  if (la_fwd_workspace_bytes(&s) == 0) return 7;  /* two: one start state per sequence */
  r = la_step_gated(2, 3, 64, 64, LA_BF16, 0, 0, 0, 0, 0, 0, 0, 0);
  if (r != LA_ERR_INVALID_ARG) return 6;
  printf("ok %s\n", la_last_error());
  return 0;
}
'''


@pytest.mark.skipif(not os.path.exists(LIB), reason="the library is not built")
def test_a_c99_program_calls_the_library(tmp_path):
    src = tmp_path / "caller.c"
    exe = tmp_path / "caller"
    src.write_text(SRC)
    libdir = os.path.dirname(LIB)
    subprocess.check_call(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                           "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe),
                           "-L", libdir, "-llinattn", "-Wl,-rpath," + libdir])
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, (out.returncode, out.stdout, out.stderr)
    assert out.stdout.startswith("ok ")
