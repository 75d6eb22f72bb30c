"""The boundary from C: include/lopt.h compiles as C99 with warnings as errors,
and a C program linked against liblopt.so calls the host-only entry points
(config defaults, sizes, workspace planning and its validation).  No device
call is made."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "learned_optimizer_step_amd")

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "lopt.h"

int main(void) {
  lopt_config cfg;
  if (lopt_default_config(&cfg) != LOPT_OK) return 1;
  if (cfg.n_feat != LOPT_N_FEATURES || cfg.n_time != 11 || cfg.mlp_impl != LOPT_MLP_AUTO) return 2;
  if (lopt_mlp_floats(LOPT_N_FEATURES, 11) != 2402 || lopt_mlp_floats(LOPT_VELO_FEATURES, 11) != 2114) return 3;
  if (lopt_state_floats(4, 5) != 4 * 20 + 3 * 9) return 4;
  /* two tensors at fake, never dereferenced device addresses */
  lopt_tensor ts[2];
  memset(ts, 0, sizeof(ts));
  ts[0].param = (float*)(size_t)0x10000000000ull; ts[0].state = (float*)(size_t)0x20000000000ull;
  ts[0].rows = 16; ts[0].cols = 16;
  ts[1].param = (float*)(size_t)0x30000000000ull; ts[1].state = (float*)(size_t)0x40000000000ull;
  ts[1].rows = 1; ts[1].cols = 9;
  size_t bytes = 0;
  if (lopt_workspace_bytes(NULL, ts, 2, &bytes) != LOPT_OK || bytes == 0 || bytes % 256 != 0) return 5;
  ts[1].rows = 0;
  if (lopt_workspace_bytes(NULL, ts, 2, &bytes) != LOPT_ERR_INVALID_ARGUMENT) return 6;
  if (strlen(lopt_last_error()) == 0) return 7;
  lopt_destroy(NULL);
  printf("ok %zu\n", bytes);
  return 0;
}
"""


def test_c_program_links_and_calls_the_library(tmp_path):
    if not os.path.exists(os.path.join(LIBDIR, "liblopt.so")):
        pytest.skip("liblopt.so not built")
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "abi.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "abi"
    res = subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
                          str(src), "-L", LIBDIR, "-llopt", "-Wl,-rpath," + LIBDIR, "-o", str(exe)],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0 and run.stdout.startswith("ok "), (run.returncode, run.stdout, run.stderr)
