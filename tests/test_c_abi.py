"""The boundary from plain C: include/flce.h compiles as C11 with all
warnings as errors, and a C program links libflce.so and exercises the
host-only entry points (sizes, validation, strings) without a GPU."""
import os
import subprocess

import pytest

from linear_cross_entropy_fwd_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")

C_SRC = r"""
#include <stdio.h>
#include <string.h>
#include "flce.h"

static flce_problem_t problem(int64_t n, int64_t h, int64_t v) {
  flce_problem_t p;
  memset(&p, 0, sizeof p);
  p.n_tokens = n;
  p.hidden = h;
  p.vocab = v;
  p.ignore_index = -100;
  p.dtype = FLCE_BF16;
  p.reduction = FLCE_MEAN;
  p.logit_scale = 1.0f;
  return p;
}

int main(void) {
  if (flce_problem_size() != sizeof(flce_problem_t)) { puts("size mismatch"); return 1; }
  if (strncmp(flce_version(), "flce-gfx950", 11) != 0) { puts("version"); return 2; }
  flce_problem_t p = problem(4096, 4096, 128256);
  size_t f = flce_forward_workspace_size(&p), b = flce_backward_workspace_size(&p);
  size_t fb = flce_forward_backward_workspace_size(&p);
  if (f == 0 || b == 0 || fb < f + b) { puts("workspace sizes"); return 3; }
  /* an invalid problem: size 0 and a status before any launch */
  flce_problem_t bad = problem(64, 100, 1000);   /* 200-byte bf16 rows: not a multiple of 16 */
  if (flce_forward_workspace_size(&bad) != 0) { puts("bad size"); return 4; }
  float loss;
  flce_status_t s = flce_forward(&bad, (void*)0x100000, (void*)0x100000, (const int64_t*)0x100000, NULL,
                                 &loss, NULL, NULL, (void*)0x100000, 1 << 20, NULL);
  if (s != FLCE_ERR_UNSUPPORTED || strlen(flce_last_error()) == 0) { puts("status"); return 5; }
  if (strcmp(flce_status_str(FLCE_ERR_WORKSPACE), "FLCE_ERR_WORKSPACE") != 0) { puts("status str"); return 6; }
  printf("ok %zu %zu %zu\n", f, b, fb);
  return 0;
}
"""


def test_header_is_c11_and_links_from_c(tmp_path):
    lib = _abi.library()  # builds nothing; raises if the library is missing
    assert lib is not None
    src = tmp_path / "abi.c"
    src.write_text(C_SRC)
    exe = tmp_path / "abi"
    libdir = os.path.dirname(_abi.LIB_PATH)
    cmd = ["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", INCLUDE, str(src), "-o", str(exe),
           "-L", libdir, "-l:libflce.so", "-Wl,-rpath," + libdir]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0 and "cannot find" in res.stderr and "amdhip" in res.stderr:
        pytest.skip("HIP runtime library not found for linking")
    assert res.returncode == 0, res.stderr
    env = dict(os.environ)
    env["LD_LIBRARY_PATH"] = ":".join(filter(None, [libdir, "/opt/rocm/lib", env.get("LD_LIBRARY_PATH", "")]))
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=60)
    assert run.returncode == 0, (run.returncode, run.stdout, run.stderr)
    assert run.stdout.startswith("ok ")
    f, b, fb = (int(x) for x in run.stdout.split()[1:4])
    p = _abi.make_problem(4096, 4096, 128256, _abi.BF16)
    assert (f, b, fb) == (_abi.flce_forward_workspace_size(p), _abi.flce_backward_workspace_size(p),
                          _abi.flce_forward_backward_workspace_size(p))
