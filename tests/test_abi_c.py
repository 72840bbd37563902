"""The C ABI from C: a C99 program includes include/sla.h, links libsla.so and
makes the host-only calls (version, block counts, workspace sizes, status
text and the error paths that return before any device work, including those
of the SLA backward, the training pair and the allocation-free forward)."""

import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "sparse_linear_attention_block_amd")

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "sla.h"

int main(void) {
  sla_problem p = {1, 12, 32760, 128, SLA_BF16, SLA_QUANT_NONE, 0, SLA_PHI_SOFTMAX, 0.05, 0.10};
  int32_t nb = 0, nh = 0, nl = 0;
  size_t fwd = 0, bwd = 0;
  if ((sla_version() >> 16) != 1) return 1;
  if (sla_block_counts(&p, &nb, &nh, &nl) != SLA_OK || nb != 512 || nh != 25 || nl != 51) return 2;
  if (sla_workspace_bytes(&p, &fwd) != SLA_OK || fwd == 0 || fwd % 256) return 3;
  if (sla_backward_workspace_bytes(&p, &bwd) != SLA_OK || bwd <= fwd) return 4;
  p.d = 96;
  if (sla_workspace_bytes(&p, &fwd) != SLA_ERR_UNSUPPORTED || !strlen(sla_last_error())) return 5;
  p.d = 128;
  p.phi = 7;
  if (sla_forward(&p, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0) != SLA_ERR_ARG) return 6;
  p.phi = SLA_PHI_ELU1;
  size_t bwd1 = 0;
  if (sla_backward_workspace_bytes(&p, &bwd) != SLA_OK || sla1_backward_workspace_bytes(&p, &bwd1) != SLA_OK ||
      bwd1 <= bwd) return 7;
  p.quant = SLA_QUANT_I8QK_F8PV;
  if (sla1_backward_workspace_bytes(&p, &bwd1) != SLA_ERR_UNSUPPORTED) return 11;
  if (sla1_backward(&p, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0) != SLA_ERR_ARG) return 12;
  if (sla_forward_noalloc(&p, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0) != SLA_ERR_WORKSPACE) return 13;  /* too big */
  p.quant = SLA_QUANT_NONE;
  if (sla1_forward(&p, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0) != SLA_ERR_ARG) return 8;
  if (sla_soft_topk(0, 1, 1, 0.5, 1.0, 0, 0, 0) != SLA_ERR_ARG) return 9;
  if (!strstr(sla_status_str(SLA_ERR_WORKSPACE), "WORKSPACE")) return 10;
  /* the training pair: bf16 only, and the backward's workspace for the saving forward */
  p.dtype = SLA_F32;
  if (sla_forward_train(&p, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0) != SLA_ERR_UNSUPPORTED) return 14;
  if (sla_backward_saved(&p, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0) != SLA_ERR_UNSUPPORTED) return 15;
  p.dtype = SLA_BF16;
  if (sla1_forward_train(&p, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0) != SLA_ERR_ARG) return 16;  /* no proj_o */
  if (sla1_backward_saved(&p, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0) != SLA_ERR_ARG) return 17;
  printf("ok\n");
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_c_program_uses_the_abi():
    lib = os.path.join(LIBDIR, "libsla.so")
    if not os.path.exists(lib):
        pytest.skip("libsla.so is not built")
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "t.c"), os.path.join(d, "t")
        with open(src, "w") as f:
            f.write(PROGRAM)
        subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), src,
                        "-L", LIBDIR, "-lsla", f"-Wl,-rpath,{LIBDIR}", "-o", exe], check=True)
        r = subprocess.run([exe], capture_output=True, text=True)
        assert r.returncode == 0 and r.stdout.strip() == "ok", (r.returncode, r.stdout, r.stderr)
