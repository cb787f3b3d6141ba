"""The public header is plain C: a C11 program includes it, links against the
library and runs calls that fail in argument checking (no GPU needed: those
paths make no HIP call)."""
import os
import shutil
import subprocess

import pytest

import sparse_mixture_experts_logits_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "moe_mi355x.h"

int main(void)
{
    moe_opts o;
    moe_opts_init(&o);
    if (o.struct_size != sizeof(moe_opts) || o.routed_scale != 1.0f) return 10;
    int64_t ws = moe_workspace_bytes(32, 4096, 6400, 16, 2, &o);
    if (ws <= 0 || ws % 256) return 11;
    if (moe_workspace_bytes(32, 4096, 6400, 16, 0, &o) != MOE_ERR_INVALID_ARG) return 12;
    if (strstr(moe_last_error(), "k = 0") == NULL) return 13;
    /* T = 0 is a successful no-op, whatever the pointers */
    if (moe_forward(NULL, NULL, NULL, NULL, 0, 64, 32, 4, 2, &o, NULL) != MOE_OK) return 14;
    /* a NULL opts is an argument error */
    if (moe_forward(NULL, NULL, NULL, NULL, 4, 64, 32, 4, 2, NULL, NULL) != MOE_ERR_INVALID_ARG) return 15;
    if (moe_quantize_fp8_rows(NULL, 4, 8, NULL, NULL, NULL) != MOE_ERR_INVALID_ARG) return 16;
    if (moe_quantize_mxfp4_rows(NULL, 4, 16, NULL, NULL, NULL) != MOE_ERR_INVALID_ARG) return 17;
    printf("ok %lld\n", (long long)ws);
    return 0;
}
"""


@pytest.mark.skipif(not os.path.exists(moe.LIB_PATH) or shutil.which("gcc") is None,
                    reason="library not built or no C compiler")
def test_header_compiles_as_c11_and_links(tmp_path):
    src = tmp_path / "use_abi.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "use_abi"
    libdir = os.path.dirname(moe.LIB_PATH)
    cmd = ["gcc", "-std=c11", "-Wall", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"), str(src),
           "-o", str(exe), "-L", libdir, "-l:" + os.path.basename(moe.LIB_PATH), "-Wl,-rpath," + libdir]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ)
    env["LD_LIBRARY_PATH"] = "/opt/rocm/lib:" + env.get("LD_LIBRARY_PATH", "")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0 and r.stdout.startswith("ok"), (r.returncode, r.stdout, r.stderr)
