"""The CPU side under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU
code runs): the oracle's pins against a sanitized build of the oracle, and a
C program driving the library's argument checks, workspace sizing and
entry-point plumbing through a copy of the library whose host code is
sanitized. Every finding is fatal."""
import os
import subprocess
import sys

import pytest

import oracle
import sparse_mixture_experts_logits_amd as moe
from sparse_mixture_experts_logits_amd import build as hipbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"


def _gcc_runtime(name):
    r = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(not (_gcc_runtime("libasan.so") and _gcc_runtime("libubsan.so")),
                    reason="gcc sanitizer runtimes not installed")
def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    lib = oracle.build_sanitized(str(tmp_path / "libmoe_oracle_san.so"))
    env = dict(os.environ)
    env.update(LD_PRELOAD=_gcc_runtime("libasan.so") + ":" + _gcc_runtime("libubsan.so"),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               MOE_ORACLE_LIB=lib, OMP_NUM_THREADS="4")
    files = [os.path.join("tests", f) for f in ("test_oracle_pins.py", "test_oracle_fp8.py", "test_oracle_mxfp4.py",
                                                "test_oracle_stats.py", "test_oracle_scoring.py")]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not slow and not gpu",
                        "-p", "no:cacheprovider", *files], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=900)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert " passed" in r.stdout and "error" not in r.stdout.lower().split("passed")[-1]


PROGRAM = r"""
#include <stdint.h>
#include <stdio.h>
#include <string.h>
#include "moe_mi355x.h"

#define FAKE(n) ((void *)(((uintptr_t)1 << 40) + ((uintptr_t)(n) << 30)))
#define EXPECT(c, code) do { if (!(c)) { printf("check %d failed: %s\n", code, moe_last_error()); return code; } } while (0)

int main(void)
{
    moe_opts o;
    moe_opts_init(&o);
    /* workspace sizes over every shape class (pure host arithmetic) */
    for (int64_t T = 0; T <= 20000; T = T * 3 + 1)
        for (int k = 1; k <= 8; k *= 2) {
            int64_t ws = moe_workspace_bytes(T, 4096, 6400, 16, k, &o);
            EXPECT(ws >= 0 && ws % 256 == 0, 1);
        }
    o.shared_I = 2048;
    EXPECT(moe_workspace_bytes(2048, 2048, 1024, 64, 6, &o) > 0, 2);
    o.shared_I = 0;
    EXPECT(moe_workspace_bytes(32, 4096, 6400, 16, 0, &o) == MOE_ERR_INVALID_ARG, 3);
    EXPECT(moe_workspace_bytes(32, 4100, 6400, 16, 2, &o) == MOE_ERR_INVALID_ARG, 4);
    /* argument checks of moe_forward, each stopping before any HIP call */
    EXPECT(moe_forward(NULL, NULL, NULL, NULL, 0, 64, 32, 4, 2, &o, NULL) == MOE_OK, 5);
    EXPECT(moe_forward(NULL, NULL, NULL, NULL, 4, 64, 32, 4, 2, NULL, NULL) == MOE_ERR_INVALID_ARG, 6);
    EXPECT(moe_forward(NULL, FAKE(1), FAKE(2), FAKE(3), 4, 64, 32, 4, 2, &o, FAKE(4)) == MOE_ERR_INVALID_ARG, 7);
    o.workspace = FAKE(8);
    o.workspace_bytes = 100;
    EXPECT(moe_forward(FAKE(0), FAKE(1), FAKE(2), FAKE(3), 4, 64, 32, 4, 2, &o, FAKE(4)) == MOE_ERR_WORKSPACE, 8);
    EXPECT(strstr(moe_last_error(), "needed") != NULL, 9);
    EXPECT(moe_forward(FAKE(0), FAKE(1), FAKE(2), FAKE(3), 4, 64, 32, 4, 2, &o, FAKE(0)) == MOE_ERR_INVALID_ARG, 10);
    o.topk_ids = (int32_t *)FAKE(8);
    EXPECT(moe_forward(FAKE(0), FAKE(1), FAKE(2), FAKE(3), 4, 64, 32, 4, 2, &o, FAKE(4)) == MOE_ERR_INVALID_ARG, 11);
    o.topk_ids = NULL;
    o.workspace_bytes = (size_t)1 << 30;
    o.workspace = FAKE(3);
    EXPECT(moe_forward(FAKE(0), FAKE(1), FAKE(2), FAKE(3), 4, 64, 32, 4, 2, &o, FAKE(4)) == MOE_ERR_INVALID_ARG, 12);
    o.workspace = NULL;
    o.workspace_bytes = 0;
    o.struct_size = 8;
    EXPECT(moe_forward(FAKE(0), FAKE(1), FAKE(2), FAKE(3), 4, 64, 32, 4, 2, &o, FAKE(4)) == MOE_ERR_INVALID_ARG, 13);
    moe_opts_init(&o);
    o.score_func = MOE_SCORE_SIGMOID;
    o.n_group = 8;
    o.topk_group = 1;
    EXPECT(moe_forward(FAKE(0), FAKE(1), FAKE(2), FAKE(3), 4, 64, 32, 16, 4, &o, FAKE(4)) == MOE_ERR_INVALID_ARG, 14);
    moe_opts_init(&o);
    o.weight_format = MOE_WEIGHTS_MXFP4;
    EXPECT(moe_forward(FAKE(0), FAKE(1), FAKE(2), FAKE(3), 4, 80, 32, 4, 2, &o, FAKE(4)) == MOE_ERR_UNSUPPORTED, 15);
    /* the quantisers' checks */
    EXPECT(moe_quantize_fp8_rows(NULL, 4, 8, NULL, NULL, NULL) == MOE_ERR_INVALID_ARG, 16);
    EXPECT(moe_quantize_mxfp4_rows(FAKE(0), 4, 64, FAKE(0), FAKE(1), NULL) == MOE_ERR_INVALID_ARG, 17);
    /* the message buffer is never overrun */
    EXPECT(moe_workspace_bytes(-1, 64, 32, 4, 2, NULL) == MOE_ERR_INVALID_ARG, 18);
    EXPECT(strlen(moe_last_error()) < 512, 19);
    printf("ok\n");
    return 0;
}
"""


@pytest.mark.skipif(not os.path.exists(CLANG), reason="no ROCm clang")
def test_library_host_code_under_asan_and_ubsan(tmp_path):
    lib = hipbuild.build_host_sanitized(str(tmp_path / "libmoe_mi355x_hostsan.so"))
    src = tmp_path / "drive_abi.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "drive_abi"
    cmd = [CLANG, "-std=c11", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe), "-L", str(tmp_path),
           "-l:" + os.path.basename(lib), "-Wl,-rpath," + str(tmp_path), "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ)
    env.update(ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), (r.returncode, r.stdout, r.stderr[-3000:])
