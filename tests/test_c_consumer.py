"""The boundary as a C program sees it (no GPU needed): include/logra.h
compiles as C99 and C++17 with warnings as errors, and a C program linked
against liblogra.so gets the documented answers from the host-only entry
points and from argument validation (which returns before any device work).
"""

import os
import shutil
import subprocess

import pytest

import rank_gradient_sketching_accumulate_amd as lg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")
ROCM_INCLUDE = "/opt/rocm/include"
ROCM_LIB = "/opt/rocm/lib"

PROGRAM = r"""
#include <math.h>
#include <stdio.h>
#include <string.h>
#include "logra.h"

#define CHECK(c) do { if (!(c)) { fprintf(stderr, "failed: %s (line %d)\n", #c, __LINE__); return 1; } } while (0)

int main(void) {
  CHECK(logra_abi_version() == LOGRA_ABI_VERSION);
  CHECK(strcmp(logra_status_string(LOGRA_OK), "ok") == 0);
  CHECK(strcmp(logra_status_string((logra_status)99), "unknown status") == 0);
  /* equation 7: a proposal predicting four times the budget is halved */
  CHECK(logra_kl_step_scale(4e-4, 1e-4, 10.0) == 0.5);
  CHECK(isnan(logra_kl_step_scale(-1.0, 1e-4, 1.0)));
  CHECK(fabs(logra_kl_budget(1, 300, 2e-4, 2e-5) - 2e-4) < 1e-18);
  CHECK(logra_kl_effective_budget(1e-4, 9e-5) == 5e-5);
  CHECK(logra_projection_bytes(4096, 64) == (size_t)4 * 4096 * 64);
  CHECK(logra_workspace_bytes(4096, 1536, 1536, 64) >= (size_t)4 * 4096 * 64);
  CHECK(logra_workspace_reserve(4096, 1536, 1536, 0, 0) == LOGRA_ERR_RANGE);
  /* validation returns before any device work */
  void* fake = (void*)(uintptr_t)0x10000;
  CHECK(logra_sketch_accumulate(fake, 512, fake, 256, 16, 512, 256, 0, 0, (float*)fake, 16, 0) == LOGRA_ERR_RANGE);
  CHECK(strlen(logra_last_error()) > 0);
  CHECK(logra_sketch_accumulate(NULL, 512, NULL, 256, 0, 512, 256, 0, 16, NULL, 16, 0) == LOGRA_OK);
  CHECK(logra_merge_update(fake, 500, (const float*)fake, 16, 256, 512, 0, 16, 1e-3f, 0) == LOGRA_ERR_SHAPE);
  CHECK(logra_merge_update_grouped(NULL, 0, 16, 0) == LOGRA_OK);
  CHECK(logra_project(fake, 512, 16, 512, 0, 16, fake, 16, 0) == LOGRA_ERR_SHAPE);
  CHECK(logra_predicted_kl(fake, 1024, fake, 1024, 16, 1000, 7, 1.0f, NULL, (float*)fake, 0) == LOGRA_ERR_RANGE);
  CHECK(logra_set_deterministic(1) == 0);
  CHECK(logra_set_deterministic(0) == 1);
  logra_merge_item item;
  memset(&item, 0, sizeof(item));
  CHECK(logra_merge_update_grouped(&item, 1, 16, 0) == LOGRA_ERR_SHAPE); /* ldu < r, checked first */
  item.ldu = 16;
  CHECK(logra_merge_update_grouped(&item, 1, 16, 0) == LOGRA_OK); /* d = 0: nothing to do */
  printf("ok\n");
  return 0;
}
"""


def _need_tools():
    if shutil.which("gcc") is None or shutil.which("g++") is None:
        pytest.skip("gcc / g++ not available")
    if not os.path.isdir(ROCM_INCLUDE):
        pytest.skip("ROCm headers not available")


@pytest.mark.parametrize("lang", ["c", "c++"])
def test_header_compiles(tmp_path, lang):
    _need_tools()
    src = tmp_path / ("h.c" if lang == "c" else "h.cpp")
    src.write_text('#include "logra.h"\nint main(void) { logra_merge_item it; (void)it; return 0; }\n')
    cc = ["gcc", "-std=c99"] if lang == "c" else ["g++", "-std=c++17"]
    cmd = cc + ["-Wall", "-Wextra", "-Werror", "-fsyntax-only", "-D__HIP_PLATFORM_AMD__", "-I", INCLUDE, "-I",
                ROCM_INCLUDE, str(src)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_c_program_against_the_library(tmp_path):
    _need_tools()
    if not os.path.exists(lg.LIB_PATH):
        pytest.skip("liblogra.so not built")
    src = tmp_path / "consumer.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "consumer"
    libdir = os.path.dirname(lg.LIB_PATH)
    cmd = ["gcc", "-std=c99", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I", INCLUDE, "-I", ROCM_INCLUDE,
           str(src), "-o", str(exe), "-L", libdir, "-llogra", "-L", ROCM_LIB, "-lamdhip64", "-lm",
           f"-Wl,-rpath,{libdir}", f"-Wl,-rpath,{ROCM_LIB}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "cannot find -llogra" in r.stderr:
        pytest.skip("the library is not named for the linker")
    assert r.returncode == 0, r.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stderr
    assert run.stdout.strip() == "ok"
