"""The host side of the library under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only; no device work).

The library sources are compiled as usual for gfx950 with the sanitizers on
the host pass only (each -fsanitize= behind -Xarch_host), and linked into a
small C++ driver that walks every host-side path that runs before device
work: the launch planners over a grid of shapes (through
logra_workspace_bytes and logra_projection_bytes), the argument checks of
every entry point, the sync payload's layout and parser (with truncated and
corrupted headers in exactly sized heap buffers, so any over-read lands in a
redzone), and the predicted-KL host helpers.  Any sanitizer report aborts the
driver.
"""

import os
import shutil
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "rank_gradient_sketching_accumulate_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"

DRIVER = textwrap.dedent(r"""
    #include "logra.h"
    #include <cstdint>
    #include <cstdio>
    #include <cstdlib>
    #include <cstring>
    #include <vector>

    static uint64_t lcg = 0x9E3779B97F4A7C15ull;
    static uint32_t rnd() { lcg = lcg * 6364136223846793005ull + 1442695040888963407ull; return (uint32_t)(lcg >> 33); }
    #define CHECK(c) do { if (!(c)) { fprintf(stderr, "failed: %s (line %d)\n", #c, __LINE__); return 1; } } while (0)

    int main() {
      void* F = (void*)(uintptr_t)0x10000;  // aligned, never dereferenced on these paths
      // Planners over a grid of shapes.
      const int64_t Ts[] = {1, 31, 32, 33, 700, 4096, 16384, 65536};
      const int64_t Ds[] = {1, 17, 256, 3584, 5120, 17408, 65536};
      const int rs[] = {1, 5, 16, 64, 128, 200, 256, 257, 300, 512};
      size_t acc = 0;
      for (int64_t T : Ts)
        for (int64_t d : Ds)
          for (int64_t k : Ds)
            for (int r : rs) {
              for (int det = 0; det < 2; ++det)
                for (int prec = 0; prec < 2; ++prec) {
                  logra_set_deterministic(det);
                  logra_set_precision(prec);
                  acc += logra_workspace_bytes(T, d, k, r);
                }
              acc += logra_projection_bytes(T, r);
            }
      logra_set_deterministic(0);
      logra_set_precision(0);
      CHECK(acc > 0);
      CHECK(logra_workspace_bytes(0, 5, 5, 5) == 0 && logra_workspace_bytes(5, 5, 5, 513) == 0);
      // Argument checks (all fail before any device call).
      CHECK(logra_sketch_accumulate(F, 512, F, 256, 16, 512, 256, 0, 0, (float*)F, 16, 0) == LOGRA_ERR_RANGE);
      CHECK(logra_sketch_accumulate(F, 500, F, 256, 16, 512, 256, 0, 16, (float*)F, 16, 0) == LOGRA_ERR_SHAPE);
      CHECK(logra_sketch_accumulate_noalloc(F, 512, F, 256, 16, 512, 256, 0, 600, (float*)F, 600, 0) == LOGRA_ERR_RANGE);
      CHECK(logra_project(F, 512, 16, 512, 0, 16, F, 16, 0) == LOGRA_ERR_SHAPE);
      CHECK(logra_contract(F, 256, 16, 256, F, 16, 16, (float*)F, 16, 0) == LOGRA_ERR_SHAPE);
      CHECK(logra_merge_update(F, 500, (const float*)F, 16, 256, 512, 0, 16, 1e-3f, 0) == LOGRA_ERR_SHAPE);
      CHECK(logra_rowadam_scale((float*)F, 16, (float*)F, 256, 16, 0, 0.9f, 1e-8f, 0) == LOGRA_ERR_RANGE);
      CHECK(logra_signs(0, 0, 16, (int8_t*)F, 0) == LOGRA_ERR_RANGE);
      CHECK(logra_basis_normals(0, 4, -1, (float*)F, 0) == LOGRA_ERR_SHAPE);
      CHECK(logra_workspace_reserve(-1, 1, 1, 1, 0) == LOGRA_ERR_SHAPE);
      logra_merge_item items[3];
      memset(items, 0, sizeof(items));
      for (int j = 0; j < 3; ++j) {
        items[j].W = (char*)F + 0x100000 * j; items[j].ldw = 512; items[j].U = (const float*)((char*)F + 0x2000000);
        items[j].ldu = 16; items[j].d = 64; items[j].k = 512; items[j].scale = 1e-3f;
      }
      items[2].W = items[0].W;  // two items write one W
      CHECK(logra_merge_update_grouped(items, 3, 16, 0) == LOGRA_ERR_ALIAS);
      CHECK(logra_payload_pack(items, 40, 16, F, 1 << 20, 0) == LOGRA_ERR_RANGE);
      for (int s = -2; s < 12; ++s) CHECK(logra_status_string((logra_status)s) != NULL);
      CHECK(logra_last_error() != NULL);
      // Payload layout sizes with random items.
      for (int it = 0; it < 2000; ++it) {
        logra_merge_item m[32];
        memset(m, 0, sizeof(m));
        const int n = 1 + (int)(rnd() % 32);
        for (int j = 0; j < n; ++j) { m[j].d = (int64_t)(rnd() % 70000) - 5; m[j].k = rnd() % 9000; }
        (void)logra_payload_bytes(m, n, 1 + (int)(rnd() % 600));
      }
      // A valid header, then truncations and corruptions in exact-size heap buffers.
      const int n = 5, r = 64;
      const size_t hb = logra_payload_header_bytes(n);
      std::vector<unsigned char> good(hb, 0);
      logra_payload_header h; memset(&h, 0, sizeof(h));
      h.magic = LOGRA_PAYLOAD_MAGIC; h.version = LOGRA_PAYLOAD_VERSION; h.count = n; h.r = r;
      uint64_t off = hb;
      logra_payload_entry e[n]; memset(e, 0, sizeof(e));
      for (int j = 0; j < n; ++j) {
        e[j].seed = 100 + j; e[j].d = 10 + j; e[j].k = 20; e[j].scale = 1e-3f; e[j].u_offset = off;
        off += ((uint64_t)e[j].d * r * 4 + 255) / 256 * 256;
      }
      h.total_bytes = off;
      memcpy(good.data(), &h, sizeof(h));
      memcpy(good.data() + 32, e, sizeof(e));
      logra_payload_header ho; logra_payload_entry eo[32];
      CHECK(logra_payload_parse(good.data(), good.size(), &ho, eo, 32) == LOGRA_OK);
      int ok = 0, bad = 0;
      for (int it = 0; it < 20000; ++it) {
        size_t len = good.size();
        if (rnd() % 3 == 0) len = rnd() % (good.size() + 1);
        unsigned char* b = new unsigned char[len ? len : 1];
        memcpy(b, good.data(), len);
        const int flips = rnd() % 4;
        for (int f = 0; f < flips && len; ++f) b[rnd() % len] ^= (unsigned char)(1u << (rnd() % 8));
        const logra_status st = logra_payload_parse(b, len, &ho, eo, (int32_t)(rnd() % 40));
        CHECK(st == LOGRA_OK || st == LOGRA_ERR_SHAPE || st == LOGRA_ERR_RANGE || st == LOGRA_ERR_NULL);
        (st == LOGRA_OK ? ok : bad) += 1;
        delete[] b;
      }
      CHECK(ok > 0 && bad > 0);
      // Predicted-KL host helpers.
      CHECK(logra_kl_step_scale(4e-4, 1e-4, 10.0) == 0.5);
      (void)logra_kl_budget(7, 300, 2e-4, 2e-5);
      (void)logra_kl_effective_budget(1e-4, 9e-5);
      printf("ok %zu\n", acc);
      return 0;
    }
    """)

SOURCES = ["logra_api", "sketch_kernels", "merge_kernels", "misc_kernels", "kl_kernels"]


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG)):
        pytest.skip("ROCm compilers not found")
    out = tmp_path_factory.mktemp("sanitized")
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    procs = []
    for name in SOURCES:
        cmd = [HIPCC, "--offload-arch=gfx950", "-O2", "-g", "-fPIC", "-std=c++17", "-munsafe-fp-atomics",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *host_san,
               "-I", os.path.join(ROOT, "include"), "-c", os.path.join(CSRC, name + ".hip"),
               "-o", str(out / (name + ".o"))]
        procs.append((name, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    for name, p in procs:
        log, _ = p.communicate()
        assert p.returncode == 0, f"{name}: {log[-3000:]}"
    (out / "driver.cpp").write_text(DRIVER)
    link = [CLANG, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
            "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
            str(out / "driver.cpp"), *[str(out / (n + ".o")) for n in SOURCES],
            "-L", "/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", str(out / "driver")]
    r = subprocess.run(link, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    yield out / "driver"
    shutil.rmtree(out, ignore_errors=True)


def test_host_paths_clean_under_asan_and_ubsan(driver):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([str(driver)], capture_output=True, text=True, env=env, timeout=300)
    sys.stdout.write(r.stdout[-500:])
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert r.stdout.startswith("ok ")
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
