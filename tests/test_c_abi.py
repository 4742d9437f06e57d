"""The C ABI from C: include/zha.h compiles as C99 with gcc (-Wall -Werror), and a C
program linked against libzha.so gets the sizes and the host-side argument checks the
header describes. No GPU: every call here returns before anything is enqueued."""

import os
import shutil
import subprocess

import pytest

from tree_indexed_sparse_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "zha.h"

static int fails = 0;
#define EXPECT(c) do { if (!(c)) { printf("FAIL %s:%d %s\n", __FILE__, __LINE__, #c); ++fails; } } while (0)

int main(void) {
  /* pyramid bytes: levels of B*Hkv*(N/b^l)*d floats, each rounded up to 256 bytes */
  size_t want = 0, n = 4096;
  for (int l = 1; l <= 3; ++l) { n /= 4; want = (want + 4 * 2 * n * 64 + 255) / 256 * 256; }
  EXPECT(zha_tree_bytes(1, 2, 4096, 64, 4, 3) == want);
  EXPECT(zha_tree_bytes(1, 2, 4000, 64, 4, 3) == 0);
  EXPECT(zha_router_bytes(1, 2, 4096, 96, 4, 3) == 0);
  EXPECT(zha_router_bytes(1, 2, 4096, 64, 4, 3) > 0);

  void* fake = (void*)0x1000;
  /* the library lays the view out: over zero tokens the build enqueues nothing */
  zha_tree t;
  memset(&t, 0, sizeof t);
  EXPECT(zha_build_tree(fake, fake, ZHA_BF16, 1, 2, 0, 4096, 64, 4, 3, fake, 1 << 30, &t,
                        NULL) == ZHA_OK);
  EXPECT(t.N == 0 && t.level_off[1] == 0 && t.level_off[2] == 2 * 1024 * 64);
  t.N = 4096;
  EXPECT(zha_attend_workspace_bytes(&t, 1, 8) > 0);
  EXPECT(zha_attend_workspace_bytes(&t, 1, 7) == 0);  /* Hq % Hkv != 0 */
  t.level_off[3] += 1;                                  /* not the library's layout */
  EXPECT(zha_attend_workspace_bytes(&t, 1, 8) == 0);
  t.level_off[3] -= 1;

  EXPECT(zha_attend(NULL, fake, 1, 8, fake, fake, 0.9f, 1, (float*)fake, NULL, 4096,
                    (int32_t*)fake, fake, 1 << 30, NULL) == ZHA_ERR_INVALID_ARG);
  EXPECT(strlen(zha_last_error()) > 0);
  EXPECT(zha_attend(&t, fake, 1, 8, fake, fake, 1.5f, 1, (float*)fake, NULL, 4096,
                    (int32_t*)fake, fake, 1 << 30, NULL) == ZHA_ERR_INVALID_ARG);
  EXPECT(zha_attend(&t, fake, 1, 8, fake, fake, 0.9f, 1, (float*)fake, (int32_t*)fake, 100,
                    (int32_t*)fake, fake, 1 << 30, NULL) == ZHA_ERR_CAPACITY);
  EXPECT(zha_attend_causal(&t, fake, 1, 8, NULL, fake, fake, 0.9f, 1, (float*)fake, NULL, 4096,
                           (int32_t*)fake, fake, 1 << 30, NULL) == ZHA_ERR_INVALID_ARG);
  t.router = ZHA_ROUTER_MXFP4;  /* no router copy */
  EXPECT(zha_attend(&t, fake, 1, 8, fake, fake, 0.9f, 1, (float*)fake, NULL, 4096,
                    (int32_t*)fake, fake, 1 << 30, NULL) == ZHA_ERR_INVALID_ARG);
  EXPECT(zha_build_tree(fake, fake, ZHA_BF16, 1, 2, 4096, 4096, 96, 4, 3, fake, 1 << 30, &t,
                        NULL) == ZHA_ERR_UNSUPPORTED);
  double ms = 0.0;
  int64_t launches = 0;
  EXPECT(zha_timing_read(ZHA_K_DECODE, 0, &ms, &launches) == ZHA_OK && launches == 0);
  printf("%s\n", fails ? "FAILED" : "OK");
  return fails != 0;
}
"""


@pytest.fixture(scope="module")
def built(tmp_path_factory):
    if not os.path.exists(L.LIB_PATH):
        pytest.skip("libzha.so not built")
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    d = tmp_path_factory.mktemp("cabi")
    src = d / "main.c"
    src.write_text(PROGRAM)
    exe = d / "main"
    libdir = os.path.dirname(L.LIB_PATH)
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
           str(src), "-o", str(exe), f"-L{libdir}", "-lzha", f"-Wl,-rpath,{libdir}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def test_header_is_c99_and_the_library_links(built):
    assert built.exists()


def test_host_checks_from_c(built):
    r = subprocess.run([str(built)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith("OK")
