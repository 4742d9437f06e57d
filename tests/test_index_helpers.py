"""Integer helpers of the library's internal header that every kernel relies on, compiled
for the host from the header's own code (hipcc's host pass; CPU only):

* the division by a runtime constant that maps a frontier entry or a token to its node
  (zha::FastDiv, a round-up multiply-shift method), against the integer quotient,
  exhaustively for small numerators and at every multiple-boundary and random pair up to
  the 2^31 its comment states;
* the numbering of query heads as (unit, member) pairs (unit = sequence, KV head and block
  of queries; members = the query heads and queries sharing one union frontier), which
  must be a bijection onto the members each unit has, with every member reading its own
  KV head's cache slice."""

import os
import shutil
import subprocess

import pytest

from tree_indexed_sparse_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROGRAM = r"""
#include <cstdint>
#include <cstdio>
#include <hip/hip_runtime.h>
// the header's division calls the device intrinsic __umulhi; this host-only build gives it
// the same definition (high 32 bits of the 64-bit product)
static inline unsigned int host_umulhi(unsigned int x, unsigned int y) {
  return (unsigned int)(((unsigned long long)x * y) >> 32);
}
#define __umulhi host_umulhi
#include "zha_internal.h"

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint64_t next() {  // xorshift64*
  state ^= state >> 12; state ^= state << 25; state ^= state >> 27;
  return state * 0x2545F4914F6CDD1Dull;
}

int main() {
  long long bad = 0, checked = 0;
  auto check = [&](uint32_t n, uint32_t d, const zha::FastDiv& f) {
    ++checked;
    if (f.div(n) != n / d) {
      if (bad < 5) printf("FAIL n=%u d=%u got %u want %u\n", n, d, f.div(n), n / d);
      ++bad;
    }
  };
  // every numerator below 2^16 for every divisor up to 1024
  for (uint32_t d = 1; d <= 1024; ++d) {
    const zha::FastDiv f = zha::make_fastdiv(d);
    for (uint32_t n = 0; n < 65536; ++n) check(n, d, f);
  }
  // around multiples of d up to 2^31 - 1, for divisors up to 2^20 and near powers of two
  const uint32_t top = 0x7fffffffu;
  for (int pass = 0; pass < 2; ++pass) {
    for (uint32_t i = 1; i <= (pass ? 62u : 4096u); ++i) {
      uint32_t d = pass ? ((1u << (1 + (i - 1) / 2)) + ((i & 1) ? 1u : 0u) - ((i & 2) ? 1u : 0u))
                        : i;
      if (d == 0 || d > top) continue;
      const zha::FastDiv f = zha::make_fastdiv(d);
      for (int k = 0; k < 600; ++k) {
        const uint64_t q = (uint64_t)(next() % ((uint64_t)top / d + 1));
        const uint64_t base = q * d;
        for (int64_t e = -1; e <= 1; ++e) {
          const int64_t n = (int64_t)base + e;
          if (n >= 0 && n <= (int64_t)top) check((uint32_t)n, d, f);
        }
      }
      check(top, d, f);
      check(top - 1, d, f);
    }
  }
  // random pairs
  for (int i = 0; i < 4000000; ++i) {
    const uint32_t d = 1u + (uint32_t)(next() % (1u << 20));
    const uint32_t n = (uint32_t)(next() & top);
    check(n, d, zha::make_fastdiv(d));
  }
  printf("%s %lld checked\n", bad ? "FAILED" : "OK", checked);
  return bad != 0;
}
"""


def test_fastdiv_matches_integer_division(tmp_path):
    cc = B.hipcc()
    if not os.path.exists(cc) and shutil.which(cc) is None:
        pytest.skip("hipcc not available")
    src = tmp_path / "fastdiv.hip"
    src.write_text(PROGRAM)
    exe = tmp_path / "fastdiv"
    r = subprocess.run([cc, "--offload-host-only", "-O2", "-std=c++17",
                        "-I", os.path.join(ROOT, "include"),
                        "-I", os.path.join(ROOT, "tree_indexed_sparse_amd", "csrc"),
                        str(src), "-o", str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.startswith("OK"), r.stdout[-2000:]


UNITS = r"""
#include <cstdio>
#include <hip/hip_runtime.h>
#include "zha_internal.h"

int main() {
  long long bad = 0, checked = 0;
  for (int B = 1; B <= 3; ++B)
    for (int Hkv = 1; Hkv <= 4; ++Hkv)
      for (int G = 1; G <= zha::kMaxMembers; ++G)
        for (int T = 1; T <= 37; T += (T < 8 ? 1 : 9)) {
          zha::Geom g{};
          g.B = B; g.T = T; g.Hkv = Hkv; g.G = G; g.Hq = G * Hkv;
          g.Tb = T < zha::kMaxMembers / G ? T : zha::kMaxMembers / G;  // as the host sets it
          g.nTB = (T + g.Tb - 1) / g.Tb;
          g.U = B * Hkv * g.nTB;
          const int QH = B * T * g.Hq;
          // every query head lands on a valid (unit, member) and back
          for (int qh = 0; qh < QH; ++qh) {
            int u, m;
            zha::unit_member_of(g, qh, &u, &m);
            const int h = qh % g.Hq, bb = qh / (g.Hq * T);
            ++checked;
            if (u < 0 || u >= g.U || m < 0 || m >= zha::members_of(g, u) ||
                zha::qh_of(g, u, m) != qh || zha::bg_of(g, u) != bb * Hkv + h / G) {
              if (bad < 5) printf("FAIL B=%d Hkv=%d G=%d T=%d qh=%d u=%d m=%d\n", B, Hkv, G, T, qh, u, m);
              ++bad;
            }
          }
          // every member of every unit is one query head, and the members cover them all
          long long members = 0;
          for (int u = 0; u < g.U; ++u) {
            const int Mu = zha::members_of(g, u);
            if (Mu < 1 || Mu > zha::kMaxMembers) ++bad;
            for (int m = 0; m < Mu; ++m) {
              int u2, m2;
              zha::unit_member_of(g, zha::qh_of(g, u, m), &u2, &m2);
              ++checked;
              if (u2 != u || m2 != m) ++bad;
            }
            members += Mu;
          }
          if (members != QH) ++bad;
        }
  printf("%s %lld checked\n", bad ? "FAILED" : "OK", checked);
  return bad != 0;
}
"""


def test_query_heads_are_numbered_as_unit_members_one_to_one(tmp_path):
    cc = B.hipcc()
    if not os.path.exists(cc) and shutil.which(cc) is None:
        pytest.skip("hipcc not available")
    src = tmp_path / "units.hip"
    src.write_text(UNITS)
    exe = tmp_path / "units"
    r = subprocess.run([cc, "--offload-host-only", "-O2", "-std=c++17",
                        "-I", os.path.join(ROOT, "include"),
                        "-I", os.path.join(ROOT, "tree_indexed_sparse_amd", "csrc"),
                        str(src), "-o", str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.startswith("OK"), r.stdout[-2000:]
