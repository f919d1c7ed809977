"""The host index builder (csrc/index.cpp) built with g++ under AddressSanitizer
and UndefinedBehaviorSanitizer, driven over valid and invalid inputs with
output buffers of exactly the documented sizes.  Host code only: no GPU and no
HIP runtime (a stub stands in for the library's error-message helpers)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "context_causal_attention_amd", "csrc")

STUB = r"""
#include <cstdarg>
#include <cstdio>
namespace cpattn {
int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  return code;
}
void clear_error() {}
}  // namespace cpattn
"""

DRIVER = r"""
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <memory>
#include <vector>
#include "cpattn.h"

static uint64_t rng = 88172645463325252ull;
static uint32_t next_u32() { rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17; return (uint32_t)rng; }
static int failures = 0;
#define CHECK(c) do { if (!(c)) { std::fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); ++failures; } } while (0)

// Every rank's positions, each written into a heap buffer of exactly S/cp
// int32 (so an overrun is caught); returns false if any call fails.
static bool deal(const std::vector<int32_t>& cu, int cp, int mode, std::vector<int32_t>* all) {
  const int64_t S = cu.back();
  const int64_t n = S / cp;
  all->clear();
  for (int r = 0; r < cp; ++r) {
    std::unique_ptr<int32_t[]> pos(new int32_t[n > 0 ? n : 1]), lo(new int32_t[n > 0 ? n : 1]);
    const int rc = cp_varlen_index(cu.data(), (int32_t)cu.size() - 1, cp, r, mode, pos.get(), lo.get());
    if (rc != CP_OK) return false;
    for (int64_t i = 0; i < n; ++i) {
      CHECK(pos[i] >= 0 && pos[i] < S);
      CHECK(lo[i] <= pos[i]);
      all->push_back(pos[i]);
    }
  }
  return true;
}

int main() {
  // Zigzag deal: every rank's S/cp positions; together a permutation of [0, S).
  for (int64_t S : {0, 2, 16, 48, 4096, 6144}) {
    for (int cp : {1, 2, 3, 8}) {
      const bool ok = S % (2 * cp) == 0;
      const int64_t n = S / cp;
      std::vector<int> seen(S > 0 ? S : 1, 0);
      for (int r = 0; r < cp; ++r) {
        std::unique_ptr<int32_t[]> pos(new int32_t[n > 0 ? n : 1]);
        const int rc = cp_shard_zigzag(S, cp, r, pos.get());
        CHECK(ok ? rc == CP_OK : rc == CP_ESHAPE);
        if (rc == CP_OK)
          for (int64_t i = 0; i < n; ++i) seen[pos[i]]++;
      }
      if (ok) {
        for (int64_t i = 0; i < S; ++i) CHECK(seen[i] == 1);
        std::unique_ptr<int32_t[]> perm(new int32_t[S > 0 ? S : 1]);
        CHECK(cp_unshard_zigzag(S, cp, perm.get()) == CP_OK);
      }
    }
  }
  CHECK(cp_shard_zigzag(16, 0, 0, nullptr) == CP_EINVAL);
  CHECK(cp_shard_zigzag(16, 2, 2, nullptr) == CP_EINVAL);
  CHECK(cp_shard_zigzag(-4, 2, 0, nullptr) == CP_EINVAL);

  // Packed documents, three deals, random lengths.
  for (int trial = 0; trial < 300; ++trial) {
    const int cp = 1 << (next_u32() % 4);  // 1, 2, 4, 8
    const int docs = 1 + next_u32() % 40;
    const bool per_doc_ok = trial % 2 == 0;  // every length a multiple of 2cp
    std::vector<int32_t> cu(1, 0);
    for (int d = 0; d < docs; ++d) {
      int len = 1 + next_u32() % 700;
      if (per_doc_ok) len = (len / (2 * cp) + 1) * (2 * cp);
      cu.push_back(cu.back() + len);
    }
    const int pad = (int)((2 * cp - cu.back() % (2 * cp)) % (2 * cp));
    if (pad) cu.back() += pad;  // the last document absorbs the rounding
    std::vector<int32_t> all;
    for (int mode : {CP_STREAM, CP_PER_DOC, CP_WHOLE_DOC}) {
      const bool ok = deal(cu, cp, mode, &all);
      if (mode == CP_PER_DOC && !(per_doc_ok && pad == 0)) continue;
      CHECK(ok);
      if (!ok) continue;
      std::vector<int> seen(cu.back(), 0);
      for (int32_t p : all) seen[p]++;
      for (int32_t i = 0; i < cu.back(); ++i) CHECK(seen[i] == 1);
    }
  }
  // Invalid boundaries: errors, no out-of-bounds access.
  {
    std::unique_ptr<int32_t[]> pos(new int32_t[64]), lo(new int32_t[64]);
    const int32_t bad_start[] = {4, 32, 64};
    const int32_t not_monotone[] = {0, 40, 32, 64};
    const int32_t not_multiple[] = {0, 30, 63};
    CHECK(cp_varlen_index(bad_start, 2, 2, 0, CP_STREAM, pos.get(), lo.get()) != CP_OK);
    CHECK(cp_varlen_index(not_monotone, 3, 2, 0, CP_STREAM, pos.get(), lo.get()) != CP_OK);
    CHECK(cp_varlen_index(not_multiple, 2, 2, 0, CP_STREAM, pos.get(), lo.get()) != CP_OK);
    CHECK(cp_varlen_index(not_monotone, 0, 2, 0, CP_STREAM, pos.get(), lo.get()) != CP_OK);
    CHECK(cp_varlen_index(nullptr, 2, 2, 0, CP_STREAM, pos.get(), lo.get()) != CP_OK);
    const int32_t fine[] = {0, 32, 64};
    CHECK(cp_varlen_index(fine, 2, 2, 0, 7, pos.get(), lo.get()) != CP_OK);
    CHECK(cp_varlen_index(fine, 2, 2, 5, CP_STREAM, pos.get(), lo.get()) != CP_OK);
  }

  // Pair counts over exact-size arrays, against a direct count.
  for (int trial = 0; trial < 50; ++trial) {
    const int nq = 1 + next_u32() % 300, nk = 1 + next_u32() % 300;
    std::unique_ptr<int32_t[]> qp(new int32_t[nq]), ql(new int32_t[nq]), kp(new int32_t[nk]);
    for (int i = 0; i < nq; ++i) { qp[i] = next_u32() % 500; ql[i] = qp[i] - (int)(next_u32() % 100); }
    for (int j = 0; j < nk; ++j) kp[j] = next_u32() % 500;
    int64_t want = 0;
    for (int i = 0; i < nq; ++i)
      for (int j = 0; j < nk; ++j) want += (ql[i] <= kp[j] && kp[j] <= qp[i]);
    CHECK(cp_pairs(qp.get(), ql.get(), nq, kp.get(), nk) == want);
  }
  CHECK(cp_pairs(nullptr, nullptr, 3, nullptr, 3) == -1);
  CHECK(cp_ring_source(8, 0, 1) == 7);
  CHECK(cp_ring_source(8, 8, 0) == -1);

  if (failures) { std::fprintf(stderr, "%d checks failed\n", failures); return 1; }
  std::printf("index builder ok\n");
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_index_builder_under_address_and_ub_sanitizers(tmp_path):
    (tmp_path / "stub.cpp").write_text(STUB)
    (tmp_path / "driver.cpp").write_text(DRIVER)
    exe = tmp_path / "drv"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, "-I", "/opt/rocm/include", os.path.join(CSRC, "index.cpp"), str(tmp_path / "stub.cpp"),
           str(tmp_path / "driver.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    assert "index builder ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
