"""The C ABI's host code (csrc/api.cpp with the index builder) built with g++
under AddressSanitizer and UndefinedBehaviorSanitizer.  The kernel launchers
and the six HIP runtime calls the host code makes are stubs that succeed
without touching memory, so every entry point runs its whole host path
(validation, workspace layout, the stepwise ring's event and copy ordering)
on fake device addresses; extreme sizes and strides probe the size arithmetic.
Host code only: no GPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "context_causal_attention_amd", "csrc")

STUBS = r"""
#include <hip/hip_runtime_api.h>
#include "internal.h"

namespace cpattn {
hipError_t launch_bwd(const BwdArgs&, hipStream_t) { return hipSuccess; }
hipError_t launch_delta(const BwdArgs&, hipStream_t) { return hipSuccess; }
hipError_t launch_fwd(const FwdArgs&, hipStream_t) { return hipSuccess; }
hipError_t launch_a2a(int32_t, int32_t, int64_t, int32_t, int32_t, const void*, void*, int64_t, int32_t, int32_t,
                      hipStream_t) { return hipSuccess; }
hipError_t launch_merge(int64_t, int32_t, float*, float*, const float*, const float*, hipStream_t) {
  return hipSuccess;
}
hipError_t fwd_noalloc_scratch(void** p) {
  *p = reinterpret_cast<void*>(0x200000);  // 256-byte aligned, never dereferenced
  return hipSuccess;
}
}  // namespace cpattn

static int g_events = 0;
const char* hipGetErrorString(hipError_t) { return "stub"; }
hipError_t hipEventCreateWithFlags(hipEvent_t* event, unsigned) {
  *event = reinterpret_cast<hipEvent_t>(new int(++g_events));
  return hipSuccess;
}
hipError_t hipEventDestroy(hipEvent_t event) {
  delete reinterpret_cast<int*>(event);
  --g_events;
  return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }
hipError_t hipStreamWaitEvent(hipStream_t, hipEvent_t, unsigned int) { return hipSuccess; }
hipError_t hipMemcpy2DAsync(void*, size_t, const void*, size_t, size_t, size_t, hipMemcpyKind, hipStream_t) {
  return hipSuccess;
}
int stub_live_events() { return g_events; }
"""

DRIVER = r"""
#include <cstdint>
#include <cstdio>
#include <initializer_list>
#include <limits>
#include "cpattn.h"
#include "internal.h"

int stub_live_events();
static int failures = 0;
#define CHECK(c) do { if (!(c)) { std::fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); ++failures; } } while (0)

static void* const F = reinterpret_cast<void*>(0x10000);  // 16-byte aligned, never dereferenced
static int32_t* const FI = reinterpret_cast<int32_t*>(0x10000);
static float* const FF = reinterpret_cast<float*>(0x10000);
static void* const WS = reinterpret_cast<void*>(0x100000);  // 256-byte aligned
static const size_t BIG = size_t(1) << 40;

static cp_shape shape(int64_t sq, int64_t sk, int32_t d = 128, int32_t in = CP_BF16, int32_t out = CP_F32) {
  cp_shape s{};
  s.b = 1; s.hq = 4; s.hkv = 2; s.d = d; s.sq = sq; s.sk = sk; s.scale = 0.088f;
  s.in_dtype = in; s.out_dtype = out;
  const int64_t q[3] = {4 * sq * d, sq * d, d}, k[3] = {2 * sk * d, sk * d, d};
  for (int i = 0; i < 3; ++i) { s.q_str[i] = q[i]; s.o_str[i] = q[i]; s.k_str[i] = k[i]; s.v_str[i] = k[i]; }
  return s;
}

int main() {
  const int64_t i64max = std::numeric_limits<int64_t>::max();
  // Valid calls run their whole host path.
  for (int32_t in : {CP_BF16, CP_F32}) {
    cp_shape s = shape(256, 512, 128, in);
    CHECK(cp_attn_ring_fwd_workspace(&s, 2) > 0);
    CHECK(cp_attn_partial_fwd(&s, F, F, F, FI, nullptr, FI, FF, FF, WS, BIG, nullptr) == CP_OK);
    CHECK(cp_attn_ring_fwd(&s, 2, 1, F, F, F, FI, FI, FI, F, FF, WS, BIG, nullptr) == CP_OK);
    CHECK(cp_attn_ring_fwd_stepwise(&s, 2, 0, F, F, F, FI, nullptr, FI, FF, FF, WS, BIG, nullptr, 0, nullptr,
                                     nullptr) == CP_OK);
    CHECK(cp_attn_ring_fwd_stepwise(&s, 2, 1, F, F, F, FI, nullptr, FI, FF, FF, WS, BIG, WS, BIG, nullptr,
                                     nullptr) == CP_OK);
    cp_shape s8 = shape(256, 4096, 128, in);
    CHECK(cp_attn_ring_fwd_stepwise(&s8, 8, 3, F, F, F, FI, nullptr, FI, FF, FF, WS, BIG, WS, BIG, nullptr,
                                     nullptr) == CP_OK);
    // the allocation-free ring: valid up to its 4 MiB of tables, rejected past them
    CHECK(cp_attn_ring_fwd_noalloc(&s, 2, 1, F, F, F, FI, FI, FI, F, FF, nullptr) == CP_OK);
    cp_shape wide = shape(256, 131072, 128, in);
    CHECK(cp_attn_ring_fwd_noalloc(&wide, 8, 7, F, F, F, FI, nullptr, FI, F, FF, nullptr) == CP_OK);
    // bf16: 2^21 keys take 32768 tiles x 272 bytes; fp32: 2^24 keys, 524288 tiles x 16 bytes
    cp_shape huge = shape(256, int64_t(1) << (in == CP_BF16 ? 21 : 24), 128, in);
    CHECK(cp_attn_ring_fwd_noalloc(&huge, 8, 0, F, F, F, FI, nullptr, FI, F, FF, nullptr) == CP_EINVAL);
    CHECK(cp_attn_ring_fwd_noalloc(&s, 3, 0, F, F, F, FI, nullptr, FI, F, FF, nullptr) == CP_ESHAPE);
    CHECK(cp_attn_ring_fwd_noalloc(&s, 2, 2, F, F, F, FI, nullptr, FI, F, FF, nullptr) == CP_EINVAL);
    CHECK(cp_attn_ring_fwd_noalloc(&s, 2, 0, nullptr, F, F, FI, nullptr, FI, F, FF, nullptr) == CP_EINVAL);
  }
  CHECK(stub_live_events() == 0);  // every event the calls created was destroyed
  {
    cp_shape s = shape(256, 512);
    CHECK(cp_attn_bwd_workspace(&s, 2) > 0);
    CHECK(cp_attn_bwd_delta(&s, F, F, FF, nullptr) == CP_OK);
    CHECK(cp_attn_partial_bwd(&s, F, F, F, F, FF, FF, FI, nullptr, FI, FF, FF, FF, WS, BIG, nullptr) == CP_OK);
    CHECK(cp_attn_ring_bwd(&s, 2, 0, F, F, F, F, FF, FF, FI, FI, FI, FF, FF, FF, WS, BIG, nullptr) == CP_OK);
    CHECK(cp_attn_merge(1000, 128, FF, FF, FF, FF, nullptr) == CP_OK);
    CHECK(cp_a2a_pack(2, 32, 1024, 128, CP_BF16, F, 32 * 128, F, 0, nullptr) == CP_OK);
    CHECK(cp_a2a_unpack(8, 32, 1024, 128, CP_F32, F, F, 1, nullptr) == CP_OK);
  }
  // Extreme sizes and strides: rejected, with no overflow on the way.
  const int64_t huge[] = {i64max, i64max / 2, i64max / 16, int64_t(1) << 40, int64_t(1) << 31, -1,
                          std::numeric_limits<int64_t>::min()};
  for (int64_t h : huge) {
    for (int field = 0; field < 6; ++field) {
      cp_shape s = shape(256, 512);
      switch (field) {
        case 0: s.sq = h; break;
        case 1: s.sk = h; break;
        case 2: s.q_str[2] = h; break;
        case 3: s.k_str[1] = h; break;
        case 4: s.v_str[2] = h; break;
        case 5: s.o_str[0] = h; break;
      }
      cp_attn_ring_fwd_workspace(&s, 2);
      cp_attn_bwd_workspace(&s, 2);
      cp_attn_ring_fwd_stepwise_workspace(&s, 2);
      cp_attn_ring_stage_bytes(&s, 2);
      const int a = cp_attn_ring_fwd(&s, 2, 0, F, F, F, FI, FI, FI, F, FF, WS, BIG, nullptr);
      const int b = cp_attn_ring_bwd(&s, 2, 0, F, F, F, F, FF, FF, FI, FI, FI, FF, FF, FF, WS, BIG, nullptr);
      const int c = cp_attn_ring_fwd_stepwise(&s, 2, 0, F, F, F, FI, nullptr, FI, FF, FF, WS, BIG, WS, BIG,
                                              nullptr, nullptr);
      // Negative sizes or strides, and row counts of 2^40, are rejected
      // everywhere.  Outer strides may be huge: they are applied in 64-bit
      // pointer arithmetic, and the API cannot know how large an allocation
      // is.  The backward bounds row strides (32-bit buffer offsets).
      if (h < 0 || (field <= 1 && h >= (int64_t(1) << 40))) {
        CHECK(a != CP_OK);
        CHECK(b != CP_OK || field == 5);  // the backward does not read o
        CHECK(c != CP_OK);
      }
      if ((field == 2 || field == 4) && h >= (int64_t(1) << 31)) CHECK(b != CP_OK);
    }
  }
  for (int32_t bad : {0, -1, std::numeric_limits<int32_t>::max(), std::numeric_limits<int32_t>::min()}) {
    cp_shape s = shape(256, 512);
    s.hq = bad;  // 0 and negatives are invalid; 2^31 - 1 is not a multiple of hkv = 2
    CHECK(cp_attn_ring_fwd(&s, 2, 0, F, F, F, FI, FI, FI, F, FF, WS, BIG, nullptr) != CP_OK);
    CHECK(cp_attn_ring_fwd(&s, bad, 0, F, F, F, FI, FI, FI, F, FF, WS, BIG, nullptr) != CP_OK);
    CHECK((cp_attn_merge(bad, 128, FF, FF, FF, FF, nullptr) == CP_OK) == (bad >= 0));
    CHECK(cp_a2a_pack(2, bad, 1024, 128, CP_BF16, F, 4096, F, 0, nullptr) != CP_OK);
    CHECK(cp_a2a_unpack(bad, 32, i64max, 128, CP_BF16, F, F, 0, nullptr) != CP_OK);
  }
  CHECK(cp_attn_merge(i64max, 128, FF, FF, FF, FF, nullptr) != CP_OK);
  CHECK(cp_a2a_pack(2, 32, i64max, 128, CP_BF16, F, 4096, F, 0, nullptr) != CP_OK);
  CHECK(cp_a2a_pack(2, 32, 1024, 128, CP_BF16, F, i64max, F, 0, nullptr) != CP_OK);
  // The grid of the merge and head-exchange launches: for every row count the
  // calls accept (2^31 rows, 16-byte vectors of d = 128 fp32 rows: 2^36
  // items), one workgroup per 256 items up to the cap, and a work-item count
  // below 2^32.
  for (int64_t items : {int64_t(0), int64_t(1), int64_t(256), int64_t(257), int64_t(1) << 30, (int64_t(1) << 30) + 1,
                        int64_t(1) << 32, (int64_t(1) << 31) * 32, (int64_t(1) << 31) * 32 * 65535}) {
    const int64_t blocks = cpattn::stride_blocks(items);
    CHECK(blocks * 256 <= int64_t(0xFFFFFFFF));
    CHECK((items == 0) == (blocks == 0));
    if (items <= (int64_t(1) << 30)) CHECK(blocks * 256 >= items && (blocks - 1) * 256 < items);
  }
  CHECK(cp_attn_merge(int64_t(1) << 31, 128, FF, FF, FF, FF, nullptr) == CP_OK);
  CHECK(cp_attn_merge((int64_t(1) << 31) + 1, 128, FF, FF, FF, FF, nullptr) != CP_OK);
  CHECK(stub_live_events() == 0);
  if (failures) { std::fprintf(stderr, "%d checks failed\n", failures); return 1; }
  std::printf("api host code ok\n");
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_api_host_code_under_address_and_ub_sanitizers(tmp_path):
    (tmp_path / "stubs.cpp").write_text(STUBS)
    (tmp_path / "driver.cpp").write_text(DRIVER)
    exe = tmp_path / "drv"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, "-I", "/opt/rocm/include", os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "index.cpp"),
           str(tmp_path / "stubs.cpp"), str(tmp_path / "driver.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    assert "api host code ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
