// Host-side walk over the C ABI (include/rownorm.h, include/distill.h) for a build of
// the library's host code with AddressSanitizer and UndefinedBehaviorSanitizer, no
// device code, and tests/abi_mock_hip.cpp in place of the HIP runtime
// (tests/test_abi_sanitize.py builds and runs it).  Every argument check, plan,
// workspace layout, dispatch and launch sequence runs on the CPU; the mock checks each
// launch's configuration and runs nothing.  Device pointers are distinct addresses that
// the host code must never dereference.
//
// Checked: valid calls over a grid of shapes, types, offsets and gradient selections
// return RN_OK (never RN_ERR_INTERNAL, a plan naming a kernel instance that was not
// compiled) and launch only configurations the hardware accepts; invalid arguments return
// their documented status; the sanitizers report nothing.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "../include/distill.h"
#include "../include/rownorm.h"

namespace {

int g_calls = 0, g_fail = 0;

void* dev(int i) {  // a distinct, 256-byte aligned device-looking address
  return reinterpret_cast<void*>(static_cast<uintptr_t>(0x100000000000ull) +
                                 static_cast<uintptr_t>(i) * (static_cast<uintptr_t>(1) << 36));
}
float* devf(int i) { return static_cast<float*>(dev(i)); }

void expect(bool ok, const char* what, int rc, int64_t M, int64_t N, int a, int b) {
  ++g_calls;
  if (!ok) {
    ++g_fail;
    if (g_fail <= 20)
      std::fprintf(stderr, "FAIL %s: rc %d (%s) M %lld N %lld [%d %d]\n", what, rc,
                   rn_status_str(rc), static_cast<long long>(M), static_cast<long long>(N), a, b);
  }
}
bool launched_or_empty(int rc) { return rc == RN_OK; }

extern "C" int mock_launches();
extern "C" int mock_bad_launches();

const rn_dtype kTypes[] = {RN_F32, RN_F16, RN_BF16};

void valid_calls(int64_t M, int64_t N) {
  const float eps = 1e-6f;
  for (rn_dtype xt : kTypes) {
    for (rn_dtype wt : {xt, RN_F32}) {
      for (float off : {0.0f, 1.0f}) {
        int rc = rmsnorm_fwd(dev(1), N, dev(2), dev(3), N, devf(4), M, N, eps, off, xt, wt, nullptr);
        expect(launched_or_empty(rc), "rmsnorm_fwd", rc, M, N, xt, wt);
        rc = rmsnorm_fwd(dev(1), N, dev(2), dev(3), N, nullptr, M, N, eps, off, xt, wt, nullptr);
        expect(launched_or_empty(rc), "rmsnorm_fwd no rstd", rc, M, N, xt, wt);
        rc = fused_add_rmsnorm_fwd(dev(1), N, dev(2), N, dev(3), dev(4), N, dev(5), N, devf(6), M, N,
                                   eps, off, xt, wt, nullptr);
        expect(launched_or_empty(rc), "fused_add_rmsnorm_fwd", rc, M, N, xt, wt);
        for (int g = 0; g <= 1; ++g) {
          const size_t wsb = rn_bwd_workspace_bytes(M, N, 1);
          rc = rmsnorm_bwd(dev(1), N, dev(2), N, dev(3), dev(4), N, g ? devf(5) : nullptr,
                           g ? dev(6) : nullptr, g ? wsb : 0, M, N, eps, off, xt, wt, nullptr);
          expect(launched_or_empty(rc), "rmsnorm_bwd", rc, M, N, xt, g);
          rc = rmsnorm_bwd_noalloc(dev(1), N, dev(2), N, dev(3), dev(4), N, g ? devf(5) : nullptr,
                                   M, N, eps, off, xt, wt, nullptr);
          expect(launched_or_empty(rc) || rc == RN_ERR_SCRATCH, "rmsnorm_bwd_noalloc", rc, M, N, xt, g);
          rc = fused_add_rmsnorm_bwd(dev(1), N, g ? dev(2) : nullptr, N, dev(3), N, dev(4), dev(5), N,
                                     g ? devf(6) : nullptr, g ? dev(7) : nullptr, g ? wsb : 0, M, N,
                                     eps, off, xt, wt, nullptr);
          expect(launched_or_empty(rc), "fused_add_rmsnorm_bwd", rc, M, N, xt, g);
        }
      }
      int rc = layernorm_fwd(dev(1), N, dev(2), dev(3), dev(4), N, devf(5), devf(6), M, N, 1e-5f, xt,
                             wt, nullptr);
      expect(launched_or_empty(rc), "layernorm_fwd", rc, M, N, xt, wt);
      for (int sel = 0; sel < 4; ++sel) {  // none, dW, dB, both
        const bool gw = sel & 1, gb = sel & 2;
        const int ng = static_cast<int>(gw) + static_cast<int>(gb);
        const size_t wsb = ng ? rn_bwd_workspace_bytes(M, N, ng) : 0;
        rc = layernorm_bwd(dev(1), N, dev(2), N, dev(3), dev(4), N, gw ? devf(5) : nullptr,
                           gb ? devf(6) : nullptr, ng ? dev(7) : nullptr, wsb, M, N, 1e-5f, xt, wt,
                           nullptr);
        expect(launched_or_empty(rc), "layernorm_bwd", rc, M, N, xt, sel);
      }
    }
  }
}

void invalid_calls() {
  const int64_t M = 64, N = 4096;
  int rc = rmsnorm_fwd(nullptr, N, dev(2), dev(3), N, nullptr, M, N, 1e-6f, 0.f, RN_BF16, RN_BF16, nullptr);
  expect(rc == RN_ERR_NULL, "fwd null x", rc, M, N, 0, 0);
  rc = rmsnorm_fwd(dev(1), N, dev(2), dev(3), N, nullptr, M, 0, 1e-6f, 0.f, RN_BF16, RN_BF16, nullptr);
  expect(rc == RN_ERR_SHAPE, "fwd N = 0", rc, M, 0, 0, 0);
  rc = rmsnorm_fwd(dev(1), N, dev(2), dev(3), N, nullptr, M, RN_MAX_N + 1, 1e-6f, 0.f, RN_BF16, RN_BF16,
                   nullptr);
  expect(rc == RN_ERR_SHAPE, "fwd N too large", rc, M, RN_MAX_N + 1, 0, 0);
  rc = rmsnorm_fwd(dev(1), N, dev(2), dev(3), N, nullptr, -1, N, 1e-6f, 0.f, RN_BF16, RN_BF16, nullptr);
  expect(rc == RN_ERR_SHAPE, "fwd M < 0", rc, -1, N, 0, 0);
  rc = rmsnorm_fwd(dev(1), N - 1, dev(2), dev(3), N, nullptr, M, N, 1e-6f, 0.f, RN_BF16, RN_BF16, nullptr);
  expect(rc == RN_ERR_STRIDE, "fwd ldx < N", rc, M, N, 0, 0);
  rc = rmsnorm_fwd(dev(1), N, dev(2), dev(3), N, nullptr, M, N, 1e-6f, 0.f, RN_BF16, RN_F16, nullptr);
  expect(rc == RN_ERR_DTYPE, "fwd weight type", rc, M, N, 0, 0);
  rc = rmsnorm_fwd(dev(1), N, dev(2), dev(3), N, nullptr, M, N, 1e-6f, 0.f, static_cast<rn_dtype>(7),
                   RN_F32, nullptr);
  expect(rc == RN_ERR_DTYPE, "fwd unknown type", rc, M, N, 0, 0);
  const size_t wsb = rn_bwd_workspace_bytes(M, N, 1);
  rc = rmsnorm_bwd(dev(1), N, dev(2), N, dev(3), dev(4), N, devf(5), dev(6), wsb - 1, M, N, 1e-6f, 0.f,
                   RN_BF16, RN_BF16, nullptr);
  expect(rc == RN_ERR_WORKSPACE, "bwd workspace too small", rc, M, N, 0, 0);
  rc = rmsnorm_bwd(dev(1), N, dev(2), N, dev(3), dev(4), N, devf(5), nullptr, wsb, M, N, 1e-6f, 0.f,
                   RN_BF16, RN_BF16, nullptr);
  expect(rc == RN_ERR_WORKSPACE, "bwd workspace null", rc, M, N, 0, 0);
  rc = rmsnorm_bwd_noalloc(dev(1), 16384, dev(2), 16384, dev(3), dev(4), 16384, devf(5), int64_t(1) << 20,
                           16384, 1e-6f, 0.f, RN_BF16, RN_BF16, nullptr);  // 16 MiB of partial rows
  expect(rc == RN_ERR_SCRATCH, "noalloc beyond scratch", rc, int64_t(1) << 20, 16384, 0, 0);
  // distillation loss
  rc = fused_linear_jsd(dev(1), 64, dev(2), nullptr, dev(3), 64, dev(4), nullptr, 16, 60, 64, 100, 0.5f,
                        1.f, 8, devf(5), dev(6), 64, nullptr, nullptr, dev(7), size_t(1) << 30, nullptr);
  expect(rc == RN_ERR_SHAPE, "jsd H % 8", rc, 16, 60, 0, 0);
  rc = fused_linear_jsd(dev(1), 64, dev(2), nullptr, dev(3), 64, dev(4), nullptr, 16, 64, 64, 100, 1.5f,
                        1.f, 8, devf(5), dev(6), 64, nullptr, nullptr, dev(7), size_t(1) << 30, nullptr);
  expect(rc == RN_ERR_SHAPE, "jsd beta > 1", rc, 16, 64, 0, 0);
  rc = fused_linear_jsd(dev(1), 64, dev(2), nullptr, dev(3), 64, dev(4), nullptr, 16, 64, 64, 100, 0.5f,
                        1.f, 8, devf(5), dev(6), 64, nullptr, devf(8), dev(7), size_t(1) << 30, nullptr);
  expect(rc == RN_ERR_NULL, "jsd dB without bias", rc, 16, 64, 0, 0);
  rc = fused_linear_jsd(dev(1), 64, dev(2), nullptr, dev(3), 64, dev(4), nullptr, 16, 64, 64, 100, 0.5f,
                        1.f, 8, devf(5), dev(6), 64, nullptr, nullptr, dev(7), 16, nullptr);
  expect(rc == RN_ERR_WORKSPACE, "jsd workspace too small", rc, 16, 64, 0, 0);
}

void distill_calls() {
  struct S { int64_t BT, H, Ht, V, chunk; };
  const S shapes[] = {{0, 64, 64, 100, 8},     {1, 8, 8, 5, 1},        {257, 128, 96, 777, 100},
                      {300, 64, 64, 1000, 128}, {1000, 512, 512, 2048, 1024}, {4096, 4096, 4096, 128256, 1024},
                      {4096, 4096, 4096, 151936, 1024}, {63 * 2, 64, 64, 300, 63}};
  for (const S& s : shapes) {
    for (int sel = 0; sel < 8; ++sel) {  // dx, dW, dB requested
      const bool gx = sel & 1, gw = sel & 2, gb = sel & 4;
      const size_t need = fused_linear_jsd_workspace_bytes(s.BT, s.H, s.Ht, s.V, s.chunk, gx, gw, gb);
      expect(need > 0, "jsd workspace query", 0, s.BT, s.V, sel, 0);
      if (sel) {
        const size_t base = fused_linear_jsd_workspace_bytes(s.BT, s.H, s.Ht, s.V, s.chunk, 0, 0, 0);
        expect(need >= base, "jsd workspace grows with gradients", 0, s.BT, s.V, sel, 0);
      }
      const int rc = fused_linear_jsd(dev(1), s.H, dev(2), dev(3), dev(4), s.Ht, dev(5), dev(6), s.BT, s.H,
                                      s.Ht, s.V, 0.5f, 1.0f, s.chunk, devf(7), gx ? dev(8) : nullptr, s.H,
                                      gw ? devf(9) : nullptr, gb ? devf(10) : nullptr, dev(11), need,
                                      nullptr);
      expect(launched_or_empty(rc), "fused_linear_jsd", rc, s.BT, s.V, sel, 0);
    }
  }
}

}  // namespace

int main() {
  for (int s = -12; s <= 3; ++s) {
    const char* p = rn_status_str(s);
    expect(p != nullptr && std::strlen(p) > 0, "rn_status_str", s, 0, 0, 0, 0);
  }
  const std::vector<int64_t> Ms = {0, 1, 2, 3, 7, 33, 128, 255, 1000, 2048, 8192, 65536, int64_t(1) << 20};
  const std::vector<int64_t> Ns = {1, 7, 8, 63, 64, 100, 128, 255, 256, 1000, 2048, 4096, 4100,
                                   8192, 12288, 18432, 20000, RN_MAX_N};
  for (int64_t M : Ms)
    for (int64_t N : Ns) {
      for (int g = 0; g <= 3; ++g) {
        const size_t b = rn_bwd_workspace_bytes(M, N, g);
        expect((g >= 1 && g <= 2) ? (M == 0 || b > 0) : b == 0, "rn_bwd_workspace_bytes", 0, M, N, g, 0);
      }
      valid_calls(M, N);
    }
  invalid_calls();
  distill_calls();
  const int bad = mock_bad_launches();
  std::printf("checked %d calls, %d launches, %d bad launches, %d failures\n", g_calls,
              mock_launches(), bad, g_fail);
  return (g_fail || bad) ? 1 : 0;
}
