// A stand-in for the HIP runtime, linked instead of it with the library's host code
// built without device code (tests/test_abi_sanitize.py).  Kernel registration is
// accepted and ignored; every launch "succeeds" without running anything, after its
// configuration is checked against the hardware's limits (grid and workgroup sizes,
// dynamic LDS within what the kernel was granted and within 160 KiB); the device
// symbol lookup returns a fake address.  Nothing here touches a GPU.
#include <hip/hip_ext.h>
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstdio>
#include <map>
#include <mutex>

namespace {
std::mutex g_mu;
std::map<const void*, int>& granted() {  // kernel -> dynamic LDS bytes allowed
  static std::map<const void*, int> m;
  return m;
}
int g_launches = 0, g_bad = 0;

hipError_t check(const void* f, dim3 g, dim3 b, void** args, size_t shmem) {
  std::lock_guard<std::mutex> lk(g_mu);
  ++g_launches;
  const uint64_t threads = static_cast<uint64_t>(b.x) * b.y * b.z;
  int allowed = 64 * 1024;
  auto it = granted().find(f);
  if (it != granted().end()) allowed = it->second;
  const bool ok = f != nullptr && args != nullptr && g.x >= 1 && g.y >= 1 && g.z >= 1 &&
                  g.x <= 0x7fffffffu && g.y <= 65535u && g.z <= 65535u && threads >= 1 &&
                  threads <= 1024 && threads % 64 == 0 && shmem <= static_cast<size_t>(allowed) &&
                  shmem <= 160u * 1024u;
  if (!ok) {
    ++g_bad;
    if (g_bad <= 20)
      std::fprintf(stderr, "bad launch: grid %u %u %u block %u %u %u shmem %zu (allowed %d)\n", g.x,
                   g.y, g.z, b.x, b.y, b.z, shmem, allowed);
  }
  return hipSuccess;
}
}  // namespace

extern "C" {
int mock_launches() { return g_launches; }
int mock_bad_launches() { return g_bad; }

void** __hipRegisterFatBinary(const void*) {
  static void* handle = nullptr;
  return &handle;
}
void __hipRegisterFunction(void**, const void*, char*, const char*, unsigned int, void*, void*,
                           void*, void*, int*) {}
void __hipRegisterVar(void**, void*, char*, const char*, int, size_t, int, int) {}
void __hipUnregisterFatBinary(void**) {}
hipError_t __hipPopCallConfiguration(dim3*, dim3*, size_t*, hipStream_t*) {
  return hipErrorInvalidValue;
}

hipError_t hipGetDevice(int* d) {
  *d = 0;
  return hipSuccess;
}
hipError_t hipFuncSetAttribute(const void* f, hipFuncAttribute attr, int value) {
  if (attr == hipFuncAttributeMaxDynamicSharedMemorySize) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (value < 0 || value > 160 * 1024) return hipErrorInvalidValue;
    granted()[f] = value;
  }
  return hipSuccess;
}
hipError_t hipGetSymbolAddress(void** p, const void*) {
  *p = reinterpret_cast<void*>(static_cast<uintptr_t>(0x300000000000ull));
  return hipSuccess;
}
hipError_t hipLaunchKernel(const void* f, dim3 g, dim3 b, void** args, size_t shmem, hipStream_t) {
  return check(f, g, b, args, shmem);
}
hipError_t hipExtLaunchKernel(const void* f, dim3 g, dim3 b, void** args, size_t shmem, hipStream_t,
                              hipEvent_t, hipEvent_t, int) {
  return check(f, g, b, args, shmem);
}
}  // extern "C"
