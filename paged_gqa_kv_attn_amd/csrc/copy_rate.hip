// copy_rate.hip — the copy rate this part reaches, the ceiling for kernels that read each byte once
// and write each result once (the appends): 1 GiB device to device, by hand-written copy kernels
// with and without the non-temporal hint on loads and stores, and by the runtime's own copy.
// A standalone program (not part of the library); it prints one JSON line.
//
// Thread t of workgroup w copies the 16-byte vectors (w * PER + k) * 256 + t, k < PER; the grid
// covers exactly n16 vectors, which the host checks (n16 % (256 * PER) == 0) before any launch.

#include <hip/hip_runtime.h>

#include <cstdio>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int PER, bool NT_LOAD, bool NT_STORE>
__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ src,
                                                   u32x4* __restrict__ dst) {
  const size_t base = (size_t)blockIdx.x * PER * 256 + threadIdx.x;
  u32x4 v[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k)
    v[k] = NT_LOAD ? __builtin_nontemporal_load(src + base + k * 256) : src[base + k * 256];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    if (NT_STORE) __builtin_nontemporal_store(v[k], dst + base + k * 256);
    else dst[base + k * 256] = v[k];
  }
}

bool ok(hipError_t e, const char* what) {
  if (e == hipSuccess) return true;
  std::fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
  return false;
}

// Mean milliseconds per copy over 10 launches after 3 warm-up launches; < 0 on an error.
template <int PER, bool NT_LOAD, bool NT_STORE>
float time_kernel(const u32x4* src, u32x4* dst, size_t n16, hipEvent_t a, hipEvent_t b) {
  if (n16 % (256 * PER) != 0) return -1.f;
  const dim3 grid((unsigned)(n16 / (256 * PER)));
  for (int i = 0; i < 13; ++i) {
    if (i == 3 && !ok(hipEventRecord(a, 0), "event")) return -1.f;
    copy_kernel<PER, NT_LOAD, NT_STORE><<<grid, 256>>>(src, dst);
  }
  float ms = -1.f;
  if (!ok(hipGetLastError(), "launch") || !ok(hipEventRecord(b, 0), "event") ||
      !ok(hipEventSynchronize(b), "sync") || !ok(hipEventElapsedTime(&ms, a, b), "elapsed"))
    return -1.f;
  return ms / 10;
}

}  // namespace

int main() {
  const size_t bytes = 1ull << 30, n16 = bytes / 16;
  u32x4 *src = nullptr, *dst = nullptr;
  hipEvent_t a, b;
  if (!ok(hipMalloc(&src, bytes), "hipMalloc") || !ok(hipMalloc(&dst, bytes), "hipMalloc") ||
      !ok(hipMemset(src, 1, bytes), "hipMemset") || !ok(hipMemset(dst, 0, bytes), "hipMemset") ||
      !ok(hipEventCreate(&a), "event") || !ok(hipEventCreate(&b), "event") ||
      !ok(hipDeviceSynchronize(), "sync"))
    return 1;
  struct Row {
    const char* name;
    float ms;
  } rows[] = {
      {"kernel_plain_1x16B", time_kernel<1, false, false>(src, dst, n16, a, b)},
      {"kernel_plain_4x16B", time_kernel<4, false, false>(src, dst, n16, a, b)},
      {"kernel_nt_load_4x16B", time_kernel<4, true, false>(src, dst, n16, a, b)},
      {"kernel_nt_store_4x16B", time_kernel<4, false, true>(src, dst, n16, a, b)},
      {"kernel_nt_both_4x16B", time_kernel<4, true, true>(src, dst, n16, a, b)},
      {"kernel_nt_both_1x16B", time_kernel<1, true, true>(src, dst, n16, a, b)},
      {"runtime_memcpy", -1.f},
  };
  // The runtime's device-to-device copy, timed the same way.
  for (int i = 0; i < 13; ++i) {
    if (i == 3 && !ok(hipEventRecord(a, 0), "event")) return 1;
    if (!ok(hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, 0), "hipMemcpyAsync"))
      return 1;
  }
  float ms = -1.f;
  if (!ok(hipEventRecord(b, 0), "event") || !ok(hipEventSynchronize(b), "sync") ||
      !ok(hipEventElapsedTime(&ms, a, b), "elapsed"))
    return 1;
  rows[6].ms = ms / 10;
  std::printf("{\"bytes_each_way\": %zu, \"GB_per_s_read_plus_write\": {", bytes);
  for (int i = 0; i < 7; ++i)
    std::printf("%s\"%s\": %.1f", i ? ", " : "", rows[i].name,
                rows[i].ms > 0 ? 2.0 * bytes / (rows[i].ms * 1e-3) / 1e9 : -1.0);
  std::printf("}}\n");
  hipFree(src);
  hipFree(dst);
  for (int i = 0; i < 7; ++i)
    if (rows[i].ms <= 0) return 1;
  return 0;
}
