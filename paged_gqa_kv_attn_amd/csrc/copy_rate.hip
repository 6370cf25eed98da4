// copy_rate.hip — the copy and read rates this part reaches: the ceiling for kernels that read each
// byte once and write each result once (the appends), and for kernels that only stream their inputs
// (attention over a KV cache). Buffers of 1 GiB (or the size given in MiB): copied device to device
// by hand-written copy kernels with and without the non-temporal hint on loads and stores, and by
// the runtime's own copy; then read by a grid that covers the buffer once and by fixed grids of 1,
// 2 or 4 workgroups per CU that each stream a contiguous chunk with 8 or 16 loads per lane in
// flight. A standalone program (not part of the library); it prints one JSON line.
//
// Copy and one-pass read: thread t of workgroup w takes the 16-byte vectors (w * PER + k) * 256 + t,
// k < PER; the grid covers exactly n16 vectors, which the host checks (n16 % (256 * PER) == 0)
// before any launch. Streamed read: workgroup w takes the vectors [w * chunk, (w + 1) * chunk),
// chunk a multiple of 256 * UN with grid * chunk <= n16 (the host floors it), in rounds of UN
// vectors per lane. The read kernels add what they load and store the sum only when it equals a
// value the fill (bytes of 0x01) cannot produce, so every load stays live and nothing is written.

#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

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

constexpr unsigned kNever = 0x9e3779b9u;  // no sum of 0x01010101 words reaches it below 2^20 terms

template <int PER, bool NT>
__global__ __launch_bounds__(256) void read_kernel(const u32x4* __restrict__ src,
                                                   u32x4* __restrict__ dst) {
  const size_t base = (size_t)blockIdx.x * PER * 256 + threadIdx.x;
  u32x4 v[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k)
    v[k] = NT ? __builtin_nontemporal_load(src + base + k * 256) : src[base + k * 256];
  __builtin_amdgcn_sched_barrier(0);
  u32x4 acc = v[0];
#pragma unroll
  for (int k = 1; k < PER; ++k) acc += v[k];
  if (acc.x == kNever) dst[base] = acc;
}

template <int UN>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src,
                                                          u32x4* __restrict__ dst, size_t chunk) {
  const u32x4* p = src + (size_t)blockIdx.x * chunk + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (size_t done = 0; done < chunk; done += UN * 256) {
    u32x4 v[UN];
#pragma unroll
    for (int k = 0; k < UN; ++k) v[k] = __builtin_nontemporal_load(p + done + k * 256);
    __builtin_amdgcn_sched_barrier(0);  // every load of the round issued before the first add
#pragma unroll
    for (int k = 0; k < UN; ++k) acc += v[k];
  }
  if (acc.x == kNever) dst[(size_t)blockIdx.x * 256 + threadIdx.x] = acc;
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

template <int PER, bool NT>
float time_read(const u32x4* src, u32x4* dst, size_t n16, hipEvent_t a, hipEvent_t b) {
  if (n16 % (256 * PER) != 0) return -1.f;
  const dim3 grid((unsigned)(n16 / (256 * PER)));
  for (int i = 0; i < 13; ++i) {
    if (i == 3 && !ok(hipEventRecord(a, 0), "event")) return -1.f;
    read_kernel<PER, NT><<<grid, 256>>>(src, dst);
  }
  float ms = -1.f;
  if (!ok(hipGetLastError(), "launch") || !ok(hipEventRecord(b, 0), "event") ||
      !ok(hipEventSynchronize(b), "sync") || !ok(hipEventElapsedTime(&ms, a, b), "elapsed"))
    return -1.f;
  return ms / 10;
}

// Mean milliseconds per streamed read of *bytes (grid * chunk vectors) by `workgroups` workgroups.
template <int UN>
float time_stream(const u32x4* src, u32x4* dst, size_t n16, int workgroups, hipEvent_t a,
                  hipEvent_t b, size_t* bytes) {
  *bytes = 0;
  if (workgroups <= 0) return -1.f;
  const size_t chunk = n16 / workgroups / (256 * UN) * (256 * UN);
  // dst takes one vector per lane of the grid; it holds n16 vectors.
  if (chunk == 0 || (size_t)workgroups * 256 > n16) return -1.f;
  for (int i = 0; i < 13; ++i) {
    if (i == 3 && !ok(hipEventRecord(a, 0), "event")) return -1.f;
    stream_read_kernel<UN><<<dim3(workgroups), 256>>>(src, dst, chunk);
  }
  float ms = -1.f;
  if (!ok(hipGetLastError(), "launch") || !ok(hipEventRecord(b, 0), "event") ||
      !ok(hipEventSynchronize(b), "sync") || !ok(hipEventElapsedTime(&ms, a, b), "elapsed"))
    return -1.f;
  *bytes = (size_t)workgroups * chunk * 16;
  return ms / 10;
}

}  // namespace

// Usage: copy_rate [MiB] — the size of each buffer (default 1024, at most 16384).
int main(int argc, char** argv) {
  long mib = 1024;
  if (argc > 1) {
    char* end = nullptr;
    mib = std::strtol(argv[1], &end, 10);
    if (end == argv[1] || *end != '\0' || mib < 1 || mib > 16384) {
      std::fprintf(stderr, "copy_rate: size must be 1-16384 MiB, got '%s'\n", argv[1]);
      return 2;
    }
  }
  const size_t bytes = (size_t)mib << 20, n16 = bytes / 16;
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
  std::printf("}, ");
  int cus = 0;
  if (!ok(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0), "attribute"))
    return 1;
  struct ReadRow {
    const char* name;
    float ms;
    size_t bytes;
  } reads[9] = {
      {"one_pass_plain_1x16B", time_read<1, false>(src, dst, n16, a, b), bytes},
      {"one_pass_plain_4x16B", time_read<4, false>(src, dst, n16, a, b), bytes},
      {"one_pass_nt_1x16B", time_read<1, true>(src, dst, n16, a, b), bytes},
      {"one_pass_nt_4x16B", time_read<4, true>(src, dst, n16, a, b), bytes},
      {"stream_1wg_per_cu_8x16B", -1.f, 0},
      {"stream_1wg_per_cu_16x16B", -1.f, 0},
      {"stream_2wg_per_cu_8x16B", -1.f, 0},
      {"stream_4wg_per_cu_8x16B", -1.f, 0},
      {"stream_4wg_per_cu_16x16B", -1.f, 0},
  };
  reads[4].ms = time_stream<8>(src, dst, n16, cus, a, b, &reads[4].bytes);
  reads[5].ms = time_stream<16>(src, dst, n16, cus, a, b, &reads[5].bytes);
  reads[6].ms = time_stream<8>(src, dst, n16, 2 * cus, a, b, &reads[6].bytes);
  reads[7].ms = time_stream<8>(src, dst, n16, 4 * cus, a, b, &reads[7].bytes);
  reads[8].ms = time_stream<16>(src, dst, n16, 4 * cus, a, b, &reads[8].bytes);
  std::printf("\"cus\": %d, \"GB_per_s_read_only\": {", cus);
  for (int i = 0; i < 9; ++i)
    std::printf("%s\"%s\": %.1f", i ? ", " : "", reads[i].name,
                reads[i].ms > 0 ? reads[i].bytes / (reads[i].ms * 1e-3) / 1e9 : -1.0);
  std::printf("}}\n");
  hipFree(src);
  hipFree(dst);
  for (int i = 0; i < 7; ++i)
    if (rows[i].ms <= 0) return 1;
  for (int i = 0; i < 9; ++i)
    if (reads[i].ms <= 0) return 1;
  return 0;
}
