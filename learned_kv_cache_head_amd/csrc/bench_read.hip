// Read-only bandwidth reference for the benchmark (libkvebench.so; not part
// of libkvevict's interface). Streams a device buffer once with the load
// form the decode attention uses for its K/V rows (16-byte non-temporal
// loads, several in flight per lane) and writes nothing but one word per
// workgroup, so its rate is the read ceiling the attention kernel can be
// held against.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kDepth = 4;                              // loads in flight per lane
constexpr size_t kStep = (size_t)kThreads * 16 * kDepth;  // bytes per sweep
constexpr size_t kSpan = 64 * kStep;                   // bytes per workgroup

// Workgroup g reads bytes [g * kSpan, min((g + 1) * kSpan, n16 * 16)).
__global__ __launch_bounds__(kThreads) void read_kernel(const u32x4* p,
                                                        size_t n16,
                                                        uint32_t* sink) {
  const size_t first = (size_t)blockIdx.x * (kSpan / 16);
  const size_t last = first + kSpan / 16 < n16 ? first + kSpan / 16 : n16;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (size_t base = first + threadIdx.x; base < last;
       base += (size_t)kThreads * kDepth) {
    u32x4 t[kDepth];
#pragma unroll
    for (int u = 0; u < kDepth; ++u) {
      size_t i = base + (size_t)u * kThreads;
      i = i < last ? i : last - 1;  // clamp: every load stays in bounds
      t[u] = __builtin_nontemporal_load(p + i);
    }
#pragma unroll
    for (int u = 0; u < kDepth; ++u) acc ^= t[u];
  }
  // One word per workgroup keeps the loads live.
  const uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (threadIdx.x == 0) sink[blockIdx.x] = x;
}

}  // namespace

extern "C" {

// Workgroups (and sink words) a read of `bytes` launches.
size_t kvebench_read_blocks(size_t bytes) {
  return (bytes / 16 + kSpan / 16 - 1) / (kSpan / 16);
}

// Reads bytes (a multiple of 16, 16-byte aligned) at p on stream; sink holds
// kvebench_read_blocks(bytes) uint32 words. Returns 0 on success.
int kvebench_read(const void* p, size_t bytes, uint32_t* sink,
                  hipStream_t stream) {
  if (!p || !sink || bytes < 16 || bytes % 16 != 0 ||
      ((uintptr_t)p & 15u) != 0)
    return 1;
  const size_t blocks = kvebench_read_blocks(bytes);
  if (blocks > 0x7fffffffu) return 1;
  hipLaunchKernelGGL(read_kernel, dim3((unsigned)blocks), dim3(kThreads), 0,
                     stream, (const u32x4*)p, bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
