// Reference kernels for the benchmark (libkvebench.so; not part of
// libkvevict's interface).
//
// Read ceiling: streams a device buffer once with the load form the decode
// attention uses for its K/V rows (16-byte non-temporal loads, several in
// flight per lane) and writes nothing but one word per workgroup, so its
// rate is the read ceiling the attention kernel can be held against.
//
// Issue probe: how far MFMAs and vector ALU instructions overlap on one
// SIMD, the question that bounds a kernel which, like the masked prefill
// attention, alternates matrix products with per-element softmax arithmetic.
// Workgroups of 8 waves; waves w and w + 4 of a workgroup share a SIMD.
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

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Per iteration, a wave running MFMAs issues 8 independent
// v_mfma_f32_16x16x32_bf16; a wave running vector work issues 32 float32
// FMAs, or 32 v_exp_f32, over 8 independent chains. MODE bits: 1 waves 0-3
// run the MFMAs, 2 waves 4-7 run the vector work, 4 waves 0-3 run the vector
// work as well (in the same wave as their MFMAs), 8 the vector work is exp2.
template <int MODE>
__global__ __launch_bounds__(512) void issue_kernel(float* out, int iters) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool mfma = (MODE & 1) && wave < 4;
  const bool valu = ((MODE & 2) && wave >= 4) || ((MODE & 4) && wave < 4);
  bf16x8_t a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(threadIdx.x * 0.001f + i);
    b[i] = (__bf16)(i * 0.5f);
  }
  f32x4_t acc[8];
  float x[8];
  for (int i = 0; i < 8; ++i) {
    acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    x[i] = threadIdx.x * 1e-3f + i;
  }
  for (int it = 0; it < iters; ++it) {
    if (mfma) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[i], 0, 0, 0);
    }
    if (valu) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int i = 0; i < 8; ++i)
          x[i] = (MODE & 8) ? __builtin_amdgcn_exp2f(x[i]) * -0.5f
                            : fmaf(x[i], 0.999f, 0.001f);
    }
  }
  float r = 0.f;
  for (int i = 0; i < 8; ++i) r += acc[i][0] + acc[i][3] + x[i];
  out[(size_t)blockIdx.x * 512 + threadIdx.x] = r;
}

}  // namespace

extern "C" {

// Launches the issue probe in mode `mode` (1, 2, 3, 5, 10, 11 or 13; bits
// as above) over `blocks` workgroups of 512 threads, `iters` iterations;
// out holds blocks * 512 floats. Returns 0 on success.
int kvebench_issue(int mode, int blocks, int iters, float* out,
                   hipStream_t stream) {
  if (!out || blocks <= 0 || iters <= 0) return 1;
#define KVB_ISSUE(M)                                                        \
  if (mode == M) {                                                          \
    hipLaunchKernelGGL(issue_kernel<M>, dim3(blocks), dim3(512), 0, stream, \
                       out, iters);                                         \
    return hipGetLastError() == hipSuccess ? 0 : 2;                         \
  }
  KVB_ISSUE(1) KVB_ISSUE(2) KVB_ISSUE(3) KVB_ISSUE(5) KVB_ISSUE(10)
  KVB_ISSUE(11) KVB_ISSUE(13)
#undef KVB_ISSUE
  return 1;
}


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
