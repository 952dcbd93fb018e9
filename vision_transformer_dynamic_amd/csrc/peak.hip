// Achievable-peak probes for the benchmark, built into a library of their own
// (libbra_peak.so), beside the operator's library: the rate a plain bf16
// matrix-core loop and a plain streaming copy reach on the part, against
// which the kernels' rates are read next to the published peaks.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kChains = 8;  // independent accumulators per wave (covers the MFMA latency)

// Every wave issues iters * kChains v_mfma_f32_16x16x32_bf16 (16 * 16 * 32
// multiply-adds each) on operands built from its lane index, and writes one
// sum per lane so that nothing is optimised away.
__global__ __launch_bounds__(256) void mfma_loop_kernel(float* out, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(0.001f * (float)((lane + e) & 7));
    b[e] = (__bf16)(0.002f * (float)((lane * 3 + e) & 7));
  }
  floatx4 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = floatx4{0.f, 0.f, 0.f, (float)c};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// dst = src, 16-byte vectors, four per thread, all loads before any store.
__global__ __launch_bounds__(256) void copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst, size_t n) {
  const size_t base = (size_t)blockIdx.x * (256 * 4) + threadIdx.x;
  uint4 v[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const size_t i = base + 256 * m;
    if (i < n) v[m] = src[i];
  }
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const size_t i = base + 256 * m;
    if (i < n) dst[i] = v[m];
  }
}

}  // namespace

extern "C" {

// Flops of one bra_peak_mfma launch with these arguments.
double bra_peak_mfma_flops(int blocks, int iters) {
  return 2.0 * 16 * 16 * 32 * (double)kChains * iters * 4 /* waves */ * blocks;
}

// Launch the matrix-core loop: `blocks` workgroups of 4 waves; out holds
// blocks * 256 floats. Returns the HIP status of the launch.
int bra_peak_mfma(float* out, int blocks, int iters, hipStream_t stream) {
  if (out == nullptr || blocks <= 0 || iters <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(blocks), dim3(256), 0, stream, out, iters);
  return (int)hipGetLastError();
}

// Copy `bytes` (a multiple of 16; both pointers 16-byte aligned) from src to dst.
int bra_peak_copy(const void* src, void* dst, size_t bytes, hipStream_t stream) {
  if (src == nullptr || dst == nullptr || bytes % 16 != 0 || (uintptr_t)src % 16 || (uintptr_t)dst % 16)
    return (int)hipErrorInvalidValue;
  const size_t n = bytes / 16;
  const size_t grid = (n + 1023) / 1024;
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)grid), dim3(256), 0, stream, static_cast<const uint4*>(src),
                     static_cast<uint4*>(dst), n);
  return (int)hipGetLastError();
}

}  // extern "C"
