// Region affinity fused with top-k routing (explainer "BiFormer Reshapes
// Visual Attention with 'Bi-Level Routing'", Part 2.2 step 3, pseudocode
// steps 4-5; paper summary "BiFormer: Vision Transformer with Bi-Level
// Routing Attention", Section 3: row i of the routing index holds the k
// regions most relevant to region i).
//
// One wavefront per affinity row (image b, query region i). Lane j holds the
// candidates j, j+64, j+128, j+192 (at most 256 regions); each computes
// A[i][j] = Q^r[b,i,:] . K^r[b,j,:] in fp32 with fused multiply-adds in
// increasing channel order. The row never leaves registers: topk rounds of a
// wave-wide arg-max (butterfly over 64 lanes) pick, in turn, the largest
// remaining affinity, the lower index winning exact ties. Every lane ends each
// round with the same winner, so the result is deterministic.
#include "bra_internal.h"

#include <math.h>

namespace bra {
namespace {

struct RouteParams {
  const float* Qr;
  const float* Kr;
  int32_t* idx;
  int R, C, topk;
  int row_blocks;  // ceil(R / 4): workgroups per image
};

// (v, j) ranks above (bv, bj): larger value, or equal value and lower index.
__device__ inline bool better(float v, int j, float bv, int bj) {
  return v > bv || (v == bv && j < bj);
}

__global__ __launch_bounds__(256) void route_kernel(RouteParams p) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.x / p.row_blocks;
  const int i = (blockIdx.x - b * p.row_blocks) * 4 + wave;
  if (i >= p.R) return;  // the whole wave leaves; no barrier below

  const float* q = p.Qr + ((int64_t)b * p.R + i) * p.C;
  const float* kb = p.Kr + (int64_t)b * p.R * p.C;

  float a[4];
  uint32_t taken = 0;  // bit u: candidate lane + 64u is used or absent
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int j = lane + 64 * u;
    a[u] = -INFINITY;
    if (j < p.R) {
      const float4* kr = reinterpret_cast<const float4*>(kb + (int64_t)j * p.C);
      const float4* qr = reinterpret_cast<const float4*>(q);
      float acc = 0.f;
      for (int c = 0; c < (p.C >> 2); ++c) {
        const float4 kv = kr[c];
        const float4 qv = qr[c];
        acc = __builtin_fmaf(qv.x, kv.x, acc);
        acc = __builtin_fmaf(qv.y, kv.y, acc);
        acc = __builtin_fmaf(qv.z, kv.z, acc);
        acc = __builtin_fmaf(qv.w, kv.w, acc);
      }
      a[u] = acc;
    } else {
      taken |= 1u << u;
    }
  }

  int32_t* out = p.idx + ((int64_t)b * p.R + i) * p.topk;
  for (int round = 0; round < p.topk; ++round) {
    float bv = -INFINITY;
    int bj = 0x7fffffff;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (!(taken & (1u << u)) && better(a[u], lane + 64 * u, bv, bj)) {
        bv = a[u];
        bj = lane + 64 * u;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off, 64);
      const int oj = __shfl_xor(bj, off, 64);
      if (better(ov, oj, bv, bj)) {
        bv = ov;
        bj = oj;
      }
    }
    if (lane == 0) out[round] = bj;
    if ((bj & 63) == lane && bj < 256) taken |= 1u << (bj >> 6);
  }
}

}  // namespace

hipError_t launch_route(const float* Qr, const float* Kr, int32_t* idx,
                        const Shape& s, hipStream_t stream) {
  RouteParams p{Qr, Kr, idx, s.R, s.C, s.topk, (s.R + 3) / 4};
  dim3 grid((unsigned)(s.B * p.row_blocks));
  void* args[] = {&p};
  return hipLaunchKernel(reinterpret_cast<const void*>(&route_kernel), grid, dim3(256), args, 0, stream);
}

}  // namespace bra
