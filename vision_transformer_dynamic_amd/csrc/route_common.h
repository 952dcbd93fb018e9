// Routing arithmetic of the vector form of the route kernel: region affinity
// A[i][j] = Q^r[i,:] . K^r[j,:] in one fixed order, and the top-k tie rule
// (explainer "BiFormer Reshapes Visual Attention with 'Bi-Level Routing'",
// Part 2.2 pseudocode steps 4-5).
#pragma once

#include <hip/hip_runtime.h>

namespace bra {

// One 4-channel step of the affinity dot product. The product is accumulated
// as four fused multiply-add chains, one per channel residue mod 4, in
// increasing channel order.
__device__ inline float4 affinity_step(float4 acc, const float4 q, const float4 k) {
  acc.x = __builtin_fmaf(q.x, k.x, acc.x);
  acc.y = __builtin_fmaf(q.y, k.y, acc.y);
  acc.z = __builtin_fmaf(q.z, k.z, acc.z);
  acc.w = __builtin_fmaf(q.w, k.w, acc.w);
  return acc;
}

// The four chains combined in a fixed order.
__device__ inline float affinity_finish(const float4 acc) {
  return (acc.x + acc.y) + (acc.z + acc.w);
}

// Number of candidates among a[0..ldr) that rank above candidate j with
// affinity aj: m ranks above j when a[m] > aj, or a[m] == aj and m < j (a
// strict total order, so ranks are unique). Entries past the last region must
// hold -inf; a is 16-byte aligned and ldr a multiple of 4.
__device__ inline int affinity_rank(const float* a, int ldr, float aj, int j) {
  int rank = 0;
  for (int m = 0; m < ldr; m += 4) {
    const float4 am = *reinterpret_cast<const float4*>(a + m);
    rank += (am.x > aj) || (am.x == aj && m + 0 < j);
    rank += (am.y > aj) || (am.y == aj && m + 1 < j);
    rank += (am.z > aj) || (am.z == aj && m + 2 < j);
    rank += (am.w > aj) || (am.w == aj && m + 3 < j);
  }
  return rank;
}

}  // namespace bra
