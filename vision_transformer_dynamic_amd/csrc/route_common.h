// Routing arithmetic: region affinity A[i][j] = Q^r[i,:] . K^r[j,:] in a
// fixed order, and the top-k tie rule (explainer "BiFormer Reshapes Visual
// Attention with 'Bi-Level Routing'", Part 2.2 pseudocode steps 4-5).
//
// Matrix-core form (route kernel for up to 64 regions): a 16 x 16 tile of A
// over one half of the channels is the sequence of affinity_mfma_step over
// the half's 16-channel steps in increasing order from a zero accumulator;
// the two halves are then added, half 0 + half 1. An output element of the
// product depends only on its own query-row and candidate-row operands, so
// any kernel that puts the same rows anywhere in a tile gets the same bits.
//
// Vector form (route kernel otherwise): four fused multiply-add chains.
#pragma once

#include <hip/hip_runtime.h>

namespace bra {

typedef float floatx4 __attribute__((ext_vector_type(4)));

// One 16-channel step of a 16 x 16 affinity tile: the A lane supplies 4
// channels of its query row, the B lane the same 4 channels of its candidate
// row; four 16x16x4 fp32 products in component order.
__device__ inline floatx4 affinity_mfma_step(floatx4 acc, const float4 a, const float4 k) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, k.x, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, k.y, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, k.z, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, k.w, acc, 0, 0, 0);
  return acc;
}

// Order-preserving key of candidate j (0 <= j < 2^16) with affinity a: a
// larger key beats a smaller one exactly when the affinity is larger, or
// equal with a lower index. -0 is folded into +0 first, so zeros tie as they
// compare. Every bit pattern, NaN included, maps to a distinct key per j, so
// the keys of a row are a strict total order and every rank is unique (a NaN
// with the sign bit clear ranks above +inf, one with it set below -inf).
// A key is never 0, which marks candidates past the last region.
__device__ inline uint64_t affinity_key(float a, int j) {
  uint32_t u = __float_as_uint(a == 0.f ? 0.f : a);
  u = (u >> 31) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)j);
}

// Candidate index of a key made by affinity_key.
__device__ inline int key_index(uint64_t key) { return (int)(0xFFFFFFFFu - (uint32_t)key); }

// the larger of a and the key with halves (lo, hi)
__device__ inline uint64_t key_max(uint64_t a, uint32_t lo, uint32_t hi) {
  const uint64_t b = ((uint64_t)hi << 32) | lo;
  return b > a ? b : a;
}

// Largest key over the 64 lanes, in every lane: DPP within rows of 16 (swap
// neighbours, swap pairs, rotate by 4, rotate by 8), then the permlane swaps
// across rows. max is exact, so the order of combination does not matter.
__device__ inline uint64_t wave_max_key(uint64_t v) {
#define BRA_KEY_DPP(ctrl)                                                                         \
  v = key_max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)v, ctrl, 0xF, 0xF, false),      \
              (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(v >> 32), ctrl, 0xF, 0xF, false))
  BRA_KEY_DPP(0xB1);   // quad_perm 1,0,3,2
  BRA_KEY_DPP(0x4E);   // quad_perm 2,3,0,1
  BRA_KEY_DPP(0x124);  // row_ror:4
  BRA_KEY_DPP(0x128);  // row_ror:8
#undef BRA_KEY_DPP
  {
    const auto lo = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
    const auto hi = __builtin_amdgcn_permlane16_swap((uint32_t)(v >> 32), (uint32_t)(v >> 32), false, false);
    v = key_max(key_max(v, lo[0], hi[0]), lo[1], hi[1]);
  }
  {
    const auto lo = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
    const auto hi = __builtin_amdgcn_permlane32_swap((uint32_t)(v >> 32), (uint32_t)(v >> 32), false, false);
    v = key_max(key_max(v, lo[0], hi[0]), lo[1], hi[1]);
  }
  return v;
}

// Largest 32-bit value over the 64 lanes, in every lane (the same steps as
// wave_max_key on one word).
__device__ inline uint32_t wave_max_u32(uint32_t v) {
#define BRA_U32_DPP(ctrl) v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, ctrl, 0xF, 0xF, false))
  BRA_U32_DPP(0xB1);   // quad_perm 1,0,3,2
  BRA_U32_DPP(0x4E);   // quad_perm 2,3,0,1
  BRA_U32_DPP(0x124);  // row_ror:4
  BRA_U32_DPP(0x128);  // row_ror:8
#undef BRA_U32_DPP
  {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = max(max(v, (uint32_t)r[0]), (uint32_t)r[1]);
  }
  {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    v = max(max(v, (uint32_t)r[0]), (uint32_t)r[1]);
  }
  return v;
}

// Rank of key kj among the 64 keys of a row held in LDS (16-byte aligned):
// how many beat it. All 8 broadcast reads of a 16-key block are issued before
// its compares.
__device__ inline int key_rank64(const uint64_t* keys, uint64_t kj) {
  int rank = 0;
#pragma unroll
  for (int m0 = 0; m0 < 64; m0 += 16) {
    ulonglong2 km[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) km[e] = *reinterpret_cast<const ulonglong2*>(keys + m0 + 2 * e);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      rank += km[e].x > kj;
      rank += km[e].y > kj;
    }
  }
  return rank;
}

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

// Rank of key kj among the keys keys[0..ldr) of a row in LDS (16-byte
// aligned, ldr a multiple of 2, entries past the last region 0): how many
// beat it.
__device__ inline int key_rank(const uint64_t* keys, int ldr, uint64_t kj) {
  int rank = 0;
  for (int m = 0; m < ldr; m += 2) {
    const ulonglong2 km = *reinterpret_cast<const ulonglong2*>(keys + m);
    rank += km.x > kj;
    rank += km.y > kj;
  }
  return rank;
}

}  // namespace bra
