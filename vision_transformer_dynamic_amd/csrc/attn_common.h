// Pieces shared by the forward attention kernels and the backward kernels:
// element traits for the two dtypes (MFMA forms, 16-byte operand loads and
// stores), cross-lane-group reductions and the transposed-tile writes.
//
// MFMA operand layout used throughout (16 x 16 output tiles): lane l holds
// output rows 4*(l/16) .. 4*(l/16)+3 of column l % 16; an A operand lane
// supplies row l % 16, a B operand lane column l % 16, and both supply the
// same contraction slots for the same lane group. Only that pairing matters,
// so the code never depends on the hardware's order of slots inside the
// contraction.
#pragma once

#include "bra_internal.h"

namespace bra {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx8 __attribute__((ext_vector_type(8)));

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx2 __attribute__((ext_vector_type(2)));

constexpr int KC = 64;       // keys per chunk
constexpr int D = kHeadDim;  // 32

template <typename T>
struct Tr;

template <>
struct Tr<__bf16> {
  typedef bf16x8 op8;                 // 8 contraction slots per lane
  static constexpr int VEC = 8;       // elements per 16-byte vector
  static constexpr int PADK = 8;      // LDS row padding (elements)
  static constexpr int PADV = 8;
  __device__ static inline floatx4 mma(op8 a, op8 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static inline op8 load8(const __bf16* p) { return *reinterpret_cast<const op8*>(p); }
  // converted in pairs: one v_cvt_pk_bf16_f32 (round to nearest even) per
  // pair, with no repacking of single conversions
  __device__ static inline op8 from_f32(const float* v) {
    op8 r;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const bf16x2 t = __builtin_convertvector(floatx2{v[e], v[e + 1]}, bf16x2);
      r[e] = t[0];
      r[e + 1] = t[1];
    }
    return r;
  }
  // The rounding error of hi = from_f32(v), itself rounded: hi + lo carries
  // about 16 bits of v. The dQ products take dZ this way: dQ = sum_j dZ_j k_j
  // cancels the keys' common part (a query's dZ sum to zero), which would
  // amplify an 8-bit rounding of dZ by |k| / |k - mean k|.
  __device__ static inline op8 residual(const float* v, op8 hi) {
    float r[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = v[e] - (float)hi[e];
    return from_f32(r);
  }
  __device__ static inline op8 zero() {
    op8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (__bf16)0.0f;
    return r;
  }
  __device__ static inline op8 ones() {
    op8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (__bf16)1.0f;
    return r;
  }
  __device__ static inline void store8(__bf16* p, const float* v) {
    *reinterpret_cast<op8*>(p) = from_f32(v);
  }
  // non-temporal: the attention output is not read again by the kernel, and
  // the hint keeps it from piling up as dirty lines in L2
  __device__ static inline void store8_nt(__bf16* p, const float* v) {
    __builtin_nontemporal_store(from_f32(v), reinterpret_cast<op8*>(p));
  }
  // 16-deep contraction: 4 slots per lane
  typedef shortx4 op4;
  __device__ static inline floatx4 mma16(op4 a, op4 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
  }
  __device__ static inline op4 from_f32_4(const float* v) {
    bf16x4 r;
#pragma unroll
    for (int e = 0; e < 4; e += 2) {
      const bf16x2 t = __builtin_convertvector(floatx2{v[e], v[e + 1]}, bf16x2);
      r[e] = t[0];
      r[e + 1] = t[1];
    }
    return __builtin_bit_cast(op4, r);
  }
  __device__ static inline op4 load4(const __bf16* p) { return *reinterpret_cast<const op4*>(p); }
};

template <>
struct Tr<float> {
  typedef floatx8 op8;
  static constexpr int VEC = 4;
  static constexpr int PADK = 4;
  static constexpr int PADV = 4;
  __device__ static inline floatx4 mma(op8 a, op8 b, floatx4 c) {
#pragma unroll
    for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], c, 0, 0, 0);
    return c;
  }
  __device__ static inline op8 load8(const float* p) {
    const float4 lo = *reinterpret_cast<const float4*>(p);
    const float4 hi = *reinterpret_cast<const float4*>(p + 4);
    op8 r;
    r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
    r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
    return r;
  }
  __device__ static inline op8 from_f32(const float* v) {
    op8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = v[e];
    return r;
  }
  __device__ static inline op8 zero() {
    op8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = 0.f;
    return r;
  }
  __device__ static inline op8 ones() {
    op8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = 1.f;
    return r;
  }
  __device__ static inline void store8(float* p, const float* v) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
  __device__ static inline void store8_nt(float* p, const float* v) {
    __builtin_nontemporal_store(floatx4{v[0], v[1], v[2], v[3]}, reinterpret_cast<floatx4*>(p));
    __builtin_nontemporal_store(floatx4{v[4], v[5], v[6], v[7]}, reinterpret_cast<floatx4*>(p + 4));
  }
  typedef floatx4 op4;
  __device__ static inline floatx4 mma16(op4 a, op4 b, floatx4 c) {
#pragma unroll
    for (int e = 0; e < 4; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], c, 0, 0, 0);
    return c;
  }
  __device__ static inline op4 from_f32_4(const float* v) { return op4{v[0], v[1], v[2], v[3]}; }
  __device__ static inline op4 load4(const float* p) {
    const float4 x = *reinterpret_cast<const float4*>(p);
    return op4{x.x, x.y, x.z, x.w};
  }
};

// Cross-lane-group exchanges without LDS: v_permlane16_swap with both
// operands equal leaves {v[lane], v[lane ^ 16]} in the lane's two results,
// and v_permlane32_swap {v[lane], v[lane ^ 32]}. The two values are combined
// by a commutative operation, so the order in which the lane receives them
// does not matter and every lane of a group gets the same bits.
__device__ inline float xor16_pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float xor32_pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float xor16_pair_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ inline float xor32_pair_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Max over the 4 lane groups that share lane % 16.
__device__ inline float wave_max_groups(float v) { return xor32_pair_max(xor16_pair_max(v)); }

// Channel-row swizzle of the V^T tile: column blocks of 8 keys are permuted
// by an XOR that depends on the row's 8-row group, so the transposed writes of
// one wave spread over the LDS banks. Blocks of 8 keys stay contiguous (and
// even columns stay even), which is what the P.V operand reads and the packed
// key-pair writes need.
__device__ inline int vt_col(int row, int col) { return col ^ (((row >> 3) & 7) << 3); }

// Two keys' 16-byte vectors -> per channel e, the pair (key0, key1) as one
// 32-bit (bf16) or 64-bit (fp32) LDS word of the V^T tile.
__device__ inline void store_vt_pair(__bf16* Vt, int ldv, int row0, int col, const uint4& a, const uint4& b) {
  const uint32_t wa[4] = {a.x, a.y, a.z, a.w};
  const uint32_t wb[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t lo = (wa[e] & 0xffffu) | (wb[e] << 16);          // channel 2e
    const uint32_t hi = (wa[e] >> 16) | (wb[e] & 0xffff0000u);      // channel 2e+1
    *reinterpret_cast<uint32_t*>(Vt + (row0 + 2 * e) * ldv + col) = lo;
    *reinterpret_cast<uint32_t*>(Vt + (row0 + 2 * e + 1) * ldv + col) = hi;
  }
}

__device__ inline void store_vt_pair(float* Vt, int ldv, int row0, int col, const uint4& a, const uint4& b) {
  const uint32_t wa[4] = {a.x, a.y, a.z, a.w};
  const uint32_t wb[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
  for (int e = 0; e < 4; ++e)
    *reinterpret_cast<uint2*>(Vt + (row0 + e) * ldv + col) = make_uint2(wa[e], wb[e]);
}

// Whole-row exchange buffers ([row][8 chunks of 16 bytes], two heads' halves
// of 128-byte output rows): chunk c of row r sits at chunk c ^ (r % 8). The
// 16 lanes of a group writing one chunk of 16 consecutive rows then meet no
// LDS bank conflict; unswizzled, the 128-byte row stride puts them on the
// same banks (about 68 conflict cycles a write on gfx950, measured with
// SQ_LDS_BANK_CONFLICT).
__device__ inline int xrow_at(int row, int chunk) { return row * 8 + (chunk ^ (row & 7)); }

// Sum over the 4 lane groups that share lane % 16, as (g0 + g1) + (g2 + g3).
__device__ inline float wave_sum_groups(float v) { return xor32_pair_sum(xor16_pair_sum(v)); }

}  // namespace bra
