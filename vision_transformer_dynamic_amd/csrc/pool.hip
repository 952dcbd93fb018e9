// Region mean-pool: Q^r[b, r, :] and K^r[b, r, :] = mean of Q and K over the
// tokens of region r (explainer "BiFormer Reshapes Visual Attention with
// 'Bi-Level Routing'", Part 2.2 step 3 and pseudocode step 3; paper summary
// "BiFormer: Vision Transformer with Bi-Level Routing Attention", Section 6,
// regional representations by average pooling).
//
// HBM-bound: every input byte is read once, 2*B*R*C fp32 values are written.
// Small bf16 regions take one wave per region (pool_wave_kernel below).
// Otherwise one workgroup per (image, region) pools both Q and K; an image's regions
// go to one XCD (xcd_item), as in the route and attention kernels. (One wave
// per region with a lane-shuffle reduction measured slower at the stage-1
// shape.) A region is sh rows of one contiguous segment of sw*C elements,
// read as 16-byte vectors; every
// thread issues all of its loads (up to NL per tensor) before it adds any, so
// a workgroup has its whole region in flight at once. The block size is a
// multiple of the number of 16-byte channel groups per token, so a thread
// always accumulates the same 8 (bf16) or 4 (fp32) channels; the per-thread
// sums are then reduced across threads through LDS in a fixed order
// (deterministic, fp32 throughout).
#include "bra_internal.h"

namespace bra {
namespace {

constexpr int NL = 4;  // loads per tensor per thread per batch

struct PoolParams {
  const void* Q;
  const void* K;
  float* Qr;
  float* Kr;
  int H, W, C, S, sh, sw;
  int nregions;  // B * S * S
};

template <int VEC>
__device__ inline void accum16(float* acc, const uint4 v);

// bf16: 8 values per 16 bytes; a bf16 is the high half of an fp32.
template <>
__device__ inline void accum16<8>(float* acc, const uint4 v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    acc[2 * e] += __uint_as_float(w[e] << 16);
    acc[2 * e + 1] += __uint_as_float(w[e] & 0xffff0000u);
  }
}

// fp32: 4 values per 16 bytes.
template <>
__device__ inline void accum16<4>(float* acc, const uint4 v) {
  acc[0] += __uint_as_float(v.x);
  acc[1] += __uint_as_float(v.y);
  acc[2] += __uint_as_float(v.z);
  acc[3] += __uint_as_float(v.w);
}

template <int ESIZE>
__global__ __launch_bounds__(256) void pool_kernel(PoolParams p) {
  constexpr int VEC = 16 / ESIZE;  // elements per 16-byte vector
  // per-thread partial sums of Q and K, sized to the launched block (dynamic
  // LDS), so the LDS does not cap how many workgroups a CU holds
  extern __shared__ float red[];  // [2][blockDim.x * VEC]

  const int R = p.S * p.S;
  const int w = xcd_item(blockIdx.x, gridDim.x);
  const int b = w / R;
  const int r = w - b * R;

  const int G = p.C / VEC;                // 16-byte channel groups per token
  const int nthr = (blockDim.x / G) * G;  // active threads, multiple of G
  const int t = threadIdx.x;
  const int segv = p.sw * G;              // vectors per region row segment
  const int total = p.sh * segv;

  float acc[2][VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[0][e] = acc[1][e] = 0.f;
  if (t < nthr) {
    const int y0 = (r / p.S) * p.sh;
    const int x0 = (r - (r / p.S) * p.S) * p.sw;
    const int64_t row_elems = (int64_t)p.W * p.C;
    const int64_t base = (((int64_t)b * p.H + y0) * p.W + x0) * p.C;
    const char* Qb = static_cast<const char*>(p.Q) + base * ESIZE;
    const char* Kb = static_cast<const char*>(p.K) + base * ESIZE;
    for (int f0 = t; f0 < total; f0 += nthr * NL) {
      uint4 vq[NL], vk[NL];
#pragma unroll
      for (int m = 0; m < NL; ++m) {
        const int f = f0 + m * nthr;
        if (f < total) {
          const int y = f / segv;
          const int64_t off = (y * row_elems + (int64_t)(f - y * segv) * VEC) * ESIZE;
          vq[m] = *reinterpret_cast<const uint4*>(Qb + off);
          vk[m] = *reinterpret_cast<const uint4*>(Kb + off);
        }
      }
#pragma unroll
      for (int m = 0; m < NL; ++m) {
        if (f0 + m * nthr < total) {
          accum16<VEC>(acc[0], vq[m]);
          accum16<VEC>(acc[1], vk[m]);
        }
      }
    }
  }
  float* redq = red;
  float* redk = red + blockDim.x * VEC;
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    redq[t * VEC + e] = acc[0][e];
    redk[t * VEC + e] = acc[1][e];
  }
  __syncthreads();

  // thread t's channel group is t % G, so channel c = g*VEC + e sums
  // red[(g + j*G)*VEC + e] over j, in increasing j.
  const float inv_n = 1.0f / (float)(p.sh * p.sw);
  for (int c = t; c < 2 * p.C; c += blockDim.x) {
    const int which = c >= p.C;
    const int cc = c - which * p.C;
    const int g = cc / VEC;
    const int e = cc - g * VEC;
    float s = 0.f;
    const float* part = which ? redk : redq;
    for (int u = g; u < nthr; u += G) s += part[u * VEC + e];
    float* out = which ? p.Kr : p.Qr;
    out[((int64_t)b * R + r) * p.C + cc] = s * inv_n;
  }
}

// ---- small regions: one wave per region, four regions per workgroup ----
// For bf16 regions of at most 256 / G tokens (G = C / 8 channel groups of
// 16 bytes: the 28 x 28 and 14 x 14 stage maps), the per-region workgroups
// above are mostly launch and reduction overhead. Here lane l owns channel
// group g = l % G and the region's tokens l / G, l / G + 64 / G, ... (at most
// NB per tensor, all loaded before any is added), and the 64 / G lanes of a
// group are combined by exchanges across lane bits log2(G) .. 5 (DPP row
// rotation by 8 for bit 3, the permlane swaps for bits 4 and 5), in the same
// order every time. No LDS, no barrier.
__device__ inline float xsum8(float v) {  // v + v[lane ^ 8]
  return v + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xF, 0xF, false));
}
__device__ inline float xsum16(float v) {  // v + v[lane ^ 16]
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ inline float xsum32(float v) {  // v + v[lane ^ 32]
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int G, int NB>
__global__ __launch_bounds__(256) void pool_wave_kernel(PoolParams p) {
  constexpr int TS = 64 / G;  // token stride between a lane's tokens
  const int R = p.S * p.S;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int w = xcd_item(blockIdx.x, gridDim.x) * 4 + wave;  // region; an image's regions on one XCD
  if (w >= p.nregions) return;  // uniform; no barrier in this kernel
  const int b = w / R, r = w - b * R;
  const int y0 = (r / p.S) * p.sh, x0 = (r - (r / p.S) * p.S) * p.sw;
  const int g = lane % G, t0 = lane / G;
  const int n = p.sh * p.sw;
  const int64_t img = (int64_t)b * p.H * p.W * p.C;
  const __bf16* Qb = static_cast<const __bf16*>(p.Q) + img + 8 * g;
  const __bf16* Kb = static_cast<const __bf16*>(p.K) + img + 8 * g;
  uint4 vq[NB], vk[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int t = t0 + j * TS;
    vq[j] = vk[j] = make_uint4(0u, 0u, 0u, 0u);
    if (t < n) {
      const int ty = t / p.sw, tx = t - ty * p.sw;
      const int off = ((y0 + ty) * p.W + x0 + tx) * p.C;
      vq[j] = *reinterpret_cast<const uint4*>(Qb + off);
      vk[j] = *reinterpret_cast<const uint4*>(Kb + off);
    }
  }
  float aq[8] = {}, ak[8] = {};
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    accum16<8>(aq, vq[j]);
    accum16<8>(ak, vk[j]);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if (G <= 8) { aq[e] = xsum8(aq[e]); ak[e] = xsum8(ak[e]); }
    if (G <= 16) { aq[e] = xsum16(aq[e]); ak[e] = xsum16(ak[e]); }
    if (G <= 32) { aq[e] = xsum32(aq[e]); ak[e] = xsum32(ak[e]); }
  }
  if (lane < G) {
    const float inv = 1.0f / (float)n;
    float* oq = p.Qr + ((int64_t)b * R + r) * p.C + 8 * g;
    float* ok = p.Kr + ((int64_t)b * R + r) * p.C + 8 * g;
    *reinterpret_cast<float4*>(oq) = make_float4(aq[0] * inv, aq[1] * inv, aq[2] * inv, aq[3] * inv);
    *reinterpret_cast<float4*>(oq + 4) = make_float4(aq[4] * inv, aq[5] * inv, aq[6] * inv, aq[7] * inv);
    *reinterpret_cast<float4*>(ok) = make_float4(ak[0] * inv, ak[1] * inv, ak[2] * inv, ak[3] * inv);
    *reinterpret_cast<float4*>(ok + 4) = make_float4(ak[4] * inv, ak[5] * inv, ak[6] * inv, ak[7] * inv);
  }
}

}  // namespace

hipError_t launch_pool(const void* Q, const void* K, float* Qr, float* Kr,
                       const Shape& s, int dtype, hipStream_t stream) {
  PoolParams p{Q, K, Qr, Kr, s.H, s.W, s.C, s.S, s.sh, s.sw, s.B * s.R};
  // small bf16 regions (at most four 16-byte vectors per tensor per lane):
  // one wave per region (measured at 28 x 28, C = 128: 8.5 vs 9.2 us; at
  // 14 x 14, C = 256: 6.5 vs 8.1 us; the same at the 56 x 56 stage map, and
  // slower for 16 x 16 regions, whose tokens would take several rounds)
  const int G8 = s.C / 8;
  if (dtype == kBF16 && (G8 == 8 || G8 == 16 || G8 == 32) && s.n * G8 <= 256) {
    void* a[] = {&p};
    const unsigned grid = (unsigned)((s.B * s.R + 3) / 4);
    const void* fn = G8 == 8 ? (const void*)&pool_wave_kernel<8, 4> : G8 == 16 ? (const void*)&pool_wave_kernel<16, 4>
                                                                             : (const void*)&pool_wave_kernel<32, 4>;
    return hipLaunchKernel(fn, dim3(grid), dim3(256), a, 0, stream);
  }
  const int vec = dtype == kBF16 ? 8 : 4;
  const int G = s.C / vec;

  const int total = s.sh * s.sw * G;
  // up to 8 vectors per tensor per thread (measured against 4 at the stage-1
  // shape: pool + route 16.5 vs 16.7 us), at least one full channel-group set
  int bs = 64;
  while (bs < 256 && total > 8 * bs) bs *= 2;
  while (bs < G) bs *= 2;
  dim3 grid((unsigned)(s.B * s.R));
  void* args[] = {&p};
  const size_t lds = 2 * sizeof(float) * (size_t)bs * vec;
  if (dtype == kBF16)
    return hipLaunchKernel(reinterpret_cast<const void*>(&pool_kernel<2>), grid, dim3(bs), args, lds, stream);
  return hipLaunchKernel(reinterpret_cast<const void*>(&pool_kernel<4>), grid, dim3(bs), args, lds, stream);
}

}  // namespace bra
