// Region affinity fused with top-k routing (explainer "BiFormer Reshapes
// Visual Attention with 'Bi-Level Routing'", Part 2.2 step 3, pseudocode
// steps 4-5; paper summary "BiFormer: Vision Transformer with Bi-Level
// Routing Attention", Section 3: row i of the routing index holds the k
// regions most relevant to region i).
//
// One workgroup per (image b, block of 4 affinity rows); each of its 4 waves
// owns one row, and lane j owns the candidates j, j+64, j+128, j+192 (at most
// 256 regions). Channels are streamed in slices of CC: each slice of K^r[b]
// (all R rows) and of the block's query rows is staged in LDS with coalesced
// loads, the next slice's loads being in flight while the current one is used.
// A[i][j] = Q^r[b,i,:] . K^r[b,j,:] is accumulated as four fused
// multiply-add chains, one per channel residue mod 4, in increasing channel
// order, and combined as (s0 + s1) + (s2 + s3): a fixed order, so the values
// are bit-reproducible. The query row is read as a broadcast, K^r row j by
// lane j. The row never reaches HBM.
//
// Top-k by rank: candidate j of row i is beaten by m when A[i][m] > A[i][j],
// or A[i][m] == A[i][j] and m < j. This is a strict total order, so the number
// of candidates that beat j is a unique rank in [0, R); j is routed iff its
// rank is below k, and it is written to slot `rank`, which lists the routed
// regions in descending affinity with the lower index first on exact ties.
// Each lane counts against the whole row (broadcast LDS reads): R compares
// per candidate, independent of k.
#include "bra_internal.h"
#include "route_common.h"

#include <math.h>

namespace bra {
namespace {

constexpr int RB = 4;              // affinity rows per workgroup (one per wave)
constexpr int NT = 256;            // threads

struct RouteParams {
  const float* Qr;
  const float* Kr;
  int32_t* idx;
  int R, C, topk;
  int row_blocks;  // ceil(R / RB): workgroups per image
  int ldr;         // LDS row stride of the affinity block (R rounded up to 4)
};

// NU: candidates per lane (1 when R <= 64, 4 when R <= 256).
// CC: channels per staged slice (fewer when there are more candidate rows).
template <int NU> struct RouteCfg {
  static constexpr int CC = NU == 1 ? 64 : 32;
  static constexpr int C4 = CC / 4;        // float4 per row slice
  static constexpr int LDC = CC + 4;       // LDS row stride (floats)
};

template <int NU>
__global__ __launch_bounds__(NT) void route_kernel(RouteParams p) {
  constexpr int CC = RouteCfg<NU>::CC, C4 = RouteCfg<NU>::C4, LDC = RouteCfg<NU>::LDC;
  constexpr int KLD = 64 * NU * C4 / NT;  // float4 loads of K^r per thread per slice
  extern __shared__ __align__(16) float sm[];
  float* Ks = sm;                 // R x LDC
  float* Qs = Ks + p.R * LDC;     // RB x LDC
  float* As = Qs + RB * LDC;      // RB x ldr

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int b = blockIdx.x / p.row_blocks;
  const int i0 = (blockIdx.x - b * p.row_blocks) * RB;
  const int nrows = min(RB, p.R - i0);
  const float* kb = p.Kr + (int64_t)b * p.R * p.C;
  const float* qb = p.Qr + ((int64_t)b * p.R + i0) * p.C;

  float4 acc[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) acc[u] = make_float4(0.f, 0.f, 0.f, 0.f);

  // slice loads: element f = tid + NT*m of the slice is (row f / C4, float4 f % C4)
  float4 kreg[KLD];
  float4 qreg = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int m = 0; m < KLD; ++m) kreg[m] = make_float4(0.f, 0.f, 0.f, 0.f);
  auto slice_w4 = [&](int c0) { return min(CC, p.C - c0) >> 2; };  // valid float4 per row
  {
    const int w4 = slice_w4(0);
#pragma unroll
    for (int m = 0; m < KLD; ++m) {
      const int f = tid + NT * m, j = f / C4, c4 = f % C4;
      if (j < p.R && c4 < w4) kreg[m] = *reinterpret_cast<const float4*>(kb + (int64_t)j * p.C + 4 * c4);
    }
    const int r = tid / C4, c4 = tid % C4;
    if (r < nrows && c4 < w4) qreg = *reinterpret_cast<const float4*>(qb + (int64_t)r * p.C + 4 * c4);
  }

  for (int c0 = 0; c0 < p.C; c0 += CC) {
    const int w4 = slice_w4(c0);
    if (c0) __syncthreads();  // previous slice consumed
#pragma unroll
    for (int m = 0; m < KLD; ++m) {
      const int f = tid + NT * m, j = f / C4, c4 = f % C4;
      if (j < p.R) *reinterpret_cast<float4*>(Ks + j * LDC + 4 * c4) = kreg[m];
    }
    {
      const int r = tid / C4, c4 = tid % C4;
      if (r < RB) *reinterpret_cast<float4*>(Qs + r * LDC + 4 * c4) = qreg;
    }
    __syncthreads();
    const int n0 = c0 + CC;  // next slice, in flight while this one is used
    if (n0 < p.C) {
      const int w4n = slice_w4(n0);
#pragma unroll
      for (int m = 0; m < KLD; ++m) {
        const int f = tid + NT * m, j = f / C4, c4 = f % C4;
        if (j < p.R && c4 < w4n) kreg[m] = *reinterpret_cast<const float4*>(kb + (int64_t)j * p.C + n0 + 4 * c4);
      }
      const int r = tid / C4, c4 = tid % C4;
      if (r < nrows && c4 < w4n) qreg = *reinterpret_cast<const float4*>(qb + (int64_t)r * p.C + n0 + 4 * c4);
    }
    const float* qs = Qs + wave * LDC;
    for (int c4 = 0; c4 < w4; ++c4) {
      const float4 q = *reinterpret_cast<const float4*>(qs + 4 * c4);
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const float4 k = *reinterpret_cast<const float4*>(Ks + min(lane + 64 * u, p.R - 1) * LDC + 4 * c4);
        acc[u] = affinity_step(acc[u], q, k);
      }
    }
  }

  // affinity row to LDS (the wave's own row); columns R..ldr-1 hold -inf
  const int row = wave;
  float* a = As + row * p.ldr;
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int j = lane + 64 * u;
    if (j < p.ldr) a[j] = j < p.R ? affinity_finish(acc[u]) : -INFINITY;
  }
  __syncthreads();
  if (row >= nrows) return;  // wave-uniform; no barrier follows

  // ranks
  int32_t* out = p.idx + ((int64_t)b * p.R + i0 + row) * p.topk;
#pragma unroll 1
  for (int u = 0; u < NU; ++u) {
    const int j = lane + 64 * u;
    const float aj = j < p.R ? a[j] : -INFINITY;
    const int rank = affinity_rank(a, p.ldr, aj, j);
    if (j < p.R && rank < p.topk) out[rank] = j;
  }
}

}  // namespace

size_t route_lds_bytes(const Shape& s) {
  const int ldr = (s.R + 3) / 4 * 4;
  const int ldc = s.R <= 64 ? RouteCfg<1>::LDC : RouteCfg<4>::LDC;
  return sizeof(float) * ((size_t)s.R * ldc + (size_t)RB * ldc + (size_t)RB * ldr);
}

hipError_t launch_route(const float* Qr, const float* Kr, int32_t* idx,
                        const Shape& s, hipStream_t stream) {
  RouteParams p{Qr, Kr, idx, s.R, s.C, s.topk, (s.R + RB - 1) / RB, (s.R + 3) / 4 * 4};
  dim3 grid((unsigned)(s.B * p.row_blocks));
  void* args[] = {&p};
  const void* fn = s.R <= 64 ? reinterpret_cast<const void*>(&route_kernel<1>)
                             : reinterpret_cast<const void*>(&route_kernel<4>);
  return hipLaunchKernel(fn, grid, dim3(NT), args, route_lds_bytes(s), stream);
}

}  // namespace bra
