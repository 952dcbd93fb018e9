// Stand-alone local context enhancement pass: O += lce(V), the "+ dwconv(value)"
// term of the module output (explainer "BiFormer Reshapes Visual Attention
// with 'Bi-Level Routing'", Part 2.2 step 4 and pseudocode step 7). It runs
// after the attention kernel wherever the attention kernel cannot fuse the
// term into its epilogue (fp32, regions wider or taller than 8 tokens, or more
// than 64 keys per query). The arithmetic is the shared tile code of
// lce_tile.h; this kernel adds the fp32 result to O (read, add, one rounding
// to O's dtype, write).
//
// Work split: one wave per (image, 8 x 8 output tile, 32-channel group);
// tiles that pass the map's edge keep their in-map outputs only.
#include "lce_tile.h"

namespace bra {
namespace {

constexpr int TR = 8, TC = 8;  // output tile rows, columns

struct LceParams {
  const void* V;
  const void* w;
  const void* bias;
  void* O;
  int H, W, C;
  int tiles_x, tiles_y, ncg;
  int nitems;
};

template <typename T>
__global__ __launch_bounds__(64) void lce_kernel(LceParams p) {
  typedef Lce<T> L;
  constexpr int VEC = L::VEC;
  constexpr int CVN = 32 / VEC;
  constexpr int NB = ((TR + 4) * ((TC + 5) / 2) * CVN + 63) / 64 > 5 ? 3 : 5;  // halo items per lane per batch
  extern __shared__ __align__(16) unsigned char smem_raw[];
  const int lane = threadIdx.x;

  const int wg = xcd_item(blockIdx.x, gridDim.x);  // consecutive work to one XCD
  const int cg = wg % p.ncg;
  int rest = wg / p.ncg;
  const int tx = rest % p.tiles_x;
  rest /= p.tiles_x;
  const int ty = rest % p.tiles_y;
  const int b = rest / p.tiles_y;

  LceTile t;
  t.y0 = ty * TR;
  t.x0 = tx * TC;
  t.rows = TR;
  t.cols = TC;
  t.pw = lce_pw(TC);
  t.ps = lce_ps(TR, TC);
  t.inv_pw = 1.0f / lce_pw(TC);
  const int64_t img = (int64_t)b * p.H * p.W * p.C;
  const int ch0 = cg * 32;
  const int c = lane & 31, par = lane >> 5;

  // the attention output this tile adds to: loads issued first, consumed last
  T* Og = static_cast<T*>(p.O) + img;
  constexpr int NO = TR * TC * CVN / 64;  // 16-byte output vectors per lane
  uint4 ov[NO];
  int ooff[NO];
#pragma unroll
  for (int m = 0; m < NO; ++m) {
    const int f = lane + 64 * m;
    const int cv = f % CVN, q = f / CVN;
    const int yy = t.y0 + q / TC, xx = t.x0 + q % TC;
    ooff[m] = (yy < p.H && xx < p.W) ? (yy * p.W + xx) * p.C + ch0 + cv * VEC : -1;
    ov[m] = ooff[m] >= 0 ? *reinterpret_cast<const uint4*>(Og + ooff[m]) : make_uint4(0u, 0u, 0u, 0u);
  }
  LceW<T> lw;
  lce_weights(static_cast<const T*>(p.w), static_cast<const T*>(p.bias), ch0 + c, par, lw);
  typename L::word* halo = reinterpret_cast<typename L::word*>(smem_raw);
  lce_halo_fill<T, NB>(static_cast<const T*>(p.V) + img, p.H, p.W, p.C, ch0, t, lane, halo);
  __syncthreads();
  float acc[TR][TC / 2];
  lce_compute<T, TR, TC / 2>(halo + c * t.ps, t, lw, acc);
  __syncthreads();  // every halo read done before the results overwrite it
  float* res = reinterpret_cast<float*>(smem_raw);
  lce_store_results<TR, TC / 2>(res, t, c, par, acc);
  __syncthreads();

#pragma unroll
  for (int m = 0; m < NO; ++m) {
    const int f = lane + 64 * m;
    const int cv = f % CVN, q = f / CVN;
    if (ooff[m] >= 0) {
      const float* r = res + q * kLceRes + cv * VEC;
      if constexpr (VEC == 8) {
        typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
        bf16x8 v = __builtin_bit_cast(bf16x8, ov[m]);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (__bf16)((float)v[e] + r[e]);
        *reinterpret_cast<bf16x8*>(Og + ooff[m]) = v;
      } else {
        float4 v = __builtin_bit_cast(float4, ov[m]);
        v.x += r[0];
        v.y += r[1];
        v.z += r[2];
        v.w += r[3];
        *reinterpret_cast<float4*>(Og + ooff[m]) = v;
      }
    }
  }
}

}  // namespace

hipError_t launch_lce(const void* V, const void* weight, const void* bias, void* O, const Shape& s, int dtype,
                      hipStream_t stream) {
  LceParams p;
  p.V = V;
  p.w = weight;
  p.bias = bias;
  p.O = O;
  p.H = s.H;
  p.W = s.W;
  p.C = s.C;
  p.tiles_x = (s.W + TC - 1) / TC;
  p.tiles_y = (s.H + TR - 1) / TR;
  p.ncg = s.C / 32;
  const int64_t n = (int64_t)s.B * p.tiles_y * p.tiles_x * p.ncg;
  if (n >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  p.nitems = (int)n;
  const size_t lds = lce_lds_bytes(TR, TC, dtype == kBF16 ? 4 : 8);
  const void* fn = dtype == kBF16 ? (const void*)&lce_kernel<__bf16> : (const void*)&lce_kernel<float>;
  void* args[] = {&p};
  return hipLaunchKernel(fn, dim3((unsigned)p.nitems), dim3(64), args, lds, stream);
}

}  // namespace bra
