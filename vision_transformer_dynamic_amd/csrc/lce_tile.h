// Local context enhancement (LCE): the "+ dwconv(value)" term of the module
// output (explainer "BiFormer Reshapes Visual Attention with 'Bi-Level
// Routing'", Part 2.2 step 4 and pseudocode step 7; paper summary "BiFormer:
// Vision Transformer with Bi-Level Routing Attention", Section 3):
//
//   lce[y, x, c] = bias[c] + sum_{i,j < 5} w[c][i][j] * V[y + i - 2, x + j - 2, c]
//
// over the whole H x W map, zero outside it. Device routines shared by the
// attention kernel (fused epilogue) and the stand-alone LCE kernel. One wave
// handles one tile of at most LR x 2*LX outputs of one 32-channel head:
//
//  * halo: the tile's V neighbourhood ((rows + 4) x (cols + 4) positions) is
//    staged in LDS as 32 channel planes; a plane row holds pairs of
//    horizontally adjacent positions, one pair per 32-bit word (bf16) or
//    64-bit word (fp32). Plane stride is odd, so the 32 lanes that read the
//    same (row, word) of their own planes hit 32 different banks.
//  * compute: lane = (channel c = lane % 32, column parity par = lane / 32).
//    Output column x = 2m + par needs halo columns x .. x+4, i.e. exactly the
//    words m, m+1, m+2 of a row, whatever the parity: with the tap pairs
//    (w0,w1) (w2,w3) (w4,0) for even x and (0,w0) (w1,w2) (w3,w4) for odd x.
//    So every lane keeps ONE packed weight set of 15 pairs and the bf16 path
//    runs two taps per v_dot2c_f32_bf16 (fp32 accumulation).
//  * results: transposed through LDS into [position][channel] fp32 rows so
//    the caller can read 8 consecutive channels of one position per lane.
#pragma once

#include "bra_internal.h"

namespace bra {

typedef __bf16 lce_bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kLceRes = 36;  // floats per result row (32 channels + 4 of padding)

template <typename T>
struct Lce;

template <>
struct Lce<__bf16> {
  typedef uint32_t word;  // (V[x], V[x+1]) of one channel, low half first
  static constexpr int VEC = 8;
  __device__ static inline float dot(word v, word w, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(lce_bf16x2, v), __builtin_bit_cast(lce_bf16x2, w), acc,
                                           false);
  }
  __device__ static inline word zero() { return 0u; }
};

template <>
struct Lce<float> {
  typedef float2 word;
  static constexpr int VEC = 4;
  __device__ static inline float dot(word v, word w, float acc) {
    return __builtin_fmaf(v.y, w.y, __builtin_fmaf(v.x, w.x, acc));
  }
  __device__ static inline word zero() { return make_float2(0.f, 0.f); }
};

// Halo words per plane row for a tile `cols` wide: (cols + 4) rounded up to
// even, halved (the odd-width case carries one zero column).
__host__ __device__ inline int lce_pw(int cols) { return (cols + 5) / 2; }
// Plane stride in words: odd, at least (rows + 4) * pw.
__host__ __device__ inline int lce_ps(int rows, int cols) { return ((rows + 4) * lce_pw(cols)) | 1; }
// LDS bytes of one wave's LCE area: the halo planes (plus the words a row
// read may run past the last plane) or the result rows, whichever is larger.
__host__ __device__ inline int lce_lds_bytes(int rows, int cols, int word_bytes) {
  const int halo = (32 * lce_ps(rows, cols) + 8) * word_bytes;
  const int res = rows * cols * kLceRes * 4;
  return halo > res ? halo : res;
}

// Uniform geometry of one wave's tile.
struct LceTile {
  int y0, x0;      // image coordinates of the tile's first output
  int rows, cols;  // tile size
  int pw, ps;      // lce_pw(cols), lce_ps(rows, cols)
  float inv_pw;    // 1 / pw
};

// Halo items: f -> (halo row hy, word px, channel vector cv). The row is
// (pi + 0.5) / pw rounded down, with pi = f / CVN: for pi < 2^16 the float
// product is far closer to the true quotient than the 0.5 / pw that separates
// it from an integer, so it truncates exactly without a remainder fix-up.
template <typename T>
__device__ __forceinline__ void lce_halo_item(const LceTile& t, int f, int* hy, int* px, int* cv) {
  constexpr int CVN = 32 / Lce<T>::VEC;  // 4 (bf16) or 8 (fp32)
  *cv = f & (CVN - 1);
  const int pi = f / CVN;
  *hy = (int)(((float)pi + 0.5f) * t.inv_pw);
  *px = pi - *hy * t.pw;
}

// Each item loads the two positions of word px (16 bytes each). Positions
// outside the map are clamped to the map for the load (always in bounds, no
// branch) and their values replaced by zeros.
template <typename T, int NB>
__device__ __forceinline__ void lce_halo_load(const T* Vimg, int H, int W, int C, int ch0, const LceTile& t,
                                              int base, int lane, uint4 (&a)[NB], uint4 (&b)[NB]) {
  constexpr int CVN = 32 / Lce<T>::VEC;
  const int nitems = (t.rows + 4) * t.pw * CVN;
  const uint4 z = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
  for (int m = 0; m < NB; ++m) {
    const int f = base + lane + 64 * m;
    const bool in = f < nitems;
    int hy, px, cv;
    lce_halo_item<T>(t, in ? f : 0, &hy, &px, &cv);
    const int yy = t.y0 - 2 + hy, xx = t.x0 - 2 + 2 * px;
    const bool rok = in && (unsigned)yy < (unsigned)H;
    const bool aok = rok && (unsigned)xx < (unsigned)W;
    const bool bok = rok && (unsigned)(xx + 1) < (unsigned)W;
    const int yc = min(max(yy, 0), H - 1);
    const int xa = min(max(xx, 0), W - 1), xb = min(max(xx + 1, 0), W - 1);
    const T* row = Vimg + (yc * W) * C + ch0 + cv * Lce<T>::VEC;
    const uint4 va = *reinterpret_cast<const uint4*>(row + xa * C);
    const uint4 vb = *reinterpret_cast<const uint4*>(row + xb * C);
    a[m] = aok ? va : z;
    b[m] = bok ? vb : z;
  }
}

__device__ __forceinline__ void lce_put(uint32_t* halo, int ps, int ch, int w, const uint4& a, const uint4& b) {
  const uint32_t wa[4] = {a.x, a.y, a.z, a.w};
  const uint32_t wb[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    halo[(ch + 2 * e) * ps + w] = (wa[e] & 0xffffu) | (wb[e] << 16);
    halo[(ch + 2 * e + 1) * ps + w] = (wa[e] >> 16) | (wb[e] & 0xffff0000u);
  }
}

__device__ __forceinline__ void lce_put(float2* halo, int ps, int ch, int w, const uint4& a, const uint4& b) {
  halo[(ch + 0) * ps + w] = make_float2(__uint_as_float(a.x), __uint_as_float(b.x));
  halo[(ch + 1) * ps + w] = make_float2(__uint_as_float(a.y), __uint_as_float(b.y));
  halo[(ch + 2) * ps + w] = make_float2(__uint_as_float(a.z), __uint_as_float(b.z));
  halo[(ch + 3) * ps + w] = make_float2(__uint_as_float(a.w), __uint_as_float(b.w));
}

template <typename T, int NB>
__device__ __forceinline__ void lce_halo_store(typename Lce<T>::word* halo, const LceTile& t, int base, int lane,
                                               const uint4 (&a)[NB], const uint4 (&b)[NB]) {
  constexpr int CVN = 32 / Lce<T>::VEC;
  const int nitems = (t.rows + 4) * t.pw * CVN;
#pragma unroll
  for (int m = 0; m < NB; ++m) {
    const int f = base + lane + 64 * m;
    if (f < nitems) {
      int hy, px, cv;
      lce_halo_item<T>(t, f, &hy, &px, &cv);
      lce_put(halo, t.ps, cv * Lce<T>::VEC, hy * t.pw + px, a[m], b[m]);
    }
  }
}

// Whole halo, load then store in batches of NB items per lane.
template <typename T, int NB>
__device__ __forceinline__ void lce_halo_fill(const T* Vimg, int H, int W, int C, int ch0, const LceTile& t, int lane,
                                              typename Lce<T>::word* halo) {
  constexpr int CVN = 32 / Lce<T>::VEC;
  const int nitems = (t.rows + 4) * t.pw * CVN;
#pragma unroll 1
  for (int base = 0; base < nitems; base += 64 * NB) {
    uint4 a[NB], b[NB];
    lce_halo_load<T, NB>(Vimg, H, W, C, ch0, t, base, lane, a, b);
    lce_halo_store<T, NB>(halo, t, base, lane, a, b);
  }
}

// The lane's packed weights: w[i][k] multiplies halo word m + k of row y + i
// for output (y, 2m + par); plus the bias.
template <typename T>
struct LceW {
  typename Lce<T>::word w[5][3];
  float bias;
};

__device__ __forceinline__ uint32_t lce_half(const uint32_t (&wd)[13], int off, int k) {
  // element k of a channel's 25 weights is halfword k + off of wd
  const uint32_t e0 = (k & 1) ? (wd[k >> 1] >> 16) : (wd[k >> 1] & 0xffffu);
  const uint32_t e1 = ((k + 1) & 1) ? (wd[(k + 1) >> 1] >> 16) : (wd[(k + 1) >> 1] & 0xffffu);
  return off ? e1 : e0;
}

// weight: [C][5][5] (4-byte aligned base for bf16); bias: [C] or null.
__device__ __forceinline__ void lce_weights(const __bf16* weight, const __bf16* bias, int chg, int par,
                                            LceW<__bf16>& lw) {
  const int e0 = chg * 25;
  const int off = e0 & 1;
  // 13 words cover the channel's 25 halfwords from either parity; they never
  // pass the end of the array (the last channel, C - 1, is odd).
  const uint32_t* src = reinterpret_cast<const uint32_t*>(weight) + (e0 >> 1);
  uint32_t wd[13];
#pragma unroll
  for (int k = 0; k < 13; ++k) wd[k] = src[k];
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const uint32_t h0 = lce_half(wd, off, 5 * i), h1 = lce_half(wd, off, 5 * i + 1);
    const uint32_t h2 = lce_half(wd, off, 5 * i + 2), h3 = lce_half(wd, off, 5 * i + 3);
    const uint32_t h4 = lce_half(wd, off, 5 * i + 4);
    lw.w[i][0] = par ? (h0 << 16) : (h0 | (h1 << 16));
    lw.w[i][1] = par ? (h1 | (h2 << 16)) : (h2 | (h3 << 16));
    lw.w[i][2] = par ? (h3 | (h4 << 16)) : h4;
  }
  lw.bias = bias ? (float)bias[chg] : 0.f;
}

__device__ __forceinline__ void lce_weights(const float* weight, const float* bias, int chg, int par,
                                            LceW<float>& lw) {
  const float* src = weight + chg * 25;
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const float h0 = src[5 * i], h1 = src[5 * i + 1], h2 = src[5 * i + 2], h3 = src[5 * i + 3], h4 = src[5 * i + 4];
    lw.w[i][0] = par ? make_float2(0.f, h0) : make_float2(h0, h1);
    lw.w[i][1] = par ? make_float2(h1, h2) : make_float2(h2, h3);
    lw.w[i][2] = par ? make_float2(h3, h4) : make_float2(h4, 0.f);
  }
  lw.bias = bias ? bias[chg] : 0.f;
}

// acc[y][m] = output (y, 2m + par) of the lane's channel. plane: the lane's
// channel plane of the halo. Rows beyond t.rows are skipped (uniformly);
// columns beyond t.cols are computed from in-bounds LDS words and ignored.
template <typename T, int LR, int LX>
__device__ __forceinline__ void lce_compute(const typename Lce<T>::word* plane, const LceTile& t, const LceW<T>& lw,
                                            float (&acc)[LR][LX]) {
  typedef Lce<T> L;
#pragma unroll
  for (int y = 0; y < LR; ++y)
#pragma unroll
    for (int m = 0; m < LX; ++m) acc[y][m] = lw.bias;
#pragma unroll
  for (int hy = 0; hy < LR + 4; ++hy) {
    if (hy >= t.rows + 4) break;  // uniform
    typename L::word wd[LX + 2];
#pragma unroll
    for (int k = 0; k < LX + 2; ++k) wd[k] = plane[hy * t.pw + k];
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      const int y = hy - i;  // output row fed by halo row hy through filter row i
      if (y < 0 || y >= LR) continue;
      if (y >= t.rows) continue;  // uniform
      // consecutive instructions update different accumulators
#pragma unroll
      for (int k = 0; k < 3; ++k)
#pragma unroll
        for (int m = 0; m < LX; ++m) acc[y][m] = L::dot(wd[m + k], lw.w[i][k], acc[y][m]);
    }
  }
}

// Results to LDS rows res[(y * cols + x) * kLceRes + c]. Outputs past the
// tile's last column go to a padding slot of row 0 (no branch per store).
template <int LR, int LX>
__device__ __forceinline__ void lce_store_results(float* res, const LceTile& t, int c, int par,
                                                  const float (&acc)[LR][LX]) {
#pragma unroll
  for (int y = 0; y < LR; ++y) {
    if (y >= t.rows) break;  // uniform
#pragma unroll
    for (int m = 0; m < LX; ++m) {
      const int x = 2 * m + par;
      const int at = x < t.cols ? (y * t.cols + x) * kLceRes + c : 32 + (c & 3);
      res[at] = acc[y][m];
    }
  }
}

}  // namespace bra
