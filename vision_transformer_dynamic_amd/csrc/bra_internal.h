// Internal launch interface shared by the host API and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bra {

// Validated problem shape. Region grid S x S; each region is sh x sw tokens.
struct Shape {
  int B, H, W, C, heads, S, topk;
  int sh, sw;  // region rows / columns (H/S, W/S)
  int n;       // tokens per region
  int R;       // regions per image (S*S)
  int d;       // head dim (C/heads)
  int kv;      // keys per query (topk * n)
};

constexpr int kHeadDim = 32;       // head dim implemented by the attention kernel
constexpr int kMaxRegions = 256;   // route kernel: at most 4 candidates per lane
constexpr int kMaxChannelsBf16 = 2048;
constexpr int kMaxChannelsF32 = 1024;

// Limits that keep every in-image index and every fast division exact.
constexpr int64_t kMaxImageElems = (int64_t(1) << 31) - 1;  // H*W*C per image
constexpr int kMaxFastDiv = 1 << 22;                       // numerators of FastDiv

// Exact a / d for 0 <= a < 2^22 and 1 <= d < 2^22 through a float reciprocal:
// the float quotient is within 0.5 of a/d, so its truncation is off by at most
// one, which a single remainder check repairs. About 7 VALU instructions
// instead of the ~20 of a 32-bit integer division.
struct FastDiv {
  float inv;
  int d;
};

inline FastDiv make_fastdiv(int d) { return FastDiv{1.0f / (float)d, d}; }

// The repair is written as selects, not branches, so that it never splits a
// wave's control flow (at most one of the two applies).
__device__ inline int fdiv(int a, FastDiv f, int* rem) {
  int q = (int)((float)a * f.inv);
  int r = a - q * f.d;
  const bool lo = r < 0;
  q = lo ? q - 1 : q;
  r = lo ? r + f.d : r;
  const bool hi = r >= f.d;
  q = hi ? q + 1 : q;
  r = hi ? r - f.d : r;
  *rem = r;
  return q;
}

// dtype codes match bra_dtype in include/bra.h
// Work item of workgroup bid among n. Workgroups are dealt round-robin to the
// 8 XCDs, so XCD x = bid % 8 is given the contiguous items
// [x * (n / 8) + min(x, n % 8), ...): consecutive items (regions of one image)
// share an L2. The pool, route and attention kernels split images over the
// XCDs this same way. reverse: the XCD walks its range from the end, so the
// attention kernel starts on the images the pool kernel read last, which are
// the likeliest to be still cached.
__device__ inline int xcd_item(int bid, int n, bool reverse = false) {
  const int x = bid & 7, loc = bid >> 3, q8 = n >> 3, r8 = n & 7;
  const int cnt = q8 + (x < r8 ? 1 : 0);
  return x * q8 + (x < r8 ? x : r8) + (reverse ? cnt - 1 - loc : loc);
}

constexpr int kF32 = 0;
constexpr int kBF16 = 1;

// Region means of Q and K, fp32: Qr, Kr are [B, R, C].
hipError_t launch_pool(const void* Q, const void* K, float* Qr, float* Kr,
                       const Shape& s, int dtype, hipStream_t stream);

// Affinity Qr Kr^T per image and top-k per row: idx is [B, R, topk].
hipError_t launch_route(const float* Qr, const float* Kr, int32_t* idx,
                        const Shape& s, hipStream_t stream);

// Token attention over routed regions: O = softmax(q k_g^T / sqrt(d)) v_g,
// plus the local context term lce(V) when lce_w ([C][5][5]) is not null
// (lce_b: [C] bias or null), fused or by launch_lce afterwards.
hipError_t launch_attend(const void* Q, const void* K, const void* V,
                         const int32_t* idx, const void* lce_w, const void* lce_b, void* O,
                         const Shape& s, int dtype, hipStream_t stream);

// bf16 attention with more than 64 and at most 1024 keys per query: every
// routed key of a head staged in LDS by direct-to-LDS loads, V read with the
// transposing LDS reads (attend_dense.hip).
bool dense_attend_fits(const Shape& s, int dtype);
hipError_t launch_attend_dense(const void* Q, const void* K, const void* V, const int32_t* idx, void* O,
                               const Shape& s, hipStream_t stream);

// Name of the attention kernel launch_attend runs for this shape (the same
// dispatch decision; the convolution pass, where there is one, follows it).
const char* attend_kernel_name(const Shape& s, int dtype, bool lce);

// O += lce(V): 5x5 depthwise convolution of V over the whole map, zero
// padding, per-channel bias (lce_b may be null). C must be a multiple of 32.
hipError_t launch_lce(const void* V, const void* lce_w, const void* lce_b, void* O,
                      const Shape& s, int dtype, hipStream_t stream);

// Q, K, V = X Wqkv^T + bqkv (Wqkv [3C][C]; bqkv [3C] or null) and the region
// means Qr, Kr [B, R, C] of the rounded Q and K. C % 32 == 0, C <= 256 (bf16)
// or 128 (fp32): the X rows, region sums and per-wave tiles fit in LDS.
hipError_t launch_qkv_pool(const void* X, const void* Wqkv, const void* bqkv, void* Q, void* K, void* V, float* Qr,
                           float* Kr, const Shape& s, int dtype, hipStream_t stream);
constexpr int kMaxProjChannelsBf16 = 256;
constexpr int kMaxProjChannelsF32 = 128;

// Backward of the token attention, routing table idx held fixed: dQ, dK, dV
// from dO (and the forward output O). ws holds backward_workspace_bytes(s).
size_t backward_workspace_bytes(const Shape& s);
hipError_t launch_backward(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                           const int32_t* idx, void* dQ, void* dK, void* dV, void* ws, const Shape& s, int dtype,
                           hipStream_t stream);

// The same backward in one launch for small bf16 maps (regions of 4, 8 or 16
// tokens, at most 64 regions, the image's K, V, Q and dO rows of one head in
// LDS): backward_image.hip. launch_backward takes it when it fits.
bool backward_image_fits(const Shape& s, int dtype);
hipError_t launch_backward_image(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                                 const int32_t* idx, void* dQ, void* dK, void* dV, const Shape& s,
                                 hipStream_t stream);

// dQ, log-sum-exp and D of the backward for bf16 with 65 to 1024 routed keys
// per query: every routed key's K and V rows of a head staged in LDS by
// direct-to-LDS loads, as in the dense forward (backward_dense.hip).
// launch_backward takes it for the several-chunk dQ step when it fits.
bool backward_dq_dense_fits(const Shape& s, int dtype);
hipError_t launch_backward_dq_dense(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                                    const int32_t* idx, void* dQ, float* lse, float* dd, const Shape& s,
                                    hipStream_t stream);

// The same backward in one launch for top-1 routing (bf16, regions of 16 to
// 64 tokens): one workgroup per (image, key region, pair of heads) takes the
// query regions routed to its region and finishes their dQ and its dK, dV
// (backward_top1.hip). O is not read: D = rowsum(P * dP). launch_backward
// takes it when it fits and the image kernel does not.
bool backward_top1_fits(const Shape& s, int dtype);
hipError_t launch_backward_top1(const void* Q, const void* K, const void* V, const void* dO, const int32_t* idx,
                                void* dQ, void* dK, void* dV, const Shape& s, hipStream_t stream);

}  // namespace bra
