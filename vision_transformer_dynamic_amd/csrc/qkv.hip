// Linear QKV projection with the region pooling in its epilogue (explainer
// "BiFormer Reshapes Visual Attention with 'Bi-Level Routing'", Part 2.2
// steps 2-3 and pseudocode steps 2-3; Part 3 counts the projection as the
// 3HWC^2 term):
//
//   [Q | K | V] = X Wqkv^T + bqkv,  Q^r, K^r = region means of Q, K
//
// Wqkv is [3C, C] (a torch Linear weight: row = output feature). The region
// means are taken of the ROUNDED outputs, in fp32, so they are what the pool
// kernel would compute from the stored Q and K; the routing then needs no
// second read of Q and K.
//
// Work split: one workgroup = whole regions of one image - floor(64 / n)
// regions of n <= 64 tokens, or one region of n > 64 tokens walked in blocks
// of 64 - and waves own feature groups of 32 output features. The token
// block's X rows are staged in LDS once; a wave computes
//   out^T[32 features x 16 tokens] = Wqkv[32 x C] . X^T[C x 16]
// per 16-token tile (transposed, so each lane ends with 8 consecutive
// features of one token: one 16-byte store), with the weight rows read as
// natural MFMA operands from L2. For Q and K feature groups the rounded
// values also go to a per-wave LDS tile, from which each (region, feature)
// sum is formed in a fixed order (deterministic, no atomics).
#include "attn_common.h"

namespace bra {
namespace {

constexpr int kTokBlock = 64;  // tokens per block
constexpr int kQkvWaves = 8;   // waves per workgroup (at most)

struct QkvParams {
  const void* X;
  const void* Wt;   // [3C][C]
  const void* bias; // [3C] or null
  void* Q;
  void* K;
  void* V;
  float* Qr;  // [B, R, C]
  float* Kr;
  int H, W, C, S, sh, sw, n, R;
  int rpw;      // regions per workgroup (n <= 64), else 1
  int nsub;     // 64-token blocks per region (n > 64), else 1
  int ngroups;  // workgroups per image
  int nfg;      // feature groups (3C / 32)
  FastDiv div_n, div_sw, div_S;
};

// Token tw of block `sub` of the workgroup (regions r0.. of n tokens) ->
// token inside the image, or -1.
__device__ __forceinline__ int block_token(int sub, int tw, int r0, int nreg, int nsub, int n, int sh, int sw, int W,
                                           FastDiv div_n, FastDiv div_sw, FastDiv div_S) {
  int j, q;
  if (nsub > 1) {
    j = 0;
    q = sub * kTokBlock + tw;
    if (q >= n) return -1;
  } else {
    j = fdiv(tw, div_n, &q);
    if (j >= nreg) return -1;
  }
  int rx;
  const int ry = fdiv(r0 + j, div_S, &rx);
  int qx;
  const int qy = fdiv(q, div_sw, &qx);
  return (ry * sh + qy) * W + rx * sw + qx;
}

template <typename T>
__global__ __launch_bounds__(512) void qkv_pool_kernel(QkvParams p) {
  typedef Tr<T> TT;
  typedef typename TT::op8 op8;
  constexpr int VEC = TT::VEC;
  const int LDX = p.C + 16 / (int)sizeof(T);  // X rows in LDS, 16-byte pad
  extern __shared__ __align__(16) unsigned char smem_raw[];
  T* xs = reinterpret_cast<T*>(smem_raw);                                         // [64][LDX]
  float* pool = reinterpret_cast<float*>(xs + kTokBlock * LDX);                    // [rpw][2C] sums
  float* ptile = pool + p.rpw * 2 * p.C + (threadIdx.x >> 6) * kTokBlock * 33;     // wave's [64][33]

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nw = blockDim.x >> 6;
  const int lane = tid & 63;
  const int g = lane >> 4, col = lane & 15;

  int w;
  {
    const int nwg = gridDim.x, bid = blockIdx.x;
    const int x = bid & 7, loc = bid >> 3, q8 = nwg >> 3, r8 = nwg & 7;
    w = x * q8 + min(x, r8) + loc;
  }
  const int grp = w % p.ngroups;
  const int b = w / p.ngroups;
  const int r0 = grp * p.rpw;
  const int nreg = min(p.rpw, p.R - r0);  // regions of this workgroup
  const int64_t img = (int64_t)b * p.H * p.W * p.C;
  const T* Xg = static_cast<const T*>(p.X) + img;
  const T* Wg = static_cast<const T*>(p.Wt);
  const T* Bg = static_cast<const T*>(p.bias);

  for (int e = tid; e < p.rpw * 2 * p.C; e += blockDim.x) pool[e] = 0.f;

  const int ntok = p.nsub > 1 ? kTokBlock : nreg * p.n;  // tokens per block
  const int ks_n = p.C / 32;
  const int cvec = p.C / VEC;  // 16-byte vectors per X row
  for (int sub = 0; sub < p.nsub; ++sub) {
    __syncthreads();  // previous block's X rows consumed
    for (int f = tid; f < kTokBlock * cvec; f += blockDim.x) {
      const int tw = f / cvec, cv = f - tw * cvec;
      const int t = tw < ntok ? block_token(sub, tw, r0, nreg, p.nsub, p.n, p.sh, p.sw, p.W, p.div_n, p.div_sw, p.div_S) : -1;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (t >= 0) v = *reinterpret_cast<const uint4*>(Xg + t * p.C + cv * VEC);
      *reinterpret_cast<uint4*>(xs + tw * LDX + cv * VEC) = v;
    }
    __syncthreads();
    const int mtiles = (ntok + 15) >> 4;
    // token of this lane in each 16-token tile (stores)
    for (int fg = wave; fg < p.nfg; fg += nw) {
      // A rows: row rr = col of feature tile ct is feature 32 fg + 8 (rr/4) +
      // (rr%4) + 4 ct, so lane group g ends with features 8g..8g+7
      const int frow = fg * 32 + 8 * (col >> 2) + (col & 3);
      floatx4 acc[4][2];
      for (int m0 = 0; m0 < mtiles; m0 += 4) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int ct = 0; ct < 2; ++ct) acc[mt][ct] = floatx4{0.f, 0.f, 0.f, 0.f};
        for (int ks = 0; ks < ks_n; ++ks) {
          const op8 wa = TT::load8(Wg + (frow + 0) * p.C + ks * 32 + 8 * g);
          const op8 wb = TT::load8(Wg + (frow + 4) * p.C + ks * 32 + 8 * g);
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) {
            if (m0 + mt >= mtiles) break;  // uniform
            const op8 xb = TT::load8(xs + ((m0 + mt) * 16 + col) * LDX + ks * 32 + 8 * g);
            acc[mt][0] = TT::mma(wa, xb, acc[mt][0]);
            acc[mt][1] = TT::mma(wb, xb, acc[mt][1]);
          }
        }
        // epilogue: bias, one rounding, store; Q/K groups also keep the
        // rounded values for the region sums
        const int feat = fg * 32 + 8 * g;  // lane's first feature
        const int tensor = feat / p.C, ch = feat - tensor * p.C;
        float bv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) bv[e] = Bg ? (float)Bg[feat + e] : 0.f;
        T* dst = static_cast<T*>(tensor == 0 ? p.Q : tensor == 1 ? p.K : p.V) + img;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          if (m0 + mt >= mtiles) break;
          const int tw = (m0 + mt) * 16 + col;
          const int t = tw < ntok ? block_token(sub, tw, r0, nreg, p.nsub, p.n, p.sh, p.sw, p.W, p.div_n, p.div_sw, p.div_S) : -1;
          float o[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            o[e] = acc[mt][0][e] + bv[e];
            o[4 + e] = acc[mt][1][e] + bv[4 + e];
          }
          typename TT::op8 r = TT::from_f32(o);  // the rounded outputs
          if (t >= 0) *reinterpret_cast<op8*>(dst + t * p.C + ch) = r;
          if (fg * 32 < 2 * p.C) {
#pragma unroll
            for (int e = 0; e < 8; ++e) ptile[tw * 33 + 8 * g + e] = t >= 0 ? (float)r[e] : 0.f;
          }
        }
        if (fg * 32 < 2 * p.C) {
          // region sums over this block's tokens, one (region, feature) per
          // lane step, tokens in order
          __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
          __builtin_amdgcn_wave_barrier();
          const int t0 = m0 * 16, t1 = min(ntok, (m0 + 4) * 16);
          for (int jf = lane; jf < p.rpw * 32; jf += 64) {
            const int j = jf >> 5, f = jf & 31;
            const int a = max(t0, p.nsub > 1 ? 0 : j * p.n), z = min(t1, p.nsub > 1 ? ntok : (j + 1) * p.n);
            float sacc = 0.f;
            for (int tw = a; tw < z; ++tw) sacc += ptile[tw * 33 + f];
            if (a < z) pool[j * 2 * p.C + fg * 32 + f] += sacc;
          }
          __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
          __builtin_amdgcn_wave_barrier();
        }
      }
    }
  }
  __syncthreads();
  // means of the rounded Q and K
  const float inv = 1.0f / (float)p.n;
  for (int e = tid; e < nreg * 2 * p.C; e += blockDim.x) {
    const int j = e / (2 * p.C), f = e - j * 2 * p.C;
    const int64_t at = ((int64_t)b * p.R + r0 + j) * p.C;
    if (f < p.C)
      p.Qr[at + f] = pool[e] * inv;
    else
      p.Kr[at + f - p.C] = pool[e] * inv;
  }
}

}  // namespace

hipError_t launch_qkv_pool(const void* X, const void* Wqkv, const void* bqkv, void* Q, void* K, void* V, float* Qr,
                           float* Kr, const Shape& s, int dtype, hipStream_t stream) {
  QkvParams p;
  p.X = X; p.Wt = Wqkv; p.bias = bqkv; p.Q = Q; p.K = K; p.V = V; p.Qr = Qr; p.Kr = Kr;
  p.H = s.H; p.W = s.W; p.C = s.C; p.S = s.S; p.sh = s.sh; p.sw = s.sw; p.n = s.n; p.R = s.R;
  if (s.n <= kTokBlock) {
    // whole regions up to 64 tokens, with their sums in at most 32 KB of LDS
    p.rpw = min(kTokBlock / s.n, max(1, 4096 / s.C));
    p.nsub = 1;
  } else {
    p.rpw = 1;
    p.nsub = (s.n + kTokBlock - 1) / kTokBlock;
  }
  p.ngroups = (s.R + p.rpw - 1) / p.rpw;
  p.nfg = 3 * s.C / 32;
  p.div_n = make_fastdiv(s.n);
  p.div_sw = make_fastdiv(s.sw);
  p.div_S = make_fastdiv(s.S);
  const int64_t nwg = (int64_t)s.B * p.ngroups;
  if (nwg >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  const int waves = p.nfg < kQkvWaves ? p.nfg : kQkvWaves;
  const size_t esz = dtype == kBF16 ? 2 : 4;
  const size_t lds = esz * kTokBlock * (s.C + 16 / esz) + sizeof(float) * p.rpw * 2 * s.C +
                     sizeof(float) * waves * kTokBlock * 33;
  const void* fn = dtype == kBF16 ? (const void*)&qkv_pool_kernel<__bf16> : (const void*)&qkv_pool_kernel<float>;
  void* args[] = {&p};
  return hipLaunchKernel(fn, dim3((unsigned)nwg), dim3(waves * 64), args, lds, stream);
}

}  // namespace bra
