// Fused gather + token attention over routed regions (explainer "BiFormer
// Reshapes Visual Attention with 'Bi-Level Routing'", Part 2.2 step 4 and
// pseudocode steps 6-7 without the dwconv term; paper summary "BiFormer:
// Vision Transformer with Bi-Level Routing Attention", Section 3
// "Token-to-token attention").
//
// The pages gather the routed keys/values into a contiguous tensor and then
// run two batched matrix products. Here nothing is gathered in HBM: each
// workgroup streams the routed regions' K/V tokens from HBM straight into LDS
// through the routing table (each token's head-group channels are one
// contiguous run), and runs both products on MFMA with an online softmax.
//
// Work split. One workgroup = (image b, query region i, block of <= 64 of the
// region's queries, group of HG heads). Its 4 waves own "units" = (head, tile
// of 16 queries); each wave keeps <= 2 units' accumulators in registers.
//
// Transposed products. With d = 32 the score tile is computed as
//   S^T[16 keys x 16 queries] = K[16 x 32] . Q^T[32 x 16]
// so that each lane ends up holding scores of ONE query (column lane % 16),
// which makes the softmax statistics per lane. The output is accumulated as
//   O^T[16 channels x 16 queries] += V^T[16 x 32 keys] . P^T[32 keys x 16].
// The rows of the key tiles are permuted so that lane group g = lane / 16
// holds the scores of keys 8g..8g+7 of every 32-key step; those eight
// probabilities are exactly the eight contraction slots that lane supplies as
// the P^T operand of the next product, so P never leaves registers. Likewise
// the channel rows of the V^T tiles are permuted so that each lane owns eight
// consecutive output channels (one 16-byte store per lane).
//
// Only the contraction slots' pairing between the A and B operands matters to
// an MFMA, and both operands here are filled with the same (lane group, slot)
// -> (channel or key) map, so the code does not depend on how the hardware
// orders the slots inside the contraction.
//
// bf16: v_mfma_f32_16x16x32_bf16, P rounded to bf16 for the P.V product, fp32
// accumulation and softmax. fp32: eight v_mfma_f32_16x16x4_f32 per 32-deep
// contraction, P kept in fp32.
#include "bra_internal.h"

#include <math.h>

namespace bra {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx8 __attribute__((ext_vector_type(8)));

constexpr int KC = 64;      // keys per LDS chunk
constexpr int D = kHeadDim; // 32
constexpr int NW = 4;       // waves per workgroup
constexpr int MAXU = 2;     // units per wave
constexpr int QB = 64;      // queries per workgroup (<= 4 tiles of 16)

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
  __device__ static inline op8 from_f32(const float* v) {
    op8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (__bf16)v[e];
    return r;
  }
  __device__ static inline op8 zero() {
    op8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (__bf16)0.0f;
    return r;
  }
  __device__ static inline void store8(__bf16* p, const float* v) {
    *reinterpret_cast<op8*>(p) = from_f32(v);
  }
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
  __device__ static inline void store8(float* p, const float* v) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
};

struct AttnParams {
  const void* Q;
  const void* K;
  const void* V;
  const int32_t* idx;
  void* O;
  int H, W, C, S, topk;
  int sh, sw, n, R, kv;
  int heads;
  int nqb;   // query blocks per region
  int HG;    // heads per workgroup
  int nhg;   // head groups
  float c;   // softmax scale * log2(e)
};

__device__ inline float wave_max_groups(float v) {
  // max over the 4 lane groups that share lane % 16
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  v = fmaxf(v, __shfl_xor(v, 32, 64));
  return v;
}

__device__ inline float wave_sum_groups(float v) {
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}

template <typename T>
__global__ __launch_bounds__(256) void attend_kernel(AttnParams p) {
  typedef Tr<T> TT;
  typedef typename TT::op8 op8;
  constexpr int VEC = TT::VEC;

  extern __shared__ __align__(16) unsigned char smem_raw[];
  __shared__ int sidx[kMaxRegions];
  __shared__ int sbad;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int g = lane >> 4;      // lane group: contraction slots 8g..8g+7
  const int col = lane & 15;    // query column of the 16-query tile

  int w = blockIdx.x;
  const int hg = w % p.nhg;  w /= p.nhg;
  const int qb = w % p.nqb;  w /= p.nqb;
  const int i = w % p.R;
  const int b = w / p.R;

  const int q0 = qb * QB;
  const int nq = min(QB, p.n - q0);
  const int ntiles = (nq + 15) >> 4;
  const int h0 = hg * p.HG;
  const int nh = min(p.HG, p.heads - h0);
  const int HGC = nh * D;             // channels this workgroup touches
  const int cb = h0 * D;              // first channel
  const int U = nh * ntiles;          // units
  const int ldk = p.HG * D + TT::PADK;   // LDS row stride of K (elements)
  const int ldv = KC + TT::PADV;         // LDS row stride of V^T (elements)
  T* Ks = reinterpret_cast<T*>(smem_raw);
  T* Vt = Ks + KC * ldk;

  const T* Qg = static_cast<const T*>(p.Q);
  const T* Kg = static_cast<const T*>(p.K);
  const T* Vg = static_cast<const T*>(p.V);
  T* Og = static_cast<T*>(p.O);

  // routing row of region i
  if (tid == 0) sbad = 0;
  __syncthreads();
  for (int j = tid; j < p.topk; j += blockDim.x) {
    const int r = p.idx[((int64_t)b * p.R + i) * p.topk + j];
    const bool ok = r >= 0 && r < p.R;
    sidx[j] = ok ? r : 0;
    if (!ok) sbad = 1;
  }
  __syncthreads();

  const int ri = i / p.S, rj = i - (i / p.S) * p.S;
  // per-unit state
  op8 qop[MAXU];
  floatx4 acc[MAXU][2];
  float m[MAXU], lsum[MAXU];
  int64_t qoff[MAXU];
  bool qvalid[MAXU];
#pragma unroll
  for (int uu = 0; uu < MAXU; ++uu) {
    const int u = wave + NW * uu;
    const int hl = u / max(ntiles, 1);
    const int t = u - hl * ntiles;
    const int qi = q0 + t * 16 + col;
    qvalid[uu] = (u < U) && (qi < q0 + nq);
    qoff[uu] = 0;
    if (qvalid[uu]) {
      const int qy = ri * p.sh + qi / p.sw;
      const int qx = rj * p.sw + (qi - (qi / p.sw) * p.sw);
      qoff[uu] = (((int64_t)b * p.H + qy) * p.W + qx) * p.C + cb + hl * D + 8 * g;
      qop[uu] = TT::load8(Qg + qoff[uu]);
    } else {
      qop[uu] = TT::zero();
    }
    acc[uu][0] = floatx4{0.f, 0.f, 0.f, 0.f};
    acc[uu][1] = floatx4{0.f, 0.f, 0.f, 0.f};
    m[uu] = -INFINITY;
    lsum[uu] = 0.f;
  }

  if (sbad) {
    // a routing entry outside [0, S*S): never dereferenced; output NaN
    float nanv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) nanv[e] = __builtin_nanf("");
#pragma unroll
    for (int uu = 0; uu < MAXU; ++uu)
      if (qvalid[uu]) TT::store8(Og + qoff[uu], nanv);
    return;
  }

  const int vpk = HGC / VEC;  // 16-byte vectors per key row
  for (int c0 = 0; c0 < p.kv; c0 += KC) {
    if (c0) __syncthreads();  // previous chunk fully consumed
    // ---- gather chunk: K rows as is, V transposed, through the routing table
    for (int f = tid; f < KC * vpk; f += blockDim.x) {
      const int kl = f / vpk;
      const int cv = f - kl * vpk;
      const int kappa = c0 + kl;
      uint4 kvv = make_uint4(0u, 0u, 0u, 0u);
      uint4 vvv = make_uint4(0u, 0u, 0u, 0u);
      if (kappa < p.kv) {
        const int jr = kappa / p.n;
        const int tk = kappa - jr * p.n;
        const int r = sidx[jr];
        const int ty = tk / p.sw;
        const int y = (r / p.S) * p.sh + ty;
        const int x = (r - (r / p.S) * p.S) * p.sw + (tk - ty * p.sw);
        const int64_t off = (((int64_t)b * p.H + y) * p.W + x) * p.C + cb + cv * VEC;
        kvv = *reinterpret_cast<const uint4*>(Kg + off);
        vvv = *reinterpret_cast<const uint4*>(Vg + off);
      }
      *reinterpret_cast<uint4*>(Ks + kl * ldk + cv * VEC) = kvv;
      const T* ve = reinterpret_cast<const T*>(&vvv);
#pragma unroll
      for (int e = 0; e < VEC; ++e) Vt[(cv * VEC + e) * ldv + kl] = ve[e];
    }
    __syncthreads();

    const int nvalid = min(KC, p.kv - c0);
#pragma unroll
    for (int uu = 0; uu < MAXU; ++uu) {
      const int u = wave + NW * uu;
      if (u >= U) continue;  // wave-uniform
      const int hl = u / ntiles;
      // ---- scores S^T for 64 keys: two 32-key steps, two 16-row tiles each
      float s[KC / 32][8];
      const int rr = col;  // MFMA row supplied by this lane
      const int krow = 8 * (rr >> 2) + (rr & 3);  // key row of tile a; tile b is +4
#pragma unroll
      for (int st = 0; st < KC / 32; ++st) {
        const op8 ka = TT::load8(Ks + (st * 32 + krow) * ldk + hl * D + 8 * g);
        const op8 kb = TT::load8(Ks + (st * 32 + krow + 4) * ldk + hl * D + 8 * g);
        const floatx4 sa = TT::mma(ka, qop[uu], floatx4{0.f, 0.f, 0.f, 0.f});
        const floatx4 sb = TT::mma(kb, qop[uu], floatx4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s[st][e] = sa[e];
          s[st][4 + e] = sb[e];
        }
      }
      // lane group g holds keys st*32 + 8g + e, e = 0..7
      float mx = -INFINITY;
#pragma unroll
      for (int st = 0; st < KC / 32; ++st)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if (st * 32 + 8 * g + e >= nvalid) s[st][e] = -INFINITY;
          mx = fmaxf(mx, s[st][e]);
        }
      mx = wave_max_groups(mx);
      const float mnew = fmaxf(m[uu], mx);
      const float mc = mnew * p.c;
      const float alpha = __builtin_amdgcn_exp2f(m[uu] * p.c - mc);
      float ps = 0.f;
#pragma unroll
      for (int st = 0; st < KC / 32; ++st)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(s[st][e], p.c, -mc));
          s[st][e] = pe;
          ps += pe;
        }
      lsum[uu] = __builtin_fmaf(lsum[uu], alpha, ps);
      m[uu] = mnew;
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) acc[uu][ct] *= alpha;
      // ---- O^T += V^T P^T
      const int vrow = 8 * (rr >> 2) + (rr & 3);  // channel row of tile 0; tile 1 is +4
#pragma unroll
      for (int st = 0; st < KC / 32; ++st) {
        const op8 pop = TT::from_f32(s[st]);
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          const op8 va = TT::load8(Vt + (hl * D + vrow + 4 * ct) * ldv + st * 32 + 8 * g);
          acc[uu][ct] = TT::mma(va, pop, acc[uu][ct]);
        }
      }
    }
  }

  // ---- normalise and store: lane holds channels 8g..8g+7 of its query
#pragma unroll
  for (int uu = 0; uu < MAXU; ++uu) {
    const int u = wave + NW * uu;
    if (u >= U) continue;
    const float l = wave_sum_groups(lsum[uu]);
    const float inv = 1.0f / l;
    float o[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      o[e] = acc[uu][0][e] * inv;
      o[4 + e] = acc[uu][1][e] * inv;
    }
    if (qvalid[uu]) TT::store8(Og + qoff[uu], o);
  }
}

}  // namespace

hipError_t launch_attend(const void* Q, const void* K, const void* V,
                         const int32_t* idx, void* O, const Shape& s, int dtype,
                         hipStream_t stream) {
  AttnParams p;
  p.Q = Q; p.K = K; p.V = V; p.idx = idx; p.O = O;
  p.H = s.H; p.W = s.W; p.C = s.C; p.S = s.S; p.topk = s.topk;
  p.sh = s.sh; p.sw = s.sw; p.n = s.n; p.R = s.R; p.kv = s.kv;
  p.heads = s.heads;
  p.nqb = (s.n + QB - 1) / QB;
  const int qtiles = (min(s.n, QB) + 15) / 16;
  const int cap = dtype == kBF16 ? 4 : 2;  // keeps LDS at or below 64 KiB
  int HG = (NW * MAXU) / qtiles;
  if (HG > cap) HG = cap;
  if (HG > s.heads) HG = s.heads;
  if (HG < 1) HG = 1;
  p.HG = HG;
  p.nhg = (s.heads + HG - 1) / HG;
  p.c = 1.4426950408889634f / sqrtf((float)s.d);
  const size_t esz = dtype == kBF16 ? 2 : 4;
  const int padk = dtype == kBF16 ? Tr<__bf16>::PADK : Tr<float>::PADK;
  const int padv = dtype == kBF16 ? Tr<__bf16>::PADV : Tr<float>::PADV;
  const size_t lds = esz * ((size_t)KC * (HG * D + padk) + (size_t)HG * D * (KC + padv));
  const int64_t nwg = (int64_t)s.B * s.R * p.nqb * p.nhg;
  dim3 grid((unsigned)nwg);
  void* args[] = {&p};
  if (dtype == kBF16)
    return hipLaunchKernel(reinterpret_cast<const void*>(&attend_kernel<__bf16>), grid, dim3(NW * 64), args, lds, stream);
  return hipLaunchKernel(reinterpret_cast<const void*>(&attend_kernel<float>), grid, dim3(NW * 64), args, lds, stream);
}

}  // namespace bra
