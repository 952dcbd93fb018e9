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

#include <algorithm>

namespace bra {
namespace {

constexpr int kTokBlock = 64;  // tokens per block
constexpr int kQkvWaves = 8;   // waves per workgroup (at most)
constexpr int kXLoads = 2;     // X-row loads in flight per thread

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
  int B;
  int rpw;      // regions per workgroup (n <= 64), else 1
  int nsub;     // 64-token blocks per region (n > 64), else 1
  int ngroups;  // workgroups per image
  int nfg;      // feature groups (3C / 32)
  int nunits;   // persistent form: images x groups
  int end_mask; // persistent form: bit t set when a region ends with 16-token tile t
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

// Sum of v over aligned runs of `seg` lanes (seg = 1, 2, 4, 8 or 16) inside
// each row of 16 lanes, with DPP moves (no LDS traffic): quad permutes for
// pairs and quads, then the half-row and row mirrors, which pair every lane
// with one of the other half. The run's first lane reads the sum. (Every
// source lane lies in the row, so the out-of-row setting never applies; it is
// set so the moves fuse into the adds.)
template <int SEG>
__device__ __forceinline__ float run_sum(float v) {
  constexpr int seg = SEG;
  if (seg >= 2) v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));  // quad_perm 1,0,3,2
  if (seg >= 4) v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));  // quad_perm 2,3,0,1
  if (seg >= 8) v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, true)); // row_half_mirror
  if (seg >= 16) v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, true)); // row_mirror
  return v;
}

// SEG > 0: the region size n is a multiple of 16 or divides 16, so the tokens
// of one region inside a 16-token tile are aligned runs of SEG = min(n, 16)
// lanes and their sums come from DPP moves across those lanes. SEG = 0: the
// rounded values go through a per-wave LDS tile and are summed from there.
template <typename T, int SEG>
__global__ __launch_bounds__(512) void qkv_pool_kernel(QkvParams p) {
  typedef Tr<T> TT;
  typedef typename TT::op8 op8;
  constexpr int VEC = TT::VEC;
  constexpr int KPF = 2;  // k-steps whose weight operands are loaded together
  const int LDX = p.C + 16 / (int)sizeof(T);  // X rows in LDS, 16-byte pad
  extern __shared__ __align__(16) unsigned char smem_raw[];
  T* xs = reinterpret_cast<T*>(smem_raw);                                      // [64][LDX]
  float* pool = reinterpret_cast<float*>(xs + kTokBlock * LDX);                 // [rpw][2C] sums
  float* ptile = pool + p.rpw * 2 * p.C + (threadIdx.x >> 6) * kTokBlock * 33;  // SEG = 0: wave's [64][33]

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
  constexpr bool BFLY = SEG > 0;
  for (int sub = 0; sub < p.nsub; ++sub) {
    __syncthreads();  // previous block's X rows consumed
    // X rows of the block: every load of a thread issued before any store
    for (int f0 = 0; f0 < kTokBlock * cvec; f0 += kXLoads * blockDim.x) {
      uint4 xv[kXLoads];
#pragma unroll
      for (int m = 0; m < kXLoads; ++m) {
        const int f = f0 + m * blockDim.x + tid;
        const int tw = f / cvec, cv = f - tw * cvec;
        const int t = (f < kTokBlock * cvec && tw < ntok)
                          ? block_token(sub, tw, r0, nreg, p.nsub, p.n, p.sh, p.sw, p.W, p.div_n, p.div_sw, p.div_S)
                          : -1;
        xv[m] = make_uint4(0u, 0u, 0u, 0u);
        if (t >= 0) xv[m] = *reinterpret_cast<const uint4*>(Xg + t * p.C + cv * VEC);
      }
#pragma unroll
      for (int m = 0; m < kXLoads; ++m) {
        const int f = f0 + m * blockDim.x + tid;
        if (f < kTokBlock * cvec) {
          const int tw = f / cvec, cv = f - tw * cvec;
          *reinterpret_cast<uint4*>(xs + tw * LDX + cv * VEC) = xv[m];
        }
      }
    }
    __syncthreads();
    for (int fg = wave; fg < p.nfg; fg += nw) {
      // A rows: row rr = col of feature tile ct is feature 32 fg + 8 (rr/4) +
      // (rr%4) + 4 ct, so lane group g ends with features 8g..8g+7
      const int frow = fg * 32 + 8 * (col >> 2) + (col & 3);
      floatx4 acc[4][2];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) acc[mt][ct] = floatx4{0.f, 0.f, 0.f, 0.f};
      for (int k0 = 0; k0 < ks_n; k0 += KPF) {
        op8 wa[KPF], wb[KPF];
#pragma unroll
        for (int kk = 0; kk < KPF; ++kk) {
          wa[kk] = TT::zero();
          wb[kk] = TT::zero();
          if (k0 + kk < ks_n) {
            wa[kk] = TT::load8(Wg + (frow + 0) * p.C + (k0 + kk) * 32 + 8 * g);
            wb[kk] = TT::load8(Wg + (frow + 4) * p.C + (k0 + kk) * 32 + 8 * g);
          }
        }
#pragma unroll
        for (int kk = 0; kk < KPF; ++kk) {
          if (k0 + kk >= ks_n) break;  // uniform
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) {  // rows past the block are zeros in LDS
            const op8 xb = TT::load8(xs + (mt * 16 + col) * LDX + (k0 + kk) * 32 + 8 * g);
            acc[mt][0] = TT::mma(wa[kk], xb, acc[mt][0]);
            acc[mt][1] = TT::mma(wb[kk], xb, acc[mt][1]);
          }
        }
      }
      // epilogue: bias, one rounding, store; Q/K groups also sum the rounded
      // values per region
      const int feat = fg * 32 + 8 * g;  // lane's first feature
      const int tensor = feat / p.C, ch = feat - tensor * p.C;
      const bool pooled = fg * 32 < 2 * p.C;  // uniform
      float bv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) bv[e] = Bg ? (float)Bg[feat + e] : 0.f;
      T* dst = static_cast<T*>(tensor == 0 ? p.Q : tensor == 1 ? p.K : p.V) + img;
#pragma unroll 1
      for (int mt = 0; mt < 4; ++mt) {
        const int twl = mt * 16 + col;
        const int t = twl < ntok ? block_token(sub, twl, r0, nreg, p.nsub, p.n, p.sh, p.sw, p.W, p.div_n, p.div_sw, p.div_S)
                                 : -1;
        float o[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o[e] = acc[mt][0][e] + bv[e];
          o[4 + e] = acc[mt][1][e] + bv[4 + e];
        }
        const op8 r = TT::from_f32(o);  // the rounded outputs
        if (t >= 0) *reinterpret_cast<op8*>(dst + t * p.C + ch) = r;
        if (pooled) {
          float v[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = t >= 0 ? (float)r[e] : 0.f;
          if (BFLY) {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = run_sum<SEG>(v[e]);
            // the first lane of each run holds its region's sum for this tile
            const int tw = mt * 16 + col;
            if ((col & (SEG - 1)) == 0 && tw < ntok) {
              const int j = p.nsub > 1 ? 0 : tw / p.n;
#pragma unroll
              for (int e = 0; e < 8; ++e) pool[j * 2 * p.C + feat + e] += v[e];
            }
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) ptile[(mt * 16 + col) * 33 + 8 * g + e] = v[e];
          }
        }
      }
      if (!BFLY && pooled) {
        // region sums from the wave's tile, (region, feature) pairs over the
        // lanes, tokens in order in 4 interleaved partial sums
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
        for (int jf = lane; jf < p.rpw * 32; jf += 64) {
          const int j = jf >> 5, f = jf & 31;
          const int a = p.nsub > 1 ? 0 : j * p.n, z = min(ntok, p.nsub > 1 ? ntok : (j + 1) * p.n);
          float s4[4] = {0.f, 0.f, 0.f, 0.f};
          int tw = a;
          for (; tw + 4 <= z; tw += 4)
#pragma unroll
            for (int u = 0; u < 4; ++u) s4[u] += ptile[(tw + u) * 33 + f];
          for (; tw < z; ++tw) s4[0] += ptile[tw * 33 + f];
          if (a < z) pool[j * 2 * p.C + fg * 32 + f] += (s4[0] + s4[1]) + (s4[2] + s4[3]);
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
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

// Persistent form (bf16, C <= 128, regions of at most 64 tokens whose runs
// align with 16-token tiles): the grid is sized to the machine and every
// workgroup walks units (image, region group) u, u + gridDim.x, ... Each
// wave owns one feature group of 32 outputs (3C/32 waves) and loads its
// weight rows and bias once, keeping them in registers; X blocks alternate
// between two LDS buffers, the next block's loads in flight while the current
// one is computed (one barrier per block); region sums stay in the run
// leader's registers and are written as means when the region is complete.
//
// Token geometry that is the same for every unit is decoded once per thread:
// a token of slot tw of a unit lies in the unit's region slot j = tw / n at
// offset q = tw % n inside that region, and j is kept split as j = jy S + jx,
// so the region of slot j follows from the unit's first region (ry0, rx0)
// with one carry and no division.
constexpr int kPersistKS = 4;  // k-steps kept in registers (C <= 128)
constexpr int kPersistMaxWaves = 3 * kPersistKS;  // one wave per feature group of 32 outputs
constexpr int kTilesPerStep = 2;  // 16-token tiles per products + epilogue step
constexpr int kPersistXL = 4;  // X loads per thread per block (the host checks they cover it)

// packed slot word: bits 0-10 LDS vector index (element offset / 8), 11-16 jx,
// 17-22 jy, 23-29 j (kNoSlot: no token)
constexpr int kNoSlot = 127;

__device__ __forceinline__ int slot_j(int w) { return (w >> 23) & 127; }
__device__ __forceinline__ int slot_v8(int w) { return w & 2047; }

// First token (index inside the image) of the region in slot w's region slot
__device__ __forceinline__ int slot_region_token(int w, int ry0, int rx0, const QkvParams& p) {
  int rx = rx0 + ((w >> 11) & 63), ry = ry0 + ((w >> 17) & 63);
  if (rx >= p.S) {
    rx -= p.S;
    ++ry;
  }
  return ry * p.sh * p.W + rx * p.sw;
}

__device__ __forceinline__ int pack_slot(int v8, int j, int S) {
  if (j >= kNoSlot) return kNoSlot << 23;
  const int jy = j / S, jx = j - jy * S;  // j < 64: jx, jy < 64
  return v8 | (jx << 11) | (jy << 17) | (j << 23);
}

// The unit's image, first region (and its region row and column) and count
struct UnitGeo {
  int b, r0, nreg, ry0, rx0;
};
// (a unit past the last has no regions)
__device__ __forceinline__ UnitGeo unit_geo(int u, const QkvParams& p) {
  UnitGeo q;
  q.b = u / p.ngroups;
  q.r0 = (u - q.b * p.ngroups) * p.rpw;
  q.nreg = u < p.nunits ? min(p.rpw, p.R - q.r0) : 0;
  q.ry0 = q.r0 / p.S;
  q.rx0 = q.r0 - q.ry0 * p.S;
  return q;
}

// Raw buffer accesses. A lane with nothing to load or store uses an offset
// past the buffer's range: the buffer unit returns zeros for such a load and
// drops such a store, so every load and store instruction is issued
// unconditionally. That keeps the number of memory operations after the X
// prefetch fixed, so the wait for the prefetch at the top of the next unit
// does not also wait for this unit's output stores (vector memory counters
// count stores too).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kRawBufferWord3 = 0x00020000;  // raw (untyped) access, 32-bit data format
constexpr int kOutOfRange = (int)0x80000000u;  // past every range the host allows (< 2^31 bytes)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_buffer(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRawBufferWord3);
}

// This thread's X loads of a unit (zeros for slots with no token)
__device__ __forceinline__ void persist_load_x(const QkvParams& p, const UnitGeo& q,
                                               const int (&xoff)[kPersistXL], const int (&xslot)[kPersistXL],
                                               uint4 (&xr)[kPersistXL]) {
  const uint32_t img_bytes = (uint32_t)p.H * p.W * p.C * 2u;
  const __amdgpu_buffer_rsrc_t rx =
      raw_buffer(static_cast<const __bf16*>(p.X) + (int64_t)min(q.b, p.B - 1) * p.H * p.W * p.C, img_bytes);
#pragma unroll
  for (int m = 0; m < kPersistXL; ++m) {
    const bool ok = slot_j(xslot[m]) < q.nreg;
    const int off = ok ? (slot_region_token(xslot[m], q.ry0, q.rx0, p) * p.C + xoff[m]) * 2 : kOutOfRange;
    xr[m] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0));
  }
}

template <int KSM, int SEG, int PD>
__global__ __launch_bounds__(kPersistMaxWaves * 64) void qkv_pool_persistent(QkvParams p) {
  constexpr int FPW = 1;  // feature groups per wave
  typedef Tr<__bf16> TT;
  typedef TT::op8 op8;
  const int LDX = p.C + 8;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  __bf16* xbuf = reinterpret_cast<__bf16*>(smem_raw);  // [2][64][LDX]

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4, col = lane & 15;
  const int nthr = blockDim.x;
  const int ks_n = p.C / 32;
  const int cvec = p.C / 8;
  const int total = p.nunits;
  const __bf16* Wg = static_cast<const __bf16*>(p.Wt);
  const __bf16* Bg = static_cast<const __bf16*>(p.bias);

  // the wave's feature groups: weight rows (A operands) and bias, kept
  op8 wa[FPW][KSM], wb[FPW][KSM];
  float bv[FPW][8];
#pragma unroll
  for (int fi = 0; fi < FPW; ++fi) {
    const int fg = wave * FPW + fi;
    const int frow = fg * 32 + 8 * (col >> 2) + (col & 3);
#pragma unroll
    for (int ks = 0; ks < KSM; ++ks) {
      wa[fi][ks] = TT::zero();
      wb[fi][ks] = TT::zero();
      if (fg < p.nfg && ks < ks_n) {
        wa[fi][ks] = TT::load8(Wg + (frow + 0) * p.C + ks * 32 + 8 * g);
        wb[fi][ks] = TT::load8(Wg + (frow + 4) * p.C + ks * 32 + 8 * g);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) bv[fi][e] = (Bg && fg < p.nfg) ? (float)Bg[fg * 32 + 8 * g + e] : 0.f;
  }

  // this thread's X loads: image offset past the region's first token, slot
  int xoff[kPersistXL], xslot[kPersistXL];
#pragma unroll
  for (int m = 0; m < kPersistXL; ++m) {
    const int f = tid + m * nthr;
    const int tw = f / cvec, cv = f - tw * cvec;
    const int q = tw % p.n, qy = q / p.sw, qx = q - qy * p.sw;
    xoff[m] = (qy * p.W + qx) * p.C + cv * 8;
    xslot[m] = pack_slot((tw * LDX + cv * 8) >> 3, f < kTokBlock * cvec ? tw / p.n : kNoSlot, p.S);
  }
  // this lane's output tokens (slot mt * 16 + col): offset past the region's
  // first token, slot. With runs of 16 (n a multiple of 16) a tile lies in one
  // region, so its region slot is uniform (sj, split as sjy S + sjx) and the
  // region's address is scalar arithmetic.
  int eoff[4], eslot[4], sj[4], sjx[4], sjy[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int tw = mt * 16 + col;
    const int q = tw % p.n, qy = q / p.sw, qx = q - qy * p.sw;
    eoff[mt] = (qy * p.W + qx) * p.C;
    eslot[mt] = pack_slot(0, tw / p.n, p.S);
    sj[mt] = (mt * 16) / p.n;
    sjy[mt] = sj[mt] / p.S;
    sjx[mt] = sj[mt] - sjy[mt] * p.S;
  }

  // X rows of this thread's slots into buffer `bufi` of LDS
  auto stage_x = [&](int bufi, const uint4 (&v)[kPersistXL]) {
    __bf16* xs = xbuf + bufi * kTokBlock * LDX;
#pragma unroll
    for (int m = 0; m < kPersistXL; ++m)
      if (slot_j(xslot[m]) != kNoSlot) *reinterpret_cast<uint4*>(xs + slot_v8(xslot[m]) * 8) = v[m];
  };
  // X rows are loaded PD units ahead. PD = 1: xr receives the next unit's
  // rows during this unit. PD = 2: xr holds the next unit's rows (loaded
  // during the previous unit) and xn receives the rows of the unit after it.
  uint4 xr[kPersistXL], xn[PD == 2 ? kPersistXL : 1];
  int u = blockIdx.x;
  UnitGeo cur = unit_geo(u, p), nxt = unit_geo(u + gridDim.x, p);
  persist_load_x(p, cur, xoff, xslot, xr);
  stage_x(0, xr);
  if constexpr (PD == 2) persist_load_x(p, nxt, xoff, xslot, xr);
  int buf = 0;
  for (; u < total; u += gridDim.x, buf ^= 1) {
    // buffer `buf` holds this unit's X rows; every wave is done with the other
    // buffer (the previous unit), which receives the next unit's rows at the
    // end of this iteration, after this unit's stores (so waiting for those
    // loads there does not wait for the stores, nor for loads issued later)
    __syncthreads();
    const __bf16* xs = xbuf + buf * kTokBlock * LDX;
    UnitGeo nn;
    if constexpr (PD == 2) {
      nn = unit_geo(u + 2 * gridDim.x, p);
      persist_load_x(p, nn, xoff, xslot, xn);
    } else {
      persist_load_x(p, nxt, xoff, xslot, xr);
    }

    const int b = cur.b, r0 = cur.r0, nreg = cur.nreg, ry0 = cur.ry0, rx0 = cur.rx0;
    const int64_t img = (int64_t)b * p.H * p.W * p.C;
    const uint32_t img_bytes = (uint32_t)p.H * p.W * p.C * 2u;
    const uint32_t mean_bytes = (uint32_t)p.R * p.C * 4u;
#pragma unroll
    for (int fi = 0; fi < FPW; ++fi) {
      // a wave past the last feature group computes on zero weights and its
      // stores go out of range (no branch: the store count stays fixed)
      const bool fvalid = wave * FPW + fi < p.nfg;  // uniform
      const int fg = fvalid ? wave * FPW + fi : p.nfg - 1;
      const int feat = fg * 32 + 8 * g;
      const int tensor = fg * 32 / p.C;  // uniform: the wave's 32 features lie in one of Q, K, V
      const int ch = feat - tensor * p.C;
      const bool pooled = fvalid && tensor < 2;  // uniform
      const __amdgpu_buffer_rsrc_t rdst =
          raw_buffer(static_cast<__bf16*>(tensor == 0 ? p.Q : tensor == 1 ? p.K : p.V) + img, img_bytes);
      const float inv = 1.0f / (float)p.n;
      float racc[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) racc[e] = 0.f;
      // steps of kTilesPerStep 16-token tiles: products, then their epilogue
      // (only one step's accumulators live at a time, and a step's epilogue
      // overlaps the next step's products)
#pragma unroll
      for (int hh = 0; hh < 4 / kTilesPerStep; ++hh) {
      floatx4 acc[kTilesPerStep][2];  // accumulated onto the bias
#pragma unroll
      for (int m2 = 0; m2 < kTilesPerStep; ++m2) {
        acc[m2][0] = floatx4{bv[fi][0], bv[fi][1], bv[fi][2], bv[fi][3]};
        acc[m2][1] = floatx4{bv[fi][4], bv[fi][5], bv[fi][6], bv[fi][7]};
      }
#pragma unroll
      for (int ks = 0; ks < KSM; ++ks) {
        if (ks >= ks_n) break;  // uniform
#pragma unroll
        for (int m2 = 0; m2 < kTilesPerStep; ++m2) {  // rows past the block are zeros
          const int mt = kTilesPerStep * hh + m2;
          const op8 xb = TT::load8(xs + (mt * 16 + col) * LDX + ks * 32 + 8 * g);
          acc[m2][0] = TT::mma(wa[fi][ks], xb, acc[m2][0]);
          acc[m2][1] = TT::mma(wb[fi][ks], xb, acc[m2][1]);
        }
      }
#pragma unroll
      for (int m2 = 0; m2 < kTilesPerStep; ++m2) {
        const int mt = kTilesPerStep * hh + m2;
        int j, rtok;  // the lane's region slot and the region's first token
        if constexpr (SEG == 16) {
          j = sj[mt];
          int rx = rx0 + sjx[mt], ry = ry0 + sjy[mt];
          if (rx >= p.S) {
            rx -= p.S;
            ++ry;
          }
          rtok = ry * p.sh * p.W + rx * p.sw;
        } else {
          j = slot_j(eslot[mt]);
          rtok = slot_region_token(eslot[mt], ry0, rx0, p);
        }
        const bool ok = j < nreg;
        float o[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o[e] = acc[m2][0][e];
          o[4 + e] = acc[m2][1][e];
        }
        const op8 r = TT::from_f32(o);  // the rounded outputs
        const int soff = ok && fvalid ? rtok * p.C * 2 + (eoff[mt] + ch) * 2 : kOutOfRange;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, r), rdst, soff, 0, 0);
        if (pooled) {
          // a run that is not a region of this unit sums garbage that is never written
#pragma unroll
          for (int e = 0; e < 8; ++e) racc[e] += (float)r[e];
          // a region ends at its run's end (SEG < 16) or with its last
          // 16-token tile; its run leader then holds the sum
          if ((p.end_mask >> mt) & 1) {
#pragma unroll
            for (int e = 0; e < 8; ++e) racc[e] = run_sum<SEG>(racc[e]) * inv;
            const __amdgpu_buffer_rsrc_t rmean =
                raw_buffer((tensor == 0 ? p.Qr : p.Kr) + (int64_t)b * p.R * p.C, mean_bytes);
            const int moff = ((col & (SEG - 1)) == 0 && ok) ? (r0 + j) * p.C * 4 + ch * 4 : kOutOfRange;
            __builtin_amdgcn_raw_buffer_store_b128(
                __builtin_bit_cast(u32x4, make_float4(racc[0], racc[1], racc[2], racc[3])), rmean, moff, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b128(
                __builtin_bit_cast(u32x4, make_float4(racc[4], racc[5], racc[6], racc[7])), rmean,
                moff == kOutOfRange ? kOutOfRange : moff + 16, 0, 0);
#pragma unroll
            for (int e = 0; e < 8; ++e) racc[e] = 0.f;
          }
        }
      }
      }  // hh
    }
    stage_x(buf ^ 1, xr);
    cur = nxt;
    if constexpr (PD == 2) {
#pragma unroll
      for (int m = 0; m < kPersistXL; ++m) xr[m] = xn[m];
      nxt = nn;
    } else {
      nxt = unit_geo(u + 2 * gridDim.x, p);
    }
  }
}

}  // namespace

hipError_t launch_qkv_pool(const void* X, const void* Wqkv, const void* bqkv, void* Q, void* K, void* V, float* Qr,
                           float* Kr, const Shape& s, int dtype, hipStream_t stream) {
  QkvParams p;
  p.X = X; p.Wt = Wqkv; p.bias = bqkv; p.Q = Q; p.K = K; p.V = V; p.Qr = Qr; p.Kr = Kr;
  p.H = s.H; p.W = s.W; p.C = s.C; p.S = s.S; p.sh = s.sh; p.sw = s.sw; p.n = s.n; p.R = s.R; p.B = s.B;
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
  p.nunits = (int)nwg;
  // persistent form: bf16, C <= 128, regions of <= 64 tokens in aligned runs
  const int seg0 = s.n % 16 == 0 ? 16 : (s.n < 16 && 16 % s.n == 0) ? s.n : 0;
  const int pwaves = p.nfg;  // one wave per feature group
  const bool covered = pwaves * 64 * kPersistXL >= kTokBlock * (s.C / 8);
  // (raw buffer offsets: one image's bytes below 2^31)
  // (unit indices up to two grid strides past the last unit stay below 2^31)
  const bool fits = 2 * (int64_t)s.H * s.W * s.C < (int64_t(1) << 31) && nwg < (int64_t(1) << 30);
  if (dtype == kBF16 && s.C <= 32 * kPersistKS && s.n <= kTokBlock && seg0 > 0 && covered && fits) {
    const int waves = pwaves;
    const size_t lds = 2 * sizeof(__bf16) * kTokBlock * (s.C + 8);
    p.end_mask = 0;
    for (int t = 0; t < 4; ++t)
      if (seg0 < 16 || ((t + 1) * 16) % s.n == 0) p.end_mask |= 1 << t;
    // X prefetched one unit ahead for C <= 64 and two for C > 64 (measured:
    // 56x56 C=64 34.5 vs 39.1 us with two; 28x28 C=128 25.6 vs 26.9 us)
    const void* k2[] = {(const void*)&qkv_pool_persistent<2, 1, 1>, (const void*)&qkv_pool_persistent<2, 2, 1>,
                        (const void*)&qkv_pool_persistent<2, 4, 1>, (const void*)&qkv_pool_persistent<2, 8, 1>,
                        (const void*)&qkv_pool_persistent<2, 16, 1>};
    const void* k4[] = {(const void*)&qkv_pool_persistent<4, 1, 2>, (const void*)&qkv_pool_persistent<4, 2, 2>,
                        (const void*)&qkv_pool_persistent<4, 4, 2>, (const void*)&qkv_pool_persistent<4, 8, 2>,
                        (const void*)&qkv_pool_persistent<4, 16, 2>};
    const void* fn = (s.C <= 64 ? k2 : k4)[__builtin_ctz(seg0)];
    // as many workgroups as fit at once, each walking many units
    int dev = 0, ncu = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, waves * 64, lds) != hipSuccess)
      return hipErrorInvalidValue;
    const int grid = (int)std::min<int64_t>(nwg, (int64_t)ncu * std::max(1, per_cu));
    void* args[] = {&p};
    return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(waves * 64), args, lds, stream);
  }
  const int waves = p.nfg < kQkvWaves ? p.nfg : kQkvWaves;
  const size_t esz = dtype == kBF16 ? 2 : 4;
  // lanes per region run inside a 16-token tile, 0 when runs do not align
  const int seg = s.n % 16 == 0 ? 16 : (s.n < 16 && 16 % s.n == 0) ? s.n : 0;
  const size_t lds = esz * kTokBlock * (s.C + 16 / esz) + sizeof(float) * p.rpw * 2 * s.C +
                     (seg ? 0 : sizeof(float) * waves * kTokBlock * 33);
  const void* fn;
  if (dtype == kBF16) {
    const void* k[] = {(const void*)&qkv_pool_kernel<__bf16, 0>, (const void*)&qkv_pool_kernel<__bf16, 1>,
                       (const void*)&qkv_pool_kernel<__bf16, 2>, (const void*)&qkv_pool_kernel<__bf16, 4>,
                       (const void*)&qkv_pool_kernel<__bf16, 8>, (const void*)&qkv_pool_kernel<__bf16, 16>};
    fn = k[seg == 0 ? 0 : 1 + __builtin_ctz(seg)];
  } else {
    const void* k[] = {(const void*)&qkv_pool_kernel<float, 0>, (const void*)&qkv_pool_kernel<float, 1>,
                       (const void*)&qkv_pool_kernel<float, 2>, (const void*)&qkv_pool_kernel<float, 4>,
                       (const void*)&qkv_pool_kernel<float, 8>, (const void*)&qkv_pool_kernel<float, 16>};
    fn = k[seg == 0 ? 0 : 1 + __builtin_ctz(seg)];
  }
  void* args[] = {&p};
  return hipLaunchKernel(fn, dim3((unsigned)nwg), dim3(waves * 64), args, lds, stream);
}

}  // namespace bra
