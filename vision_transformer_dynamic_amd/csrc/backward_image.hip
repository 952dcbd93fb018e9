// Backward of the token attention for small maps, in one launch: one
// workgroup per (image, head) holds the head's K, V, Q and dO for the whole
// image in LDS and computes dQ, dK and dV from there (explainer "BiFormer
// Reshapes Visual Attention with 'Bi-Level Routing'", Part 2.2 step 4 and
// pseudocode steps 6-7 for the forward; Part 7 for training throughput). The
// routing table is held fixed, so the gradients are those of softmax
// attention of every region's queries over its routed keys:
//
//   P = softmax(c' q k^T), dP = dO V_g^T, D = rowsum(dO * O),
//   dZ = P * (dP - D), dQ = scale * dZ K_g, dK_g = scale * dZ^T Q, dV_g = P^T dO
//
// with dK, dV of a token summed over every query region routed to its region.
//
// With small regions (4, 8 or 16 tokens) the routed sets of an image's query
// regions overlap heavily, and the per-region kernels (backward.hip) gather
// the same rows from the caches many times: at 14 x 14 with 2 x 2 regions and
// k = 16 every key region is read by 16 query regions in the dQ step and
// every query row by 16 key regions in the dK/dV step, and a key region of 4
// tokens fills 4 of the 16 key columns of a matrix tile. Here:
//
//  * Staging: the head's rows of K, V, Q and dO (64 bytes each) go to LDS in
//    region-major order, position = region * n + token, so a region's tokens
//    are n consecutive positions and the 16 positions 16u .. 16u + 15 are
//    16 / n whole regions ("unit" u). The routing table becomes each routed
//    region's first position, one 64-bit mask per query region (its routed
//    regions) and one per key region (the good query regions routed to it).
//    A row with an entry outside [0, S*S) or a repeated entry is bad: its
//    queries get NaN dQ and are left out of dK and dV.
//  * Phase 1, per query unit (the forward image kernel's formulation): with
//    several regions side by side, region j's products use operands whose
//    columns outside region j are zero, so
//      S^T = sum_j K_j Q_j^T, dP^T = sum_j V_j dO_j^T, dQ^T = sum_j K_j^T dZ_j^T;
//    K_j^T comes from the K rows by gfx950's transposing LDS read. The log-sum-
//    exp and D of every query go to LDS for phase 2; dQ goes to memory.
//  * Phase 2, per key unit (16 keys of 16 / n key regions): the tiles are the
//    union of the unit's incoming query regions, 16 / n regions per 16-slot
//    tile, in ascending order. S = Q K^T and dP = dO V^T put each lane on one
//    key with 4 query slots; a (query region, key region) pair outside the
//    routing gets P = 0. dV^T += dO^T P and dK^T += Q^T dZ (16-deep products)
//    take dO^T and Q^T by the transposing read, so P and dZ never leave
//    registers. Each key's sums run in a fixed order: deterministic.
#include "bra_internal.h"
#include "attn_common.h"

#include <math.h>

#include <algorithm>

namespace bra {
namespace {

constexpr int kRowE = 40;  // LDS row stride in elements: a head's 32 channels + 16 bytes of pad
constexpr size_t kBwdImgMaxLds = 160 * 1024;

struct BwdImgParams {
  const __bf16* Q;
  const __bf16* K;
  const __bf16* V;
  const __bf16* O;
  const __bf16* dO;
  const int32_t* idx;
  __bf16* dQ;
  __bf16* dK;
  __bf16* dV;
  int H, W, C, S, topk, sh, sw, n, R, kv, heads;
  int HW;      // tokens per image
  int HW4;     // HW rounded up to 4 (the float arrays stay 16-byte aligned)
  int nunits;  // 16-position units per image
  float c;     // scale * log2(e)
  float scale; // 1 / sqrt(d)
  FastDiv div_n, div_sw, div_S, div_topk;
};

typedef __attribute__((address_space(3))) shortx4 lds_s4;

// Region-major position -> token offset inside the image.
__device__ inline int pos_token(const BwdImgParams& p, int pos) {
  int t, rx, tx;
  const int r = fdiv(pos, p.div_n, &t);
  const int ry = fdiv(r, p.div_S, &rx);
  const int ty = fdiv(t, p.div_sw, &tx);
  return (ry * p.sh + ty) * p.W + rx * p.sw + tx;
}

// Value v of lane src (src in [0, 64)).
__device__ inline int lane_value(int v, int src) { return __builtin_amdgcn_ds_bpermute(src << 2, v); }

// Transposing LDS read of 4 bf16 (8 bytes) at p: within each 16-lane group,
// lane j receives element j % 4 of the reads of lanes 4 s + j / 4, s = 0..3.
__device__ inline shortx4 read_tr(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(p));
}

// Region j of a tile packed as byte j of one word (0xFF: none), so that a
// lane-varying j is a shift and not an index into a private array (which
// would go to scratch memory).
__device__ inline int tile_region(uint32_t packed, int j) {
  const int r = (packed >> (8 * j)) & 0xFF;
  return r == 0xFF ? -1 : r;
}

// QR = 16 / n regions per unit (n = 4, 8, 16). RAGGED: kv < 64. MAXU: units
// per wave at most (wave w takes units w, w + waves, ...). SPLIT: the four
// row arrays do not fit in LDS together (28 x 28 map): K and V are staged
// for phase 1, whose query operands come from memory, and Q and dO take
// their place for phase 2, whose key operands are read from LDS into
// registers before the swap.
template <int QR, bool RAGGED, int MAXU, bool SPLIT>
__global__ __launch_bounds__(1024) void bwd_image_kernel(BwdImgParams p) {
  typedef Tr<__bf16> TT;
  typedef TT::op8 op8;
  typedef TT::op4 op4;
  constexpr int N = 16 / QR;  // tokens per region
  extern __shared__ __align__(16) unsigned char smem_raw[];
  __bf16* Ks = reinterpret_cast<__bf16*>(smem_raw);  // [HW][kRowE] each
  __bf16* Vs = Ks + p.HW * kRowE;
  __bf16* Qs = SPLIT ? Ks : Vs + p.HW * kRowE;
  __bf16* Ds = SPLIT ? Vs : Qs + p.HW * kRowE;
  float* lse_s = reinterpret_cast<float*>(Ds + p.HW * kRowE);  // [HW4]: base-2 log-sum-exp of every query
  float* dd_s = lse_s + p.HW4;                                  // [HW4]: D of every query
  uint64_t* rmask = reinterpret_cast<uint64_t*>(dd_s + p.HW4);  // [R]: routed regions of query region i
  uint64_t* imask = rmask + p.R;                                // [R]: good query regions routed to key region j
  int* rpos = reinterpret_cast<int*>(imask + p.R);              // [R * topk]: first position of the routed region, -1 out of range
  int* rout = rpos + p.R * p.topk;                              // [R]: row i has an entry out of range

  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int nw = nthr >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4, col = lane & 15;

  // (image, head), heads of an image adjacent: they share its cache lines on
  // one XCD
  const int w = xcd_item(blockIdx.x, gridDim.x, true);
  const int head = w % p.heads, b = w / p.heads;
  const int64_t img = (int64_t)b * p.HW * p.C;
  const int ch0 = head * D;

  for (int e = tid; e < p.R; e += nthr) {
    rmask[e] = 0;
    imask[e] = 0;
    rout[e] = 0;
  }

  // ---- O (for D) of the query columns of the wave's phase-1 units, and
  // with SPLIT their Q and dO
  op8 oop[MAXU], qg[SPLIT ? MAXU : 1], dg[SPLIT ? MAXU : 1];
#pragma unroll
  for (int uu = 0; uu < MAXU; ++uu) {
    const int qpos = 16 * (wave + nw * uu) + col;
    oop[uu] = TT::zero();
    if (SPLIT) qg[uu] = dg[uu] = TT::zero();
    if (qpos < p.HW) {
      const int64_t off = img + pos_token(p, qpos) * p.C + ch0 + 8 * g;
      oop[uu] = TT::load8(p.O + off);
      if (SPLIT) {
        qg[uu] = TT::load8(p.Q + off);
        dg[uu] = TT::load8(p.dO + off);
      }
    }
  }

  // ---- K and V rows of the head (and Q and dO without SPLIT): item f =
  // (position, 16-byte chunk)
  const int nitems = p.HW * 4;
  for (int f = tid; f < nitems; f += nthr) {
    const int pos = f >> 2, cv = f & 3;
    const int64_t off = img + pos_token(p, pos) * p.C + ch0 + 8 * cv;
    const int at = pos * kRowE + 8 * cv;
    const uint4 vk = *reinterpret_cast<const uint4*>(p.K + off);
    const uint4 vv = *reinterpret_cast<const uint4*>(p.V + off);
    if (SPLIT) {
      *reinterpret_cast<uint4*>(Ks + at) = vk;
      *reinterpret_cast<uint4*>(Vs + at) = vv;
    } else {
      const uint4 vq = *reinterpret_cast<const uint4*>(p.Q + off);
      const uint4 vd = *reinterpret_cast<const uint4*>(p.dO + off);
      *reinterpret_cast<uint4*>(Ks + at) = vk;
      *reinterpret_cast<uint4*>(Vs + at) = vv;
      *reinterpret_cast<uint4*>(Qs + at) = vq;
      *reinterpret_cast<uint4*>(Ds + at) = vd;
    }
  }
  __syncthreads();  // masks cleared

  // ---- routing rows -> first positions and row masks (OR is order-free)
  const int nroute = p.R * p.topk;
  for (int e = tid; e < nroute; e += nthr) {
    int slot;
    const int i = fdiv(e, p.div_topk, &slot);
    const int r = p.idx[(int64_t)b * nroute + e];
    const bool ok = r >= 0 && r < p.R;
    rpos[e] = ok ? r * N : -1;
    if (ok) atomicOr(reinterpret_cast<unsigned long long*>(&rmask[i]), 1ull << r);
    else rout[i] = 1;
  }
  __syncthreads();  // rows, masks and staged tensors complete

  // ---- inverse masks from the good rows (used after the next barrier)
  for (int e = tid; e < nroute; e += nthr) {
    int slot;
    const int i = fdiv(e, p.div_topk, &slot);
    const bool good = !rout[i] && __popcll(rmask[i]) == p.topk;
    const int rp = rpos[e];
    if (good && rp >= 0) atomicOr(reinterpret_cast<unsigned long long*>(&imask[rp / N]), 1ull << i);
  }

  const int srow = col >> 2, q4 = col & 3;  // transposing reads: slot/key row offset, 4-channel block

  // ---- phase 1: dQ, log-sum-exp and D per query unit
#pragma unroll
  for (int uu = 0; uu < MAXU; ++uu) {
    const int u = wave + nw * uu;
    if (u >= p.nunits) break;  // uniform
    const int qpos = 16 * u + col;
    const bool qv = qpos < p.HW;
    op8 qop, dop;
    if (SPLIT) {
      qop = qg[uu];
      dop = dg[uu];
    } else {
      qop = qv ? TT::load8(Qs + qpos * kRowE + 8 * g) : TT::zero();
      dop = qv ? TT::load8(Ds + qpos * kRowE + 8 * g) : TT::zero();
    }
    float dpart = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) dpart += (float)dop[e] * (float)oop[uu][e];
    const float Dq = wave_sum_groups(dpart);
    const int jl = col / N;  // the lane's region in the unit

    // position of routed key kappa = lane of each region j of the unit
    int kpos[QR];
    bool bad = false;
#pragma unroll
    for (int j = 0; j < QR; ++j) {
      const int r = u * QR + j;
      kpos[j] = 0;
      bool rb = false;
      if (r < p.R) {
        rb = rout[r] || __popcll(rmask[r]) != p.topk;
        if (lane < p.kv) {
          int tk;
          const int jr = fdiv(lane, p.div_n, &tk);
          const int base = rpos[r * p.topk + jr];
          kpos[j] = base < 0 ? 0 : base + tk;
        }
      }
      if (jl == j) bad = rb;
    }

    // S^T = sum_j K_j Q_j^T and dP^T = sum_j V_j dO_j^T. A-operand row col of
    // tile (st, tb) is key st*32 + 8*(col/4) + col%4 + 4*tb.
    floatx4 sacc[2][2], pacc[2][2];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) sacc[st][tb] = pacc[st][tb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < QR; ++j) {
      const op8 qj = (QR == 1 || jl == j) ? qop : TT::zero();
      const op8 dj = (QR == 1 || jl == j) ? dop : TT::zero();
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          const int key = st * 32 + 8 * (col >> 2) + (col & 3) + 4 * tb;
          const int pos = lane_value(kpos[j], key);
          const bool kin = !RAGGED || key < p.kv;
          const op8 kk = kin ? TT::load8(Ks + pos * kRowE + 8 * g) : TT::zero();
          const op8 vv = kin ? TT::load8(Vs + pos * kRowE + 8 * g) : TT::zero();
          sacc[st][tb] = TT::mma(kk, qj, sacc[st][tb]);
          pacc[st][tb] = TT::mma(vv, dj, pacc[st][tb]);
        }
    }
    // lane group g holds keys st*32 + 8g + e of its query
    float s[2][8], dp[2][8];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s[st][e] = sacc[st][0][e];
        s[st][4 + e] = sacc[st][1][e];
        dp[st][e] = pacc[st][0][e];
        dp[st][4 + e] = pacc[st][1][e];
      }
    if (RAGGED) {
      // scores of keys past kv to -inf by a min against +-inf made with
      // integer arithmetic (compare masks would be held in scalar registers)
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int key = st * 32 + 8 * g + e;
          const uint32_t lim = 0xff800000u ^ ((uint32_t)((key - p.kv) >> 31) & 0x80000000u);
          s[st][e] = fminf(s[st][e], __uint_as_float(lim));
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int e = 0; e < 8; ++e) mx = fmaxf(mx, s[st][e]);
    mx = wave_max_groups(mx);
    float sum = 0.f;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int e = 0; e < 8; ++e) sum += __builtin_amdgcn_exp2f((s[st][e] - mx) * p.c);
    const float lse = mx * p.c + __builtin_log2f(wave_sum_groups(sum));

    // dQ^T = sum_j K_j^T dZ_j^T: the K^T operand of tile ct (slots = keys
    // st*32 + 8g .. +7) from two transposing reads, in which lane col = 4 s + q
    // reads key row st*32 + 8g + s (+4) at channels 8 q + 4 ct .. +3, so that
    // row r of the tile is channel 8 (r / 4) + 4 ct + r % 4 and each lane ends
    // with 8 consecutive channels of its query (one 16-byte store)
    floatx4 dq[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      float dz[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[st][e], p.c, -lse));
        dz[e] = pr * (dp[st][e] - Dq);
      }
      const op8 zop = TT::from_f32(dz);
      const op8 zlo = TT::residual(dz, zop);  // dZ's low bits
#pragma unroll
      for (int j = 0; j < QR; ++j) {
        const op8 zj = (QR == 1 || jl == j) ? zop : TT::zero();
        const op8 zjl = (QR == 1 || jl == j) ? zlo : TT::zero();
        const int p0 = lane_value(kpos[j], st * 32 + 8 * g + srow);
        const int p1 = lane_value(kpos[j], st * 32 + 8 * g + 4 + srow);
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          const shortx4 lo = read_tr(Ks + p0 * kRowE + 8 * q4 + 4 * ct);
          const shortx4 hi = read_tr(Ks + p1 * kRowE + 8 * q4 + 4 * ct);
          const op8 kt = __builtin_bit_cast(op8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          dq[ct] = TT::mma(kt, zj, dq[ct]);
          dq[ct] = TT::mma(kt, zjl, dq[ct]);
        }
      }
    }
    if (qv) {
      // tile ct: this lane holds channels 8g + 4 ct .. +3 of its query
      const float f = bad ? __builtin_nanf("") : p.scale;
      float o[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[e] = dq[0][e] * f;
        o[4 + e] = dq[1][e] * f;
      }
      TT::store8_nt(p.dQ + img + pos_token(p, qpos) * p.C + ch0 + 8 * g, o);
      if (g == 0) {
        lse_s[qpos] = lse;
        dd_s[qpos] = Dq;
      }
    }
  }
  // with SPLIT: the key operands of the wave's phase-2 units (B operands of
  // S = Q K^T and dP = dO V^T: column = key col, slots = channels 8g ..)
  // from the K and V rows, then Q and dO in their place
  op8 kBs[SPLIT ? MAXU : 1], vBs[SPLIT ? MAXU : 1];
  if (SPLIT) {
#pragma unroll
    for (int uu = 0; uu < MAXU; ++uu) {
      const int kp = 16 * (wave + nw * uu) + col;
      kBs[uu] = kp < p.HW ? TT::load8(Ks + kp * kRowE + 8 * g) : TT::zero();
      vBs[uu] = kp < p.HW ? TT::load8(Vs + kp * kRowE + 8 * g) : TT::zero();
    }
    __syncthreads();  // every read of K and V done
    for (int f = tid; f < nitems; f += nthr) {
      const int pos = f >> 2, cv = f & 3;
      const int64_t off = img + pos_token(p, pos) * p.C + ch0 + 8 * cv;
      const int at = pos * kRowE + 8 * cv;
      const uint4 vq = *reinterpret_cast<const uint4*>(p.Q + off);
      const uint4 vd = *reinterpret_cast<const uint4*>(p.dO + off);
      *reinterpret_cast<uint4*>(Qs + at) = vq;
      *reinterpret_cast<uint4*>(Ds + at) = vd;
    }
  }
  __syncthreads();  // log-sum-exp, D, the inverse masks (and Q, dO) complete

  // ---- phase 2: dK, dV per key unit
#pragma unroll
  for (int uu = 0; uu < MAXU; ++uu) {
    const int u = wave + nw * uu;
    if (u >= p.nunits) break;  // uniform
    const int kp = 16 * u + col;  // the lane's key column
    const bool kvld = kp < p.HW;
    // B operands of S = Q K^T and dP = dO V^T: column = key col, slots = channels 8g ..
    const op8 kB = SPLIT ? kBs[uu] : kvld ? TT::load8(Ks + kp * kRowE + 8 * g) : TT::zero();
    const op8 vB = SPLIT ? vBs[uu] : kvld ? TT::load8(Vs + kp * kRowE + 8 * g) : TT::zero();
    const uint64_t mine = kvld ? imask[kp / N] : 0ull;
    uint64_t U = 0;  // incoming query regions of the unit's key regions (uniform)
#pragma unroll
    for (int j = 0; j < QR; ++j)
      if (u * QR + j < p.R) U |= imask[u * QR + j];
    floatx4 dv[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
    floatx4 dk[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
    while (U != 0) {  // uniform
      // the tile: the next QR incoming regions in ascending order, byte j =
      // region j of the tile (0xFF: none)
      uint32_t qpk = 0xFFFFFFFFu;
#pragma unroll
      for (int j = 0; j < QR; ++j) {
        if (U != 0) {
          qpk = (qpk & ~(0xFFu << (8 * j))) | ((uint32_t)__builtin_ctzll(U) << (8 * j));
          U &= U - 1;
        }
      }
      // slot s of the tile is token s % N of tile region s / N
      const int ar = tile_region(qpk, col / N);
      const int apos = ar >= 0 ? ar * N + col % N : 0;
      const op8 qA = TT::load8(Qs + apos * kRowE + 8 * g);
      const op8 dA = TT::load8(Ds + apos * kRowE + 8 * g);
      const floatx4 sc = TT::mma(qA, kB, floatx4{0.f, 0.f, 0.f, 0.f});
      const floatx4 dpv = TT::mma(dA, vB, floatx4{0.f, 0.f, 0.f, 0.f});
      // this lane: slots 4g .. 4g + 3, all in tile region 4g / N, of key col
      const int lr = tile_region(qpk, (4 * g) / N);
      const bool ok = lr >= 0 && ((mine >> lr) & 1ull);
      const int lpos = ok ? lr * N + (4 * g) % N : 0;
      const float4 l4 = *reinterpret_cast<const float4*>(lse_s + lpos);
      const float4 d4 = *reinterpret_cast<const float4*>(dd_s + lpos);
      const float la[4] = {l4.x, l4.y, l4.z, l4.w};
      const float da[4] = {d4.x, d4.y, d4.z, d4.w};
      float pr[4], dz[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pr[i] = ok ? __builtin_amdgcn_exp2f(__builtin_fmaf(sc[i], p.c, -la[i])) : 0.f;
        dz[i] = pr[i] * (dpv[i] - da[i]);
      }
      const op4 pB = TT::from_f32_4(pr);
      const op4 zB = TT::from_f32_4(dz);
      // dV^T += dO^T P and dK^T += Q^T dZ: A operand of tile ct (slots =
      // slots 4g .. +3) by a transposing read in which lane col = 4 s + q reads
      // slot row 4g + s at channels 8 q + 4 ct .. +3 (row r of the tile is
      // channel 8 (r / 4) + 4 ct + r % 4, as in phase 1)
      const int ts = 4 * g + srow;
      const int tr = tile_region(qpk, ts / N);
      const int tpos = tr >= 0 ? tr * N + ts % N : 0;
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const op4 dOA = read_tr(Ds + tpos * kRowE + 8 * q4 + 4 * ct);
        const op4 QA = read_tr(Qs + tpos * kRowE + 8 * q4 + 4 * ct);
        dv[ct] = TT::mma16(dOA, pB, dv[ct]);
        dk[ct] = TT::mma16(QA, zB, dk[ct]);
      }
    }
    if (kvld) {
      // tile ct: this lane holds channels 8g + 4 ct .. +3 of its key
      const int off = pos_token(p, kp) * p.C + ch0 + 8 * g;
      float ov[8], ok[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ov[e] = dv[0][e];
        ov[4 + e] = dv[1][e];
        ok[e] = dk[0][e] * p.scale;
        ok[4 + e] = dk[1][e] * p.scale;
      }
      TT::store8_nt(p.dV + img + off, ov);
      TT::store8_nt(p.dK + img + off, ok);
    }
  }
}

size_t bwd_image_lds(const Shape& s, bool split) {
  const size_t HW = (size_t)s.H * s.W, HW4 = (HW + 3) / 4 * 4;
  return (split ? 2 : 4) * 2 * HW * kRowE + 2 * 4 * HW4 + 2 * 8 * (size_t)s.R + 4 * (size_t)s.R * s.topk +
         4 * (size_t)s.R;
}

}  // namespace

bool backward_image_fits(const Shape& s, int dtype) {
  if (dtype != kBF16 || s.d != kHeadDim || s.kv > KC) return false;
  if (s.n != 4 && s.n != 8 && s.n != 16) return false;
  if (s.R > 64) return false;  // one 64-bit mask per region
  // one workgroup per (image, head): fewer than half the compute units busy
  // is slower than the per-region kernels
  if ((int64_t)s.B * s.heads < 128) return false;
  const int nunits = (s.H * s.W + 15) / 16;
  if (nunits > 64) return false;  // at most 4 units per wave
  return bwd_image_lds(s, true) <= kBwdImgMaxLds;
}

hipError_t launch_backward_image(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                                 const int32_t* idx, void* dQ, void* dK, void* dV, const Shape& s,
                                 hipStream_t stream) {
  BwdImgParams p{};
  p.Q = static_cast<const __bf16*>(Q);
  p.K = static_cast<const __bf16*>(K);
  p.V = static_cast<const __bf16*>(V);
  p.O = static_cast<const __bf16*>(O);
  p.dO = static_cast<const __bf16*>(dO);
  p.idx = idx;
  p.dQ = static_cast<__bf16*>(dQ);
  p.dK = static_cast<__bf16*>(dK);
  p.dV = static_cast<__bf16*>(dV);
  p.H = s.H; p.W = s.W; p.C = s.C; p.S = s.S; p.topk = s.topk;
  p.sh = s.sh; p.sw = s.sw; p.n = s.n; p.R = s.R; p.kv = s.kv; p.heads = s.heads;
  p.HW = s.H * s.W;
  p.HW4 = (p.HW + 3) / 4 * 4;
  p.nunits = (p.HW + 15) / 16;
  p.scale = 1.0f / sqrtf((float)s.d);
  p.c = p.scale * 1.4426950408889634f;
  p.div_n = make_fastdiv(s.n);
  p.div_sw = make_fastdiv(s.sw);
  p.div_S = make_fastdiv(s.S);
  p.div_topk = make_fastdiv(s.topk);
  // about two units per wave (13 units at 14 x 14: 7 waves), at most 16 waves
  const int waves = std::min(16, (p.nunits + 1) / 2);
  const int maxu = (p.nunits + waves - 1) / waves;  // <= 4
  const bool split = bwd_image_lds(s, false) > kBwdImgMaxLds;
  const bool ragged = s.kv < KC;
  const int form = s.n == 4 ? 0 : s.n == 8 ? 1 : 2;
  const int mu = maxu <= 1 ? 0 : maxu <= 2 ? 1 : 2;
#define BRA_BI(QR, RG, SP)                                                                   \
  {(const void*)&bwd_image_kernel<QR, RG, 1, SP>, (const void*)&bwd_image_kernel<QR, RG, 2, SP>, \
   (const void*)&bwd_image_kernel<QR, RG, 4, SP>}
  // [split][ragged][form][units per wave: 1, 2, 4]
  const void* fns[2][2][3][3] = {
      {{BRA_BI(4, false, false), BRA_BI(2, false, false), BRA_BI(1, false, false)},
       {BRA_BI(4, true, false), BRA_BI(2, true, false), BRA_BI(1, true, false)}},
      // (4-token regions never need SPLIT: at most 64 regions, 256 positions)
      {{{nullptr, nullptr, nullptr}, BRA_BI(2, false, true), BRA_BI(1, false, true)},
       {{nullptr, nullptr, nullptr}, BRA_BI(2, true, true), BRA_BI(1, true, true)}}};
#undef BRA_BI
  const void* fn = fns[split][ragged][form][mu];
  if (fn == nullptr) return hipErrorInvalidValue;
  const size_t lds = bwd_image_lds(s, split);
  // more than the default 64 KiB of dynamic LDS: raise the kernel's limit
  // to the most any launch of it uses (one value for every caller)
  if (lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kBwdImgMaxLds);
    if (e != hipSuccess) return e;
  }
  void* args[] = {&p};
  return hipLaunchKernel(fn, dim3((unsigned)(s.B * s.heads)), dim3(waves * 64), args, lds, stream);
}

}  // namespace bra
