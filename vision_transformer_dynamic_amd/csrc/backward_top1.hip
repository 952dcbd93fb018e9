// Backward of the token attention with top-1 routing (BiFormer's first
// stage: every query region attends to the tokens of exactly one key region)
// in one launch (explainer "BiFormer Reshapes Visual Attention with
// 'Bi-Level Routing'", Part 2.2 step 4 and pseudocode steps 6-7 for the
// forward; Part 4.3 for top-k = 1 at the first stage; Part 7 for training
// throughput). The routing table is held fixed:
//
//   P = softmax(c' q k^T), dP = dO V_g^T, D = rowsum(P * dP),
//   dZ = P * (dP - D), dQ = scale * dZ K_g, dK_g = scale * dZ^T Q, dV_g = P^T dO
//
// With one routed region per query region, all of a query's keys are one
// region's tokens, so the workgroup of key region r sees every key of each
// query region routed to r and finishes that region's dQ (no log-sum-exp or D
// goes through memory), and it is the only one to add to dK and dV of r's
// tokens (no atomics, no second launch). One workgroup per (image, key
// region, pair of heads), 8 waves (head of the pair, 16-row tile), the
// heaviest key regions of every image first:
//
//  * The routing column: each wave ballots idx[b, :] == r in region order, so
//    the incoming query regions are taken in ascending order (deterministic
//    sums). A region whose own row is outside [0, S*S) gets NaN dQ from its
//    own key region's workgroup and is in no list.
//  * K, V of region r and Q, dO of the incoming region go to LDS (the pair's
//    128-byte rows, 16 bytes a thread), loaded only when the list is not
//    empty; the next region's Q, dO are fetched into registers while the
//    current one is processed.
//  * Phase 1 per (head, query tile): S^T = K Q^T and dP^T = V dO^T over the
//    region's keys, then the softmax, D = rowsum(P * dP) (equal to
//    rowsum(dO * O) for O = P V, without reading O), dZ and
//    dQ^T = K^T dZ^T with K^T from gfx950's transposing LDS read. P and dZ
//    (bf16, as the products below take them) go to LDS; the pair's dQ halves
//    meet in LDS and leave as whole 128-byte rows.
//  * Phase 2 per (head, key tile): dV^T += dO^T P and dK^T += Q^T dZ
//    (16-deep products; dO^T, Q^T and the P, dZ columns of the key tile by
//    the transposing read), summed over the incoming regions in registers.
//  * dK and dV rows leave once at the end (zero for a region nobody routes to).
#include "bra_internal.h"
#include "attn_common.h"

#include <math.h>

namespace bra {
namespace {

constexpr int kRowT = 32;  // LDS row of one token and head: 32 channels, 64 bytes, no pad
constexpr int kHeadRows = 64 * kRowT;  // one head's rows of one tensor

// LDS layouts, chosen by measuring gfx950's bank conflicts
// (SQ_LDS_BANK_CONFLICT) for each access pattern of this kernel:
//  * token rows: the 16-byte chunk c of row r sits at chunk c ^ 2 when bit 3
//    of r is set. With that, the 16-byte operand reads (16 rows x 4 chunks,
//    rows col or 8 (col / 4) + col % 4) and the staging writes meet no
//    conflict, and the transposing reads 2 cycles; with 80-byte padded rows
//    they cost 4, 4 and ~9 cycles an instruction.
//  * whole-row exchange: xrow_at.
__device__ inline int row_at(int row, int chunk) { return row * kRowT + 8 * (chunk ^ ((row >> 2) & 2)); }
constexpr int kTop1Threads = 512;

struct BwdTop1Params {
  const __bf16* Q;
  const __bf16* K;
  const __bf16* V;
  const __bf16* dO;
  const int32_t* idx;
  __bf16* dQ;
  __bf16* dK;
  __bf16* dV;
  int B, H, W, C, S, sh, sw, n, R, heads;
  int nhg;      // pairs of heads
  float c;      // scale * log2(e)
  float scale;  // 1 / sqrt(d)
  FastDiv div_sw, div_S;
};

typedef __attribute__((address_space(3))) shortx4 lds_s4;

// Transposing LDS read of 4 bf16 (8 bytes) at p: within each 16-lane group,
// lane j receives element j % 4 of the reads of lanes 4 s + j / 4, s = 0..3.
__device__ inline shortx4 read_tr(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(p));
}

// Token offset of region i's top-left token inside the image.
__device__ inline int region_corner(const BwdTop1Params& p, int i) {
  int rx;
  const int ry = fdiv(i, p.div_S, &rx);
  return ry * p.sh * p.W + rx * p.sw;
}

// RAGGED: fewer than 64 tokens per region (the scores of the missing keys
// are masked; their rows are zero in LDS).
template <bool RAGGED>
__global__ __launch_bounds__(kTop1Threads) void bwd_top1_kernel(BwdTop1Params p) {
  typedef Tr<__bf16> TT;
  typedef TT::op8 op8;
  typedef TT::op4 op4;
  // K, V, Q, dO rows [head][64][kRowT] (Q and dO then hold the dK, dV rows
  // at the end), P and dZ [tensor][head][64 queries][64 keys] (bf16, 16-byte
  // chunks swizzled as in xrow_at), the dQ rows [64][8 chunks], the incoming
  // query regions
  __shared__ __align__(16) __bf16 rows_s[4 * 2 * kHeadRows];
  __shared__ __align__(16) __bf16 pz_s[2 * 2 * 64 * 64];
  __shared__ __align__(16) uint4 xq[64 * 8];
  __shared__ int qlist[kMaxRegions];
  __shared__ int degl[8 * 64];  // per wave: in-degrees of the image's key regions (R <= 64)
  __bf16* Ks = rows_s;
  __bf16* Vs = Ks + 2 * kHeadRows;
  __bf16* Qs = Vs + 2 * kHeadRows;
  __bf16* Ds = Qs + 2 * kHeadRows;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4, col = lane & 15;
  const int hl = wave >> 2, tq = wave & 3;  // head of the pair, tile
  const int srow = col >> 2, q4 = col & 3;  // transposing reads: row offset, 4-channel block
  // Lane bases of the swizzled row reads. Bit 3 of the row (the swizzle bit)
  // is the same for every row a lane reads through one base: each base plus
  // a constant number of whole rows (16, 32 or 4 of them) keeps it.
  const int a_key = row_at(8 * (col >> 2) + (col & 3), g);  // A rows of S^T, dP^T (+ 32 st + 4 tb rows)
  const int a_col = row_at(col, g);                         // rows = col (+ 16 per tile)
  const int a_tr1 = row_at(8 * g + srow, q4);               // K^T reads (+ 32 st, + 4 rows)
  const int a_tr2 = row_at(4 * g + srow, q4);               // dO^T, Q^T reads (+ 16 per tile)
  // P and dZ of a query tile as B operands of the 16-deep products: lane
  // 4 s + m of group g reads query row 4g + s (+ 16 per tile), keys
  // 16 tq + 4m .. +3 (chunk 2 tq + m / 2, half m % 2; row % 8 is the lane's)
  const int a_pz = (4 * g + srow) * 64 + 8 * ((2 * tq + (q4 >> 1)) ^ ((4 * g + srow) & 7)) + 4 * (q4 & 1);

  // workgroup -> (image b, key region r, pair of heads): images fastest, then
  // the key regions of each image by descending in-degree (ties: lower index
  // first), so every image's heaviest regions start in the first round and
  // the many unrouted ones come last. Each wave derives the order on its own
  // from the image's routing row: counts by LDS atomic adds, the largest
  // count bit by bit, then one ballot per count level. Any order gives the
  // same results, region by region. (With top-1 routing over random maps a
  // key region's in-degree runs from 0 to about 7; in image order the heavy
  // regions drained in a tail: stage-1 backward 53.1 -> 47.5 us.) With more
  // than 64 regions, region order.
  int w = blockIdx.x;
  const int hg = w % p.nhg;
  w /= p.nhg;
  const int b = w % p.B;
  const int kr = w / p.B;
  int r = kr;
  if (p.R <= 64) {  // uniform
    int* dl = degl + 64 * wave;
    dl[lane] = 0;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    const int v = lane < p.R ? p.idx[(int64_t)b * p.R + lane] : -1;
    if (v >= 0 && v < p.R) atomicAdd(&dl[v], 1);  // rows outside [0, S*S) count for no region
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    const int deg = lane < p.R ? dl[lane] : -1;
    int mx = 0;
#pragma unroll
    for (int bit = 6; bit >= 0; --bit)
      if (__builtin_amdgcn_ballot_w64(deg >= (mx | (1 << bit))) != 0) mx |= 1 << bit;
    int rank = 0, placed = 0;
    for (int d = mx; d >= 0 && placed < p.R; --d) {  // uniform
      const uint64_t h = __builtin_amdgcn_ballot_w64(deg == d);
      if (deg == d)
        rank = placed + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(h >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)h, 0));
      placed += __builtin_popcountll(h);
    }
    r = __builtin_ctzll(__builtin_amdgcn_ballot_w64(lane < p.R && rank == kr));
  }
  const int nh = min(2, p.heads - 2 * hg);  // heads in the pair (the last pair of an odd count has one)
  const int cb = 2 * hg * D;               // the pair's first channel
  const int64_t img = (int64_t)b * p.H * p.W * p.C;
  const int32_t* irow = p.idx + (int64_t)b * p.R;
  const int ntq = (p.n + 15) >> 4;         // 16-row tiles of a region (queries and keys alike)
  const bool busy = tq < ntq && hl < nh;   // the wave has rows in both phases (uniform)

  // staging item of this thread: token tid / 8 of a region, 16-byte chunk
  // tid % 8 of the pair's 128-byte row (chunk / 4 = head)
  const int st_tok = tid >> 3, st_c = tid & 7;
  const bool st_ok = st_tok < p.n && (st_c >> 2) < nh;
  int st_tx;
  const int st_off = fdiv(st_tok, p.div_sw, &st_tx) * p.W + st_tx;
  const int st_at = (st_c >> 2) * kHeadRows + row_at(st_tok, st_c & 3);
  const int64_t st_g = img + cb + 8 * st_c;  // + token * C

  // ---- the query regions routed to r, ascending (one 64-region ballot per
  // step; at most kMaxRegions regions)
  int cnt = 0, first = -1;
#pragma unroll
  for (int j = 0; j < kMaxRegions / 64; ++j) {
    if (64 * j < p.R) {  // uniform
      const int e = 64 * j + lane;
      const int v = e < p.R ? irow[e] : -1;
      const uint64_t hit = __builtin_amdgcn_ballot_w64(v == r);
      if (first < 0 && hit != 0) first = 64 * j + __builtin_ctzll(hit);
      if (wave == 0 && v == r) {
        const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(hit >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)hit, 0));
        qlist[cnt + below] = e;
      }
      cnt += __builtin_popcountll(hit);
    }
  }
  const int own = irow[r];
  const bool own_bad = own < 0 || own >= p.R;

  // ---- K and V of key region r and Q and dO of the first incoming region,
  // all issued together once the list is known (a region nobody routes to
  // reads neither: about a third of them with top-1 routing over random
  // features)
  const int rcorner = region_corner(p, r);
  uint4 qst = make_uint4(0, 0, 0, 0), dst = qst;
  if (cnt > 0) {  // uniform
    uint4 kst = make_uint4(0, 0, 0, 0), vst = kst;
    if (st_ok) {
      const int64_t koff = st_g + (int64_t)(rcorner + st_off) * p.C;
      const int64_t qoff = st_g + (int64_t)(region_corner(p, first) + st_off) * p.C;
      kst = *reinterpret_cast<const uint4*>(p.K + koff);
      vst = *reinterpret_cast<const uint4*>(p.V + koff);
      qst = *reinterpret_cast<const uint4*>(p.Q + qoff);
      dst = *reinterpret_cast<const uint4*>(p.dO + qoff);
    }
    *reinterpret_cast<uint4*>(Ks + st_at) = kst;
    *reinterpret_cast<uint4*>(Vs + st_at) = vst;
  }

  const __bf16* Kh = Ks + hl * kHeadRows;
  const __bf16* Vh = Vs + hl * kHeadRows;
  const __bf16* Qh = Qs + hl * kHeadRows;
  const __bf16* Dh = Ds + hl * kHeadRows;
  __bf16* Ph = pz_s + hl * 64 * 64;
  __bf16* Zh = pz_s + (2 + hl) * 64 * 64;

  floatx4 dv[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
  floatx4 dk[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
  for (int it = 0; it < cnt; ++it) {
    *reinterpret_cast<uint4*>(Qs + st_at) = qst;
    *reinterpret_cast<uint4*>(Ds + st_at) = dst;
    __syncthreads();  // Q, dO rows (and K, V, the list on the first pass) in LDS
    const int iq = qlist[it];
    if (it + 1 < cnt && st_ok) {
      const int64_t off = st_g + (int64_t)(region_corner(p, qlist[it + 1]) + st_off) * p.C;
      qst = *reinterpret_cast<const uint4*>(p.Q + off);
      dst = *reinterpret_cast<const uint4*>(p.dO + off);
    }

    // ---- phase 1: dQ, log-sum-exp and D of query tile tq
    if (busy) {
      const int qs = tq * 16 + col;
      const bool qv = !RAGGED || qs < p.n;
      const op8 qop = TT::load8(Qh + a_col + tq * 16 * kRowT);
      const op8 dop = TT::load8(Dh + a_col + tq * 16 * kRowT);
      // S^T = K Q^T, dP^T = V dO^T: A-operand row col of tile (st, tb) is key
      // st*32 + 8*(col/4) + col%4 + 4*tb, so lane group g holds keys
      // st*32 + 8g + e of its query
      float s[2][8], dp[2][8];
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          const op8 kk = TT::load8(Kh + a_key + (st * 32 + 4 * tb) * kRowT);
          const op8 vv = TT::load8(Vh + a_key + (st * 32 + 4 * tb) * kRowT);
          const floatx4 sa = TT::mma(kk, qop, floatx4{0.f, 0.f, 0.f, 0.f});
          const floatx4 pa = TT::mma(vv, dop, floatx4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            s[st][4 * tb + e] = sa[e];
            dp[st][4 * tb + e] = pa[e];
          }
        }
      if (RAGGED) {
        // scores of keys past n to -inf by a min against +-inf made with
        // integer arithmetic (compare masks would be held in scalar registers)
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int key = st * 32 + 8 * g + e;
            const uint32_t lim = 0xff800000u ^ ((uint32_t)((key - p.n) >> 31) & 0x80000000u);
            s[st][e] = fminf(s[st][e], __uint_as_float(lim));
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int e = 0; e < 8; ++e) mx = fmaxf(mx, s[st][e]);
      mx = wave_max_groups(mx);
      // P in place of the scores (one exponential each), then D = rowsum(P * dP)
      float sum = 0.f;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          s[st][e] = __builtin_amdgcn_exp2f((s[st][e] - mx) * p.c);
          sum += s[st][e];
        }
      const float inv = 1.0f / wave_sum_groups(sum);
      float dpart = 0.f;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          s[st][e] *= inv;
          dpart = __builtin_fmaf(s[st][e], dp[st][e], dpart);
        }
      const float Dq = wave_sum_groups(dpart);

      // dQ^T = K^T dZ^T: the K^T operand of tile ct (slots = keys st*32 + 8g
      // .. +7) from two transposing reads, in which lane col = 4 s + q reads
      // key row st*32 + 8g + s (+4) at channels 8 q + 4 ct .. +3, so that row
      // r of the tile is channel 8 (r / 4) + 4 ct + r % 4 and each lane ends
      // with 8 consecutive channels of its query
      floatx4 dq[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        float dz[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) dz[e] = s[st][e] * (dp[st][e] - Dq);
        const op8 zop = TT::from_f32(dz);
        const op8 zlo = TT::residual(dz, zop);  // dZ's low bits
        // P and dZ (bf16) of keys st*32 + 8g .. +7 for phase 2; zero for a
        // query slot past n
        *reinterpret_cast<op8*>(Ph + qs * 64 + 8 * ((4 * st + g) ^ (qs & 7))) = qv ? TT::from_f32(s[st]) : TT::zero();
        *reinterpret_cast<op8*>(Zh + qs * 64 + 8 * ((4 * st + g) ^ (qs & 7))) = qv ? zop : TT::zero();
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          const shortx4 lo = read_tr(Kh + a_tr1 + st * 32 * kRowT + 4 * ct);
          const shortx4 hi = read_tr(Kh + a_tr1 + (st * 32 + 4) * kRowT + 4 * ct);
          const op8 kt = __builtin_bit_cast(op8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          dq[ct] = TT::mma(kt, zop, dq[ct]);
          dq[ct] = TT::mma(kt, zlo, dq[ct]);
        }
      }
      float o[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[e] = dq[0][e] * p.scale;
        o[4 + e] = dq[1][e] * p.scale;
      }
      xq[xrow_at(qs, hl * 4 + g)] = __builtin_bit_cast(uint4, TT::from_f32(o));
    }
    __syncthreads();  // dQ rows, P and dZ in LDS

    if (st_ok) {
      const int64_t off = st_g + (int64_t)(region_corner(p, iq) + st_off) * p.C;
      __builtin_nontemporal_store(__builtin_bit_cast(op8, xq[xrow_at(st_tok, st_c)]), reinterpret_cast<op8*>(p.dQ + off));
    }

    // ---- phase 2: dK, dV of key tile tq over the region's query tiles
    if (busy) {
#pragma unroll
      for (int qt = 0; qt < 4; ++qt) {
        if (qt >= ntq) break;  // uniform
        // B operands: P and dZ of query slots qt*16 + 4g .. +3, key tq*16 + col
        const op4 pB = read_tr(Ph + a_pz + qt * 16 * 64);
        const op4 zB = read_tr(Zh + a_pz + qt * 16 * 64);
        // dV^T += dO^T P and dK^T += Q^T dZ: A operand of tile ct (slots =
        // query slots qt*16 + 4g .. +3) by a transposing read in which lane
        // col = 4 s + q reads query row qt*16 + 4g + s at channels 8 q + 4 ct
        // .. +3 (row r of the tile is channel 8 (r / 4) + 4 ct + r % 4)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          const op4 dOA = read_tr(Dh + a_tr2 + qt * 16 * kRowT + 4 * ct);
          const op4 QA = read_tr(Qh + a_tr2 + qt * 16 * kRowT + 4 * ct);
          dv[ct] = TT::mma16(dOA, pB, dv[ct]);
          dk[ct] = TT::mma16(QA, zB, dk[ct]);
        }
      }
    }
    __syncthreads();  // Q, dO, dQ rows, P and dZ consumed before the next region
  }

  // ---- dK and dV rows of key region r: the pair's 64-byte halves meet in
  // LDS (over the Q and dO rows) and leave as whole rows. Tile ct of a lane
  // holds channels 8g + 4 ct .. +3 of key tq*16 + col.
  uint4* xr = reinterpret_cast<uint4*>(Qs);  // [dV, dK][key][chunk]
  if (busy) {
    float ov[8], ok[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ov[e] = dv[0][e];
      ov[4 + e] = dv[1][e];
      ok[e] = dk[0][e] * p.scale;
      ok[4 + e] = dk[1][e] * p.scale;
    }
    const int at = xrow_at(tq * 16 + col, hl * 4 + g);
    xr[at] = __builtin_bit_cast(uint4, TT::from_f32(ov));
    xr[512 + at] = __builtin_bit_cast(uint4, TT::from_f32(ok));
  }
  __syncthreads();
  if (st_ok) {
    const int64_t off = st_g + (int64_t)(rcorner + st_off) * p.C;
    __builtin_nontemporal_store(__builtin_bit_cast(op8, xr[xrow_at(st_tok, st_c)]), reinterpret_cast<op8*>(p.dV + off));
    __builtin_nontemporal_store(__builtin_bit_cast(op8, xr[512 + xrow_at(st_tok, st_c)]),
                                reinterpret_cast<op8*>(p.dK + off));
    if (own_bad) {
      // this region's own routing row is out of range: NaN dQ for its queries
      float nanv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) nanv[e] = __builtin_nanf("");
      TT::store8(p.dQ + st_g + (int64_t)(rcorner + st_off) * p.C, nanv);
    }
  }
}

}  // namespace

bool backward_top1_fits(const Shape& s, int dtype) {
  if (dtype != kBF16 || s.d != kHeadDim || s.topk != 1) return false;
  // regions of 16 to 64 tokens: one to four 16-row tiles per head
  if (s.n < 16 || s.n > 64 || s.R > kMaxRegions) return false;
  const int64_t nwg = (int64_t)s.B * s.R * ((s.heads + 1) / 2);
  return nwg < (int64_t(1) << 31);
}

hipError_t launch_backward_top1(const void* Q, const void* K, const void* V, const void* dO, const int32_t* idx,
                                void* dQ, void* dK, void* dV, const Shape& s, hipStream_t stream) {
  BwdTop1Params p{};
  p.Q = static_cast<const __bf16*>(Q);
  p.K = static_cast<const __bf16*>(K);
  p.V = static_cast<const __bf16*>(V);
  p.dO = static_cast<const __bf16*>(dO);
  p.idx = idx;
  p.dQ = static_cast<__bf16*>(dQ);
  p.dK = static_cast<__bf16*>(dK);
  p.dV = static_cast<__bf16*>(dV);
  p.B = s.B; p.H = s.H; p.W = s.W; p.C = s.C; p.S = s.S;
  p.sh = s.sh; p.sw = s.sw; p.n = s.n; p.R = s.R; p.heads = s.heads;
  p.nhg = (s.heads + 1) / 2;
  p.scale = 1.0f / sqrtf((float)s.d);
  p.c = p.scale * 1.4426950408889634f;
  p.div_sw = make_fastdiv(s.sw);
  p.div_S = make_fastdiv(s.S);
  const void* fn = s.n < 64 ? (const void*)&bwd_top1_kernel<true> : (const void*)&bwd_top1_kernel<false>;
  void* args[] = {&p};
  const unsigned nwg = (unsigned)((int64_t)s.B * s.R * p.nhg);
  return hipLaunchKernel(fn, dim3(nwg), dim3(kTop1Threads), args, 0, stream);
}

}  // namespace bra
