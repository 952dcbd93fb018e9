// dQ, log-sum-exp and D of the backward for bf16 with 65 to 1024 routed keys
// per query (the dense-prediction and detection maps: explainer "BiFormer
// Reshapes Visual Attention with 'Bi-Level Routing'", Part 2.2 step 4 and
// pseudocode steps 6-7 for the forward, Part 4.3 for S = 8 and S = 16, Part 7
// for training throughput). The routing table is held fixed:
//
//   P = softmax(c' q k^T), dP = dO V_g^T, D = rowsum(dO * O),
//   dZ = P * (dP - D), dQ = scale * dZ K_g
//
// The forward dense kernel's work split and staging: one workgroup = (image,
// query region, block of up to 256 of its queries, head), one wave per
// 16-query tile. Every routed key's K and V rows of the head (64 bytes each)
// are gathered into LDS once by direct-to-LDS loads, in phases of 256 keys
// with their own buffers, so the waves never wait on the caches inside their
// loops:
//
//  * one pass, phase by phase as the loads land: S^T = K Q^T and
//    dP^T = V dO^T per 64-key chunk (K and V rows as A operands); with D from
//    O and dO before any key, the probabilities relative to a lazy running
//    maximum (moved only when a score exceeds it by more than 8 / c, as in
//    the forward; the four lane groups' maxima combined only then), their
//    running sum, dZ = P (dP - D) in registers, and dQ^T += K^T dZ^T with
//    K^T from gfx950's transposing LDS read of the same K rows; dQ and the
//    log-sum-exp come from the sum at the end. dZ enters the product as two
//    bf16 operands (hi and its rounding error), as in the other dQ products.
//    (Two passes, an exact log-sum-exp first, measured 114.9 us against
//    107.2 us for the dense map's backward.)
//
// dQ and every query's base-2 log-sum-exp and D go to memory (the dK/dV kernel
// reads the last two). A routing row with an entry outside [0, S*S) or a
// repeated entry gives NaN dQ for its region's queries.
#include "bra_internal.h"
#include "attn_common.h"
#include "lds_dma.h"

#include <math.h>

#include <algorithm>

namespace bra {
namespace {

constexpr int kPhaseRows = 256;  // key rows per phase
constexpr int kMaxPhases = 4;    // at most 1024 keys per query
constexpr int kTiles = 16;       // query tiles (waves) per workgroup at most
constexpr int kRowBytes = 64;    // one head of one key: 32 bf16

struct BwdDenseParams {
  const __bf16* Q;
  const __bf16* K;
  const __bf16* V;
  const __bf16* O;
  const __bf16* dO;
  const int32_t* idx;
  __bf16* dQ;
  float* lse;  // [B * H * W][heads]
  float* dd;   // [B * H * W][heads]
  int H, W, C, S, topk, sh, sw, n, R, kv, heads;
  int kvpad;  // kv rounded up to 64
  int nqb;    // query blocks per region
  int qblk;   // queries per block (a multiple of 16, <= 256)
  float c;     // scale * log2(e)
  float scale; // 1 / sqrt(d)
  FastDiv div_n, div_sw, div_S;
};

// Byte offset of 16-byte chunk c of key row r inside a phase buffer: the four
// chunks of a row rotate with bits 3-4 of the row, so that the 16 rows of an
// operand read (rows 8 a + b + 4 t) fall on distinct banks. Bits 3-4 of every
// row a lane reads are the same from chunk to chunk and step to step, so each
// read is the lane's base plus a constant.
__device__ __forceinline__ int row_off(int r, int c) { return r * kRowBytes + 16 * (c ^ ((r >> 3) & 3)); }

// The direct-to-LDS loads of one phase of this wave: row blocks (16 key rows,
// 1 KB per tensor) m = wave, wave + nw, ... Lane l gathers row 16 m + l / 4,
// chunk (l % 4) ^ swizzle, exactly the chunk that belongs in its LDS slot.
// Rows past kv read key 0's token (finite values; their scores are masked).
// Returns the number of loads issued.
__device__ __forceinline__ int issue_phase(const BwdDenseParams& p, const int* rtab, const __bf16* Kg,
                                           const __bf16* Vg, int ch0, int p0, int rows, unsigned char* kbuf,
                                           unsigned char* vbuf, int wave, int nw, int lane) {
  int cnt = 0;
  for (int m = wave; m * 16 < rows; m += nw) {  // uniform
    const int rl = 16 * m + (lane >> 2);
    const int r = p0 + rl;
    int tok;
    {
      int tk, tx;
      const int key = r < p.kv ? r : 0;
      const int jr = fdiv(key, p.div_n, &tk);
      const int ty = fdiv(tk, p.div_sw, &tx);
      tok = rtab[jr] + ty * p.W + tx;
    }
    const int ch = (lane & 3) ^ ((rl >> 3) & 3);
    const int64_t off = (int64_t)tok * p.C + ch0 + 8 * ch;
    dma16(Kg + off, lds_offset(kbuf + 1024 * m));
    dma16(Vg + off, lds_offset(vbuf + 1024 * m));
    cnt += 2;
  }
  return cnt;
}

// S^T (and with DP, dP^T) of one 64-key chunk: A-operand row col of tile
// (st, tb) is key st*32 + 8*(col/4) + col%4 + 4*tb, so lane group g holds
// keys st*32 + 8g + e of its query. kl / vl: this lane's row base in the chunk.
template <bool DP>
__device__ __forceinline__ void chunk_products(const unsigned char* kl, const unsigned char* vl, const bf16x8& qop,
                                               const bf16x8& dop, float (&s)[2][8], float (&dp)[2][8]) {
  typedef Tr<__bf16> TT;
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const int ro = (st * 32 + 4 * tb) * kRowBytes;
      const floatx4 sa = TT::mma(*reinterpret_cast<const bf16x8*>(kl + ro), qop, floatx4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int e = 0; e < 4; ++e) s[st][4 * tb + e] = sa[e];
      if (DP) {
        const floatx4 pa = TT::mma(*reinterpret_cast<const bf16x8*>(vl + ro), dop, floatx4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int e = 0; e < 4; ++e) dp[st][4 * tb + e] = pa[e];
      }
    }
}

template <bool RAGGED, int NPH>
__global__ __launch_bounds__(kTiles * 64) void bwd_dq_dense_kernel(BwdDenseParams p) {
  typedef Tr<__bf16> TT;
  typedef TT::op8 op8;
  // one K and one V buffer per phase, each its own array
  __shared__ __align__(16) unsigned char k0[kPhaseRows * kRowBytes], v0[kPhaseRows * kRowBytes];
  __shared__ __align__(16) unsigned char k1[NPH > 1 ? kPhaseRows * kRowBytes : 16], v1[NPH > 1 ? kPhaseRows * kRowBytes : 16];
  __shared__ __align__(16) unsigned char k2[NPH > 2 ? kPhaseRows * kRowBytes : 16], v2[NPH > 2 ? kPhaseRows * kRowBytes : 16];
  __shared__ __align__(16) unsigned char k3[NPH > 3 ? kPhaseRows * kRowBytes : 16], v3[NPH > 3 ? kPhaseRows * kRowBytes : 16];
  __shared__ int rtab[kMaxRegions];
  __shared__ uint32_t rmask[kMaxRegions / 32];  // the row's regions, for the repeated-entry check
  __shared__ int sbad;

  const int tid = threadIdx.x;
  const int nw = blockDim.x >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4, col = lane & 15;

  // item (image, region, query block, head), heads fastest; an image's items
  // on one XCD (xcd_item)
  int w = xcd_item(blockIdx.x, gridDim.x);
  const int head = w % p.heads;
  w /= p.heads;
  const int qb = w % p.nqb;
  w /= p.nqb;
  const int i = w % p.R;
  const int b = w / p.R;
  const int64_t img = (int64_t)b * p.H * p.W * p.C;
  const int ch0 = head * D;
  int rix;
  const int riy = fdiv(i, p.div_S, &rix);
  const int qcorner = riy * p.sh * p.W + rix * p.sw;

  // ---- the wave's queries: B operands of q and dO (column = query col,
  // slots = channels 8g .. 8g + 7), and D = dO . O per query
  const int qi = qb * p.qblk + wave * 16 + col;
  const bool qvalid = qi < p.n;
  int qtok = 0;
  op8 qop = TT::zero(), dop = TT::zero();
  float dpart = 0.f;
  if (qvalid) {
    int qx;
    const int qy = fdiv(qi, p.div_sw, &qx);
    qtok = qcorner + qy * p.W + qx;
    const int64_t off = img + (int64_t)qtok * p.C + ch0 + 8 * g;
    qop = TT::load8(p.Q + off);
    dop = TT::load8(p.dO + off);
    const op8 o = TT::load8(p.O + off);
#pragma unroll
    for (int e = 0; e < 8; ++e) dpart += (float)dop[e] * (float)o[e];
  }
  const float Dq = wave_sum_groups(dpart);

  // ---- routing row -> region corners; an entry outside [0, S*S) or a
  // repeated one makes the region's dQ NaN
  if (tid == 0) sbad = 0;
  if (tid < kMaxRegions / 32) rmask[tid] = 0u;
  __syncthreads();
  for (int j = tid; j < p.topk; j += blockDim.x) {
    const int r = p.idx[((int64_t)b * p.R + i) * p.topk + j];
    const bool ok = r >= 0 && r < p.R;
    int rx;
    const int ry = fdiv(ok ? r : 0, p.div_S, &rx);
    rtab[j] = ry * p.sh * p.W + rx * p.sw;
    if (!ok) sbad = 1;
    else atomicOr(&rmask[r >> 5], 1u << (r & 31));
  }
  __syncthreads();
  int distinct = 0;
#pragma unroll
  for (int e = 0; e < kMaxRegions / 32; ++e) distinct += __popc(rmask[e]);
  __bf16* dQg = p.dQ + img;
  if (sbad || distinct != p.topk) {  // uniform over the workgroup; no load issued yet
    if (qvalid) {
      float nanv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) nanv[e] = __builtin_nanf("");
      TT::store8(dQg + qtok * p.C + ch0 + 8 * g, nanv);
    }
    return;
  }

  // ---- every phase's direct-to-LDS loads, in phase order. The query loads
  // have landed first: from here on the only vector-memory loads in flight are
  // these, so the waits below count them alone.
  wait_vmcnt<0>();
  const __bf16* Kg = p.K + img;
  const __bf16* Vg = p.V + img;
  int cnt[NPH];
  unsigned char* kb[4] = {k0, k1, k2, k3};
  unsigned char* vb[4] = {v0, v1, v2, v3};
#pragma unroll
  for (int ph = 0; ph < NPH; ++ph) {
    const int p0 = ph * kPhaseRows;
    cnt[ph] = issue_phase(p, rtab, Kg, Vg, ch0, p0, min(kPhaseRows, p.kvpad - p0), kb[ph], vb[ph], wave, nw, lane);
  }

  // this lane's read bases (bits 3-4 of the rows do not change from chunk to
  // chunk): A rows 8 (col / 4) + col % 4 at chunk g; transposing reads of
  // K^T, in which lane col = 4 s + q reads key row 8g + s (+4) at channels
  // 8 q + 4 ct .. +3 (row r of the tile is channel 8 (r / 4) + 4 ct + r % 4)
  const int a_row = row_off(8 * (col >> 2) + (col & 3), g);
  const int a_tr = row_off(8 * g + (col >> 2), col & 3);

  // ---- one pass, phase by phase as the loads land: S^T, dP^T, and with a
  // lazy running maximum m (moved only when a score exceeds it by more than
  // 8 / c, the four lane groups' maxima combined only then) the unnormalised
  // P = exp2(c s - c m), its running sum, dZ = P (dP - D) and
  // dQ^T += K^T dZ^T; at the end dQ and the log-sum-exp from the sum
  const float lazy = 8.0f / p.c;
  float m_run = -INFINITY, lsum = 0.f;
  float s[2][8], dp[2][8];
  floatx4 dq[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
  int after = 0;
#pragma unroll
  for (int ph = 0; ph < NPH; ++ph) after += cnt[ph];
#pragma unroll
  for (int ph = 0; ph < NPH; ++ph) {
    after -= cnt[ph];
    if (ph == 0) {
      wait_vmcnt_at_most(after);
      __builtin_amdgcn_s_barrier();
    } else if (ph == 1) {
      wait_vmcnt<0>();
      __builtin_amdgcn_s_barrier();
    }
    const int p0 = ph * kPhaseRows;
    const int rows = min(kPhaseRows, p.kvpad - p0);
    const unsigned char* kl = kb[ph] + a_row;
    const unsigned char* vl = vb[ph] + a_row;
    const unsigned char* kt = kb[ph] + a_tr;
#pragma unroll
    for (int c = 0; c < kPhaseRows / KC; ++c) {
      const int r0 = c * KC;
      if (r0 >= rows) break;  // uniform
      chunk_products<true>(kl + r0 * kRowBytes, vl + r0 * kRowBytes, qop, dop, s, dp);
      const int nvalid = p.kv - (p0 + r0);
      if (RAGGED && nvalid < KC) {  // uniform
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (st * 32 + 8 * g + e >= nvalid) s[st][e] = -INFINITY;
      }
      float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
      for (int e = 2; e < 16; ++e) mx = fmaxf(mx, s[e >> 3][e & 7]);
      if (__builtin_amdgcn_ballot_w64(mx > m_run + lazy) != 0) {  // uniform; always at the first chunk
        mx = wave_max_groups(mx);
        const float mnew = mx > m_run + lazy ? mx : m_run;
        const float alpha = __builtin_amdgcn_exp2f((m_run - mnew) * p.c);  // 0 at the start
        dq[0] *= alpha;
        dq[1] *= alpha;
        lsum *= alpha;
        m_run = mnew;
      }
      const float mc = m_run * p.c;
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        float dz[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[st][e], p.c, -mc));
          lsum += pr;
          dz[e] = pr * (dp[st][e] - Dq);
        }
        const op8 zop = TT::from_f32(dz);
        const op8 zlo = TT::residual(dz, zop);  // dZ's low bits
        const unsigned char* kr = kt + (r0 + st * 32) * kRowBytes;
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(kr + 8 * ct));
          const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(kr + 4 * kRowBytes + 8 * ct));
          const op8 ka = __builtin_bit_cast(op8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          dq[ct] = TT::mma(ka, zop, dq[ct]);
          dq[ct] = TT::mma(ka, zlo, dq[ct]);
        }
      }
    }
  }
  const float ltot = wave_sum_groups(lsum);
  const float lse = m_run * p.c + __builtin_log2f(ltot);
  const float inv_l = 1.0f / ltot;
  dq[0] *= inv_l;
  dq[1] *= inv_l;
  if (qvalid) {
    // tile ct: this lane holds channels 8g + 4 ct .. +3 of its query
    float o[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      o[e] = dq[0][e] * p.scale;
      o[4 + e] = dq[1][e] * p.scale;
    }
    TT::store8_nt(dQg + qtok * p.C + ch0 + 8 * g, o);
    if (g == 0) {
      const int64_t at = ((int64_t)b * p.H * p.W + qtok) * p.heads + head;
      p.lse[at] = lse;
      p.dd[at] = Dq;
    }
  }
}

}  // namespace

bool backward_dq_dense_fits(const Shape& s, int dtype) {
  return dtype == kBF16 && s.d == kHeadDim && s.kv > KC && s.kv <= kMaxPhases * kPhaseRows;
}

hipError_t launch_backward_dq_dense(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                                    const int32_t* idx, void* dQ, float* lse, float* dd, const Shape& s,
                                    hipStream_t stream) {
  BwdDenseParams p{};
  p.Q = static_cast<const __bf16*>(Q);
  p.K = static_cast<const __bf16*>(K);
  p.V = static_cast<const __bf16*>(V);
  p.O = static_cast<const __bf16*>(O);
  p.dO = static_cast<const __bf16*>(dO);
  p.idx = idx;
  p.dQ = static_cast<__bf16*>(dQ);
  p.lse = lse;
  p.dd = dd;
  p.H = s.H; p.W = s.W; p.C = s.C; p.S = s.S; p.topk = s.topk;
  p.sh = s.sh; p.sw = s.sw; p.n = s.n; p.R = s.R; p.kv = s.kv; p.heads = s.heads;
  p.kvpad = (s.kv + KC - 1) / KC * KC;
  p.qblk = std::min(16 * kTiles, (s.n + 15) / 16 * 16);
  p.nqb = (s.n + p.qblk - 1) / p.qblk;
  p.scale = 1.0f / sqrtf((float)s.d);
  p.c = p.scale * 1.4426950408889634f;
  p.div_n = make_fastdiv(s.n);
  p.div_sw = make_fastdiv(s.sw);
  p.div_S = make_fastdiv(s.S);
  const int nph = (p.kvpad + kPhaseRows - 1) / kPhaseRows;
  const bool ragged = s.kv % KC != 0;
  const void* fns[2][4] = {
      {(const void*)&bwd_dq_dense_kernel<false, 1>, (const void*)&bwd_dq_dense_kernel<false, 2>,
       (const void*)&bwd_dq_dense_kernel<false, 3>, (const void*)&bwd_dq_dense_kernel<false, 4>},
      {(const void*)&bwd_dq_dense_kernel<true, 1>, (const void*)&bwd_dq_dense_kernel<true, 2>,
       (const void*)&bwd_dq_dense_kernel<true, 3>, (const void*)&bwd_dq_dense_kernel<true, 4>}};
  const int64_t nitems = (int64_t)s.B * s.R * p.nqb * s.heads;
  if (nitems >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  void* args[] = {&p};
  return hipLaunchKernel(fns[ragged][nph - 1], dim3((unsigned)nitems), dim3(p.qblk / 16 * 64), args, 0, stream);
}

}  // namespace bra
