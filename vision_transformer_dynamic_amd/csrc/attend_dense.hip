// Fused gather + token attention for regions that route more than 64 keys
// per query (bf16): the dense-prediction shapes, e.g. 16 x 16 regions with
// four routed regions, 1024 keys per query (explainer "BiFormer Reshapes
// Visual Attention with 'Bi-Level Routing'", Part 2.2 step 4 and pseudocode
// steps 6-7; Part 4.3: S = 8 for segmentation, S = 16 for detection).
//
// One workgroup = one work item (image b, query region i, block of up to 256
// of its queries, head m); one wave per 16-query tile. Every routed key of
// the head is staged in LDS once, and the waves then run through all of them
// with no barrier inside a phase:
//
//  * Staging by direct-to-LDS loads (global_load_lds_dwordx4): each wave
//    instruction gathers 16 key rows (64 bytes each: the head's 32 channels)
//    straight from K or V into a 1 KB block of LDS, no registers involved.
//    Rows are split into phases of 256 keys, each with its own K and V
//    buffers; every wave issues its loads phase by phase. Before phase 0 a
//    wave waits only for its own loads of phase 0, then one barrier; before
//    phase 1 for all of its loads, then a second barrier. The later phases'
//    loads stay in flight under phase 0's products.
//  * K rows are the A operands of S^T = K Q^T (16-byte reads, chunks of a
//    row swizzled so that the 16 lanes of a read pass hit distinct banks).
//  * V stays key-major as loaded: the A operand of O^T = V^T P^T (row =
//    channel, contraction slots = keys) is read with gfx950's transposing
//    LDS read ds_read_b64_tr_b16, which hands lane j of a 16-lane group
//    element j % 4 of the 8-byte reads of lanes 4 s + j / 4, s = 0..3: the
//    16 lanes read 4 keys x 16 channels and each ends up with 4 keys of one
//    channel. Two such reads give a lane its 8 contraction slots.
//  * Scores, softmax and P are as in the other attention kernels: S^T tiles
//    put a query's 8 keys of each 32-key step in one lane, whose
//    probabilities are exactly the P^T slots the lane supplies next, so P
//    never leaves registers; online softmax over 64-key chunks with a lazy
//    running maximum (below); the denominator is a matrix product against an
//    all-ones operand, from the same bf16 P.
//  * Row r of output tile ct of O^T is channel 8 (r / 4) + 4 ct + r % 4, so
//    a lane holds 8 consecutive channels of its query over the two tiles
//    (one 16-byte store; with 4 channels per tile and two 8-byte stores, 1.8
//    times O's bytes reached memory).
#include "bra_internal.h"
#include "attn_common.h"
#include "lds_dma.h"

#include <math.h>

#include <algorithm>

namespace bra {
namespace {

constexpr int kPhaseRows = 256;   // key rows per phase
constexpr int kMaxPhases = 4;     // at most 1024 keys per query
constexpr int kDenseTiles = 16;   // query tiles (waves) per workgroup at most
constexpr int kRowBytes = 64;     // one head of one key: 32 bf16

struct DenseParams {
  const __bf16* Q;
  const __bf16* K;
  const __bf16* V;
  const int32_t* idx;
  __bf16* O;
  int H, W, C, S, topk, sh, sw, n, R, kv, heads;
  int kvpad;   // kv rounded up to 64
  int nqb;     // query blocks per region
  int qblk;    // queries per block (a multiple of 16, <= 256)
  float c;     // softmax scale * log2(e)
  float lazy;  // kLazy / c: how far a score may exceed the running maximum
  FastDiv div_n, div_sw, div_S;
};

// Byte offset of 16-byte chunk c of key row r inside a phase buffer. K: the
// four chunks of a row rotate with bits 3-4 of the row, so that the 16 rows
// of an operand read (rows 8 a + b + 4 t, a, b in 0..3) fall on distinct
// banks. V: chunk pairs swap with bit 3 of the row, so that the two 16-lane
// groups of a transposing read pass (rows 8 g + s and 8 (g + 1) + s) use
// different banks.
__device__ __forceinline__ int k_off(int r, int c) { return r * kRowBytes + 16 * (c ^ ((r >> 3) & 3)); }
__device__ __forceinline__ int v_off(int r, int c) { return r * kRowBytes + 16 * (c ^ (((r >> 3) & 1) << 1)); }

// Issue the direct-to-LDS loads of one phase of this wave: row blocks (16 key
// rows, 1 KB per tensor) m = wave, wave + nw, ... of the phase. Lane l
// gathers row 16 m + l / 4, chunk (l % 4) ^ swizzle: exactly the chunk that
// belongs in its fixed LDS slot. Rows past kv read key 0's token (finite
// values; their scores are masked). Returns the number of loads issued.
__device__ __forceinline__ int issue_phase(const DenseParams& p, const int* rtab, const __bf16* Kg, const __bf16* Vg,
                                           int ch0, int p0, int rows, unsigned char* kbuf, unsigned char* vbuf,
                                           int wave, int nw, int lane) {
  int cnt = 0;
  for (int m = wave; m * 16 < rows; m += nw) {  // uniform
    const int rl = 16 * m + (lane >> 2);        // row inside the phase
    const int r = p0 + rl;                      // routed key
    int tok;
    {
      int tk, tx;
      const int key = r < p.kv ? r : 0;
      const int jr = fdiv(key, p.div_n, &tk);
      const int ty = fdiv(tk, p.div_sw, &tx);
      tok = rtab[jr] + ty * p.W + tx;
    }
    const int ck = (lane & 3) ^ ((rl >> 3) & 3);
    const int cv = (lane & 3) ^ (((rl >> 3) & 1) << 1);
    const int64_t off = (int64_t)tok * p.C + ch0;
    dma16(Kg + off + 8 * ck, lds_offset(kbuf + 1024 * m));
    dma16(Vg + off + 8 * cv, lds_offset(vbuf + 1024 * m));
    cnt += 2;
  }
  return cnt;
}

// Scores, softmax and P.V for one 64-key chunk. kl: this lane's K operand
// row of the chunk (key 8 (col / 4) + col % 4, chunk g swizzled), vl[ct]:
// this lane's transposing-read address of tile ct (key row 8g + col / 4,
// channels 8 (col % 4) + 4 ct); the rest of each address is a constant.
// nvalid: keys of the chunk below kv (RAGGED only).
//
// Online softmax with a lazy maximum: a lane's running maximum m moves only
// when a score exceeds it by more than kLazy / c (2^8 in the exponent), so
// the probabilities exp2(c (s - m)) stay below 2^8 (exact enough in fp32 and
// in bf16, whose relative rounding does not depend on the magnitude) and the
// accumulators are rescaled far less often than the maximum grows.
constexpr float kLazy = 8.0f;

template <bool RAGGED>
__device__ __forceinline__ void dense_chunk(const DenseParams& p, const unsigned char* kl, const unsigned char* vl0,
                                            const unsigned char* vl1, int nvalid, int g, const bf16x8& qop,
                                            const bf16x8& ones, floatx4 (&acc)[3], float& m_run) {
  typedef Tr<__bf16> TT;
  // ---- S^T: rows of tile (st, tb) are keys st*32 + 8*(col/4) + col%4 + 4*tb
  float s[2][8];
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    floatx4 sab[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const bf16x8 k = *reinterpret_cast<const bf16x8*>(kl + (st * 32 + 4 * tb) * kRowBytes);
      sab[tb] = TT::mma(k, qop, floatx4{0.f, 0.f, 0.f, 0.f});
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s[st][e] = sab[0][e];
      s[st][4 + e] = sab[1][e];
    }
  }
  // lane group g holds keys st*32 + 8g + e of its query
  if (RAGGED && nvalid < KC) {  // uniform
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (st * 32 + 8 * g + e >= nvalid) s[st][e] = -INFINITY;
  }
  // the lane's own maximum; the 4 lane groups' maxima are combined only when
  // some lane's exceeds the lazy bound (always at the first chunk, where
  // m_run = -inf), so the common case has no cross-lane exchange (dense map:
  // 23.4 -> 22.0 us)
  float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
  for (int e = 2; e < 16; ++e) mx = fmaxf(mx, s[e >> 3][e & 7]);
  if (__builtin_amdgcn_ballot_w64(mx > m_run + p.lazy) != 0) {  // uniform
    mx = wave_max_groups(mx);
    const bool grow = mx > m_run + p.lazy;
    const float mnew = grow ? mx : m_run;
    const float alpha = __builtin_amdgcn_exp2f((m_run - mnew) * p.c);  // 1 where m stays, 0 at the start
#pragma unroll
    for (int ct = 0; ct < 3; ++ct) acc[ct] *= alpha;
    m_run = mnew;
  }
  const float mc = m_run * p.c;
  // ---- O^T += V^T P^T over the chunk's two 32-key steps. The V^T operand
  // of tile ct, lane group g: slots = keys st*32 + 8g .. +7, from two
  // transposing reads (keys +0..3, +4..7). In a read, lane col = 4 s + q of
  // the group reads key row 8g + s at channels 8 q + 4 ct .. +3, so that lane
  // j of the group receives channel 8 (j / 4) + 4 ct + j % 4 of the four keys.
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    float pe[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) pe[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[st][e], p.c, -mc));
    const bf16x8 pop = TT::from_f32(pe);
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const unsigned char* va_p = (ct == 0 ? vl0 : vl1) + st * 32 * kRowBytes;
      const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(va_p));
      const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(va_p + 4 * kRowBytes));
      const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      acc[ct] = TT::mma(va, pop, acc[ct]);
    }
    acc[2] = TT::mma(ones, pop, acc[2]);
  }
}

template <bool RAGGED, int NPH>
__global__ __launch_bounds__(kDenseTiles * 64) void attend_dense_kernel(DenseParams p) {
  typedef Tr<__bf16> TT;
  // one K and one V buffer per phase, each its own array
  __shared__ __align__(16) unsigned char k0[kPhaseRows * kRowBytes], v0[kPhaseRows * kRowBytes];
  __shared__ __align__(16) unsigned char k1[NPH > 1 ? kPhaseRows * kRowBytes : 16], v1[NPH > 1 ? kPhaseRows * kRowBytes : 16];
  __shared__ __align__(16) unsigned char k2[NPH > 2 ? kPhaseRows * kRowBytes : 16], v2[NPH > 2 ? kPhaseRows * kRowBytes : 16];
  __shared__ __align__(16) unsigned char k3[NPH > 3 ? kPhaseRows * kRowBytes : 16], v3[NPH > 3 ? kPhaseRows * kRowBytes : 16];
  __shared__ int rtab[kMaxRegions];
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

  // ---- the wave's query operand (B operand of S^T: column = query col,
  // slots = channels 8g .. 8g + 7)
  const int qi = qb * p.qblk + wave * 16 + col;
  const bool qvalid = qi < p.n;
  int qoff = 0;
  bf16x8 qop = TT::zero();
  if (qvalid) {
    int qx;
    const int qy = fdiv(qi, p.div_sw, &qx);
    qoff = (qcorner + qy * p.W + qx) * p.C + ch0;
    qop = TT::load8(p.Q + img + qoff + 8 * g);
  }

  // ---- routing row -> region corners; an entry outside [0, S*S) is never
  // dereferenced (corner 0) and makes the item's output NaN
  if (tid == 0) sbad = 0;
  __syncthreads();
  for (int j = tid; j < p.topk; j += blockDim.x) {
    const int r = p.idx[((int64_t)b * p.R + i) * p.topk + j];
    const bool ok = r >= 0 && r < p.R;
    int rx;
    const int ry = fdiv(ok ? r : 0, p.div_S, &rx);
    rtab[j] = ry * p.sh * p.W + rx * p.sw;
    if (!ok) sbad = 1;
  }
  __syncthreads();
  const bool bad = sbad;

  // ---- every phase's direct-to-LDS loads, in phase order. The query load
  // has landed first: from here on the only vector-memory loads in flight are
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
    const int rows = min(kPhaseRows, p.kvpad - p0);
    cnt[ph] = issue_phase(p, rtab, Kg, Vg, ch0, p0, rows, kb[ph], vb[ph], wave, nw, lane);
  }

  const bf16x8 ones = TT::ones();
  floatx4 acc[3] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
  float m_run = -INFINITY;
  int after = 0;
#pragma unroll
  for (int ph = 0; ph < NPH; ++ph) after += cnt[ph];
#pragma unroll
  for (int ph = 0; ph < NPH; ++ph) {
    after -= cnt[ph];
    // Phase 0 waits for its own loads. By the end of its products the later
    // phases have landed as well (measured per workgroup with timestamps),
    // so phase 1 waits once for all the rest and phases 2 and 3 need no
    // barrier, whose waits would idle the waves that finish a phase first
    // (dense map: 22.0 -> 21.8 us).
    if (ph == 0) {
      wait_vmcnt_at_most(after);  // this wave's loads of phase 0 have landed
      __builtin_amdgcn_s_barrier();  // and every other wave's
    } else if (ph == 1) {
      wait_vmcnt<0>();
      __builtin_amdgcn_s_barrier();
    }
    const int p0 = ph * kPhaseRows;
    const int rows = min(kPhaseRows, p.kvpad - p0);
    const unsigned char* kbuf = ph == 0 ? k0 : ph == 1 ? k1 : ph == 2 ? k2 : k3;
    const unsigned char* vbuf = ph == 0 ? v0 : ph == 1 ? v1 : ph == 2 ? v2 : v3;
    // this lane's operand addresses in the phase's first chunk (k_off and
    // v_off with the chunk-independent part of the row: bits 3-4 of the key
    // rows a lane reads do not change from chunk to chunk)
    const unsigned char* kl = kbuf + k_off(8 * (col >> 2) + (col & 3), g);
    const int srow = col >> 2, q = col & 3;
    const unsigned char* vl0 = vbuf + v_off(8 * g + srow, q);      // channels 8 q .. +3
    const unsigned char* vl1 = vbuf + v_off(8 * g + srow, q) + 8;  // channels 8 q + 4 .. +7
    // the phase's chunks unrolled, so every operand address is the lane's
    // base plus a constant (dense map: 24.0 -> 23.4 us)
#pragma unroll
    for (int c = 0; c < kPhaseRows / KC; ++c) {
      const int r0 = c * KC;
      if (r0 >= rows) break;  // uniform
      const int nvalid = p.kv - (p0 + r0);
      const int db = r0 * kRowBytes;
      if (RAGGED && nvalid < KC)
        dense_chunk<true>(p, kl + db, vl0 + db, vl1 + db, nvalid, g, qop, ones, acc, m_run);
      else
        dense_chunk<false>(p, kl + db, vl0 + db, vl1 + db, KC, g, qop, ones, acc, m_run);
    }
  }

  // ---- normalise and store: tile ct holds channels 8 g + 4 ct .. + 3, so
  // the lane's 8 channels are one 16-byte store
  if (!qvalid) return;
  const float inv = bad ? __builtin_nanf("") : 1.0f / acc[2][0];
  float o[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    o[e] = acc[0][e] * inv;
    o[4 + e] = acc[1][e] * inv;
  }
  TT::store8_nt(p.O + img + qoff + 8 * g, o);
}

}  // namespace

bool dense_attend_fits(const Shape& s, int dtype) {
  return dtype == kBF16 && s.kv > KC && s.kv <= kMaxPhases * kPhaseRows;
}

hipError_t launch_attend_dense(const void* Q, const void* K, const void* V, const int32_t* idx, void* O,
                               const Shape& s, hipStream_t stream) {
  DenseParams p{};
  p.Q = static_cast<const __bf16*>(Q);
  p.K = static_cast<const __bf16*>(K);
  p.V = static_cast<const __bf16*>(V);
  p.idx = idx;
  p.O = static_cast<__bf16*>(O);
  p.H = s.H; p.W = s.W; p.C = s.C; p.S = s.S; p.topk = s.topk;
  p.sh = s.sh; p.sw = s.sw; p.n = s.n; p.R = s.R; p.kv = s.kv; p.heads = s.heads;
  p.kvpad = (s.kv + KC - 1) / KC * KC;
  p.qblk = std::min(16 * kDenseTiles, (s.n + 15) / 16 * 16);
  p.nqb = (s.n + p.qblk - 1) / p.qblk;
  p.c = 1.4426950408889634f / sqrtf((float)s.d);
  p.lazy = kLazy / p.c;
  p.div_n = make_fastdiv(s.n);
  p.div_sw = make_fastdiv(s.sw);
  p.div_S = make_fastdiv(s.S);
  const int nph = (p.kvpad + kPhaseRows - 1) / kPhaseRows;
  const bool ragged = s.kv % KC != 0;
  const void* fns[2][4] = {
      {(const void*)&attend_dense_kernel<false, 1>, (const void*)&attend_dense_kernel<false, 2>,
       (const void*)&attend_dense_kernel<false, 3>, (const void*)&attend_dense_kernel<false, 4>},
      {(const void*)&attend_dense_kernel<true, 1>, (const void*)&attend_dense_kernel<true, 2>,
       (const void*)&attend_dense_kernel<true, 3>, (const void*)&attend_dense_kernel<true, 4>}};
  const int64_t nitems = (int64_t)s.B * s.R * p.nqb * s.heads;
  void* args[] = {&p};
  return hipLaunchKernel(fns[ragged][nph - 1], dim3((unsigned)nitems), dim3(p.qblk / 16 * 64), args, 0, stream);
}

}  // namespace bra
