// Backward of the token attention over routed regions, with the routing
// table held fixed (explainer "BiFormer Reshapes Visual Attention with
// 'Bi-Level Routing'", Part 2.2 step 4 and pseudocode steps 6-7 for the
// forward; Part 7 reports training throughput, i.e. the module is trained
// through this path). The top-k indices carry no gradient, so neither does the
// region pooling; the gradients are those of ordinary softmax attention of
// every region's queries over its routed keys:
//
//   P = softmax(Z), Z = scale * q k^T;  dV_g = P^T dO;  dP = dO V_g^T;
//   dZ = P * (dP - D), D = rowsum(dO * O) = rowsum(P * dP);
//   dQ = scale * dZ K_g;  dK_g = scale * dZ^T Q
//
// with dK, dV of a token summed over every query region routed to its region.
//
// Three steps, all deterministic (no atomics on gradients):
//  1. inverse_table: per image, the inverse routing table - for every key
//     region, the ascending list of query regions whose rows hold it. A row
//     with an entry outside [0, S*S), or a repeated entry, is marked bad and
//     left out (the dQ kernels give its queries NaN). With at most 64 keys
//     per query and 64 regions it runs as B leading workgroups of the dQ
//     launch (only step 3 needs it); otherwise bwd_routes_kernel, a launch of
//     its own.
//  2. dQ: the forward's transposed products (S^T = K Q^T, dP^T = V dO^T,
//     dQ^T = K^T dZ^T with K^T through LDS), D from O and dO, and the base-2
//     log-sum-exp of every query, written for kernel 3. With at most 64 keys
//     per query, bwd_dq_head_kernel: one wave per head looping over the
//     query tiles, as in the forward. With several 64-key chunks,
//     bwd_dq_kernel: one wave per (head, 16-query tile), two passes
//     (log-sum-exp first); in bf16 with head dim 32 and at most 1024 keys,
//     the dense form of backward_dense.hip (every routed key staged in LDS).
//  3. bwd_dkv_kernel: per (head, 32 keys of one key region), a loop over the
//     queries of the inverse table's regions, staged in LDS (small regions
//     share a tile): S = Q K^T and dP = dO V^T put each lane on one key with
//     4 queries, exactly the contraction slots of the 16-deep products
//     dV^T += dO^T P and dK^T += Q^T dZ (dO^T, Q^T through LDS), so P and dZ
//     never leave registers. fp32: one wave, stages of 64 queries; bf16: two
//     waves, stages of 128 queries, each wave taking half the 16-query tiles,
//     the second wave's partial sums added to the first's through LDS.
// With top-1 routing and small regions, backward_top1.hip does all three in
// one launch.
#include "attn_common.h"

#include <math.h>

#include <algorithm>

namespace bra {
namespace {

struct BwdParams {
  const void* Q;
  const void* K;
  const void* V;
  const void* O;
  const void* dO;
  const int32_t* idx;
  void* dQ;
  void* dK;
  void* dV;
  float* lse;     // [B*H*W*heads]: base-2 log-sum-exp of c * q.k over the query's keys
  float* dd;      // [B*H*W*heads]: D = dO . O
  int* inv_cnt;   // [B*R]
  int* inv_list;  // [B*R*R]
  int* bad;       // [B*R]
  int* order;     // [B*R]: per image, the key regions by descending in-degree (ties: lower index first)
  int B, H, W, C, S, topk;
  int sh, sw, n, R, kv, heads;
  int HG, nhg, nqb, ntq, nitems_q;    // dq kernel
  int ntab;                           // dq head kernel: leading workgroups that build the inverse table (0 or B)
  int HGk, nhgk, nkb, nitems_kv;      // dkv kernel
  float c;      // scale * log2(e)
  float scale;  // 1 / sqrt(d)
  FastDiv div_n, div_sw, div_S;
};

__device__ inline int corner_of(const BwdParams& p, int r) {
  int rx;
  const int ry = fdiv(r, p.div_S, &rx);
  return ry * p.sh * p.W + rx * p.sw;
}

// workgroup id -> work item (consecutive items to one XCD), for the grid past
// its first `skip` workgroups
__device__ inline int xcd_remap(int skip = 0) { return xcd_item(blockIdx.x - skip, gridDim.x - skip); }

// ---------------------------------------------------------------------------
// 1. Inverse routing table of image b, key regions [r0, r1), by one
// workgroup (a multiple of 64 threads) in lds: R rows of (R + 31) / 32 mask
// words, then R row flags, R in-degrees and R places. Each routing row becomes
// a bit mask of its regions (bitwise OR is order-free); the in-degree of every
// key region is an LDS count over the good rows' entries (integer adds, so the
// order does not matter); then one wave per key region of the range tests 64
// rows at a time and places the good rows that hold it with a ballot prefix
// count, so each list comes out ascending. Every loop is spread over the
// workgroup's threads: no thread walks all R rows or regions (at 256 regions
// a thread per region doing so took about 30 us).
__device__ void inverse_table(const BwdParams& p, int b, uint32_t* lds, int r0, int r1) {
  const int tid = threadIdx.x, nt = blockDim.x;
  const int R = p.R, k = p.topk, nw = (R + 31) >> 5;
  uint32_t* mask = lds;                                  // [R][nw]
  int* rowbad = reinterpret_cast<int*>(lds + R * nw);    // [R]
  int* deg = rowbad + R;                                 // [R]: in-degree of each key region
  int* place = deg + R;                                  // [R]: place of key region r0 + j in the order
  const int32_t* idx = p.idx + (int64_t)b * R * k;
  for (int e = tid; e < R * nw; e += nt) mask[e] = 0u;
  for (int i = tid; i < R; i += nt) rowbad[i] = deg[i] = place[i] = 0;
  __syncthreads();
  for (int e = tid; e < R * k; e += nt) {
    const int i = e / k, r = idx[e];
    if (r < 0 || r >= R)
      rowbad[i] = 1;
    else
      atomicOr(&mask[i * nw + (r >> 5)], 1u << (r & 31));
  }
  __syncthreads();
  // a row with a repeated entry holds fewer than k distinct regions: bad too
  for (int i = tid; i < R; i += nt) {
    int cnt = 0;
    for (int e = 0; e < nw; ++e) cnt += __popc(mask[i * nw + e]);
    if (cnt != k) rowbad[i] = 1;
  }
  __syncthreads();
  // in-degrees: one count per entry of a good row (its entries are distinct)
  for (int e = tid; e < R * k; e += nt) {
    const int i = e / k;
    if (!rowbad[i]) atomicAdd(&deg[idx[e]], 1);
  }
  __syncthreads();
  // wave w compacts the lists of key regions r0 + w, r0 + w + nwaves, ...
  const int wave = tid >> 6, lane = tid & 63, nwaves = nt >> 6;
  const uint64_t below = (uint64_t(1) << lane) - 1;
  for (int r = r0 + wave; r < r1; r += nwaves) {
    int* L = p.inv_list + ((int64_t)b * R + r) * R;
    int m = 0;
    for (int i0 = 0; i0 < R; i0 += 64) {
      const int i = i0 + lane;
      const bool hit = i < R && !rowbad[i] && ((mask[i * nw + (r >> 5)] >> (r & 31)) & 1u);
      const uint64_t bal = __ballot(hit);
      if (hit) L[m + __popcll(bal & below)] = i;
      m += __popcll(bal);
    }
    if (lane == 0) p.inv_cnt[b * R + r] = m;
  }
  // the dK/dV kernel's order: key region r goes to place #{heavier, or as
  // heavy with a lower index}, counted over (r, q) pairs spread over the
  // threads
  const int nr = r1 - r0;
  for (int e = tid; e < nr * R; e += nt) {
    const int j = e / R, q = e - j * R, r = r0 + j;
    const int dq = deg[q], dr = deg[r];
    if (dq > dr || (dq == dr && q < r)) atomicAdd(&place[j], 1);
  }
  __syncthreads();
  for (int j = tid; j < nr; j += nt) {
    const int r = r0 + j;
    p.bad[b * R + r] = rowbad[r];
    p.order[b * R + place[j]] = r;
  }
}

// LDS bytes of inverse_table
constexpr size_t inverse_table_lds(int R) { return sizeof(uint32_t) * ((size_t)R * ((R + 31) / 32) + 3 * R); }

// For more than 64 regions: a launch of its own, one workgroup per (image,
// block of kRoutesBlock key regions); each rebuilds the image's masks.
constexpr int kRoutesBlock = 16;
__global__ __launch_bounds__(256) void bwd_routes_kernel(BwdParams p) {
  __shared__ uint32_t lds[kMaxRegions * (kMaxRegions / 32) + 3 * kMaxRegions];
  const int nblk = (p.R + kRoutesBlock - 1) / kRoutesBlock;
  const int b = blockIdx.x / nblk, r0 = (blockIdx.x - b * nblk) * kRoutesBlock;
  inverse_table(p, b, lds, r0, min(p.R, r0 + kRoutesBlock));
}

// Chunk token table: tok[kappa - c0] = token (inside the image) of routed key
// kappa of the chunk starting at c0, -1 past kv. rb holds the routed regions'
// corners.
__device__ __forceinline__ void build_tok(int* tok, const int* rb, int tid, int c0, int kv, int W, FastDiv div_n,
                                          FastDiv div_sw) {
  if (tid < KC) {
    const int kappa = c0 + tid;
    int t = -1;
    if (kappa < kv) {
      int tk, tx;
      const int jr = fdiv(kappa, div_n, &tk);
      const int ty = fdiv(tk, div_sw, &tx);
      t = rb[jr] + ty * W + tx;
    }
    tok[tid] = t;
  }
}

// A-operand row rr = col of the (32-key step st, tile tb) is key
// st*32 + 8*(rr/4) + (rr%4) + 4*tb, so lane group g holds keys 8g..8g+7 of
// every 32-key step: the slots of the dZ^T operand.
__device__ __forceinline__ int key_of(int col, int st, int tb) { return st * 32 + 8 * (col >> 2) + (col & 3) + 4 * tb; }

// ---------------------------------------------------------------------------
// 2. dQ, log-sum-exp and D when the keys span several 64-key chunks.
// Workgroup = (image b, query region i, block of <= 64 queries, group of HG
// heads); wave w = (head w / ntq, tile w % ntq). Pass 1 takes the log-sum-exp
// over all chunks, pass 2 the gradient.
template <typename T, bool RAGGED>
__global__ __launch_bounds__(512) void bwd_dq_kernel(BwdParams p) {
  typedef Tr<T> TT;
  typedef typename TT::op8 op8;
  constexpr int VEC = TT::VEC;
  constexpr int CVH = D / VEC;
  constexpr int ITEMS = KC / 2 * CVH;  // (key pair, vector) items of one K^T tile
  extern __shared__ __align__(16) unsigned char smem_raw[];
  __shared__ int tok[KC];
  __shared__ int rb[kMaxRegions];
  __shared__ uint32_t rmask[kMaxRegions / 32];  // the row's regions, for the repeated-entry check
  __shared__ int sbad;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4, col = lane & 15;
  const int ldk = KC + TT::PADV;

  int w = xcd_remap();
  const int hg = w % p.nhg;
  w /= p.nhg;
  const int qb = w % p.nqb;
  w /= p.nqb;
  const int i = w % p.R;
  const int b = w / p.R;
  const int hl = wave / p.ntq, t = wave - hl * p.ntq;
  const int head = hg * p.HG + hl;
  const bool head_ok = head < p.heads;
  const int ch0 = head * D;
  const int64_t img = (int64_t)b * p.H * p.W * p.C;
  const T* Kg = static_cast<const T*>(p.K) + img;
  const T* Vg = static_cast<const T*>(p.V) + img;
  T* Kt = reinterpret_cast<T*>(smem_raw) + hl * D * ldk;  // K^T tile of this wave's head

  // the routed regions' corners
  if (tid == 0) sbad = 0;
  if (tid < kMaxRegions / 32) rmask[tid] = 0u;
  __syncthreads();
  for (int j = tid; j < p.topk; j += blockDim.x) {
    const int r = p.idx[((int64_t)b * p.R + i) * p.topk + j];
    const bool ok = r >= 0 && r < p.R;
    rb[j] = corner_of(p, ok ? r : 0);
    if (!ok) sbad = 1;
    else atomicOr(&rmask[r >> 5], 1u << (r & 31));
  }

  // the wave's queries: B operands of q and dO, and D = dO . O per query
  const int q0 = qb * 64;
  const int qi = q0 + t * 16 + col;
  const bool qvalid = head_ok && t * 16 < min(64, p.n - q0) && qi < p.n;
  int qtok = 0;
  op8 qop = TT::zero(), dop = TT::zero();
  float dpart = 0.f;
  {
    int qx;
    const int qy = fdiv(qi < p.n ? qi : 0, p.div_sw, &qx);
    int rx;
    const int ry = fdiv(i, p.div_S, &rx);
    qtok = (ry * p.sh + qy) * p.W + rx * p.sw + qx;
    if (qvalid) {
      const int off = qtok * p.C + ch0 + 8 * g;
      qop = TT::load8(static_cast<const T*>(p.Q) + img + off);
      dop = TT::load8(static_cast<const T*>(p.dO) + img + off);
      const op8 o = TT::load8(static_cast<const T*>(p.O) + img + off);
#pragma unroll
      for (int e = 0; e < 8; ++e) dpart += (float)dop[e] * (float)o[e];
    }
  }
  const float Dq = wave_sum_groups(dpart);
  __syncthreads();
  // an entry outside [0, S*S), or a repeated one (fewer distinct regions than topk)
  int distinct = 0;
#pragma unroll
  for (int e = 0; e < kMaxRegions / 32; ++e) distinct += __popc(rmask[e]);
  const bool bad = sbad || distinct != p.topk;
  T* dQg = static_cast<T*>(p.dQ) + img;
  if (bad) {
    // a routing entry outside [0, S*S): gradient NaN for the region's queries
    if (qvalid) {
      float nanv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) nanv[e] = __builtin_nanf("");
      TT::store8(dQg + qtok * p.C + ch0 + 8 * g, nanv);
    }
    return;  // uniform over the workgroup
  }

  const int nchunks = (p.kv + KC - 1) / KC;
  const int kv = p.kv, W = p.W;
  const FastDiv div_n = p.div_n, div_sw = p.div_sw;

  // ---- pass 1: running max and sum per query
  float m = -INFINITY, l = 0.f;
  {
    for (int ch = 0; ch < nchunks; ++ch) {
      build_tok(tok, rb, tid, ch * KC, kv, W, div_n, div_sw);
      __syncthreads();
      float s[2][8];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        op8 ka = TT::zero(), kb = TT::zero();
        const int t0 = tok[key_of(col, st, 0)], t1 = tok[key_of(col, st, 1)];
        if (head_ok && t0 >= 0) ka = TT::load8(Kg + t0 * p.C + ch0 + 8 * g);
        if (head_ok && t1 >= 0) kb = TT::load8(Kg + t1 * p.C + ch0 + 8 * g);
        const floatx4 sa = TT::mma(ka, qop, floatx4{0.f, 0.f, 0.f, 0.f});
        const floatx4 sb = TT::mma(kb, qop, floatx4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s[st][e] = sa[e];
          s[st][4 + e] = sb[e];
        }
      }
      const int c0 = ch * KC;
      float mx = -INFINITY;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if (RAGGED && c0 + st * 32 + 8 * g + e >= p.kv) s[st][e] = -INFINITY;
          mx = fmaxf(mx, s[st][e]);
        }
      mx = wave_max_groups(mx);
      const float mn = fmaxf(m, mx);
      float add = 0.f;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int e = 0; e < 8; ++e) add += __builtin_amdgcn_exp2f((s[st][e] - mn) * p.c);
      l = l * __builtin_amdgcn_exp2f((m - mn) * p.c) + add;
      m = mn;
      __syncthreads();  // tok reused by the next chunk
    }
  }
  const float lse = m * p.c + __builtin_log2f(wave_sum_groups(l));

  // ---- pass 2: P, dP, dZ and dQ^T += K^T dZ^T
  floatx4 dq[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
  for (int ch = 0; ch < nchunks; ++ch) {
    const int c0 = ch * KC;
    build_tok(tok, rb, tid, c0, kv, W, div_n, div_sw);
    __syncthreads();
    // K^T tile of this head, written by the head's ntq waves together
    for (int f = t * 64 + lane; f < ITEMS; f += p.ntq * 64) {
      const int cv = f % CVH, p2 = f / CVH;
      const int ta = tok[2 * p2], tb2 = tok[2 * p2 + 1];
      uint4 va = make_uint4(0u, 0u, 0u, 0u), vb = va;
      if (head_ok && ta >= 0) va = *reinterpret_cast<const uint4*>(Kg + ta * p.C + ch0 + cv * VEC);
      if (head_ok && tb2 >= 0) vb = *reinterpret_cast<const uint4*>(Kg + tb2 * p.C + ch0 + cv * VEC);
      const int row0 = cv * VEC;
      store_vt_pair(Kt, ldk, row0, vt_col(row0, 2 * p2), va, vb);
    }
    float s[2][8], dp[2][8];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int t0 = tok[key_of(col, st, 0)], t1 = tok[key_of(col, st, 1)];
      op8 ka = TT::zero(), kb = TT::zero(), va = TT::zero(), vb = TT::zero();
      if (head_ok && t0 >= 0) {
        ka = TT::load8(Kg + t0 * p.C + ch0 + 8 * g);
        va = TT::load8(Vg + t0 * p.C + ch0 + 8 * g);
      }
      if (head_ok && t1 >= 0) {
        kb = TT::load8(Kg + t1 * p.C + ch0 + 8 * g);
        vb = TT::load8(Vg + t1 * p.C + ch0 + 8 * g);
      }
      const floatx4 sa = TT::mma(ka, qop, floatx4{0.f, 0.f, 0.f, 0.f});
      const floatx4 sb = TT::mma(kb, qop, floatx4{0.f, 0.f, 0.f, 0.f});
      const floatx4 pa = TT::mma(va, dop, floatx4{0.f, 0.f, 0.f, 0.f});
      const floatx4 pb = TT::mma(vb, dop, floatx4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s[st][e] = sa[e];
        s[st][4 + e] = sb[e];
        dp[st][e] = pa[e];
        dp[st][4 + e] = pb[e];
      }
    }
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (RAGGED && c0 + st * 32 + 8 * g + e >= p.kv) s[st][e] = -INFINITY;
    __syncthreads();  // K^T tile complete
    const int vrow = 8 * (col >> 2) + (col & 3);
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      float dz[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[st][e], p.c, -lse));
        dz[e] = pr * (dp[st][e] - Dq);
      }
      const op8 zop = TT::from_f32(dz);
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const int row = vrow + 4 * ct;
        const op8 kt = TT::load8(Kt + row * ldk + vt_col(row, st * 32 + 8 * g));
        dq[ct] = TT::mma(kt, zop, dq[ct]);
        if constexpr (sizeof(T) == 2) dq[ct] = TT::mma(kt, TT::residual(dz, zop), dq[ct]);  // dZ's low bits
      }
    }
    __syncthreads();  // tok and K^T reused by the next chunk
  }

  if (qvalid) {
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

// ---------------------------------------------------------------------------
// 2b. dQ, log-sum-exp and D with a single chunk (at most 64 routed keys per
// query): the forward head kernel's work split. Workgroup = (image b, query
// region i, block of <= 64 queries, group of HG heads), one wave per head that
// loops over the block's <= 4 query tiles. The K and V operands of the 64 keys
// are loaded once per head wave and serve every tile; K^T goes through the
// wave's own LDS tile once; each wave turns the routing row into its own key
// table, so the kernel has no workgroup barrier.
template <typename T, bool RAGGED, int MAXT>
__global__ __launch_bounds__(512) void bwd_dq_head_kernel(BwdParams p) {
  typedef Tr<T> TT;
  typedef typename TT::op8 op8;
  constexpr int VEC = TT::VEC;
  constexpr int CVH = D / VEC;
  constexpr int PAIRS = KC / 2 * CVH / 64;  // (key pair, vector) items of the K^T tile per lane
  extern __shared__ __align__(16) unsigned char smem_raw[];
  __shared__ int wtok[8 * KC];  // per wave: token of every routed key, -1 past kv
  // two heads' dQ halves of a tile's query rows, per tile parity (bf16: 16
  // queries x 8 chunks of 16 bytes)
  __shared__ __align__(16) uint4 xrow[sizeof(T) == 2 ? 2 * 16 * 8 : 1];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, col = lane & 15;
  const int ldk = KC + TT::PADV;

  if ((int)blockIdx.x < p.ntab) {
    // one of the first B workgroups (when the launch builds the inverse
    // routing table): the table of image blockIdx.x, in this kernel's dynamic
    // LDS. They come first in dispatch order, so their slots free up at once.
    inverse_table(p, blockIdx.x, reinterpret_cast<uint32_t*>(smem_raw), 0, p.R);
    return;
  }
  int w = xcd_remap(p.ntab);
  const int hg = w % p.nhg;
  w /= p.nhg;
  const int qb = w % p.nqb;
  w /= p.nqb;
  const int i = w % p.R;
  const int b = w / p.R;
  const int head = hg * p.HG + wave;
  if (head >= p.heads) return;  // wave-uniform; the only barrier below needs both heads present
  // bf16 with two heads per workgroup: the head waves exchange their halves
  // of every dQ row through LDS and store whole 128-byte rows (uniform per
  // workgroup: both waves are present and share the routing row)
  const bool rows = sizeof(T) == 2 && p.HG == 2 && hg * 2 + 1 < p.heads;
  const int ch0 = head * D;
  const int64_t img = (int64_t)b * p.H * p.W * p.C;
  const T* Kg = static_cast<const T*>(p.K) + img;
  const T* Vg = static_cast<const T*>(p.V) + img;
  T* Kt = reinterpret_cast<T*>(smem_raw) + wave * D * ldk;  // this head's K^T tile

  // routing entry of key kappa = lane first (the K/V addresses wait on it)
  int rid = 0, ktok = 0;
  if (lane < p.kv) {
    int tk, tx;
    const int jr = fdiv(lane, p.div_n, &tk);
    const int ty = fdiv(tk, p.div_sw, &tx);
    ktok = ty * p.W + tx;
    rid = p.idx[((int64_t)b * p.R + i) * p.topk + jr];
  }
  // then the query rows of every tile: q and dO as B operands, O for D
  const int q0 = qb * 64;
  const int nq = min(64, p.n - q0);
  const int ntiles = (nq + 15) >> 4;
  int qcorner;
  {
    int rx;
    const int ry = fdiv(i, p.div_S, &rx);
    qcorner = ry * p.sh * p.W + rx * p.sw;
  }
  op8 qop[MAXT], dop[MAXT];
  int qtok[MAXT];
  float Dq[MAXT];
  {
    op8 oop[MAXT];
#pragma unroll
    for (int t = 0; t < MAXT; ++t) {
      const int qi = q0 + t * 16 + col;
      qtok[t] = -1;
      qop[t] = TT::zero();
      dop[t] = TT::zero();
      oop[t] = TT::zero();
      if (t < ntiles && qi < q0 + nq) {
        int qx;
        const int qy = fdiv(qi, p.div_sw, &qx);
        qtok[t] = qcorner + qy * p.W + qx;
        const int off = qtok[t] * p.C + ch0 + 8 * g;
        qop[t] = TT::load8(static_cast<const T*>(p.Q) + img + off);
        dop[t] = TT::load8(static_cast<const T*>(p.dO) + img + off);
        oop[t] = TT::load8(static_cast<const T*>(p.O) + img + off);
      }
    }
#pragma unroll
    for (int t = 0; t < MAXT; ++t) {
      float dpart = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) dpart += (float)dop[t][e] * (float)oop[t][e];
      Dq[t] = wave_sum_groups(dpart);
    }
  }

  // the wave's key table
  const bool ok = rid >= 0 && rid < p.R;
  bool bad = __builtin_amdgcn_ballot_w64(lane < p.kv && !ok) != 0;  // uniform
  // a repeated entry: slot j's region (held by lane j * n, the slot's first
  // key) is held by more than one slot's first key
  if (p.topk > 1) {
    int tk;
    (void)fdiv(lane, p.div_n, &tk);
    const bool first = lane < p.kv && tk == 0;
    for (int j = 0; j < p.topk; ++j) {  // uniform; topk * n <= 64
      const int rj = __builtin_amdgcn_readlane(rid, j * p.n);
      bad |= __popcll(__builtin_amdgcn_ballot_w64(first && rid == rj)) > 1;
    }
  }
  int* wt = wtok + wave * KC;
  wt[lane] = lane < p.kv ? corner_of(p, ok ? rid : 0) + ktok : -1;
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  T* dQg = static_cast<T*>(p.dQ) + img;
  if (bad) {
    // a routing entry outside [0, S*S): gradient NaN for the region's queries
    float nanv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) nanv[e] = __builtin_nanf("");
#pragma unroll
    for (int t = 0; t < MAXT; ++t)
      if (qtok[t] >= 0) TT::store8(dQg + qtok[t] * p.C + ch0 + 8 * g, nanv);
    return;
  }

  // K and V operands (A operands of S^T = K Q^T and dP^T = V dO^T), then the
  // K^T tile (A operands of dQ^T += K^T dZ^T) through LDS
  op8 kop[2][2], vop[2][2];
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const int tk = wt[key_of(col, st, tb)];
      kop[st][tb] = TT::zero();
      vop[st][tb] = TT::zero();
      if (tk >= 0) {
        kop[st][tb] = TT::load8(Kg + tk * p.C + ch0 + 8 * g);
        vop[st][tb] = TT::load8(Vg + tk * p.C + ch0 + 8 * g);
      }
    }
#pragma unroll
  for (int m = 0; m < PAIRS; ++m) {
    const int f = lane + 64 * m;
    const int cv = f % CVH, p2 = f / CVH;
    const int ta = wt[2 * p2], tb2 = wt[2 * p2 + 1];
    uint4 va = make_uint4(0u, 0u, 0u, 0u), vb = va;
    if (ta >= 0) va = *reinterpret_cast<const uint4*>(Kg + ta * p.C + ch0 + cv * VEC);
    if (tb2 >= 0) vb = *reinterpret_cast<const uint4*>(Kg + tb2 * p.C + ch0 + cv * VEC);
    const int row0 = cv * VEC;
    store_vt_pair(Kt, ldk, row0, vt_col(row0, 2 * p2), va, vb);
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  const int vrow = 8 * (col >> 2) + (col & 3);

#pragma unroll
  for (int t = 0; t < MAXT; ++t) {
    if (t >= ntiles) break;  // uniform
    float s[2][8], dp[2][8];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const floatx4 sa = TT::mma(kop[st][0], qop[t], floatx4{0.f, 0.f, 0.f, 0.f});
      const floatx4 sb = TT::mma(kop[st][1], qop[t], floatx4{0.f, 0.f, 0.f, 0.f});
      const floatx4 pa = TT::mma(vop[st][0], dop[t], floatx4{0.f, 0.f, 0.f, 0.f});
      const floatx4 pb = TT::mma(vop[st][1], dop[t], floatx4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s[st][e] = sa[e];
        s[st][4 + e] = sb[e];
        dp[st][e] = pa[e];
        dp[st][4 + e] = pb[e];
      }
    }
    if (RAGGED) {
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (st * 32 + 8 * g + e >= p.kv) s[st][e] = -INFINITY;
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
    floatx4 dq[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      float dz[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[st][e], p.c, -lse));
        dz[e] = pr * (dp[st][e] - Dq[t]);
      }
      const op8 zop = TT::from_f32(dz);
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const int row = vrow + 4 * ct;
        const op8 kt = TT::load8(Kt + row * ldk + vt_col(row, st * 32 + 8 * g));
        dq[ct] = TT::mma(kt, zop, dq[ct]);
        if constexpr (sizeof(T) == 2) dq[ct] = TT::mma(kt, TT::residual(dz, zop), dq[ct]);  // dZ's low bits
      }
    }
    if (qtok[t] >= 0) {
      float o[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[e] = dq[0][e] * p.scale;
        o[4 + e] = dq[1][e] * p.scale;
      }
      if constexpr (sizeof(T) == 2) {
        if (rows) xrow[(t & 1) * 128 + xrow_at(col, wave * 4 + g)] = __builtin_bit_cast(uint4, TT::from_f32(o));
        else TT::store8_nt(dQg + qtok[t] * p.C + ch0 + 8 * g, o);
      } else {
        TT::store8_nt(dQg + qtok[t] * p.C + ch0 + 8 * g, o);
      }
      if (g == 0) {
        const int64_t at = ((int64_t)b * p.H * p.W + qtok[t]) * p.heads + head;
        p.lse[at] = lse;
        p.dd[at] = Dq[t];
      }
    }
    if constexpr (sizeof(T) == 2) {
      if (rows) {
        // whole 128-byte rows of the two heads: wave h stores queries 8h ..
        // 8h + 7 of the tile (tile parities alternate: one barrier per tile)
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        const int q = 8 * wave + (lane >> 3), c = lane & 7;
        const int tq = __builtin_amdgcn_ds_bpermute(q << 2, qtok[t]);  // lane q holds query q's token
        if (tq >= 0) {
          const uint4 v = xrow[(t & 1) * 128 + xrow_at(q, c)];
          __builtin_nontemporal_store(__builtin_bit_cast(op8, v),
                                      reinterpret_cast<op8*>(dQg + tq * p.C + hg * p.HG * D + 8 * c));
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 3. dK, dV. Workgroup = (image b, key region r, block of <= 64 of its keys,
// group of HGk heads); wave = (head, key half of 32 keys, slot group).
// The queries of the key region's incoming query regions (inverse table, in
// order) form one flat sequence of slots, taken 64 SPL at a time ("stages"),
// with SPL slot groups each taking a 1 / SPL share of a stage's 16-slot
// tiles. Each stage's Q and dO rows go to LDS as rows (A operands of
// S = Q K^T and dP = dO V^T); the A operands of dV^T += dO^T P and
// dK^T += Q^T dZ are their transposes: in fp32 (SPL = 1) transposed copies
// written beside the rows, in bf16 (SPL = 2) the transposing LDS read of the
// rows. With the slots' log-sum-exp and D, all loads of a stage are in flight
// together, and the next stage's loads are issued before the current one is
// computed. Small regions share a 16-query tile.
constexpr int kStage = 64;  // query slots per stage and slot group

// bf16 stage rows: 64-byte rows (a head's 32 channels), the 16-byte chunk c of
// row r at c ^ 2 when bit 3 of r is set. The transposed operands come from
// these rows by gfx950's transposing LDS read, so no transposed copy is
// written. (Measured with SQ_LDS_BANK_CONFLICT: 16-byte reads of 16
// consecutive rows meet no bank conflict this way, transposing reads 2 cycles;
// the padded rows and transposed copies cost 4 and more.)
__device__ inline int stage_row(int r, int c) { return r * D + 8 * (c ^ ((r >> 2) & 2)); }

typedef __attribute__((address_space(3))) shortx4 lds_s4;

// Transposing LDS read of 4 bf16 (8 bytes) at p: within each 16-lane group,
// lane j receives element j % 4 of the reads of lanes 4 s + j / 4, s = 0..3.
__device__ inline shortx4 read_tr(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(p));
}

// slot s -> token of the query (inside the image), or -1 past the last slot
__device__ __forceinline__ int slot_token(int s, int nslots, const int* corners, FastDiv div_n, FastDiv div_sw,
                                          int W) {
  if (s >= nslots) return -1;
  int qi, qx;
  const int e = fdiv(s, div_n, &qi);
  const int qy = fdiv(qi, div_sw, &qx);
  return corners[e] + qy * W + qx;
}

// Per-lane share of one stage's loads: NI (slot pair, channel vector, tensor)
// items of two 16-byte vectors, plus one log-sum-exp or D value.
template <int NI>
struct StageRegs {
  uint4 a[NI], b[NI];
  float v;
};

// STG: query slots per stage; the head's 2 STG threads (lane lt) share its
// loads.
template <typename T, int NI, int STG>
__device__ __forceinline__ void stage_load(const BwdParams& p, int s0, int nslots, const int* corners, bool head_ok,
                                           int lt, int ch0, int64_t img, int64_t imgrow, int head,
                                           StageRegs<NI>& R) {
  constexpr int VEC = Tr<T>::VEC;
  constexpr int CVH = D / VEC;
  const T* Qg = static_cast<const T*>(p.Q) + img;
  const T* dOg = static_cast<const T*>(p.dO) + img;
#pragma unroll
  for (int m = 0; m < NI; ++m) {
    const int f = lt + 2 * STG * m;  // < 2 * (STG / 2) * CVH
    const int cv = f % CVH, rest = f / CVH;
    const int qp = rest % (STG / 2), tensor = rest / (STG / 2);
    const T* src = tensor == 0 ? Qg : dOg;
    R.a[m] = make_uint4(0u, 0u, 0u, 0u);
    R.b[m] = R.a[m];
    const int ta = slot_token(s0 + 2 * qp, nslots, corners, p.div_n, p.div_sw, p.W);
    const int tb = slot_token(s0 + 2 * qp + 1, nslots, corners, p.div_n, p.div_sw, p.W);
    if (head_ok && ta >= 0) R.a[m] = *reinterpret_cast<const uint4*>(src + ta * p.C + ch0 + cv * VEC);
    if (head_ok && tb >= 0) R.b[m] = *reinterpret_cast<const uint4*>(src + tb * p.C + ch0 + cv * VEC);
  }
  // lanes 0 .. STG-1: log-sum-exp of slot s0 + lt; the next STG: D of slot s0 + lt - STG
  const int sl = lt % STG;
  const int tr = slot_token(s0 + sl, nslots, corners, p.div_n, p.div_sw, p.W);
  R.v = lt < STG ? INFINITY : 0.f;  // past the last slot: P = 0 and dZ = 0
  if (head_ok && tr >= 0) R.v = (lt < STG ? p.lse : p.dd)[(imgrow + tr) * p.heads + head];
}

template <typename T, int NI, int STG>
__device__ __forceinline__ void stage_store(T* Qn, T* dOn, T* Qt, T* dOt, float* lse, float* dd, int lt,
                                            const StageRegs<NI>& R) {
  constexpr int VEC = Tr<T>::VEC;
  constexpr int CVH = D / VEC;
  constexpr int LDN = D + 16 / (int)sizeof(T);  // row tiles: one 16-byte pad per row
  constexpr int LDT = STG + 16 / (int)sizeof(T);
#pragma unroll
  for (int m = 0; m < NI; ++m) {
    const int f = lt + 2 * STG * m;
    const int cv = f % CVH, rest = f / CVH;
    const int qp = rest % (STG / 2), tensor = rest / (STG / 2);
    T* rows = tensor == 0 ? Qn : dOn;
    if constexpr (sizeof(T) == 2) {
      *reinterpret_cast<uint4*>(rows + stage_row(2 * qp, cv)) = R.a[m];
      *reinterpret_cast<uint4*>(rows + stage_row(2 * qp + 1, cv)) = R.b[m];
    } else {
      *reinterpret_cast<uint4*>(rows + (2 * qp) * LDN + cv * VEC) = R.a[m];
      *reinterpret_cast<uint4*>(rows + (2 * qp + 1) * LDN + cv * VEC) = R.b[m];
      store_vt_pair(tensor == 0 ? Qt : dOt, LDT, cv * VEC, 2 * qp, R.a[m], R.b[m]);
    }
  }
  (lt < STG ? lse : dd)[lt % STG] = R.v;
}

// SPL: waves per (head, key half), each taking its own 4 of the stage's
// 16-slot tiles (stages of 64 SPL slots); their partial sums meet in LDS at
// the end in a fixed order.
template <typename T, int SPL>
__global__ __launch_bounds__(512) void bwd_dkv_kernel(BwdParams p) {
  typedef Tr<T> TT;
  typedef typename TT::op8 op8;
  typedef typename TT::op4 op4;
  constexpr int VEC = TT::VEC;
  constexpr int CVH = D / VEC;
  constexpr int STG = kStage * SPL;  // query slots per stage
  constexpr int NI = 2 * (STG / 2) * CVH / (128 * SPL);  // stage items per lane (2 bf16, 4 fp32)
  constexpr bool TRR = sizeof(T) == 2;  // bf16: swizzled rows and transposing reads, no transposed copies
  static_assert(TRR || SPL == 1, "the fp32 form keeps one wave per (head, key half)");
  constexpr int LDN = TRR ? D : D + 16 / (int)sizeof(T);
  constexpr int LDT = STG + 16 / (int)sizeof(T);
  constexpr int HEAD_ELEMS = 2 * STG * LDN + (TRR ? 0 : 2 * D * LDT);  // Qn, dOn (, Qt, dOt)
  extern __shared__ __align__(16) unsigned char smem_raw[];
  __shared__ int corners[kMaxRegions];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4, col = lane & 15;

  // workgroup -> (place t, image b, key block, head group), images fastest
  // after the key blocks and head groups: the heaviest key regions of every
  // image start first. (When B * nkb * nhgk is a multiple of 8, an image's
  // workgroups all land on one XCD, since workgroups are dealt round-robin.)
  int w = blockIdx.x;
  const int hg = w % p.nhgk;
  w /= p.nhgk;
  const int kb = w % p.nkb;
  w /= p.nkb;
  const int b = w % p.B;
  const int r = p.order[b * p.R + w / p.B];
  const int hl = wave / (2 * SPL), kh = (wave / SPL) & 1, sh = wave % SPL;
  const int lt = (wave % (2 * SPL)) * 64 + lane;  // lane within the head's 2 SPL waves
  const int head = hg * p.HGk + hl;
  const bool head_ok = head < p.heads;
  const int ch0 = head * D;
  const int64_t img = (int64_t)b * p.H * p.W * p.C;
  const int64_t imgrow = (int64_t)b * p.H * p.W;
  T* Qn = reinterpret_cast<T*>(smem_raw) + hl * HEAD_ELEMS;
  T* dOn = Qn + STG * LDN;
  T* Qt = dOn + STG * LDN;
  T* dOt = Qt + D * LDT;
  float* lse = reinterpret_cast<float*>(reinterpret_cast<T*>(smem_raw) + p.HGk * HEAD_ELEMS) + hl * 2 * STG;
  float* dd = lse + STG;

  const int cnt = p.inv_cnt[b * p.R + r];
  const int* list = p.inv_list + ((int64_t)b * p.R + r) * p.R;
  for (int e = tid; e < cnt; e += blockDim.x) corners[e] = corner_of(p, list[e]);
  const int nslots = cnt * p.n;
  const int nstages = (nslots + STG - 1) / STG;

  // the wave's 32 keys: key tile kt2 column col is key kb*64 + kh*32 + kt2*16 + col
  const int rcorner = corner_of(p, r);
  op8 kB[2], vB[2];
  int ktok[2];
  bool kval[2];
#pragma unroll
  for (int kt2 = 0; kt2 < 2; ++kt2) {
    const int key = kb * 64 + kh * 32 + kt2 * 16 + col;
    kval[kt2] = head_ok && key < p.n;
    int tx;
    const int ty = fdiv(key < p.n ? key : 0, p.div_sw, &tx);
    ktok[kt2] = rcorner + ty * p.W + tx;
    const int off = ktok[kt2] * p.C + ch0 + 8 * g;
    kB[kt2] = kval[kt2] ? TT::load8(static_cast<const T*>(p.K) + img + off) : TT::zero();
    vB[kt2] = kval[kt2] ? TT::load8(static_cast<const T*>(p.V) + img + off) : TT::zero();
  }
  // key tiles with no key of the region skip their products (uniform per wave)
  const bool kt_live0 = kb * 64 + kh * 32 < p.n;
  const bool kt_live1 = kb * 64 + kh * 32 + 16 < p.n;
  floatx4 dv[2][2], dk[2][2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int kt2 = 0; kt2 < 2; ++kt2) {
      dv[ct][kt2] = floatx4{0.f, 0.f, 0.f, 0.f};
      dk[ct][kt2] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
  __syncthreads();  // corners

  const int vrow = 8 * (col >> 2) + (col & 3);
  // bf16: lane bases of the row reads (row col, chunk g) and of the
  // transposing reads (lane 4 s + q of group g: row 4g + s, chunk q); a whole
  // number of 16-row tiles added keeps bit 3 of the row
  const int a_row = TRR ? stage_row(col, g) : col * LDN + 8 * g;
  const int a_tr = TRR ? stage_row(4 * g + (col >> 2), col & 3) : 0;
  StageRegs<NI> st;
  if (nstages > 0) stage_load<T, NI, STG>(p, 0, nslots, corners, head_ok, lt, ch0, img, imgrow, head, st);
  for (int sg = 0; sg < nstages; ++sg) {
    stage_store<T, NI, STG>(Qn, dOn, Qt, dOt, lse, dd, lt, st);
    __syncthreads();  // stage in LDS
    if (sg + 1 < nstages)
      stage_load<T, NI, STG>(p, (sg + 1) * STG, nslots, corners, head_ok, lt, ch0, img, imgrow, head, st);
    // this wave's tiles of the stage: 4 sh .. 4 sh + 3
    const int tiles = min(4 * sh + 4, (nslots - sg * STG + 15) >> 4);
    if (kt_live0) {
      for (int t = 4 * sh; t < tiles; ++t) {
        const op8 qA = TT::load8(Qn + a_row + t * 16 * LDN);
        const op8 dA = TT::load8(dOn + a_row + t * 16 * LDN);
        const float4 lq = *reinterpret_cast<const float4*>(lse + t * 16 + 4 * g);
        const float4 dq4 = *reinterpret_cast<const float4*>(dd + t * 16 + 4 * g);
        const float lqa[4] = {lq.x, lq.y, lq.z, lq.w};
        const float dqa[4] = {dq4.x, dq4.y, dq4.z, dq4.w};
        op4 pB[2], zB[2];
#pragma unroll
        for (int kt2 = 0; kt2 < 2; ++kt2) {
          if (kt2 == 1 && !kt_live1) continue;
          const floatx4 sc = TT::mma(qA, kB[kt2], floatx4{0.f, 0.f, 0.f, 0.f});
          const floatx4 dpv = TT::mma(dA, vB[kt2], floatx4{0.f, 0.f, 0.f, 0.f});
          float pr[4], dz[4];
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            pr[ii] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[ii], p.c, -lqa[ii]));
            dz[ii] = pr[ii] * (dpv[ii] - dqa[ii]);
          }
          pB[kt2] = TT::from_f32_4(pr);
          zB[kt2] = TT::from_f32_4(dz);
        }
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          // A operand row col = channel vrow + 4 ct; slots = query slots t*16 + 4g .. +3
          op4 dOA, QA;
          if constexpr (TRR) {
            // lane 4 s + q reads slot row t*16 + 4g + s at channels 8 q + 4 ct .. +3
            dOA = read_tr(dOn + a_tr + t * 16 * LDN + 4 * ct);
            QA = read_tr(Qn + a_tr + t * 16 * LDN + 4 * ct);
          } else {
            const int row = vrow + 4 * ct;
            dOA = TT::load4(dOt + row * LDT + t * 16 + 4 * g);
            QA = TT::load4(Qt + row * LDT + t * 16 + 4 * g);
          }
#pragma unroll
          for (int kt2 = 0; kt2 < 2; ++kt2) {
            if (kt2 == 1 && !kt_live1) continue;
            dv[ct][kt2] = TT::mma16(dOA, pB[kt2], dv[ct][kt2]);
            dk[ct][kt2] = TT::mma16(QA, zB[kt2], dk[ct][kt2]);
          }
        }
      }
    }
    __syncthreads();  // stage consumed before the next one is stored
  }

  if constexpr (SPL == 2) {
    // the second slot half's partial sums join the first's (the stage area is
    // free after the loop's last barrier): [head][key half][lane][dV 16 | dK 16
    // floats], 32 KB, inside the 2 x 16 KB of the heads' stage rows
    float* red = reinterpret_cast<float*>(smem_raw) + ((hl * 2 + kh) * 64 + lane) * 32;
    if (sh == 1) {
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int kt2 = 0; kt2 < 2; ++kt2) {
          *reinterpret_cast<floatx4*>(red + (ct * 2 + kt2) * 4) = dv[ct][kt2];
          *reinterpret_cast<floatx4*>(red + 16 + (ct * 2 + kt2) * 4) = dk[ct][kt2];
        }
    }
    __syncthreads();
    if (sh == 0) {
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int kt2 = 0; kt2 < 2; ++kt2) {
          dv[ct][kt2] += *reinterpret_cast<const floatx4*>(red + (ct * 2 + kt2) * 4);
          dk[ct][kt2] += *reinterpret_cast<const floatx4*>(red + 16 + (ct * 2 + kt2) * 4);
        }
    }
    __syncthreads();  // the area is reused below
  }
  const bool holder = sh == 0;  // this wave holds the finished sums of its (head, key half)

  T* dKg = static_cast<T*>(p.dK) + img;
  T* dVg = static_cast<T*>(p.dV) + img;
  // bf16 with two heads: the head waves of one key half exchange their
  // 64-byte halves of every dK and dV row through the (now free) stage LDS,
  // and wave (head h, key half kh) stores whole 128-byte rows of key tile h
  // of that half (uniform per workgroup)
  const bool rows = sizeof(T) == 2 && p.HGk == 2 && hg * 2 + 1 < p.heads;
#pragma unroll
  for (int kt2 = 0; kt2 < 2; ++kt2) {
    float ov[8], ok[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ov[e] = dv[0][kt2][e];
      ov[4 + e] = dv[1][kt2][e];
      ok[e] = dk[0][kt2][e] * p.scale;
      ok[4 + e] = dk[1][kt2][e] * p.scale;
    }
    if constexpr (sizeof(T) == 2) {
      if (rows) {
        // [tensor][key half][key tile][key][head][chunk], chunks swizzled (xrow_at)
        uint4* xr = reinterpret_cast<uint4*>(smem_raw);
        const int at = xrow_at((kh * 2 + kt2) * 16 + col, hl * 4 + g);
        if (holder) {
          xr[at] = __builtin_bit_cast(uint4, TT::from_f32(ov));
          xr[512 + at] = __builtin_bit_cast(uint4, TT::from_f32(ok));
        }
        continue;
      }
    }
    if (!kval[kt2] || !holder) continue;
    const int off = ktok[kt2] * p.C + ch0 + 8 * g;
    TT::store8_nt(dVg + off, ov);
    TT::store8_nt(dKg + off, ok);
  }
  if constexpr (sizeof(T) == 2) {
    if (rows) {
      __syncthreads();
      const uint4* xr = reinterpret_cast<const uint4*>(smem_raw);
      const int kt2 = hl;  // this wave stores key tile hl of its key half
#pragma unroll
      for (int h8 = 0; h8 < 2; ++h8) {
        if (!holder) break;
        const int kc = 8 * h8 + (lane >> 3), c = lane & 7;  // key of the tile, 16-byte chunk of the row
        const int key = kb * 64 + kh * 32 + kt2 * 16 + kc;
        if (key < p.n) {
          int tx;
          const int ty = fdiv(key, p.div_sw, &tx);
          const int off = (rcorner + ty * p.W + tx) * p.C + hg * 2 * D + 8 * c;
          const int at = xrow_at((kh * 2 + kt2) * 16 + kc, c);
          __builtin_nontemporal_store(__builtin_bit_cast(op8, xr[at]), reinterpret_cast<op8*>(dVg + off));
          __builtin_nontemporal_store(__builtin_bit_cast(op8, xr[512 + at]), reinterpret_cast<op8*>(dKg + off));
        }
      }
    }
  }
}

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

}  // namespace

size_t backward_workspace_bytes(const Shape& s) {
  const size_t tok = (size_t)s.B * s.H * s.W * s.heads;
  const size_t reg = (size_t)s.B * s.R;
  return 2 * align256(4 * tok) + 3 * align256(4 * reg) + align256(4 * reg * s.R);
}

hipError_t launch_backward(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                           const int32_t* idx, void* dQ, void* dK, void* dV, void* ws, const Shape& s, int dtype,
                           hipStream_t stream) {
  if (backward_image_fits(s, dtype)) return launch_backward_image(Q, K, V, O, dO, idx, dQ, dK, dV, s, stream);
  if (backward_top1_fits(s, dtype)) return launch_backward_top1(Q, K, V, dO, idx, dQ, dK, dV, s, stream);
  BwdParams p{};
  p.Q = Q; p.K = K; p.V = V; p.O = O; p.dO = dO; p.idx = idx;
  p.dQ = dQ; p.dK = dK; p.dV = dV;
  char* w = static_cast<char*>(ws);
  const size_t tok = (size_t)s.B * s.H * s.W * s.heads;
  const size_t reg = (size_t)s.B * s.R;
  p.lse = reinterpret_cast<float*>(w);
  w += align256(4 * tok);
  p.dd = reinterpret_cast<float*>(w);
  w += align256(4 * tok);
  p.inv_cnt = reinterpret_cast<int*>(w);
  w += align256(4 * reg);
  p.bad = reinterpret_cast<int*>(w);
  w += align256(4 * reg);
  p.order = reinterpret_cast<int*>(w);
  w += align256(4 * reg);
  p.inv_list = reinterpret_cast<int*>(w);
  p.B = s.B;
  p.H = s.H; p.W = s.W; p.C = s.C; p.S = s.S; p.topk = s.topk;
  p.sh = s.sh; p.sw = s.sw; p.n = s.n; p.R = s.R; p.kv = s.kv; p.heads = s.heads;
  p.scale = 1.0f / sqrtf((float)s.d);
  p.c = p.scale * 1.4426950408889634f;
  p.div_n = make_fastdiv(s.n);
  p.div_sw = make_fastdiv(s.sw);
  p.div_S = make_fastdiv(s.S);
  // several-chunk dq kernel: query blocks of 64, one wave per (head, tile), <= 8 waves
  p.nqb = (s.n + 63) / 64;
  p.ntq = (min(s.n, 64) + 15) / 16;
  int HG = 1;
  while (2 * HG * p.ntq <= 8 && 2 * HG <= s.heads) HG *= 2;
  p.HG = HG;
  p.nhg = (s.heads + HG - 1) / HG;
  const int64_t nq = (int64_t)s.B * s.R * p.nqb * p.nhg;
  // dkv kernel: key blocks of 64 (two 32-key halves), up to 2 heads
  p.nkb = (s.n + 63) / 64;
  const int HGk = s.heads >= 2 ? 2 : 1;
  p.HGk = HGk;
  p.nhgk = (s.heads + HGk - 1) / HGk;
  const int64_t nk = (int64_t)s.B * s.R * p.nkb * p.nhgk;
  if (nq >= (int64_t(1) << 31) || nk >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  p.nitems_q = (int)nq;
  p.nitems_kv = (int)nk;
  const size_t esz = dtype == kBF16 ? 2 : 4;
  const int padv = dtype == kBF16 ? Tr<__bf16>::PADV : Tr<float>::PADV;

  void* args[] = {&p};
  hipError_t e = hipSuccess;
  // The inverse routing table: for the single-chunk dQ kernel (many short
  // workgroups) with at most 64 regions, its LDS fits in the dQ kernel's and B
  // workgroups put ahead of the dQ grid build it there, one launch fewer.
  // Otherwise a launch of its own: the several-chunk dQ kernel's few long
  // workgroups can fill the machine in one round, and extra ones would push
  // some of them into a second.
  const bool multi = s.kv > KC, ragged = s.kv % KC != 0;
  const bool fold = !multi && s.R <= 64;
  const int extra = fold ? s.B : 0;
  if (!fold) {
    const unsigned nblk = (unsigned)((s.R + kRoutesBlock - 1) / kRoutesBlock);
    e = hipLaunchKernel((const void*)&bwd_routes_kernel, dim3(s.B * nblk), dim3(256), args, 0, stream);
    if (e != hipSuccess) return e;
  }

  const void* fq;
  size_t ldsq;
  if (!multi) {
    // one wave per head, up to 8 heads per workgroup, looping over the tiles
    BwdParams ph = p;
    int H8 = 1;
    while (2 * H8 <= 8 && 2 * H8 <= s.heads) H8 *= 2;
    ph.HG = H8;
    ph.nhg = (s.heads + H8 - 1) / H8;
    const int64_t nqh = (int64_t)s.B * s.R * p.nqb * ph.nhg;
    if (nqh + extra >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    ph.nitems_q = (int)nqh;
    ph.ntab = extra;
    const bool one = s.n <= 16;
    if (dtype == kBF16)
      fq = ragged ? (one ? (const void*)&bwd_dq_head_kernel<__bf16, true, 1> : (const void*)&bwd_dq_head_kernel<__bf16, true, 4>)
                  : (one ? (const void*)&bwd_dq_head_kernel<__bf16, false, 1> : (const void*)&bwd_dq_head_kernel<__bf16, false, 4>);
    else
      fq = ragged ? (one ? (const void*)&bwd_dq_head_kernel<float, true, 1> : (const void*)&bwd_dq_head_kernel<float, true, 4>)
                  : (one ? (const void*)&bwd_dq_head_kernel<float, false, 1> : (const void*)&bwd_dq_head_kernel<float, false, 4>);
    ldsq = std::max(esz * (size_t)H8 * D * (KC + padv), fold ? inverse_table_lds(s.R) : 0);
    void* hargs[] = {&ph};
    e = hipLaunchKernel(fq, dim3((unsigned)(ph.nitems_q + extra)), dim3(H8 * 64), hargs, ldsq, stream);
  } else if (backward_dq_dense_fits(s, dtype)) {
    e = launch_backward_dq_dense(Q, K, V, O, dO, idx, dQ, p.lse, p.dd, s, stream);
  } else {
    if (dtype == kBF16)
      fq = ragged ? (const void*)&bwd_dq_kernel<__bf16, true> : (const void*)&bwd_dq_kernel<__bf16, false>;
    else
      fq = ragged ? (const void*)&bwd_dq_kernel<float, true> : (const void*)&bwd_dq_kernel<float, false>;
    ldsq = esz * (size_t)HG * D * (KC + padv);
    e = hipLaunchKernel(fq, dim3((unsigned)p.nitems_q), dim3(HG * p.ntq * 64), args, ldsq, stream);
  }
  if (e != hipSuccess) return e;

  // bf16: two waves per (head, key half), each on its own half of 128-slot stages
  const int spl = dtype == kBF16 ? 2 : 1;
  const void* fk = dtype == kBF16 ? (const void*)&bwd_dkv_kernel<__bf16, 2> : (const void*)&bwd_dkv_kernel<float, 1>;
  // per head: Q and dO stage rows (bf16: [128][32], 64-byte rows read by the
  // transposing read; fp32: [64][32 + pad] and transposed copies
  // [32][64 + pad]), then the stage's log-sum-exp and D
  const size_t stg = 64 * (size_t)spl;
  const size_t pad = 16 / esz;
  const size_t head_elems = dtype == kBF16 ? 2 * stg * D : 2 * stg * (D + pad) + 2 * D * (stg + pad);
  const size_t ldsk = esz * HGk * head_elems + sizeof(float) * HGk * 2 * stg;
  return hipLaunchKernel(fk, dim3((unsigned)p.nitems_kv), dim3(HGk * 2 * spl * 64), args, ldsk, stream);
}

}  // namespace bra
