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
// Work split (the chunked kernel, more than 64 keys per query). One
// workgroup = one work item (image b, query region i, block of <= 128 of the
// region's queries, group of HG heads); each of its waves owns one "unit" =
// (head, tile of 16 queries) and keeps its accumulators in registers, and the
// waves share every staged 64-key chunk. The single-chunk kernel and the
// image-resident kernel below have their own splits.
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
#include "attn_common.h"
#include "lce_tile.h"

#include <math.h>

#include <algorithm>

namespace bra {
namespace {

constexpr int MAXU = 1;       // chunked kernel: (head, 16-query tile) units per wave
constexpr int kMaxUnits = 16; // chunked kernel: units (= waves) per workgroup
constexpr int kMinWaves = 4;  // chunked kernel: waves per workgroup at least (they share the chunk loads)
constexpr int QB = 64;        // single-chunk kernel: queries per work item (<= 4 tiles of 16)
constexpr int QBM = 128;      // chunked kernel: queries per work item (<= 8 tiles of 16; 2 * QBM for large regions)
constexpr size_t kChunkMaxLds = 156 * 1024;  // chunked kernel: LDS of its four chunk buffers at most (static LDS on top)

struct AttnParams {
  const void* Q;
  const void* K;
  const void* V;
  const int32_t* idx;
  void* O;
  int H, W, C, S, topk;
  int sh, sw, n, R, kv;
  int heads;
  int nqb;     // query blocks per region
  int HG;      // heads per workgroup (a power of two)
  int nhg;     // head groups
  int nitems;  // B * R * nqb * nhg
  int lg_oct;  // log2(8 * HG * D / VEC): pair items per 8-pair octet of a chunk
  int nbuf;    // LDS chunk buffers (2: double-buffered; 4: two chunks per barrier)
  int own_tab; // single-chunk kernel: every attention wave builds its own key table
  int rtab_off; // single-chunk kernel: byte offset of the key tables in dynamic LDS (< 0: in the exchange rows)
  int qblk;    // queries per work item
  float c;     // softmax scale * log2(e)
  FastDiv div_n, div_sw, div_S;
  // local context term fused into the single-chunk kernel's epilogue
  const void* lw;   // [C][5][5] depthwise filter
  const void* lb;   // [C] bias or null
  int wave_lds;     // LDS bytes of one head's convolution area
  int lce_pw, lce_ps;
  float lce_inv_pw;
};

// Geometry of one work item; every field is uniform over the workgroup.
struct Item {
  bool valid;
  int b, i, qb, hg;
  int q0, nq, ntiles, nh, cb, U, qcorner;
  int ry0, rx0;  // image coordinates of the region's first token
  int64_t img;  // element offset of image b
};

__device__ inline Item item_at(const AttnParams& p, int w) {
  Item it;
  it.valid = w < p.nitems;
  if (!it.valid) w = 0;
  it.hg = w % p.nhg;  w /= p.nhg;
  it.qb = w % p.nqb;  w /= p.nqb;
  it.i = w % p.R;
  it.b = w / p.R;
  it.q0 = it.qb * p.qblk;
  it.nq = min(p.qblk, p.n - it.q0);
  it.ntiles = (it.nq + 15) >> 4;
  const int h0 = it.hg * p.HG;
  it.nh = min(p.HG, p.heads - h0);
  it.cb = h0 * D;
  it.U = it.valid ? it.nh * it.ntiles : 0;
  const int ri = it.i / p.S, rj = it.i - ri * p.S;
  it.qcorner = ri * p.sh * p.W + rj * p.sw;
  it.ry0 = ri * p.sh;
  it.rx0 = rj * p.sw;
  it.img = (int64_t)it.b * p.H * p.W * p.C;
  return it;
}

// Per-wave state of one item: the wave's units (head hl, query tile t).
template <typename T>
struct Units {
  typename Tr<T>::op8 qop[MAXU];
  // acc[u][0..1]: O^T tiles (channels 8g..8g+3 and 8g+4..8g+7 of the lane's
  // query); acc[u][2]: an all-ones 16 x 32 A operand against the same P^T, so
  // every element holds the softmax denominator sum_k P[k] of the lane's
  // query, computed by the matrix cores from exactly the P the numerator used.
  floatx4 acc[MAXU][3];
  float m[MAXU];
  int qoff[MAXU];
  bool qvalid[MAXU];
};

// Query operands of the wave's units (they do not depend on the routing).
template <typename T>
__device__ __forceinline__ void load_queries(const AttnParams& p, const Item& it, int wave, int g, int col,
                                             Units<T>& us) {
  typedef Tr<T> TT;
  const T* Qg = static_cast<const T*>(p.Q) + it.img;
#pragma unroll
  for (int uu = 0; uu < MAXU; ++uu) {
    const int u = wave + (int)(blockDim.x >> 6) * uu;  // uniform
    const int hl = u / max(it.ntiles, 1);
    const int t = u - hl * it.ntiles;
    const int qi = it.q0 + t * 16 + col;
    us.qvalid[uu] = (u < it.U) && (qi < it.q0 + it.nq);
    us.qoff[uu] = 0;
    if (us.qvalid[uu]) {
      int qx;
      const int qy = fdiv(qi, p.div_sw, &qx);
      us.qoff[uu] = (it.qcorner + qy * p.W + qx) * p.C + it.cb + hl * D + 8 * g;
      us.qop[uu] = TT::load8(Qg + us.qoff[uu]);
    } else {
      us.qop[uu] = TT::zero();
    }
#pragma unroll
    for (int ct = 0; ct < 3; ++ct) us.acc[uu][ct] = floatx4{0.f, 0.f, 0.f, 0.f};
    us.m[uu] = -INFINITY;
  }
}

// Token offset of region r's top-left corner inside its image.
__device__ inline int region_corner(const AttnParams& p, int r) {
  int rx;
  const int ry = fdiv(r, p.div_S, &rx);
  return ry * p.sh * p.W + rx * p.sw;
}

// Routing row of the item's region, read from the table: corner offsets into
// rb[0..topk); returns (through LDS flag *bad) whether an entry is out of range.
__device__ __forceinline__ void read_routes(const AttnParams& p, const Item& it, int tid, int* rb, int* bad) {
  for (int j = tid; j < p.topk; j += blockDim.x) {
    const int r = it.valid ? p.idx[((int64_t)it.b * p.R + it.i) * p.topk + j] : 0;
    const bool ok = r >= 0 && r < p.R;
    rb[j] = region_corner(p, ok ? r : 0);
    if (!ok) *bad = 1;
  }
}

// Single chunk (kv <= 64): token offset (inside the image) of every routed key
// kappa < kv, straight from the routing table: tok[kappa] = corner of region
// idx[b][i][kappa / n] + the (kappa % n)-th token of that region. Sets *bad
// (LDS) for an entry outside [0, S*S).
__device__ __forceinline__ void read_route_tokens(const AttnParams& p, const Item& it, int tid, int* tok, int* bad) {
  for (int kappa = tid; kappa < p.kv; kappa += blockDim.x) {
    int tk, tx;
    const int jr = fdiv(kappa, p.div_n, &tk);
    const int ty = fdiv(tk, p.div_sw, &tx);
    const int r = it.valid ? p.idx[((int64_t)it.b * p.R + it.i) * p.topk + jr] : 0;
    const bool ok = r >= 0 && r < p.R;
    tok[kappa] = region_corner(p, ok ? r : 0) + ty * p.W + tx;
    if (!ok) *bad = 1;
  }
}

// K/V loads of one 64-key chunk into registers. A thread owns NV/2 (key pair,
// 16-byte channel vector) items: pair item f = tid + blockDim.x q covers keys 2p and
// 2p+1 of channel vector cv, with 8 consecutive pairs per channel vector so
// one wave instruction reads 8 whole token rows; slot 2q holds key 2p, slot
// 2q+1 key 2p+1. (f -> p, cv by shifts: the head group spans a power-of-two
// number of 16-byte vectors.)
// TOK: rb holds the token offset of every key (single chunk) instead of the
// routed regions' corners.
template <typename T, int NV, bool TOK>
__device__ __forceinline__ void load_kv(const AttnParams& p, const Item& it, int tid, const int* rb, int c0,
                                        uint4 (&kreg)[NV], uint4 (&vreg)[NV]) {
  constexpr int VEC = Tr<T>::VEC;
  const T* Kg = static_cast<const T*>(p.K) + it.img;
  const T* Vg = static_cast<const T*>(p.V) + it.img;
  const int vpk = it.nh * (D / VEC);  // valid vectors per key row
#pragma unroll
  for (int s2 = 0; s2 < NV; ++s2) {
    const int f = tid + blockDim.x * (s2 >> 1);
    const int oct = f >> p.lg_oct;
    const int rem = f & ((1 << p.lg_oct) - 1);
    const int cv = rem >> 3;
    const int kappa = c0 + 2 * (oct * 8 + (rem & 7)) + (s2 & 1);
    kreg[s2] = make_uint4(0u, 0u, 0u, 0u);
    vreg[s2] = make_uint4(0u, 0u, 0u, 0u);
    if (it.valid && oct < KC / 16 && cv < vpk && kappa < p.kv) {
      int token;
      if (TOK) {
        token = rb[kappa];
      } else {
        int tk, tx;
        const int jr = fdiv(kappa, p.div_n, &tk);
        const int ty = fdiv(tk, p.div_sw, &tx);
        token = rb[jr] + ty * p.W + tx;
      }
      const int off = token * p.C + it.cb + cv * VEC;
      kreg[s2] = *reinterpret_cast<const uint4*>(Kg + off);
      vreg[s2] = *reinterpret_cast<const uint4*>(Vg + off);
    }
  }
}

template <typename T, int NV>
__device__ __forceinline__ void store_kv(const AttnParams& p, int tid, T* Ks, T* Vt, int ldk, int ldv,
                                         const uint4 (&kreg)[NV], const uint4 (&vreg)[NV]) {
  constexpr int VEC = Tr<T>::VEC;
#pragma unroll
  for (int q = 0; q < NV / 2; ++q) {
    const int f = tid + blockDim.x * q;
    const int oct = f >> p.lg_oct;
    if (oct < KC / 16) {
      const int rem = f & ((1 << p.lg_oct) - 1);
      const int cv = rem >> 3;
      const int k0 = 2 * (oct * 8 + (rem & 7));
      *reinterpret_cast<uint4*>(Ks + k0 * ldk + cv * VEC) = kreg[2 * q];
      *reinterpret_cast<uint4*>(Ks + (k0 + 1) * ldk + cv * VEC) = kreg[2 * q + 1];
      const int row0 = cv * VEC;
      store_vt_pair(Vt, ldv, row0, vt_col(row0, k0), vreg[2 * q], vreg[2 * q + 1]);
    }
  }
}

// Scores, softmax and P.V for the wave's units over one staged chunk.
template <typename T, bool MULTI, bool RAGGED>
__device__ __forceinline__ void compute_chunk(const AttnParams& p, const Item& it, int wave, int g, int col,
                                              const T* Ks, const T* Vt, int ldk, int ldv, int nvalid,
                                              const typename Tr<T>::op8& ones,
                                              Units<T>& us) {
  typedef Tr<T> TT;
  typedef typename TT::op8 op8;
#pragma unroll
  for (int uu = 0; uu < MAXU; ++uu) {
    const int u = wave + (int)(blockDim.x >> 6) * uu;
    if (u >= it.U) continue;  // uniform
    const int hl = u / it.ntiles;
    // ---- scores S^T for 64 keys: two 32-key steps, two 16-row tiles each
    float s[KC / 32][8];
    const int rr = col;  // MFMA row supplied by this lane
    const int krow = 8 * (rr >> 2) + (rr & 3);  // key row of tile a; tile b is +4
#pragma unroll
    for (int st = 0; st < KC / 32; ++st) {
      const op8 ka = TT::load8(Ks + (st * 32 + krow) * ldk + hl * D + 8 * g);
      const op8 kb = TT::load8(Ks + (st * 32 + krow + 4) * ldk + hl * D + 8 * g);
      const floatx4 sa = TT::mma(ka, us.qop[uu], floatx4{0.f, 0.f, 0.f, 0.f});
      const floatx4 sb = TT::mma(kb, us.qop[uu], floatx4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s[st][e] = sa[e];
        s[st][4 + e] = sb[e];
      }
    }
    // lane group g holds keys st*32 + 8g + e, e = 0..7
    if (RAGGED && nvalid < KC) {  // ragged last chunk (uniform branch)
#pragma unroll
      for (int st = 0; st < KC / 32; ++st)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (st * 32 + 8 * g + e >= nvalid) s[st][e] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int st = 0; st < KC / 32; ++st)
#pragma unroll
      for (int e = 0; e < 8; ++e) mx = fmaxf(mx, s[st][e]);
    mx = wave_max_groups(mx);
    // online softmax: with a single chunk the running max starts at -inf and
    // the accumulators at 0, so there is nothing to rescale
    const float mnew = MULTI ? fmaxf(us.m[uu], mx) : mx;
    const float mc = mnew * p.c;
    // rescale only when some lane's running max grew: otherwise every alpha
    // is exp2(0) = 1 and the product would leave the accumulators unchanged
    if (MULTI && __builtin_amdgcn_ballot_w64(mnew > us.m[uu]) != 0) {
      const float alpha = __builtin_amdgcn_exp2f(us.m[uu] * p.c - mc);
#pragma unroll
      for (int ct = 0; ct < 3; ++ct) us.acc[uu][ct] *= alpha;
      us.m[uu] = mnew;
    }
#pragma unroll
    for (int st = 0; st < KC / 32; ++st)
#pragma unroll
      for (int e = 0; e < 8; ++e) s[st][e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[st][e], p.c, -mc));
    // ---- O^T += V^T P^T (and the all-ones row-sum tile)
    const int vrow = 8 * (rr >> 2) + (rr & 3);  // channel row of tile 0; tile 1 is +4
#pragma unroll
    for (int st = 0; st < KC / 32; ++st) {
      const op8 pop = TT::from_f32(s[st]);
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const int row = hl * D + vrow + 4 * ct;
        const op8 va = TT::load8(Vt + row * ldv + vt_col(row, st * 32 + 8 * g));
        us.acc[uu][ct] = TT::mma(va, pop, us.acc[uu][ct]);
      }
      us.acc[uu][2] = TT::mma(ones, pop, us.acc[uu][2]);
    }
  }
}

// Normalise and store: the lane holds channels 8g..8g+7 of its query.
template <typename T>
__device__ __forceinline__ void store_outputs(const AttnParams& p, const Item& it, const Units<T>& us, bool nan_rows) {
  typedef Tr<T> TT;
  T* Og = static_cast<T*>(p.O) + it.img;
#pragma unroll
  for (int uu = 0; uu < MAXU; ++uu) {
    if (!us.qvalid[uu]) continue;
    float o[8];
    if (nan_rows) {
      // a routing entry outside [0, S*S): never dereferenced; output NaN
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = __builtin_nanf("");
    } else {
      const float inv = 1.0f / us.acc[uu][2][0];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[e] = us.acc[uu][0][e] * inv;
        o[4 + e] = us.acc[uu][1][e] * inv;
      }
    }
    TT::store8_nt(Og + us.qoff[uu], o);
  }
}

// NV: 16-byte vectors per tensor per thread per chunk (2 or 4, even).
// MULTI: kv spans more than one chunk (prefetch the next chunk during compute).
// RAGGED: kv is not a multiple of 64 (the last chunk masks its missing keys).
// PAIR: four LDS chunk buffers, two chunks staged per barrier (p.nbuf == 4).
template <typename T, int NV, bool MULTI, bool RAGGED, bool PAIR>
__global__ __launch_bounds__(NV == 2 ? kMaxUnits * 64 : 512) void attend_kernel(AttnParams p) {
  typedef Tr<T> TT;
  typedef typename TT::op8 op8;
  // single chunk: the routed keys' token offsets; several chunks: the routed
  // regions' corner offsets
  constexpr bool TOK = !MULTI;

  extern __shared__ __align__(16) unsigned char smem_raw[];
  __shared__ int rtab[kMaxRegions];
  __shared__ int sbad;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4;      // lane group: contraction slots 8g..8g+7
  const int col = lane & 15;    // query column of the 16-query tile
  const op8 ones = TT::ones();

  // XCD-aware order, each XCD's range walked from its end (xcd_item)
  const int wg = xcd_item(blockIdx.x, gridDim.x, true);
  const int ldk = p.HG * D + TT::PADK;   // LDS row stride of K (elements)
  const int ldv = KC + TT::PADV;         // LDS row stride of V^T (elements)
  const int bufsz = KC * ldk + p.HG * D * ldv;

  const Item it = item_at(p, wg);
  Units<T> us;
  load_queries<T>(p, it, wave, g, col, us);

  // ---- routing row -> token offsets of the routed keys (or region corners)
  if (tid == 0) sbad = 0;
  __syncthreads();
  if (TOK) read_route_tokens(p, it, tid, rtab, &sbad);
  else read_routes(p, it, tid, rtab, &sbad);
  __syncthreads();
  const bool bad = sbad;

  if (!bad) {
    // chunks are loaded two ahead into two register sets, A for even chunks
    // and B for odd ones (the loop is unrolled by two, so neither set is
    // copied, which would wait for its loads early); only the waves that hold
    // chunk items do the loads and the LDS staging
    uint4 kA[NV], vA[NV], kB[NV], vB[NV];
    const int nchunks = MULTI ? (p.kv + KC - 1) / KC : 1;
    const bool loader = wave * 64 < ((KC / 16) << p.lg_oct);  // uniform
    if (loader) {
      load_kv<T, NV, TOK>(p, it, tid, rtab, 0, kA, vA);
      if (MULTI && nchunks > 1) load_kv<T, NV, TOK>(p, it, tid, rtab, KC, kB, vB);
    }
    if constexpr (MULTI && PAIR) {
      // four LDS buffers: both chunks of a pair are staged behind one
      // barrier. Pair s uses buffers 2s, 2s + 1 (mod 4); pair s + 2 reuses
      // them only after the barrier of pair s + 1, which every wave reaches
      // after computing pair s.
      for (int ch = 0; ch < nchunks; ch += 2) {
        T* K0 = reinterpret_cast<T*>(smem_raw) + (ch & 3) * bufsz;
        T* K1 = reinterpret_cast<T*>(smem_raw) + ((ch + 1) & 3) * bufsz;
        const bool two = ch + 1 < nchunks;  // uniform
        if (loader) {
          store_kv<T, NV>(p, tid, K0, K0 + KC * ldk, ldk, ldv, kA, vA);
          if (two) store_kv<T, NV>(p, tid, K1, K1 + KC * ldk, ldk, ldv, kB, vB);
        }
        __syncthreads();
        // the next pair's loads: set A now, set B after the first chunk's
        // products (set B is free from its store until then)
        if (loader && ch + 2 < nchunks) load_kv<T, NV, TOK>(p, it, tid, rtab, (ch + 2) * KC, kA, vA);
        compute_chunk<T, MULTI, RAGGED>(p, it, wave, g, col, K0, K0 + KC * ldk, ldk, ldv, min(KC, p.kv - ch * KC),
                                        ones, us);
        if (loader && ch + 3 < nchunks) load_kv<T, NV, TOK>(p, it, tid, rtab, (ch + 3) * KC, kB, vB);
        if (two)
          compute_chunk<T, MULTI, RAGGED>(p, it, wave, g, col, K1, K1 + KC * ldk, ldk, ldv,
                                          min(KC, p.kv - (ch + 1) * KC), ones, us);
      }
    } else {
    for (int ch = 0; ch < nchunks; ch += 2) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int cc = ch + half;
        if (cc >= nchunks) break;  // uniform
        const int c0 = cc * KC;
        T* Ks = reinterpret_cast<T*>(smem_raw) + (p.nbuf == 2 ? (cc & 1) * bufsz : 0);
        T* Vt = Ks + KC * ldk;
        if (cc > 0 && p.nbuf == 1) __syncthreads();  // single buffer: previous chunk consumed
        if (loader) {
          if (half == 0)
            store_kv<T, NV>(p, tid, Ks, Vt, ldk, ldv, kA, vA);
          else
            store_kv<T, NV>(p, tid, Ks, Vt, ldk, ldv, kB, vB);
        }
        __syncthreads();
        if (loader && MULTI && cc + 2 < nchunks) {  // the chunk after next in flight
          if (half == 0)
            load_kv<T, NV, TOK>(p, it, tid, rtab, c0 + 2 * KC, kA, vA);
          else
            load_kv<T, NV, TOK>(p, it, tid, rtab, c0 + 2 * KC, kB, vB);
        }
        compute_chunk<T, MULTI, RAGGED>(p, it, wave, g, col, Ks, Vt, ldk, ldv, min(KC, p.kv - c0), ones, us);
      }
    }
    }
  }
  store_outputs<T>(p, it, us, bad);
}

// ---------------------------------------------------------------------------
// Single-chunk kernel (kv <= 64 routed keys per query), one wave per head.
// A workgroup = one work item with HG heads = HG waves; wave h owns head h of
// the group and loops over the item's <= 4 query tiles. Its K operands (the
// A operands of S^T, 64 keys x 32 channels) come straight from HBM into
// registers once and serve every tile; its V slice goes through the wave's
// own V^T tile in LDS once (the transpose) and then also lives in registers.
// Per tile only the query operand is loaded: 10 MFMAs, the softmax and the
// 16-byte output stores, with no LDS traffic.
// MAXT: query tiles per item the kernel is built for (1, or 4 = 64 queries).
//
// LR, LX > 0: the local context term is fused (bf16, regions of at most LR
// rows and 2*LX columns). The workgroup then has 2*HG waves: waves 0..HG-1
// compute attention as above, and wave HG + h computes the 5x5 depthwise
// convolution of head h over the region (lce_tile.h: V halo staged in the
// wave's own LDS area, results transposed into fp32 [query][channel] rows in
// the same area) concurrently with the attention waves' loads and products.
// The attention epilogue of head h reads its lanes' 8 channels per query from
// that area and adds them before the one rounding to bf16. The two roles
// never hold registers at the same time, so the kernel's register budget is
// the larger of the two, not their sum.
template <typename T, bool RAGGED, int MAXT, int LR, int LX>
__global__ __launch_bounds__(1024) void attend_head_kernel(AttnParams p) {
  typedef Tr<T> TT;
  typedef typename TT::op8 op8;
  constexpr int VEC = TT::VEC;
  constexpr int CVH = D / VEC;  // 16-byte vectors per key row of one head
  constexpr int PAIRS = KC / 2 * CVH / 64;  // (key pair, vector) items per lane
  constexpr bool LCE = LR > 0;
  static_assert(!LCE || sizeof(T) == 2, "the fused local context term is built for bf16");
  constexpr int LNB = LCE ? ((LR + 4) * ((2 * LX + 5) / 2) * 4 + 63) / 64 : 1;  // halo items per lane

  extern __shared__ __align__(16) unsigned char smem_raw[];
  // two heads' output halves of a tile's query rows, per tile parity (bf16
  // without the convolution term: 16 queries x 8 chunks of 16 bytes, 4 KB)
  __shared__ __align__(16) uint4 xrow[(!LCE && sizeof(T) == 2) ? 2 * 16 * 8 : 1];
  // token offset of every routed key (one table per attention wave, or one
  // shared), then the bad-row flag: in dynamic LDS after the V^T tiles and
  // convolution areas, or (rtab_off < 0: bf16, two heads, no convolution
  // term) in the exchange rows' array, which the table precedes in time. A
  // stage-1 workgroup then takes 9216 + 4096 bytes of LDS and 74 VGPRs, so
  // 12 fit per CU (3,072 of the 3,136 regions in the first round); with the
  // V operands held in registers (88 VGPRs) and the table sized for 8 heads,
  // 9 fitted (forward 35.6 -> 34.7 us over the two steps).
  const bool tab_in_x = !LCE && sizeof(T) == 2 && p.rtab_off < 0;  // uniform
  int* rtab = tab_in_x ? reinterpret_cast<int*>(xrow) : reinterpret_cast<int*>(smem_raw + max(p.rtab_off, 0));
  int& sbad = rtab[(p.own_tab ? p.HG : 1) * KC];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int col = lane & 15;
  const op8 ones = TT::ones();
  const int ldv = KC + TT::PADV;

  const int wg = xcd_item(blockIdx.x, gridDim.x, true);  // XCD-aware order, each range walked from its end
  const Item it = item_at(p, wg);
  // role: attention wave for head `head`, or (LCE) convolution wave for it
  const bool att = !LCE || wave < p.HG;
  const int head = att ? wave : wave - p.HG;
  const bool head_ok = head < it.nh;
  const int ch0 = it.cb + head * D;  // first channel of the wave's head
  T* Vt = reinterpret_cast<T*>(smem_raw) + head * D * ldv;  // head's V^T tile
  unsigned char* larea = smem_raw + p.HG * D * ldv * (int)sizeof(T) + head * p.wave_lds;  // head's LCE area
  const T* Kg = static_cast<const T*>(p.K) + it.img;
  const T* Vg = static_cast<const T*>(p.V) + it.img;
  const T* Qg = static_cast<const T*>(p.Q) + it.img;

  // ---- attention waves: query operands of all (<= 4) tiles first (they do
  // not depend on the routing, so their loads overlap the routing-table
  // round trip); convolution waves: the V halo and the filter
  // ---- attention waves that build a key table: the routing entry of key
  // kappa = lane first (the K/V addresses wait on it; vector loads complete in
  // order, so anything issued before it would delay it); attention waves: the
  // query operands of all (<= 4) tiles; convolution waves: the V halo and the
  // filter
  const bool own = p.own_tab;  // uniform: every attention wave builds its own key table
  const bool builds = att && head_ok && (own || head == 0);
  op8 qop[MAXT];
  int qoff[MAXT];
  int rid = 0, ktok = 0;  // key lane's routed region, token offset inside it
  LceTile lt;
  uint4 ha[LNB], hb[LNB];
  LceW<T> lw;
  if (att) {
    if (builds && lane < p.kv) {
      int tk, tx;
      const int jr = fdiv(lane, p.div_n, &tk);
      const int ty = fdiv(tk, p.div_sw, &tx);
      ktok = ty * p.W + tx;
      rid = p.idx[((int64_t)it.b * p.R + it.i) * p.topk + jr];
    }
#pragma unroll
    for (int t = 0; t < MAXT; ++t) {
      const int qi = it.q0 + t * 16 + col;
      qoff[t] = -1;
      qop[t] = TT::zero();
      if (head_ok && t < it.ntiles && qi < it.q0 + it.nq) {
        int qx;
        const int qy = fdiv(qi, p.div_sw, &qx);
        qoff[t] = (it.qcorner + qy * p.W + qx) * p.C + ch0 + 8 * g;
        qop[t] = TT::load8(Qg + qoff[t]);
      }
    }
  } else if constexpr (LCE) {
    lt.y0 = it.ry0;
    lt.x0 = it.rx0;
    lt.rows = p.sh;
    lt.cols = p.sw;
    lt.pw = p.lce_pw;
    lt.ps = p.lce_ps;
    lt.inv_pw = p.lce_inv_pw;
    if (head_ok) {
      lce_halo_load<T, LNB>(Vg, p.H, p.W, p.C, ch0, lt, 0, lane, ha, hb);
      lce_weights(static_cast<const T*>(p.lw), static_cast<const T*>(p.lb), ch0 + (lane & 31), (lane >> 5) & 1, lw);
    }
  }

  // ---- the routing row -> a table of key token offsets: built by every
  // attention wave for itself (no workgroup barrier; measured faster with 8
  // heads per workgroup) or by wave 0 for the whole workgroup
  bool bad = false;
  if (builds) {
    const bool ok = rid >= 0 && rid < p.R;
    bad = __builtin_amdgcn_ballot_w64(lane < p.kv && !ok) != 0;  // uniform
    rtab[(own ? head : 0) * KC + lane] = region_corner(p, ok ? rid : 0) + ktok;
    if (!own && lane == 0) sbad = bad;
  }
  if (own) {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
  } else {
    __syncthreads();
    bad = sbad;
  }
  op8 kop[2][2];
  if (att && head_ok) {
    const int* wtab = rtab + (own ? head : 0) * KC;
    if (!bad) {
      // V slice first (it is transposed through LDS before any product):
      // pair item f = lane + 64 m -> channel vector cv = f % CVH, key pair
      // p2 = f / CVH (keys 2 p2, 2 p2 + 1)
      uint4 vreg[PAIRS][2];
#pragma unroll
      for (int m = 0; m < PAIRS; ++m) {
        const int f = lane + 64 * m;
        const int cv = f % CVH, p2 = f / CVH;
#pragma unroll
        for (int k1 = 0; k1 < 2; ++k1) {
          const int key = 2 * p2 + k1;
          vreg[m][k1] = (!RAGGED || key < p.kv) ? *reinterpret_cast<const uint4*>(Vg + wtab[key] * p.C + ch0 + cv * VEC)
                                               : make_uint4(0u, 0u, 0u, 0u);
        }
      }
      // K operands: row rr = col of the tile for (32-key step st, tile tb) is
      // key st*32 + 8*(rr/4) + (rr%4) + 4*tb; slots = channels 8g..8g+7
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          const int key = st * 32 + 8 * (col >> 2) + (col & 3) + 4 * tb;
          kop[st][tb] = (!RAGGED || key < p.kv) ? TT::load8(Kg + wtab[key] * p.C + ch0 + 8 * g) : TT::zero();
        }
#pragma unroll
      for (int m = 0; m < PAIRS; ++m) {
        const int f = lane + 64 * m;
        const int cv = f % CVH, p2 = f / CVH;
        const int row0 = cv * VEC;
        store_vt_pair(Vt, ldv, row0, vt_col(row0, 2 * p2), vreg[m][0], vreg[m][1]);
      }
    }
  } else if constexpr (LCE) {
    // ---- convolution of the region for this head, all inside the wave's
    // own LDS area (LDS operations of one wave complete in order; the fences
    // keep the compiler from reordering them across the phase changes)
    if (head_ok) {
      typedef typename Lce<T>::word LWord;
      LWord* halo = reinterpret_cast<LWord*>(larea);
      lce_halo_store<T, LNB>(halo, lt, 0, lane, ha, hb);
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
      float acc[LR][LX];
      lce_compute<T, LR, LX>(halo + (lane & 31) * lt.ps, lt, lw, acc);
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
      lce_store_results<LR, LX>(reinterpret_cast<float*>(larea), lt, lane & 31, (lane >> 5) & 1, acc);
    }
  }
  if constexpr (LCE) {
    __syncthreads();  // convolution results (and V^T tiles) written
  } else {
    // the wave reads only its own V^T tile
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
  }
  if (!att || !head_ok) return;

  // bf16, two heads per workgroup, no convolution term: the two head waves
  // exchange their 64-byte halves of every query row through LDS and each
  // stores whole 128-byte rows, so every line is written once, by one
  // instruction (with halves, 1.22x O's bytes reached memory at the stage-1
  // shape; whole rows: 1.00x, and 23.6 -> 23.2 us)
  const bool rows = !LCE && sizeof(T) == 2 && p.HG == 2 && it.nh == 2;  // uniform per workgroup
  T* Og = static_cast<T*>(p.O) + it.img;
  if (bad) {
    // a routing entry outside [0, S*S): never dereferenced; output NaN
    float nanv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) nanv[e] = __builtin_nanf("");
#pragma unroll
    for (int t = 0; t < MAXT; ++t)
      if (qoff[t] >= 0) TT::store8(Og + qoff[t], nanv);
    return;
  }

  // ---- V operands, read from the wave's V^T tile at each use (holding all
  // four in registers cost 14 VGPRs, one wave per SIMD): row rr = col is
  // channel 8*(rr/4) + (rr%4) + 4*ct; slots = keys st*32 + 8g .. +7
  const int vrow = 8 * (col >> 2) + (col & 3);
  auto vop_at = [&](int st, int ct) {
    const int row = vrow + 4 * ct;
    return TT::load8(Vt + row * ldv + vt_col(row, st * 32 + 8 * g));
  };
  if constexpr (!LCE && sizeof(T) == 2) {
    if (tab_in_x && rows) {  // uniform: both head waves are done with the key table before xrow takes its place
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
      __builtin_amdgcn_s_barrier();
    }
  }

#pragma unroll
  for (int t = 0; t < MAXT; ++t) {
    if (t >= it.ntiles) break;  // uniform
    float s[2][8];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const floatx4 sa = TT::mma(kop[st][0], qop[t], floatx4{0.f, 0.f, 0.f, 0.f});
      const floatx4 sb = TT::mma(kop[st][1], qop[t], floatx4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s[st][e] = sa[e];
        s[st][4 + e] = sb[e];
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
    const float mc = mx * p.c;
    floatx4 acc[3] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      float pe[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) pe[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[st][e], p.c, -mc));
      const op8 pop = TT::from_f32(pe);
      acc[0] = TT::mma(vop_at(st, 0), pop, acc[0]);
      acc[1] = TT::mma(vop_at(st, 1), pop, acc[1]);
      acc[2] = TT::mma(ones, pop, acc[2]);
    }
    if (qoff[t] >= 0) {
      const float inv = 1.0f / acc[2][0];
      float o[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[e] = acc[0][e] * inv;
        o[4 + e] = acc[1][e] * inv;
      }
      if constexpr (LCE) {
        // the head's convolution results, query t*16 + col, channels 8g..8g+7
        const float* r = reinterpret_cast<const float*>(larea) + (t * 16 + col) * kLceRes + 8 * g;
        const float4 lo = *reinterpret_cast<const float4*>(r);
        const float4 hi = *reinterpret_cast<const float4*>(r + 4);
        o[0] += lo.x; o[1] += lo.y; o[2] += lo.z; o[3] += lo.w;
        o[4] += hi.x; o[5] += hi.y; o[6] += hi.z; o[7] += hi.w;
      }
      if constexpr (sizeof(T) == 2) {
        if (rows) xrow[(t & 1) * 128 + xrow_at(col, head * 4 + g)] = __builtin_bit_cast(uint4, TT::from_f32(o));
        else TT::store8_nt(Og + qoff[t], o);
      } else {
        TT::store8_nt(Og + qoff[t], o);
      }
    }
    if constexpr (sizeof(T) == 2) {
      if (rows) {
        // head wave h stores queries 8h .. 8h + 7 of the tile: lane = (query,
        // 16-byte chunk of the 128-byte row). Tile parities alternate, so
        // one barrier per tile suffices: a wave writes parity t & 1 again
        // only after the next barrier, which the other wave reaches after
        // its reads of it.
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS reads and writes done
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        const int q = 8 * head + (lane >> 3), c = lane & 7;
        const int qi = it.q0 + t * 16 + q;
        if (qi < it.q0 + it.nq) {
          int qx;
          const int qy = fdiv(qi, p.div_sw, &qx);
          const uint4 v = xrow[(t & 1) * 128 + xrow_at(q, c)];
          __builtin_nontemporal_store(__builtin_bit_cast(op8, v),
                                      reinterpret_cast<op8*>(Og + (it.qcorner + qy * p.W + qx) * p.C + it.cb + 8 * c));
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Image-resident kernel (bf16, kv <= 64 routed keys, n a multiple of 4, no
// fused local context term). With small regions the routed sets of an
// image's query regions overlap heavily: at 28x28 with 16-token regions and 4
// routed regions each head's key is gathered about 4 times per image, at
// 14x14 with 4-token regions and 16 routed regions about 16 times, and the
// per-region kernels above fetch it through the caches every time. Here one
// workgroup = one (image, head): it stages that head's K (a row per token)
// and V^T (a column per token) for the whole image in LDS once, in
// region-major order (position = region * n + token inside the region, so a
// routed region's keys are n consecutive positions), together with the
// image's routing table; then each wave takes units of 16 query columns and
// reads the routed keys' operands from LDS. Every query operand is loaded
// before the staging, so no unit waits on HBM.
//
// A unit is one 16-query tile of one region (n >= 12), or QR = 16 / n whole
// regions side by side (n = 4 or 8: 4 or 2 regions), so that no query column
// of the products is idle and the softmax work per query is not repeated for
// empty columns. With several regions in a tile, region j's products use the
// query operand and the probabilities with every column outside region j set
// to zero:
//   S^T  = sum_j K_j Q_j^T       (each column only meets its own region's keys)
//   O^T  = sum_j V_j^T P_j^T     (each column only gathers its own region's values)
// and the denominator tile uses the unmasked P^T (each column holds only its
// own region's probabilities). The matrix-core work equals that of QR
// separate units; the softmax and the stores are done once.
constexpr int kImgUnits = 4;   // units per wave at most
constexpr int kImgLdk = D + 8; // LDS row stride of K (elements)

struct ImgParams {
  const __bf16* Q;
  const __bf16* K;
  const __bf16* V;
  const int32_t* idx;
  __bf16* O;
  int H, W, C, S, topk, sh, sw, n, R, kv, heads;
  int HW;      // tokens per image
  int nunits;  // units per image
  int ldv;     // LDS row stride of V^T (elements, a multiple of 8)
  float c;     // softmax scale * log2(e)
  FastDiv div_n, div_sw, div_S, div_nt;  // div_nt: 16-query tiles per region (one region per unit)
};

// Region-major position -> token offset inside the image.
__device__ inline int img_token(const ImgParams& p, int pos) {
  int t, rx, tx;
  const int r = fdiv(pos, p.div_n, &t);
  const int ry = fdiv(r, p.div_S, &rx);
  const int ty = fdiv(t, p.div_sw, &tx);
  return (ry * p.sh + ty) * p.W + rx * p.sw + tx;
}

// Value v of lane src (src in [0, 64)).
__device__ inline int lane_value(int v, int src) { return __builtin_amdgcn_ds_bpermute(src << 2, v); }

// Region and query (inside the region) of query column col of unit u; false
// when the column holds no query.
template <int QR>
__device__ inline bool image_query(const ImgParams& p, int u, int col, int* r, int* qi) {
  if (QR == 1) {
    int t;
    *r = fdiv(u, p.div_nt, &t);
    *qi = t * 16 + col;
    return *qi < p.n;
  }
  constexpr int NQ = 16 / QR;  // = n
  *r = u * QR + col / NQ;
  *qi = col % NQ;
  return *r < p.R;
}

// One unit u: the routed keys' operands from the staged K and V^T, both
// products, the softmax and the output stores (qoff < 0: the lane's column
// holds no query).
template <bool RAGGED, bool N8, int QR>
__device__ __forceinline__ void image_unit(const ImgParams& p, int u, int lane, int g, int col,
                                           const __bf16* Ks, const __bf16* Vt, const int* rpos,
                                           Tr<__bf16>::op8 qop, int qoff, __bf16* Og) {
  typedef Tr<__bf16> TT;
  typedef TT::op8 op8;
  const op8 ones = TT::ones();
  const op8 zero = TT::zero();
  const int vrow = 8 * (col >> 2) + (col & 3);  // channel row of V^T tile 0; tile 1 is +4
  int r0, t;
  if (QR == 1) r0 = fdiv(u, p.div_nt, &t);
  else r0 = u * QR;
  const int jl = QR == 1 ? 0 : col / (16 / QR);  // the lane's region in the unit

  // position of routed key kappa = lane of each region j; a region with an
  // entry outside [0, S*S) reads position 0 and its queries are set to NaN
  int kpos[QR];
  bool bad = false;
#pragma unroll
  for (int j = 0; j < QR; ++j) {
    const int r = r0 + j;
    kpos[j] = 0;
    bool kbad = false;
    if (lane < p.kv && r < p.R) {
      int tk;
      const int jr = fdiv(lane, p.div_n, &tk);
      const int base = rpos[r * p.topk + jr];
      kbad = base < 0;
      kpos[j] = kbad ? 0 : base + tk;
    }
    const bool rbad = __builtin_amdgcn_ballot_w64(kbad) != 0;
    if (jl == j) bad = rbad;
  }

  // ---- S^T = sum_j K_j Q_j^T. K operand row col of tile (st, tb) is key
  // st*32 + 8*(col/4) + col%4 + 4*tb; slots are channels 8g..8g+7
  floatx4 sacc[2][2];
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) sacc[st][tb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < QR; ++j) {
    const op8 qj = (QR == 1 || jl == j) ? qop : zero;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const int key = st * 32 + 8 * (col >> 2) + (col & 3) + 4 * tb;
        const int pos = lane_value(kpos[j], key);
        const op8 k = (!RAGGED || key < p.kv) ? TT::load8(Ks + pos * kImgLdk + 8 * g) : zero;
        sacc[st][tb] = TT::mma(k, qj, sacc[st][tb]);
      }
  }
  // lane group g holds keys st*32 + 8g + e, e = 0..7, of its column
  float s[2][8];
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s[st][e] = sacc[st][0][e];
      s[st][4 + e] = sacc[st][1][e];
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
  const float mc = mx * p.c;
  op8 pop[2];
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    float pe[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) pe[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[st][e], p.c, -mc));
    pop[st] = TT::from_f32(pe);
  }

  // ---- O^T = sum_j V_j^T P_j^T. V operand row col of tile (st, ct) is
  // channel vrow + 4*ct; slots are keys st*32 + 8g .. +7
  floatx4 acc[3] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int j = 0; j < QR; ++j) {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const op8 pj = (QR == 1 || jl == j) ? pop[st] : zero;
      const int key0 = st * 32 + 8 * g;
      const int pos0 = lane_value(kpos[j], key0);
      const int pos1 = N8 ? 0 : lane_value(kpos[j], key0 + 4);
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const int row = vrow + 4 * ct;
        const __bf16* vr = Vt + row * p.ldv;
        op8 v;
        if (N8) {
          v = (!RAGGED || key0 < p.kv) ? TT::load8(vr + vt_col(row, pos0)) : zero;
        } else {
          bf16x4 lo = *reinterpret_cast<const bf16x4*>(vr + vt_col(row, pos0));
          bf16x4 hi = *reinterpret_cast<const bf16x4*>(vr + vt_col(row, pos1));
          if (RAGGED && key0 >= p.kv) lo = bf16x4{};
          if (RAGGED && key0 + 4 >= p.kv) hi = bf16x4{};
          v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
        acc[ct] = TT::mma(v, pj, acc[ct]);
      }
    }
  }
#pragma unroll
  for (int st = 0; st < 2; ++st) acc[2] = TT::mma(ones, pop[st], acc[2]);

  // v_rcp_f32 (within 1 ulp) for the denominator: the output is rounded to
  // bf16 after the multiply
  const float inv = __builtin_amdgcn_rcpf(acc[2][0]);
  float o[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    o[e] = acc[0][e] * inv;
    o[4 + e] = acc[1][e] * inv;
  }
  if (__builtin_amdgcn_ballot_w64(bad) != 0) {  // uniform; rare
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = bad ? __builtin_nanf("") : o[e];
  }
  if (qoff >= 0) TT::store8_nt(Og + qoff, o);
}

// N8: n is a multiple of 8, so each block of 8 keys 8g..8g+7 is 8 consecutive
// positions (one 16-byte V^T read); otherwise (n a multiple of 4) it is two
// runs of 4. RAGGED: kv < 64 (whole runs of 4 or 8 keys are past kv). QR:
// regions per unit. The workgroup has between 1 and 16 waves; wave w takes
// units w, w + waves, ... (at most MAXU: 1 when an image has at most 16
// units, each in a wave of its own; else kImgUnits).
template <bool RAGGED, bool N8, int QR, int MAXU>
__global__ __launch_bounds__(1024) void attend_image_kernel(ImgParams p) {
  typedef Tr<__bf16> TT;
  typedef TT::op8 op8;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  __bf16* Ks = reinterpret_cast<__bf16*>(smem_raw);            // [HW][kImgLdk]
  __bf16* Vt = Ks + p.HW * kImgLdk;                              // [D][ldv]
  int* rpos = reinterpret_cast<int*>(Vt + D * p.ldv);           // [R][topk]: first position of the routed region, -1 if out of range

  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int nwaves = nthr >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int col = lane & 15;

  // items (image, head), heads of one image adjacent: they share the image's
  // cache lines on one XCD (xcd_item)
  const int w = xcd_item(blockIdx.x, gridDim.x, true);
  const int head = w % p.heads, b = w / p.heads;
  const int64_t img = (int64_t)b * p.HW * p.C;
  const int ch0 = head * D;

  // ---- query operands of the wave's units
  op8 qop[MAXU];
  int qoff[MAXU];
#pragma unroll
  for (int uu = 0; uu < MAXU; ++uu) {
    const int u = wave + nwaves * uu;
    qoff[uu] = -1;
    qop[uu] = TT::zero();
    int r, qi;
    if (u < p.nunits && image_query<QR>(p, u, col, &r, &qi)) {
      int rx, qx;
      const int ry = fdiv(r, p.div_S, &rx);
      const int qy = fdiv(qi, p.div_sw, &qx);
      qoff[uu] = ((ry * p.sh + qy) * p.W + rx * p.sw + qx) * p.C + ch0 + 8 * g;
      qop[uu] = TT::load8(p.Q + img + qoff[uu]);
    }
  }

  // ---- the image's routing table
  const int nroute = p.R * p.topk;
  for (int e = tid; e < nroute; e += nthr) {
    const int r = p.idx[(int64_t)b * nroute + e];
    rpos[e] = (r >= 0 && r < p.R) ? r * p.n : -1;
  }

  // ---- K rows and V^T columns of the head: item f = (position pair pp,
  // 16-byte channel vector cv); four lanes read a token's 64 bytes
  const int nitems = p.HW * 2;  // HW / 2 pairs x 4 vectors
  const __bf16* Kg = p.K + img + ch0;
  const __bf16* Vg = p.V + img + ch0;
  for (int base = 0; base < nitems; base += 2 * nthr) {
    uint4 kr[2][2], vr[2][2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int f = base + tid + nthr * j;
      kr[j][0] = kr[j][1] = vr[j][0] = vr[j][1] = make_uint4(0u, 0u, 0u, 0u);
      if (f < nitems) {
        const int cv = f & 3, pp = f >> 2;
        const int t0 = img_token(p, 2 * pp), t1 = img_token(p, 2 * pp + 1);
        kr[j][0] = *reinterpret_cast<const uint4*>(Kg + t0 * p.C + 8 * cv);
        kr[j][1] = *reinterpret_cast<const uint4*>(Kg + t1 * p.C + 8 * cv);
        vr[j][0] = *reinterpret_cast<const uint4*>(Vg + t0 * p.C + 8 * cv);
        vr[j][1] = *reinterpret_cast<const uint4*>(Vg + t1 * p.C + 8 * cv);
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int f = base + tid + nthr * j;
      if (f < nitems) {
        const int cv = f & 3, pp = f >> 2;
        *reinterpret_cast<uint4*>(Ks + (2 * pp) * kImgLdk + 8 * cv) = kr[j][0];
        *reinterpret_cast<uint4*>(Ks + (2 * pp + 1) * kImgLdk + 8 * cv) = kr[j][1];
        store_vt_pair(Vt, p.ldv, 8 * cv, vt_col(8 * cv, 2 * pp), vr[j][0], vr[j][1]);
      }
    }
  }
  __syncthreads();

  __bf16* Og = p.O + img;
#pragma unroll
  for (int uu = 0; uu < MAXU; ++uu) {
    const int u = wave + nwaves * uu;
    if (u < p.nunits)  // uniform
      image_unit<RAGGED, N8, QR>(p, u, lane, g, col, Ks, Vt, rpos, qop[uu], qoff[uu], Og);
  }
}

}  // namespace

namespace {

// Attention launch shape: head grouping, LDS, kernel variant.
struct AttnLaunch {
  AttnParams p;
  size_t lds;
  int waves;
  int nv;
  bool multi;
  int64_t nwg;
};

AttnLaunch plan_attend(const Shape& s, int dtype) {
  AttnLaunch L;
  AttnParams& p = L.p;
  p = AttnParams{};
  p.H = s.H; p.W = s.W; p.C = s.C; p.S = s.S; p.topk = s.topk;
  p.sh = s.sh; p.sw = s.sw; p.n = s.n; p.R = s.R; p.kv = s.kv;
  p.heads = s.heads;
  // chunked kernel: 128-query items, one wave per (head, 16-query tile) unit
  // (more queries per staged chunk measured faster at the dense 128x128
  // shape: 30.1 us with 128, 39.4 with 64 queries and two units per wave,
  // 43.3 with 32); regions of 256 tokens or more take 256-query items of one
  // head (16 waves, each chunk staged for twice the queries: 28.0 -> 26.9 us
  // at the dense shape)
  p.qblk = s.kv > KC ? (s.n >= 2 * QBM ? 2 * QBM : QBM) : QB;
  p.nqb = (s.n + p.qblk - 1) / p.qblk;
  const int qtiles = (min(s.n, p.qblk) + 15) / 16;
  const int cap = dtype == kBF16 ? 4 : 2;  // keeps LDS at or below 64 KiB
  int HG = 1;  // largest power of two <= min(units budget, cap, heads)
  while (2 * HG <= (kMaxUnits * MAXU) / qtiles && 2 * HG <= cap && 2 * HG <= s.heads) HG *= 2;
  p.HG = HG;
  p.nhg = (s.heads + HG - 1) / HG;
  p.nitems = s.B * s.R * p.nqb * p.nhg;
  const int vec = dtype == kBF16 ? 8 : 4;
  int lg = 0;
  while ((1 << lg) < 8 * (HG * D / vec)) ++lg;
  p.lg_oct = lg;
  p.c = 1.4426950408889634f / sqrtf((float)s.d);
  p.div_n = make_fastdiv(s.n);
  p.div_sw = make_fastdiv(s.sw);
  p.div_S = make_fastdiv(s.S);
  const size_t esz = dtype == kBF16 ? 2 : 4;
  const int padk = dtype == kBF16 ? Tr<__bf16>::PADK : Tr<float>::PADK;
  const int padv = dtype == kBF16 ? Tr<__bf16>::PADV : Tr<float>::PADV;
  const size_t buf = esz * ((size_t)KC * (HG * D + padk) + (size_t)HG * D * (KC + padv));
  // four buffers (two chunks per barrier) from four chunks on, when they
  // fit; else two (double-buffered) within the default 64 KiB; else one
  const int nch = (s.kv + KC - 1) / KC;
  p.nbuf = s.kv <= KC ? 1 : (nch >= 4 && 4 * buf <= kChunkMaxLds) ? 4 : (2 * buf <= 65536 ? 2 : 1);
  L.lds = p.nbuf * buf;
  L.waves = std::max(kMinWaves, std::min(kMaxUnits, HG * qtiles));
  L.nv = (KC * (HG * D / vec) + L.waves * 64 - 1) / (L.waves * 64);  // <= 4: at least 4 waves
  L.multi = s.kv > KC;
  // One item per workgroup. (Two items per workgroup, with all loads of both
  // in flight before either is computed, measured slower at the stage-1
  // shape: the extra registers cut occupancy from 8 to 5 waves per SIMD and
  // the kernel is issue-bound.)
  L.nwg = p.nitems;
  return L;
}

template <typename T, bool RAGGED>
const void* pick_attend_r(int nv, bool multi, bool pair) {
  if (multi && pair)
    return nv <= 2 ? (const void*)&attend_kernel<T, 2, true, RAGGED, true> : (const void*)&attend_kernel<T, 4, true, RAGGED, true>;
  if (multi)
    return nv <= 2 ? (const void*)&attend_kernel<T, 2, true, RAGGED, false> : (const void*)&attend_kernel<T, 4, true, RAGGED, false>;
  return nv <= 2 ? (const void*)&attend_kernel<T, 2, false, RAGGED, false> : (const void*)&attend_kernel<T, 4, false, RAGGED, false>;
}

const void* pick_attend(int dtype, const AttnLaunch& L) {
  const bool ragged = L.p.kv % KC != 0, pair = L.p.nbuf == 4;
  if (dtype == kBF16)
    return ragged ? pick_attend_r<__bf16, true>(L.nv, L.multi, pair) : pick_attend_r<__bf16, false>(L.nv, L.multi, pair);
  return ragged ? pick_attend_r<float, true>(L.nv, L.multi, pair) : pick_attend_r<float, false>(L.nv, L.multi, pair);
}

// Image-resident kernel: the shape conditions, the V^T row stride and the LDS
// size. False when the per-region kernels take the shape.
constexpr size_t kImgMaxLds = 160 * 1024;

// V^T row stride: the image's positions rounded up to 32 plus the pad (a
// multiple of 8 elements) whose operand reads spread best over the LDS banks
// (a 16-byte read is served 16 lanes per pass over 64 four-byte banks; the 16
// lanes of a pass read the same key block from 16 channel rows).
int image_ldv(int HW) {
  const int base = (HW + 31) / 32 * 32;
  int best = base, bestc = 1 << 30;
  for (int pad = 0; pad < 64; pad += 8) {
    const int L = (base + pad) / 2;  // dwords per row
    int cost = 0;
    for (int P = 0; P < 16; P += 4)  // key block offset (dwords); higher bits shift every lane alike
      for (int ct = 0; ct < 2; ++ct) {
        int cnt[64] = {0}, m = 0;
        for (int c = 0; c < 16; ++c) {
          const int row = 8 * (c >> 2) + (c & 3) + 4 * ct;
          const int w0 = row * L + (P ^ (((row >> 3) & 7) << 2));
          for (int x = 0; x < 4; ++x) m = std::max(m, ++cnt[(w0 + x) & 63]);
        }
        cost += m;
      }
    if (cost < bestc) {
      bestc = cost;
      best = base + pad;
    }
  }
  return best;
}

struct ImgLaunch {
  ImgParams p;
  size_t lds;
  int waves;  // per workgroup
  int qr;     // regions per unit
};

bool plan_image(const Shape& s, ImgLaunch* L) {
  if (s.kv > KC || s.n % 4 != 0) return false;
  const int qr = s.n == 4 ? 4 : s.n == 8 ? 2 : 1;
  const int ntiles = (s.n + 15) / 16;
  const int nunits = qr > 1 ? (s.R + qr - 1) / qr : s.R * ntiles;
  if (nunits > 16 * kImgUnits) return false;
  // one workgroup per (image, head): fewer than half the compute units busy
  // is slower than the per-region split
  if ((int64_t)s.B * s.heads < 128) return false;
  const int HW = s.H * s.W;
  const int ldv = image_ldv(HW);
  const size_t bytes = 2 * (size_t)HW * kImgLdk + 2 * (size_t)D * ldv + 4 * (size_t)s.R * s.topk;
  if (bytes > kImgMaxLds) return false;
  ImgParams& p = L->p;
  p = ImgParams{};
  p.H = s.H; p.W = s.W; p.C = s.C; p.S = s.S; p.topk = s.topk;
  p.sh = s.sh; p.sw = s.sw; p.n = s.n; p.R = s.R; p.kv = s.kv; p.heads = s.heads;
  p.HW = HW;
  p.nunits = nunits;
  p.ldv = ldv;
  p.c = 1.4426950408889634f / sqrtf((float)s.d);
  p.div_n = make_fastdiv(s.n);
  p.div_sw = make_fastdiv(s.sw);
  p.div_S = make_fastdiv(s.S);
  p.div_nt = make_fastdiv(ntiles);
  L->lds = bytes;
  L->qr = qr;
  // one unit per wave when an image has at most 16 (14x14 map, 2 x 2
  // regions: 13 waves, 12.5 vs 14.0 us with about two units per wave); else
  // about two units per wave, at most 16 waves (a wave takes up to kImgUnits)
  L->waves = nunits <= 16 ? nunits : std::min(16, (nunits + 1) / 2);
  return true;
}

hipError_t launch_image(const ImgLaunch& L, int B, hipStream_t stream) {
  ImgParams p = L.p;
  const bool ragged = p.kv % KC != 0;
  // [one unit per wave][RAGGED][form]; form (N8, QR): n = 8 has two
  // regions per unit, n = 4 four, other multiples of 4 one (N8 when a
  // multiple of 8)
  const void* fns[2][2][4] = {
      {{(const void*)&attend_image_kernel<false, true, 1, kImgUnits>, (const void*)&attend_image_kernel<false, false, 1, kImgUnits>,
        (const void*)&attend_image_kernel<false, true, 2, kImgUnits>, (const void*)&attend_image_kernel<false, false, 4, kImgUnits>},
       {(const void*)&attend_image_kernel<true, true, 1, kImgUnits>, (const void*)&attend_image_kernel<true, false, 1, kImgUnits>,
        (const void*)&attend_image_kernel<true, true, 2, kImgUnits>, (const void*)&attend_image_kernel<true, false, 4, kImgUnits>}},
      {{(const void*)&attend_image_kernel<false, true, 1, 1>, (const void*)&attend_image_kernel<false, false, 1, 1>,
        (const void*)&attend_image_kernel<false, true, 2, 1>, (const void*)&attend_image_kernel<false, false, 4, 1>},
       {(const void*)&attend_image_kernel<true, true, 1, 1>, (const void*)&attend_image_kernel<true, false, 1, 1>,
        (const void*)&attend_image_kernel<true, true, 2, 1>, (const void*)&attend_image_kernel<true, false, 4, 1>}}};
  const int form = L.qr == 2 ? 2 : L.qr == 4 ? 3 : (p.n % 8 == 0 ? 0 : 1);
  const void* fn = fns[p.nunits <= 16][ragged][form];
  // more than the default 64 KiB of dynamic LDS: raise the kernel's limit
  // (an attribute of the kernel, set on every launch: no state is kept) to
  // the most any launch of it uses, one value for every caller
  if (L.lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kImgMaxLds);
    if (e != hipSuccess) return e;
  }
  void* args[] = {&p};
  return hipLaunchKernel(fn, dim3((unsigned)(B * p.heads)), dim3(L.waves * 64), args, L.lds, stream);
}

}  // namespace

namespace {

// The local context term is fused into the single-chunk kernel for bf16
// regions of 16 to 64 tokens (at most 8 x 8). For smaller regions the halo
// is several times the region (6 x 6 positions around 2 x 2) and the
// separate pass after the attention kernel measured faster (14x14 map,
// 2 x 2 regions: 38 us for attention + pass vs 47 us fused).
bool fuse_lce(const Shape& s, int dtype, bool lce) {
  return lce && dtype == kBF16 && s.kv <= KC && s.sh <= 8 && s.sw <= 8 && s.n >= 16;
}

}  // namespace

const char* attend_kernel_name(const Shape& s, int dtype, bool lce) {
  if (!fuse_lce(s, dtype, lce) && dtype == kBF16) {
    ImgLaunch L;
    if (plan_image(s, &L)) return "attend_image_kernel";
  }
  if (s.kv <= KC) return "attend_head_kernel";
  return dense_attend_fits(s, dtype) ? "attend_dense_kernel" : "attend_kernel";
}

hipError_t launch_attend(const void* Q, const void* K, const void* V,
                         const int32_t* idx, const void* lce_w, const void* lce_b, void* O,
                         const Shape& s, int dtype, hipStream_t stream) {
  const bool lce = lce_w != nullptr;
  const bool fuse = fuse_lce(s, dtype, lce);
  if (!fuse && dtype == kBF16) {
    ImgLaunch L;
    if (plan_image(s, &L)) {
      L.p.Q = static_cast<const __bf16*>(Q);
      L.p.K = static_cast<const __bf16*>(K);
      L.p.V = static_cast<const __bf16*>(V);
      L.p.idx = idx;
      L.p.O = static_cast<__bf16*>(O);
      const hipError_t e = launch_image(L, s.B, stream);
      if (e != hipSuccess || !lce) return e;
      return launch_lce(V, lce_w, lce_b, O, s, dtype, stream);
    }
  }
  if (s.kv <= KC) {
    // single chunk: one wave per head, up to 8 heads per workgroup
    AttnParams p = plan_attend(s, dtype).p;
    int HG = 1;
    while (2 * HG <= 8 && 2 * HG <= s.heads) HG *= 2;
    p.HG = HG;
    p.nhg = (s.heads + HG - 1) / HG;
    p.nitems = s.B * s.R * p.nqb * p.nhg;
    p.Q = Q; p.K = K; p.V = V; p.idx = idx; p.O = O;
    const size_t esz = dtype == kBF16 ? 2 : 4;
    const int padv = dtype == kBF16 ? Tr<__bf16>::PADV : Tr<float>::PADV;
    const bool ragged = s.kv % KC != 0;
    const bool one = s.n <= 16;  // one query tile per item
    const bool small = s.sh <= 4 && s.sw <= 4;
    size_t lds = esz * (size_t)HG * D * (KC + padv);  // V^T tiles
    int waves = HG;
    const void* fn;
    if (fuse) {
      // one convolution wave per head beside each attention wave; at most 4
      // heads per workgroup keeps workgroups at 8 waves
      if (HG > 4) {
        HG = 4;
        p.HG = HG;
        p.nhg = (s.heads + HG - 1) / HG;
        p.nitems = s.B * s.R * p.nqb * p.nhg;
      }
      p.lw = lce_w;
      p.lb = lce_b;
      p.lce_pw = lce_pw(s.sw);
      p.lce_ps = lce_ps(s.sh, s.sw);
      p.lce_inv_pw = 1.0f / p.lce_pw;
      p.wave_lds = lce_lds_bytes(s.sh, s.sw, 4);
      lds = esz * (size_t)HG * D * (KC + padv) + (size_t)HG * p.wave_lds;
      waves = 2 * HG;
      if (small)
        fn = ragged ? (const void*)&attend_head_kernel<__bf16, true, 1, 4, 2> : (const void*)&attend_head_kernel<__bf16, false, 1, 4, 2>;
      else if (one)
        fn = ragged ? (const void*)&attend_head_kernel<__bf16, true, 1, 8, 4> : (const void*)&attend_head_kernel<__bf16, false, 1, 8, 4>;
      else
        fn = ragged ? (const void*)&attend_head_kernel<__bf16, true, 4, 8, 4> : (const void*)&attend_head_kernel<__bf16, false, 4, 8, 4>;
    } else if (dtype == kBF16) {
      fn = ragged ? (one ? (const void*)&attend_head_kernel<__bf16, true, 1, 0, 0> : (const void*)&attend_head_kernel<__bf16, true, 4, 0, 0>)
                  : (one ? (const void*)&attend_head_kernel<__bf16, false, 1, 0, 0> : (const void*)&attend_head_kernel<__bf16, false, 4, 0, 0>);
    } else {
      fn = ragged ? (one ? (const void*)&attend_head_kernel<float, true, 1, 0, 0> : (const void*)&attend_head_kernel<float, true, 4, 0, 0>)
                  : (one ? (const void*)&attend_head_kernel<float, false, 1, 0, 0> : (const void*)&attend_head_kernel<float, false, 4, 0, 0>);
    }
    // per-wave key tables pay off when many head waves would otherwise wait on
    // one: 8 heads per workgroup measured faster, 2 and 4 slower
    p.own_tab = p.HG >= 8;
    if (dtype == kBF16 && !fuse && p.HG == 2) {
      p.rtab_off = -1;  // the table and flag live in the exchange rows' static array
    } else {
      p.rtab_off = (int)lds;
      lds += sizeof(int) * ((size_t)(p.own_tab ? p.HG : 1) * KC + 1);
    }
    void* args[] = {&p};
    hipError_t e = hipLaunchKernel(fn, dim3((unsigned)p.nitems), dim3(waves * 64), args, lds, stream);
    if (e != hipSuccess || !lce || fuse) return e;
    return launch_lce(V, lce_w, lce_b, O, s, dtype, stream);
  }
  if (dense_attend_fits(s, dtype)) {
    const hipError_t e = launch_attend_dense(Q, K, V, idx, O, s, stream);
    if (e != hipSuccess || !lce) return e;
    return launch_lce(V, lce_w, lce_b, O, s, dtype, stream);
  }
  AttnLaunch L = plan_attend(s, dtype);
  L.p.Q = Q; L.p.K = K; L.p.V = V; L.p.idx = idx; L.p.O = O;
  void* args[] = {&L.p};
  if (L.nv > 4 || (L.nv > 2 && L.waves > 8)) return hipErrorInvalidValue;  // the kernels' launch bounds
  const void* fn = pick_attend(dtype, L);
  hipError_t e;
  if (L.lds > 64 * 1024) {
    // more than the default 64 KiB of dynamic LDS: raise the kernel's limit
    // to the most any launch of it uses (one value for every caller, so
    // concurrent calls cannot lower it under each other; the kernel's static
    // LDS comes on top)
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kChunkMaxLds);
    if (e != hipSuccess) return e;
  }
  e = hipLaunchKernel(fn, dim3((unsigned)L.nwg), dim3(L.waves * 64), args, L.lds, stream);
  if (e != hipSuccess || !lce) return e;
  return launch_lce(V, lce_w, lce_b, O, s, dtype, stream);
}

}  // namespace bra
