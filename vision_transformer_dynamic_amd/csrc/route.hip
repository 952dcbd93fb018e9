// Region affinity fused with top-k routing (explainer "BiFormer Reshapes
// Visual Attention with 'Bi-Level Routing'", Part 2.2 step 3, pseudocode
// steps 4-5; paper summary "BiFormer: Vision Transformer with Bi-Level
// Routing Attention", Section 3: row i of the routing index holds the k
// regions most relevant to region i).
//
// Top-k by rank: candidate j of row i is beaten by m when A[i][m] > A[i][j],
// or A[i][m] == A[i][j] and m < j. This is a strict total order, so the number
// of candidates that beat j is a unique rank in [0, R); j is routed iff its
// rank is below k, and it is written to slot `rank`, which lists the routed
// regions in descending affinity with the lower index first on exact ties.
// The affinity rows never reach HBM.
//
// Three forms; each shape always takes the same one, so every routing table
// of a shape is the same bits.
//
// R <= 64 and C a multiple of 32 (matrix-core form; every shape with heads of
// 32 channels). The affinity of one image is a 64 x 64 (padded)
// fp32 product over C channels, done with 16x16x4 fp32 MFMA. One workgroup
// per (image, block of 16 rows), 8 waves: wave w computes the 16 x 16 tile of
// candidates 16 (w % 4) .. +15 over channel half w / 4, its operands loaded
// straight from memory as 16-byte vectors (one round trip for C <= 256); the
// two halves are added in a fixed order through LDS. Each affinity becomes a
// 64-bit key (order-preserving bits of the value, then a decreasing function
// of j), so "beats" is one unsigned compare; k = 1 is a wave-wide maximum of
// the keys. The row
// blocks of one image run on one XCD (xcd_item) and share its L2 copy of
// K^r[b]; images are split over the XCDs as in the pool and attention kernels.
//
// 64 < R <= 256 and C a multiple of 32 (matrix-core form for many regions,
// route_mfma256_kernel below): one 16-candidate tile per wave over all
// channels, and the k best taken one at a time for k <= 32.
//
// Other shapes (vector form). One workgroup per (image b, block of 4 affinity rows);
// each of its 4 waves owns one row, and lane j owns the candidates j, j+64,
// j+128, j+192 (at most 256 regions). Channels are streamed in slices of CC:
// each slice of K^r[b] (all R rows) and of the block's query rows is staged
// in LDS with coalesced loads, the next slice's loads being in flight while
// the current one is used. A[i][j] is accumulated as four fused multiply-add
// chains, one per channel residue mod 4, in increasing channel order, and
// combined as (s0 + s1) + (s2 + s3). The query row is read as a broadcast,
// K^r row j by lane j. The row's affinities become the same 64-bit keys as
// in the matrix-core form (so both forms order NaN alike and every slot is
// written), and each lane counts its rank against the whole row (broadcast
// LDS reads): R compares per candidate, independent of k.
#include "bra_internal.h"
#include "route_common.h"

#include <math.h>

namespace bra {
namespace {

constexpr int RB = 4;              // affinity rows per workgroup (one per wave)
constexpr int NT = 256;            // threads

struct RouteParams {
  const float* Qr;
  const float* Kr;
  int32_t* idx;
  int B, R, C, topk;
  int row_blocks;  // ceil(R / RB): workgroups per image
  int ldr;         // LDS row stride of the affinity block (R rounded up to 4)
};

// ---- vector form ----
// NU: candidates per lane (1 when R <= 64, 4 when R <= 256).
// CC: channels per staged slice (fewer when there are more candidate rows).
template <int NU> struct RouteCfg {
  static constexpr int CC = NU == 1 ? 64 : 32;
  static constexpr int C4 = CC / 4;        // float4 per row slice
  static constexpr int LDC = CC + 4;       // LDS row stride (floats)
};

template <int NU>
__global__ __launch_bounds__(NT) void route_kernel(RouteParams p) {
  constexpr int CC = RouteCfg<NU>::CC, C4 = RouteCfg<NU>::C4, LDC = RouteCfg<NU>::LDC;
  constexpr int KLD = 64 * NU * C4 / NT;  // float4 loads of K^r per thread per slice
  extern __shared__ __align__(16) float sm[];
  float* Ks = sm;                 // R x LDC
  float* Qs = Ks + p.R * LDC;     // RB x LDC
  uint64_t* As = reinterpret_cast<uint64_t*>(Qs + RB * LDC);  // RB x ldr keys

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int b = blockIdx.x / p.row_blocks;
  const int i0 = (blockIdx.x - b * p.row_blocks) * RB;
  const int nrows = min(RB, p.R - i0);
  const float* kb = p.Kr + (int64_t)b * p.R * p.C;
  const float* qb = p.Qr + ((int64_t)b * p.R + i0) * p.C;

  float4 acc[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) acc[u] = make_float4(0.f, 0.f, 0.f, 0.f);

  // slice loads: element f = tid + NT*m of the slice is (row f / C4, float4 f % C4)
  float4 kreg[KLD];
  float4 qreg = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int m = 0; m < KLD; ++m) kreg[m] = make_float4(0.f, 0.f, 0.f, 0.f);
  auto slice_w4 = [&](int c0) { return min(CC, p.C - c0) >> 2; };  // valid float4 per row
  {
    const int w4 = slice_w4(0);
#pragma unroll
    for (int m = 0; m < KLD; ++m) {
      const int f = tid + NT * m, j = f / C4, c4 = f % C4;
      if (j < p.R && c4 < w4) kreg[m] = *reinterpret_cast<const float4*>(kb + (int64_t)j * p.C + 4 * c4);
    }
    const int r = tid / C4, c4 = tid % C4;
    if (r < nrows && c4 < w4) qreg = *reinterpret_cast<const float4*>(qb + (int64_t)r * p.C + 4 * c4);
  }

  for (int c0 = 0; c0 < p.C; c0 += CC) {
    const int w4 = slice_w4(c0);
    if (c0) __syncthreads();  // previous slice consumed
#pragma unroll
    for (int m = 0; m < KLD; ++m) {
      const int f = tid + NT * m, j = f / C4, c4 = f % C4;
      if (j < p.R) *reinterpret_cast<float4*>(Ks + j * LDC + 4 * c4) = kreg[m];
    }
    {
      const int r = tid / C4, c4 = tid % C4;
      if (r < RB) *reinterpret_cast<float4*>(Qs + r * LDC + 4 * c4) = qreg;
    }
    __syncthreads();
    const int n0 = c0 + CC;  // next slice, in flight while this one is used
    if (n0 < p.C) {
      const int w4n = slice_w4(n0);
#pragma unroll
      for (int m = 0; m < KLD; ++m) {
        const int f = tid + NT * m, j = f / C4, c4 = f % C4;
        if (j < p.R && c4 < w4n) kreg[m] = *reinterpret_cast<const float4*>(kb + (int64_t)j * p.C + n0 + 4 * c4);
      }
      const int r = tid / C4, c4 = tid % C4;
      if (r < nrows && c4 < w4n) qreg = *reinterpret_cast<const float4*>(qb + (int64_t)r * p.C + n0 + 4 * c4);
    }
    const float* qs = Qs + wave * LDC;
    for (int c4 = 0; c4 < w4; ++c4) {
      const float4 q = *reinterpret_cast<const float4*>(qs + 4 * c4);
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const float4 k = *reinterpret_cast<const float4*>(Ks + min(lane + 64 * u, p.R - 1) * LDC + 4 * c4);
        acc[u] = affinity_step(acc[u], q, k);
      }
    }
  }

  // the wave's affinity row as keys in LDS; columns R..ldr-1 hold key 0
  const int row = wave;
  uint64_t* a = As + row * p.ldr;
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int j = lane + 64 * u;
    if (j < p.ldr) a[j] = j < p.R ? affinity_key(affinity_finish(acc[u]), j) : 0ull;
  }
  __syncthreads();
  if (row >= nrows) return;  // wave-uniform; no barrier follows

  // ranks (the keys are a strict total order, so every slot is written once)
  int32_t* out = p.idx + ((int64_t)b * p.R + i0 + row) * p.topk;
#pragma unroll 1
  for (int u = 0; u < NU; ++u) {
    const int j = lane + 64 * u;
    if (j >= p.R) break;
    const int rank = key_rank(a, p.ldr, a[j]);
    if (rank < p.topk) out[rank] = j;
  }
}

// ---- matrix-core form (R <= 64, C a multiple of 32) ----
constexpr int MR = 16;    // affinity rows per workgroup
constexpr int MW = 8;     // waves: 4 candidate tiles x 2 channel halves

// The block's 16 query rows are read from memory once per workgroup into
// LDS (rows of C + 4 floats, so the 16 rows of an operand read start on
// different banks), instead of once per candidate-tile wave: the kernel is
// bound by each CU's load rate, and the query rows were most of its bytes
// (4 of the 8 waves read the same rows of each channel half). Each wave's
// first chunk of candidate rows is issued before the staging barrier.
constexpr int kQPad = 4;  // floats of padding per staged query row
constexpr int kQLdsMaxC = 256;  // channels up to which the query rows are staged (LDS stays under 64 KB)

// Stage query rows i0 .. i0 + 15 of image row offset img (rows past R repeat
// row R - 1, whose results are never used) into qs[16][C + kQPad].
__device__ inline void stage_query_rows(const RouteParams& p, int64_t img, int i0, float* qs) {
  const int c4n = p.C >> 2;
  for (int f = threadIdx.x; f < 16 * c4n; f += blockDim.x) {
    const int r = f / c4n, c4 = f - r * c4n;
    const float4 v = *reinterpret_cast<const float4*>(p.Qr + (img + min(i0 + r, p.R - 1)) * p.C + 4 * c4);
    *reinterpret_cast<float4*>(qs + r * (p.C + kQPad) + 4 * c4) = v;
  }
}

// NS: 16-channel steps per wave loaded at once (a divisor of C / 32; all of a
// chunk's loads are issued before its products). QLDS: query rows staged in
// LDS (dynamic, 16 x (C + kQPad) floats).
template <int NS, bool QLDS>
__global__ __launch_bounds__(MW * 64) void route_mfma_kernel(RouteParams p) {
  __shared__ float part[MR][64];                    // channel half 1 of each tile
  __shared__ __align__(16) uint64_t keys[MR][64];   // keys of the block's rows
  extern __shared__ __align__(16) float qs[];       // QLDS: [16][C + kQPad]
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int tile = wave & 3, half = wave >> 2;
  const int g = lane >> 4, l16 = lane & 15;
  const int w = xcd_item(blockIdx.x, gridDim.x);  // (image, row block), an image's blocks on one XCD
  const int b = w / p.row_blocks;
  const int i0 = (w - b * p.row_blocks) * MR;
  const int ncol = (p.R + 15) & ~15;
  const int j0 = tile * 16;
  const bool active = j0 < ncol;

  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  // A operand: lane supplies query row i0 + l16, B operand candidate row
  // j0 + l16, both the channels 16 t + 4 g .. + 3 of the half at step t
  // (rows past R read row R - 1; their results are never used)
  const int nh = p.C >> 5;  // 16-channel steps per half
  const int64_t img = (int64_t)b * p.R;
  const float* krow = p.Kr + (img + min(j0 + l16, p.R - 1)) * p.C + half * (p.C >> 1) + 4 * g;
  float4 k[NS];
  if (QLDS) {
    if (active) {
#pragma unroll
      for (int m = 0; m < NS; ++m) k[m] = *reinterpret_cast<const float4*>(krow + 16 * m);
    }
    stage_query_rows(p, img, i0, qs);
    __syncthreads();
  }
  if (active) {
    const float* qrow = QLDS ? qs + l16 * (p.C + kQPad) + half * (p.C >> 1) + 4 * g
                             : p.Qr + (img + min(i0 + l16, p.R - 1)) * p.C + half * (p.C >> 1) + 4 * g;
    for (int t0 = 0; t0 < nh; t0 += NS) {
      float4 a[NS];
      if (!QLDS || t0 > 0) {
#pragma unroll
        for (int m = 0; m < NS; ++m) k[m] = *reinterpret_cast<const float4*>(krow + 16 * (t0 + m));
      }
#pragma unroll
      for (int m = 0; m < NS; ++m) a[m] = *reinterpret_cast<const float4*>(qrow + 16 * (t0 + m));
      __builtin_amdgcn_sched_barrier(0);  // keep every load of the chunk ahead of the products
#pragma unroll
      for (int m = 0; m < NS; ++m) acc = affinity_mfma_step(acc, a[m], k[m]);
    }
    // lane holds rows 4 g .. 4 g + 3 of candidate column j0 + l16
    if (half == 1) {
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) part[4 * g + ii][j0 + l16] = acc[ii];
    }
  }
  __syncthreads();
  if (half == 0) {
    // every one of the 64 key columns is written: columns past R (including
    // whole tiles past ncol, whose waves computed nothing) get key 0
    const int col = j0 + l16;
    const uint64_t valid = active && col < p.R ? ~0ull : 0ull;
    float ph[4];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) ph[ii] = part[4 * g + ii][col];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) keys[4 * g + ii][col] = affinity_key(acc[ii] + ph[ii], col) & valid;
  }
  __syncthreads();

  // wave w ranks rows 2w and 2w + 1 of the block; lane j is candidate j
#pragma unroll
  for (int q = 0; q < MR / MW; ++q) {
    const int row = (MR / MW) * wave + q;
    if (i0 + row >= p.R) break;  // uniform
    int32_t* out = p.idx + ((int64_t)b * p.R + i0 + row) * p.topk;
    const uint64_t kj = keys[row][lane];
    if (p.topk == 1) {
      const uint64_t best = wave_max_key(kj);
      if (lane == 0) out[0] = key_index(best);
    } else {
      const int rank = key_rank64(&keys[row][0], kj);
      if (lane < p.R && rank < p.topk) out[rank] = lane;
    }
  }
}

// ---- matrix-core form for 64 < R <= 256 (C a multiple of 32) ----
// One workgroup per (image, block of 16 rows), 16 waves: wave t computes the
// 16 x 16 tile of candidates 16 t .. 16 t + 15 over all C channels (the
// 16-channel steps in increasing order from a zero accumulator, with the
// same 16x16x4 fp32 products), so each affinity is one fixed sequence. The
// tile's keys go to LDS ([16 rows][256]: key 0 past R), then wave t ranks row
// t of the block: lane l holds candidates l, l + 64, l + 128, l + 192. For k
// up to 32 the k best are taken one at a time (a wave-wide maximum of the
// keys, then the winner's key cleared), k rounds of a few dozen
// instructions; for larger k every candidate counts the keys that beat it
// (256 compares each), as in the other forms. Keys are unique, so both give
// the same table: descending affinity, the lower index first on ties.
constexpr int BR = 16;     // affinity rows per workgroup
constexpr int BW = 16;     // waves: one 16-candidate tile each
constexpr int BMAX = 256;  // candidates

// QLDS: the block's query rows staged once in LDS (dynamic, 16 x (C + kQPad)
// floats), as in route_mfma_kernel: all 16 waves read the same rows.
template <int NS, bool QLDS>
__global__ __launch_bounds__(BW * 64) void route_mfma256_kernel(RouteParams p) {
  __shared__ __align__(16) uint64_t keys[BR][BMAX];
  extern __shared__ __align__(16) float qs[];  // QLDS: [16][C + kQPad]
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, l16 = lane & 15;
  const int w = xcd_item(blockIdx.x, gridDim.x);  // (image, row block), an image's blocks on one XCD
  const int b = w / p.row_blocks;
  const int i0 = (w - b * p.row_blocks) * BR;
  const int j0 = wave * 16;
  const int64_t img = (int64_t)b * p.R;

  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  // A operand: query row i0 + l16; B operand: candidate row j0 + l16;
  // channels 16 t + 4 g .. + 3 at step t (rows past R read row R - 1;
  // their results are never used)
  const float* krow = p.Kr + (img + min(j0 + l16, p.R - 1)) * p.C + 4 * g;
  const int nsteps = p.C >> 4;
  float4 k[NS];
  if (QLDS) {
    if (j0 < p.R) {  // uniform
#pragma unroll
      for (int m = 0; m < NS; ++m) k[m] = *reinterpret_cast<const float4*>(krow + 16 * m);
    }
    stage_query_rows(p, img, i0, qs);
    __syncthreads();
  }
  if (j0 < p.R) {  // uniform
    const float* qrow = QLDS ? qs + l16 * (p.C + kQPad) + 4 * g : p.Qr + (img + min(i0 + l16, p.R - 1)) * p.C + 4 * g;
    for (int t0 = 0; t0 < nsteps; t0 += NS) {
      float4 a[NS];
      if (!QLDS || t0 > 0) {
#pragma unroll
        for (int m = 0; m < NS; ++m) k[m] = *reinterpret_cast<const float4*>(krow + 16 * (t0 + m));
      }
#pragma unroll
      for (int m = 0; m < NS; ++m) a[m] = *reinterpret_cast<const float4*>(qrow + 16 * (t0 + m));
      __builtin_amdgcn_sched_barrier(0);  // keep every load of the chunk ahead of the products
#pragma unroll
      for (int m = 0; m < NS; ++m) acc = affinity_mfma_step(acc, a[m], k[m]);
    }
  }
  {
    // every one of the 256 key columns is written: columns past R get key 0
    const int col = j0 + l16;
    const uint64_t valid = col < p.R ? ~0ull : 0ull;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) keys[4 * g + ii][col] = affinity_key(acc[ii], col) & valid;
  }
  __syncthreads();

  const int row = wave;
  if (i0 + row >= p.R) return;  // uniform; no barrier follows
  int32_t* out = p.idx + (img + i0 + row) * p.topk;
  uint64_t kc[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) kc[u] = keys[row][lane + 64 * u];
  if (p.topk <= 32) {
    // each lane's four keys in descending order (a five-step exchange
    // network), then k rounds: the largest head key of the wave wins and
    // its lane moves to its next key. A round compares the high halves only
    // (the affinity's order bits: one 32-bit maximum across the wave, single
    // instructions per step); the low halves (the index) decide only when
    // several lanes hold the same high half. The winners are the 64-bit key
    // maxima, so the table is the one the one-by-one extraction gives.
#define BRA_CSWAP(a, b)                         \
  {                                             \
    const uint64_t hi_ = kc[a] > kc[b] ? kc[a] : kc[b]; \
    const uint64_t lo_ = kc[a] > kc[b] ? kc[b] : kc[a]; \
    kc[a] = hi_;                                \
    kc[b] = lo_;                                \
  }
    BRA_CSWAP(0, 1) BRA_CSWAP(2, 3) BRA_CSWAP(0, 2) BRA_CSWAP(1, 3) BRA_CSWAP(1, 2)
#undef BRA_CSWAP
    for (int r = 0; r < p.topk; ++r) {  // uniform
      const uint32_t hi = (uint32_t)(kc[0] >> 32);
      const uint32_t m = wave_max_u32(hi);
      const uint64_t tied = __builtin_amdgcn_ballot_w64(hi == m);
      uint64_t win = tied;
      if (__builtin_popcountll(tied) > 1) {  // uniform; equal high halves: the larger low half
        const uint32_t lo = hi == m ? (uint32_t)kc[0] : 0u;
        const uint32_t ml = wave_max_u32(lo);
        win = __builtin_amdgcn_ballot_w64(hi == m && lo == ml);
      }
      const int wl = __builtin_ctzll(win);
      if (lane == 0) out[r] = key_index(((uint64_t)m << 32) | (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)kc[0], wl));
      if (lane == wl) {
        kc[0] = kc[1];
        kc[1] = kc[2];
        kc[2] = kc[3];
        kc[3] = 0ull;
      }
    }
  } else {
#pragma unroll 1
    for (int u = 0; u < 4; ++u) {
      const int j = lane + 64 * u;
      if (j >= p.R) break;
      const int rank = key_rank(&keys[row][0], BMAX, kc[u]);
      if (rank < p.topk) out[rank] = j;
    }
  }
}

}  // namespace

// dynamic LDS of the vector form: the staged slices (floats), then the key
// rows (16-byte aligned: R * ldc + RB * ldc floats is a multiple of 4)
size_t route_lds_bytes(const Shape& s) {
  const int ldr = (s.R + 3) / 4 * 4;
  const int ldc = s.R <= 64 ? RouteCfg<1>::LDC : RouteCfg<4>::LDC;
  return sizeof(float) * ((size_t)s.R * ldc + (size_t)RB * ldc) + sizeof(uint64_t) * (size_t)RB * ldr;
}

hipError_t launch_route(const float* Qr, const float* Kr, int32_t* idx,
                        const Shape& s, hipStream_t stream) {
  void* args[1];
  if (s.R <= 64 && s.C % 32 == 0) {
    RouteParams p{Qr, Kr, idx, s.B, s.R, s.C, s.topk, (s.R + MR - 1) / MR, 0};
    args[0] = &p;
    const unsigned grid = (unsigned)(s.B * p.row_blocks);
    const int nh = s.C / 32;
    const bool ql = s.C <= kQLdsMaxC;
    const void* fns[2][4] = {
        {reinterpret_cast<const void*>(&route_mfma_kernel<8, false>), reinterpret_cast<const void*>(&route_mfma_kernel<4, false>),
         reinterpret_cast<const void*>(&route_mfma_kernel<2, false>), reinterpret_cast<const void*>(&route_mfma_kernel<1, false>)},
        {reinterpret_cast<const void*>(&route_mfma_kernel<8, true>), reinterpret_cast<const void*>(&route_mfma_kernel<4, true>),
         reinterpret_cast<const void*>(&route_mfma_kernel<2, true>), reinterpret_cast<const void*>(&route_mfma_kernel<1, true>)}};
    const void* fn = fns[ql][nh % 8 == 0 ? 0 : nh % 4 == 0 ? 1 : nh % 2 == 0 ? 2 : 3];
    const size_t lds = ql ? sizeof(float) * 16 * (size_t)(s.C + kQPad) : 0;
    return hipLaunchKernel(fn, dim3(grid), dim3(MW * 64), args, lds, stream);
  }
  if (s.R <= BMAX && s.C % 32 == 0) {
    RouteParams p{Qr, Kr, idx, s.B, s.R, s.C, s.topk, (s.R + BR - 1) / BR, 0};
    args[0] = &p;
    const int nsteps = s.C / 16;  // even
    const bool ql = s.C <= kQLdsMaxC;
    const void* fns[2][3] = {
        {reinterpret_cast<const void*>(&route_mfma256_kernel<8, false>), reinterpret_cast<const void*>(&route_mfma256_kernel<4, false>),
         reinterpret_cast<const void*>(&route_mfma256_kernel<2, false>)},
        {reinterpret_cast<const void*>(&route_mfma256_kernel<8, true>), reinterpret_cast<const void*>(&route_mfma256_kernel<4, true>),
         reinterpret_cast<const void*>(&route_mfma256_kernel<2, true>)}};
    const void* fn = fns[ql][nsteps % 8 == 0 ? 0 : nsteps % 4 == 0 ? 1 : 2];
    const size_t lds = ql ? sizeof(float) * 16 * (size_t)(s.C + kQPad) : 0;
    return hipLaunchKernel(fn, dim3((unsigned)(s.B * p.row_blocks)), dim3(BW * 64), args, lds, stream);
  }
  RouteParams p{Qr, Kr, idx, s.B, s.R, s.C, s.topk, (s.R + RB - 1) / RB, (s.R + 3) / 4 * 4};
  args[0] = &p;
  const void* fn = s.R <= 64 ? reinterpret_cast<const void*>(&route_kernel<1>)
                             : reinterpret_cast<const void*>(&route_kernel<4>);
  return hipLaunchKernel(fn, dim3((unsigned)(s.B * p.row_blocks)), dim3(NT), args, route_lds_bytes(s), stream);
}

}  // namespace bra
