// Host side of the C ABI declared in include/bra.h: argument validation,
// workspace handling and kernel dispatch. No torch types, no global state.
#include "bra.h"
#include "bra_internal.h"

#include <stdint.h>

#include <mutex>

namespace {

using bra::Shape;

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Shape checks shared by every entry point. `heads` < 0 means "not an
// argument of this call" (bra_route: routing is shared by all heads).
bra_status check_shape(int B, int H, int W, int C, int heads, int S, int topk, int dtype, Shape* out) {
  if (B <= 0 || H <= 0 || W <= 0 || C <= 0 || S <= 0 || topk <= 0) return BRA_EINVAL;
  if (heads == 0 || heads < -1) return BRA_EINVAL;
  if (H % S != 0 || W % S != 0) return BRA_EINVAL;  // regions must tile the map
  if (heads > 0 && C % heads != 0) return BRA_EINVAL;
  const int64_t R = (int64_t)S * S;
  if (topk > R) return BRA_EINVAL;
  if ((int64_t)B * H * W * C >= (int64_t(1) << 40)) return BRA_EINVAL;
  if ((int64_t)H * W * C > bra::kMaxImageElems) return BRA_EINVAL;
  if ((int64_t)B * R * topk >= (int64_t(1) << 31)) return BRA_EINVAL;
  if (dtype != bra::kF32 && dtype != bra::kBF16) return BRA_EUNSUPPORTED;
  if (R > bra::kMaxRegions) return BRA_EUNSUPPORTED;
  if (C % 8 != 0) return BRA_EUNSUPPORTED;
  if (C > (dtype == bra::kBF16 ? bra::kMaxChannelsBf16 : bra::kMaxChannelsF32)) return BRA_EUNSUPPORTED;
  if (heads > 0 && C / heads != bra::kHeadDim) return BRA_EUNSUPPORTED;
  Shape s;
  s.B = B; s.H = H; s.W = W; s.C = C; s.heads = heads > 0 ? heads : 1; s.S = S; s.topk = topk;
  s.sh = H / S; s.sw = W / S; s.n = s.sh * s.sw; s.R = (int)R;
  s.d = heads > 0 ? C / heads : C;
  const int64_t kv = (int64_t)topk * s.n;
  if (kv >= bra::kMaxFastDiv) return BRA_EINVAL;
  s.kv = (int)kv;
  *out = s;
  return BRA_OK;
}

size_t pooled_bytes(const Shape& s) { return align_up(sizeof(float) * (size_t)s.B * s.R * s.C); }
size_t index_bytes(const Shape& s) { return align_up(sizeof(int32_t) * (size_t)s.B * s.R * s.topk); }

// Workspace: [Qr | Kr | idx], each 256-byte aligned.
size_t workspace_for(const Shape& s) { return 2 * pooled_bytes(s) + index_bytes(s); }

// Holds the workspace for one call: the caller's, or a stream-ordered one
// (only where `may_alloc`; the *_ws entry points never allocate).
struct Workspace {
  char* ptr = nullptr;
  bool owned = false;
  hipStream_t stream = nullptr;
  bra_status acquire(void* user, size_t user_bytes, size_t need, hipStream_t s, bool may_alloc = true) {
    stream = s;
    if (user != nullptr) {
      if (user_bytes < need || !aligned(user, kAlign)) return BRA_EINVAL;
      ptr = static_cast<char*>(user);
      return BRA_OK;
    }
    if (user_bytes != 0 || !may_alloc) return BRA_EINVAL;
    void* p = nullptr;
    if (hipMallocAsync(&p, need, s) != hipSuccess || p == nullptr) return BRA_ENOMEM;
    ptr = static_cast<char*>(p);
    owned = true;
    return BRA_OK;
  }
  ~Workspace() {
    if (owned) (void)hipFreeAsync(ptr, stream);
  }
};

bool bad_tensor(const void* p) { return p == nullptr || !aligned(p, 16); }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// Bytes of one [B, H, W, C] map and of the routing table.
size_t map_bytes(const Shape& s, int dtype) { return (dtype == bra::kBF16 ? 2 : 4) * (size_t)s.B * s.H * s.W * s.C; }
size_t table_bytes(const Shape& s) { return sizeof(int32_t) * (size_t)s.B * s.R * s.topk; }

// A caller workspace (ws, nbytes) must not overlap any of the tensors
// (p[i], n[i]); a null workspace is the library's own.
bool workspace_overlaps(const void* ws, size_t nbytes, const void* const* p, const size_t* n, int count) {
  if (ws == nullptr) return false;
  for (int i = 0; i < count; ++i)
    if (p[i] != nullptr && overlaps(ws, nbytes, p[i], n[i])) return true;
  return false;
}

// Local-context filter arguments: weight [C][5][5] (4-byte aligned), bias [C]
// or null (element aligned); neither may overlap O.
bra_status check_lce(const void* weight, const void* bias, const void* O, const Shape& s, int dtype) {
  const size_t esz = dtype == bra::kBF16 ? 2 : 4;
  if (weight == nullptr || !aligned(weight, 4)) return BRA_EINVAL;
  if (bias != nullptr && !aligned(bias, esz)) return BRA_EINVAL;
  const size_t obytes = esz * (size_t)s.B * s.H * s.W * s.C;
  if (overlaps(weight, esz * 25 * (size_t)s.C, O, obytes)) return BRA_EINVAL;
  if (bias != nullptr && overlaps(bias, esz * (size_t)s.C, O, obytes)) return BRA_EINVAL;
  return BRA_OK;
}

// ---- scratch of the entry point that allocates nothing (bra_forward_static)
// A file-scope device array: each GPU the library runs on holds its own copy
// until the process ends. Its device address is looked up once per device,
// with that device current; host code never uses the array's name itself
// (on the host it only stands for the symbol).
constexpr size_t kStaticScratchBytes = size_t(16) << 20;  // BRA_STATIC_SCRATCH_BYTES
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];

// The device address of the current device's copy of `scratch`; `stream`
// must belong to the current device (NULL: the current device's default).
bra_status static_scratch(hipStream_t stream, char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return BRA_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return BRA_EUNSUPPORTED;
  if (stream != nullptr) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return BRA_EHIP;
    if (sdev != dev) return BRA_EINVAL;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return BRA_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = static_cast<char*>(g_scratch_ptr[dev]);
  return BRA_OK;
}

bra_status enqueue_route(const void* Q, const void* K, int32_t* idx, const Shape& s, int dtype,
                         char* ws, hipStream_t stream) {
  float* Qr = reinterpret_cast<float*>(ws);
  float* Kr = reinterpret_cast<float*>(ws + pooled_bytes(s));
  if (bra::launch_pool(Q, K, Qr, Kr, s, dtype, stream) != hipSuccess) return BRA_EHIP;
  if (bra::launch_route(Qr, Kr, idx, s, stream) != hipSuccess) return BRA_EHIP;
  return BRA_OK;
}

}  // namespace

extern "C" {

const char* bra_status_string(bra_status status) {
  switch (status) {
    case BRA_OK: return "success";
    case BRA_EINVAL: return "invalid argument (null or misaligned pointer, non-positive size, S not dividing H or W, heads not dividing C, topk outside [1, S*S], or workspace too small)";
    case BRA_EUNSUPPORTED: return "unsupported configuration (head dim other than 32, more than 256 regions, C not a multiple of 8 or too large, or unknown dtype)";
    case BRA_EHIP: return "HIP runtime error while enqueueing a kernel";
    case BRA_ENOMEM: return "device workspace allocation failed";
    case BRA_ESCRATCH: return "the problem needs more scratch than the static buffer of bra_forward_static holds (BRA_STATIC_SCRATCH_BYTES = 16 MiB)";
  }
  return "unknown status";
}

const char* bra_attend_kernel(int B, int H, int W, int C, int heads, int S, int topk, bra_dtype dtype,
                              int with_lce) {
  Shape s;
  if (check_shape(B, H, W, C, heads, S, topk, (int)dtype, &s) != BRA_OK) return nullptr;
  return bra::attend_kernel_name(s, (int)dtype, with_lce != 0);
}

bra_status bra_pool(const void* Q, const void* K, float* Qr, float* Kr, int B, int H, int W, int C, int S,
                    bra_dtype dtype, hipStream_t stream) {
  Shape s;
  bra_status st = check_shape(B, H, W, C, -1, S, 1, (int)dtype, &s);
  if (st != BRA_OK) return st;
  if (bad_tensor(Q) || bad_tensor(K) || bad_tensor(Qr) || bad_tensor(Kr)) return BRA_EINVAL;
  const size_t mb = map_bytes(s, (int)dtype), pb = sizeof(float) * (size_t)s.B * s.R * s.C;
  if (overlaps(Qr, pb, Kr, pb)) return BRA_EINVAL;
  for (const void* o : {(const void*)Qr, (const void*)Kr})
    if (overlaps(o, pb, Q, mb) || overlaps(o, pb, K, mb)) return BRA_EINVAL;
  if (bra::launch_pool(Q, K, Qr, Kr, s, (int)dtype, stream) != hipSuccess) return BRA_EHIP;
  return BRA_OK;
}

bra_status bra_route_pooled(const float* Qr, const float* Kr, int32_t* idx, int B, int S, int C, int topk,
                            hipStream_t stream) {
  Shape s;
  // the map size does not enter the routing: a map of one token per region
  bra_status st = check_shape(B, S, S, C, -1, S, topk, bra::kBF16, &s);  // the limits of bra_route's C
  if (st != BRA_OK) return st;
  if (bad_tensor(Qr) || bad_tensor(Kr)) return BRA_EINVAL;
  if (idx == nullptr || !aligned(idx, 4)) return BRA_EINVAL;
  const size_t pb = sizeof(float) * (size_t)s.B * s.R * s.C, tb = table_bytes(s);
  if (overlaps(idx, tb, Qr, pb) || overlaps(idx, tb, Kr, pb)) return BRA_EINVAL;
  if (bra::launch_route(Qr, Kr, idx, s, stream) != hipSuccess) return BRA_EHIP;
  return BRA_OK;
}

size_t bra_workspace_bytes(int B, int H, int W, int C, int S, int topk) {
  Shape s;
  if (check_shape(B, H, W, C, -1, S, topk, bra::kBF16, &s) != BRA_OK) return 0;
  return workspace_for(s);
}

}  // extern "C"

namespace {

bra_status route_impl(const void* Q, const void* K, int32_t* idx, int B, int H, int W, int C, int S, int topk,
                      int dtype, void* workspace, size_t workspace_bytes, bool may_alloc, hipStream_t stream) {
  Shape s;
  bra_status st = check_shape(B, H, W, C, -1, S, topk, dtype, &s);
  if (st != BRA_OK) return st;
  if (bad_tensor(Q) || bad_tensor(K)) return BRA_EINVAL;
  if (idx == nullptr || !aligned(idx, 4)) return BRA_EINVAL;
  const size_t mb = map_bytes(s, dtype), tb = table_bytes(s);
  if (overlaps(idx, tb, Q, mb) || overlaps(idx, tb, K, mb)) return BRA_EINVAL;
  const void* ts[] = {Q, K, idx};
  const size_t ns[] = {mb, mb, tb};
  if (workspace_overlaps(workspace, workspace_bytes, ts, ns, 3)) return BRA_EINVAL;
  Workspace ws;
  st = ws.acquire(workspace, workspace_bytes, 2 * pooled_bytes(s), stream, may_alloc);
  if (st != BRA_OK) return st;
  return enqueue_route(Q, K, idx, s, dtype, ws.ptr, stream);
}

}  // namespace

extern "C" {

bra_status bra_route(const void* Q, const void* K, int32_t* idx,
                     int B, int H, int W, int C, int S, int topk,
                     bra_dtype dtype, hipStream_t stream) {
  return route_impl(Q, K, idx, B, H, W, C, S, topk, (int)dtype, nullptr, 0, true, stream);
}

bra_status bra_route_ws(const void* Q, const void* K, int32_t* idx,
                        int B, int H, int W, int C, int S, int topk,
                        bra_dtype dtype, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
  return route_impl(Q, K, idx, B, H, W, C, S, topk, (int)dtype, workspace, workspace_bytes, false, stream);
}

}  // extern "C"

namespace {

bra_status attend_impl(const void* Q, const void* K, const void* V, const int32_t* idx, const void* weight,
                       const void* bias, void* O, int B, int H, int W, int C, int heads, int S, int topk, int dtype,
                       hipStream_t stream) {
  Shape s;
  bra_status st = check_shape(B, H, W, C, heads, S, topk, dtype, &s);
  if (st != BRA_OK) return st;
  if (bad_tensor(Q) || bad_tensor(K) || bad_tensor(V) || bad_tensor(O))
    return BRA_EINVAL;
  if (idx == nullptr || !aligned(idx, 4)) return BRA_EINVAL;
  const size_t mb = map_bytes(s, dtype);
  if (overlaps(O, mb, Q, mb) || overlaps(O, mb, K, mb) || overlaps(O, mb, V, mb) ||
      overlaps(O, mb, idx, table_bytes(s)))
    return BRA_EINVAL;
  if (weight != nullptr && (st = check_lce(weight, bias, O, s, dtype)) != BRA_OK) return st;
  if (bra::launch_attend(Q, K, V, idx, weight, bias, O, s, dtype, stream) != hipSuccess) return BRA_EHIP;
  return BRA_OK;
}

bra_status forward_impl(const void* Q, const void* K, const void* V, const void* weight, const void* bias, void* O,
                        int B, int H, int W, int C, int heads, int S, int topk, int dtype, void* workspace,
                        size_t workspace_bytes, bool may_alloc, hipStream_t stream) {
  Shape s;
  bra_status st = check_shape(B, H, W, C, heads, S, topk, dtype, &s);
  if (st != BRA_OK) return st;
  if (bad_tensor(Q) || bad_tensor(K) || bad_tensor(V) || bad_tensor(O))
    return BRA_EINVAL;
  const size_t mb = map_bytes(s, dtype);
  if (overlaps(O, mb, Q, mb) || overlaps(O, mb, K, mb) || overlaps(O, mb, V, mb)) return BRA_EINVAL;
  if (weight != nullptr && (st = check_lce(weight, bias, O, s, dtype)) != BRA_OK) return st;
  {
    const size_t esz = dtype == bra::kBF16 ? 2 : 4;
    const void* ts[] = {Q, K, V, O, weight, bias};
    const size_t ns[] = {mb, mb, mb, mb, esz * 25 * (size_t)s.C, esz * (size_t)s.C};
    if (workspace_overlaps(workspace, workspace_bytes, ts, ns, 6)) return BRA_EINVAL;
  }
  Workspace ws;
  st = ws.acquire(workspace, workspace_bytes, workspace_for(s), stream, may_alloc);
  if (st != BRA_OK) return st;
  int32_t* idx = reinterpret_cast<int32_t*>(ws.ptr + 2 * pooled_bytes(s));
  st = enqueue_route(Q, K, idx, s, dtype, ws.ptr, stream);
  if (st != BRA_OK) return st;
  if (bra::launch_attend(Q, K, V, idx, weight, bias, O, s, dtype, stream) != hipSuccess) return BRA_EHIP;
  return BRA_OK;
}

}  // namespace

extern "C" {

bra_status bra_attend(const void* Q, const void* K, const void* V,
                      const int32_t* idx, void* O,
                      int B, int H, int W, int C, int heads, int S, int topk,
                      bra_dtype dtype, hipStream_t stream) {
  return attend_impl(Q, K, V, idx, nullptr, nullptr, O, B, H, W, C, heads, S, topk, (int)dtype, stream);
}

bra_status bra_forward(const void* Q, const void* K, const void* V, void* O,
                       int B, int H, int W, int C, int heads, int S, int topk,
                       bra_dtype dtype, hipStream_t stream) {
  return forward_impl(Q, K, V, nullptr, nullptr, O, B, H, W, C, heads, S, topk, (int)dtype, nullptr, 0, true,
                      stream);
}

bra_status bra_forward_ws(const void* Q, const void* K, const void* V, void* O,
                          int B, int H, int W, int C, int heads, int S, int topk,
                          bra_dtype dtype, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  return forward_impl(Q, K, V, nullptr, nullptr, O, B, H, W, C, heads, S, topk, (int)dtype, workspace,
                      workspace_bytes, false, stream);
}

bra_status bra_forward_static(const void* Q, const void* K, const void* V, void* O,
                              int B, int H, int W, int C, int heads, int S, int topk,
                              bra_dtype dtype, hipStream_t stream) {
  Shape s;
  bra_status st = check_shape(B, H, W, C, heads, S, topk, (int)dtype, &s);
  if (st != BRA_OK) return st;
  if (bad_tensor(Q) || bad_tensor(K) || bad_tensor(V) || bad_tensor(O)) return BRA_EINVAL;
  if (workspace_for(s) > kStaticScratchBytes) return BRA_ESCRATCH;
  // every other argument check happens in forward_impl, before any launch;
  // the pointer lookup below makes no allocation
  char* ws = nullptr;
  if ((st = static_scratch(stream, &ws)) != BRA_OK) return st;
  return forward_impl(Q, K, V, nullptr, nullptr, O, B, H, W, C, heads, S, topk, (int)dtype, ws, kStaticScratchBytes,
                      false, stream);
}

bra_status bra_attend_lce(const void* Q, const void* K, const void* V,
                          const int32_t* idx, const void* weight, const void* bias, void* O,
                          int B, int H, int W, int C, int heads, int S, int topk,
                          bra_dtype dtype, hipStream_t stream) {
  if (weight == nullptr) return BRA_EINVAL;
  return attend_impl(Q, K, V, idx, weight, bias, O, B, H, W, C, heads, S, topk, (int)dtype, stream);
}

bra_status bra_forward_lce(const void* Q, const void* K, const void* V,
                           const void* weight, const void* bias, void* O,
                           int B, int H, int W, int C, int heads, int S, int topk,
                           bra_dtype dtype, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  if (weight == nullptr) return BRA_EINVAL;
  return forward_impl(Q, K, V, weight, bias, O, B, H, W, C, heads, S, topk, (int)dtype, workspace,
                      workspace_bytes, true, stream);
}

}  // extern "C"

extern "C" {

size_t bra_backward_workspace_bytes(int B, int H, int W, int C, int heads, int S, int topk) {
  Shape s;
  if (heads <= 0 || check_shape(B, H, W, C, heads, S, topk, bra::kBF16, &s) != BRA_OK) return 0;
  return bra::backward_workspace_bytes(s);
}

bra_status bra_attend_backward(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                               const int32_t* idx, void* dQ, void* dK, void* dV,
                               int B, int H, int W, int C, int heads, int S, int topk,
                               bra_dtype dtype, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  Shape s;
  bra_status st = check_shape(B, H, W, C, heads, S, topk, (int)dtype, &s);
  if (st != BRA_OK) return st;
  const void* ins[] = {Q, K, V, O, dO};
  void* outs[] = {dQ, dK, dV};
  const size_t mb = map_bytes(s, (int)dtype), tb = table_bytes(s);
  for (const void* t : ins)
    if (bad_tensor(t)) return BRA_EINVAL;
  if (idx == nullptr || !aligned(idx, 4)) return BRA_EINVAL;
  for (int i = 0; i < 3; ++i) {
    if (bad_tensor(outs[i])) return BRA_EINVAL;
    for (const void* u : ins)
      if (overlaps(outs[i], mb, u, mb)) return BRA_EINVAL;
    if (overlaps(outs[i], mb, idx, tb)) return BRA_EINVAL;
    for (int j = 0; j < i; ++j)
      if (overlaps(outs[i], mb, outs[j], mb)) return BRA_EINVAL;
  }
  {
    const void* ts[] = {Q, K, V, O, dO, dQ, dK, dV, idx};
    const size_t ns[] = {mb, mb, mb, mb, mb, mb, mb, mb, tb};
    if (workspace_overlaps(workspace, workspace_bytes, ts, ns, 9)) return BRA_EINVAL;
  }
  Workspace ws;
  st = ws.acquire(workspace, workspace_bytes, bra::backward_workspace_bytes(s), stream);
  if (st != BRA_OK) return st;
  if (bra::launch_backward(Q, K, V, O, dO, idx, dQ, dK, dV, ws.ptr, s, (int)dtype, stream) != hipSuccess)
    return BRA_EHIP;
  return BRA_OK;
}

}  // extern "C"

namespace {

// Projection arguments: C a multiple of 32 and at most 256 (bf16) or 128 (fp32);
// X and the outputs 16-byte aligned and distinct; the weight 16-byte
// aligned, the bias element-aligned or null; no output overlapping X or the
// weights.
bra_status check_proj(const void* X, const void* Wqkv, const void* bqkv, void* const* outs, int nout,
                      const Shape& s, int dtype) {
  if (s.C % 32 != 0 || s.C > (dtype == bra::kBF16 ? bra::kMaxProjChannelsBf16 : bra::kMaxProjChannelsF32))
    return BRA_EUNSUPPORTED;
  const size_t esz = dtype == bra::kBF16 ? 2 : 4;
  if (bad_tensor(X) || bad_tensor(Wqkv)) return BRA_EINVAL;
  if (bqkv != nullptr && !aligned(bqkv, esz)) return BRA_EINVAL;
  const size_t map = esz * (size_t)s.B * s.H * s.W * s.C;
  for (int i = 0; i < nout; ++i) {
    if (bad_tensor(outs[i])) return BRA_EINVAL;
    if (overlaps(outs[i], map, X, map)) return BRA_EINVAL;
    if (overlaps(outs[i], map, Wqkv, esz * 3 * (size_t)s.C * s.C)) return BRA_EINVAL;
    if (bqkv != nullptr && overlaps(outs[i], map, bqkv, esz * 3 * (size_t)s.C)) return BRA_EINVAL;
    for (int j = 0; j < i; ++j)
      if (overlaps(outs[i], map, outs[j], map)) return BRA_EINVAL;
  }
  return BRA_OK;
}

}  // namespace

extern "C" {

bra_status bra_qkv_pool(const void* X, const void* Wqkv, const void* bqkv, void* Q, void* K, void* V,
                        float* Qr, float* Kr, int B, int H, int W, int C, int S,
                        bra_dtype dtype, hipStream_t stream) {
  Shape s;
  bra_status st = check_shape(B, H, W, C, -1, S, 1, (int)dtype, &s);
  if (st != BRA_OK) return st;
  void* outs[] = {Q, K, V};
  if ((st = check_proj(X, Wqkv, bqkv, outs, 3, s, (int)dtype)) != BRA_OK) return st;
  if (bad_tensor(Qr) || bad_tensor(Kr)) return BRA_EINVAL;
  const size_t pooled = sizeof(float) * (size_t)s.B * s.R * s.C;
  if (overlaps(Qr, pooled, Kr, pooled)) return BRA_EINVAL;
  if (bra::launch_qkv_pool(X, Wqkv, bqkv, Q, K, V, Qr, Kr, s, (int)dtype, stream) != hipSuccess) return BRA_EHIP;
  return BRA_OK;
}

bra_status bra_forward_qkv(const void* X, const void* Wqkv, const void* bqkv, void* Q, void* K, void* V, void* O,
                           int B, int H, int W, int C, int heads, int S, int topk,
                           bra_dtype dtype, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  Shape s;
  bra_status st = check_shape(B, H, W, C, heads, S, topk, (int)dtype, &s);
  if (st != BRA_OK) return st;
  void* outs[] = {Q, K, V, O};
  if ((st = check_proj(X, Wqkv, bqkv, outs, 4, s, (int)dtype)) != BRA_OK) return st;
  {
    const size_t mb = map_bytes(s, (int)dtype), esz = dtype == BRA_BF16 ? 2 : 4;
    const void* ts[] = {X, Wqkv, bqkv, Q, K, V, O};
    const size_t ns[] = {mb, esz * 3 * (size_t)s.C * s.C, esz * 3 * (size_t)s.C, mb, mb, mb, mb};
    if (workspace_overlaps(workspace, workspace_bytes, ts, ns, 7)) return BRA_EINVAL;
  }
  Workspace ws;
  st = ws.acquire(workspace, workspace_bytes, workspace_for(s), stream);
  if (st != BRA_OK) return st;
  float* Qr = reinterpret_cast<float*>(ws.ptr);
  float* Kr = reinterpret_cast<float*>(ws.ptr + pooled_bytes(s));
  int32_t* idx = reinterpret_cast<int32_t*>(ws.ptr + 2 * pooled_bytes(s));
  if (bra::launch_qkv_pool(X, Wqkv, bqkv, Q, K, V, Qr, Kr, s, (int)dtype, stream) != hipSuccess) return BRA_EHIP;
  if (bra::launch_route(Qr, Kr, idx, s, stream) != hipSuccess) return BRA_EHIP;
  if (bra::launch_attend(Q, K, V, idx, nullptr, nullptr, O, s, (int)dtype, stream) != hipSuccess) return BRA_EHIP;
  return BRA_OK;
}

}  // extern "C"
