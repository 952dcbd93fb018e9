/*
 * bra.h - C ABI of the MI355X (gfx950) Bi-Level Routing Attention forward pass.
 *
 * Bi-Level Routing Attention (BRA), from BiFormer (CVPR 2023, arXiv 2303.08810),
 * as described by the explainer "BiFormer Reshapes Visual Attention with
 * 'Bi-Level Routing'", Part 2.2 "The Overall BRA Flow" (steps 1-4 and the
 * PyTorch-style pseudocode), and by the paper summary "BiFormer: Vision
 * Transformer with Bi-Level Routing Attention", Section 3 "Our Approach".
 * Q, K, V are taken as already projected (the pseudocode's linear_qkv output).
 * bra_attend / bra_forward compute the attention alone; bra_attend_lce /
 * bra_forward_lce add the local-context term (+ dwconv(V)), whose filter
 * weights they take as arguments.
 *
 * Tensors
 *   Q, K, V, O : [B, H, W, C] row-major, channels fastest, all of one dtype,
 *                caller-owned device memory, 16-byte aligned. O must not
 *                overlap Q, K, V or idx (BRA_EINVAL).
 *   idx        : [B, S*S, topk] int32 device memory, 4-byte aligned; as the
 *                output of bra_route it must not overlap Q or K.
 * Regions      : S must divide H and W (no padding). Region r covers rows
 *                [(r/S)*H/S, (r/S+1)*H/S) and columns [(r%S)*W/S, (r%S+1)*W/S);
 *                n = (H/S)*(W/S) tokens per region.
 * Heads        : head m owns channels [m*d, (m+1)*d), d = C/heads. Supported:
 *                d == 32. Routing is shared by all heads and uses all C channels.
 * Scale        : softmax(q k^T / sqrt(d)).
 * Limits       : 1 <= S*S <= 256, 1 <= topk <= S*S, C % 8 == 0,
 *                C <= 2048 (bf16) or 1024 (fp32), H*W*C < 2^31 per image,
 *                topk*n < 2^22 keys per query, B*H*W*C < 2^40.
 *
 * Streams and errors
 *   Every call only enqueues work on `stream` (NULL = the legacy default
 *   stream) and returns; none synchronises. Arguments are checked on the host
 *   before anything is enqueued: a null pointer, a non-positive size, S not
 *   dividing H or W, heads not dividing C, topk outside [1, S*S], a
 *   misaligned pointer, a too-small workspace or sizes beyond the size limits
 *   give BRA_EINVAL; a head dim, region count, channel count or dtype this
 *   build does not implement gives BRA_EUNSUPPORTED. A HIP error reported while enqueueing gives BRA_EHIP;
 *   a failed workspace allocation gives BRA_ENOMEM. On any error nothing has
 *   been enqueued, except for BRA_EHIP, where earlier launches of the same
 *   call may already be queued. The library is thread-safe; its only state
 *   is the static scratch of bra_forward_static (one buffer per GPU and the
 *   cached device address of each). Calls that share a workspace must be
 *   ordered by the caller.
 *
 * Workspace
 *   The routing step keeps the fp32 region means Q^r, K^r (and, in
 *   bra_forward, the routing table) in device scratch of
 *   bra_workspace_bytes(...) bytes. bra_route and bra_forward allocate it
 *   and free it stream-ordered (hipMallocAsync / hipFreeAsync) on `stream`;
 *   bra_route_ws and bra_forward_ws take a caller-owned buffer (256-byte
 *   aligned, not overlapping any tensor argument) instead and allocate
 *   nothing.
 */
#ifndef BRA_H_
#define BRA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* HIP's own stream handle type; repeated here so the header needs no HIP headers. */
typedef struct ihipStream_t* hipStream_t;

typedef enum bra_dtype {
  BRA_F32 = 0,  /* IEEE binary32 in, binary32 out */
  BRA_BF16 = 1  /* bfloat16 in, bfloat16 out (round to nearest even) */
} bra_dtype;

typedef enum bra_status {
  BRA_OK = 0,
  BRA_EINVAL = 1,
  BRA_EUNSUPPORTED = 2,
  BRA_EHIP = 3,
  BRA_ENOMEM = 4,
  BRA_ESCRATCH = 5  /* bra_forward_static: more scratch than its static buffer holds */
} bra_status;

/* Static, NUL-terminated description of a status code. Never NULL. */
const char* bra_status_string(bra_status status);

/* Diagnostics: the name of the attention kernel that bra_attend (with_lce
 * = 0) or bra_attend_lce (with_lce != 0) launches for these sizes, as
 * profilers list it; NULL if the sizes are invalid or unsupported. A static
 * string; no device work. */
const char* bra_attend_kernel(int B, int H, int W, int C, int heads, int S, int topk,
                              bra_dtype dtype, int with_lce);

/* Bytes of device workspace that bra_route_ws and bra_forward_ws need for
 * these sizes (0 if the sizes are invalid). */
size_t bra_workspace_bytes(int B, int H, int W, int C, int S, int topk);

/*
 * bra_route - region-level routing (explainer Part 2.2, step 3, pseudocode
 * steps 3-5; paper summary Section 3 "Region partition and routing").
 *
 * Computes the region means Q^r, K^r of Q and K (fp32 accumulation), the
 * affinity A = Q^r (K^r)^T over all C channels in fp32, and writes to idx the
 * topk largest entries of each row of A: idx[b][i][0..topk) in descending
 * affinity, the lower region index first on exact ties. Deterministic: the
 * same inputs give bit-identical idx, and bra_forward routes with exactly
 * this table.
 */
bra_status bra_route(const void* Q, const void* K, int32_t* idx,
                     int B, int H, int W, int C, int S, int topk,
                     bra_dtype dtype, hipStream_t stream);

/* bra_route_ws - bra_route with the caller's workspace (at least
 * bra_workspace_bytes(B, H, W, C, S, topk) bytes, 256-byte aligned; a null
 * or too small buffer gives BRA_EINVAL). Same table, bit for bit. */
bra_status bra_route_ws(const void* Q, const void* K, int32_t* idx,
                        int B, int H, int W, int C, int S, int topk,
                        bra_dtype dtype, void* workspace, size_t workspace_bytes,
                        hipStream_t stream);

/*
 * bra_pool - the region means alone (explainer Part 2.2 step 3 and
 * pseudocode step 3; paper summary Section 6, regional representations by
 * averaging): Qr[b][r][:] and Kr[b][r][:] are the means of Q and K over the
 * n tokens of region r, accumulated in fp32 in a fixed order: exactly the
 * means bra_route computes before it routes.
 *   Qr, Kr : [B, S*S, C] fp32 device memory, 16-byte aligned, not
 *            overlapping each other, Q or K (BRA_EINVAL).
 */
bra_status bra_pool(const void* Q, const void* K, float* Qr, float* Kr,
                    int B, int H, int W, int C, int S,
                    bra_dtype dtype, hipStream_t stream);

/*
 * bra_route_pooled - the routing step from given region means (explainer
 * Part 2.2 pseudocode steps 4-5): the affinity A = Qr Kr^T of every image
 * over all C channels in fp32 and the topk largest entries of each row, in
 * the order and with the tie rule of bra_route. bra_route is bra_pool
 * followed by this call, bit for bit.
 *   Qr, Kr : [B, S*S, C] fp32 device memory, 16-byte aligned.
 *   idx    : [B, S*S, topk] int32 output, 4-byte aligned, not overlapping
 *            Qr or Kr (BRA_EINVAL).
 * Same limits on S, C and topk as bra_route.
 */
bra_status bra_route_pooled(const float* Qr, const float* Kr, int32_t* idx,
                            int B, int S, int C, int topk, hipStream_t stream);

/*
 * bra_attend - token-level attention over routed regions (explainer Part 2.2,
 * step 4, pseudocode steps 6-7 without the dwconv term; paper summary
 * Section 3 "Token-to-token attention").
 *
 * For every image b, region i and head m, the queries of region i attend with
 * softmax(q k^T / sqrt(d)) to the keys/values of the tokens of regions
 * idx[b][i][0..topk), which are read straight from K and V (no gathered copy
 * is made). fp32 accumulation and softmax; bf16 P for the P.V product on the
 * bf16 path. idx entries are read from device memory: an entry outside
 * [0, S*S) is never dereferenced and makes region i's output NaN.
 */
bra_status bra_attend(const void* Q, const void* K, const void* V,
                      const int32_t* idx, void* O,
                      int B, int H, int W, int C, int heads, int S, int topk,
                      bra_dtype dtype, hipStream_t stream);

/*
 * bra_forward - the whole BRA forward: bra_route into the workspace, then
 * bra_attend with that table (explainer Part 2.2 pseudocode steps 1 and
 * 3-7 without the dwconv term). O = BRA(Q, K, V).
 */
bra_status bra_forward(const void* Q, const void* K, const void* V, void* O,
                       int B, int H, int W, int C, int heads, int S, int topk,
                       bra_dtype dtype, hipStream_t stream);

/* bra_forward_ws - bra_forward with the caller's workspace (at least
 * bra_workspace_bytes(B, H, W, C, S, topk) bytes, 256-byte aligned; a null
 * or too small buffer gives BRA_EINVAL). The routing table is left in the
 * workspace at byte offset 2 * align256(4 * B * S*S * C), [B, S*S, topk]
 * int32, after the region means Q^r and K^r ([B, S*S, C] fp32 each, at
 * offsets 0 and align256(4 * B * S*S * C)). Same output, bit for bit. */
bra_status bra_forward_ws(const void* Q, const void* K, const void* V, void* O,
                          int B, int H, int W, int C, int heads, int S, int topk,
                          bra_dtype dtype, void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

/*
 * bra_forward_static - bra_forward for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc. The same kernels and the same output, bit for bit; the
 * region means and the routing table go to a library-owned static device
 * buffer of BRA_STATIC_SCRATCH_BYTES instead of a workspace. The call
 * allocates nothing.
 *
 * The buffer is one file-scope device array: each GPU the library runs on
 * holds its own copy until the process ends, and every call on that GPU
 * shares it (its contents are the last call's; nothing in it needs to start
 * at zero). Calls that overlap in time on one GPU (unordered streams, host
 * threads) race on it and give undefined results: order them. `stream` must
 * belong to the current device (BRA_EINVAL otherwise). Sizes whose
 * bra_workspace_bytes(...) exceeds BRA_STATIC_SCRATCH_BYTES give
 * BRA_ESCRATCH; every other check is bra_forward's.
 */
#define BRA_STATIC_SCRATCH_BYTES ((size_t)16 << 20)
bra_status bra_forward_static(const void* Q, const void* K, const void* V, void* O,
                              int B, int H, int W, int C, int heads, int S, int topk,
                              bra_dtype dtype, hipStream_t stream);

/*
 * Local context enhancement (LCE): the "+ dwconv(value)" term of the module
 * output (explainer Part 2.2 step 4, third bullet, and pseudocode step 7;
 * paper summary Section 3, the depthwise-convolution local context term):
 *
 *   lce[b, y, x, c] = bias[c] + sum_{i, j in 0..4} weight[c][i][j]
 *                                * V[b, y + i - 2, x + j - 2, c]
 *
 * over the whole H x W map with zero padding (terms outside the map are
 * dropped), stride 1, one 5 x 5 filter per channel (PyTorch's depthwise
 * Conv2d convention: cross-correlation, weight [C, 1, 5, 5] stored as
 * [C][5][5]).
 *
 *   weight : [C][5][5] in `dtype`, device memory, 4-byte aligned.
 *   bias   : [C] in `dtype`, device memory, or NULL for no bias.
 *   Neither may overlap O (BRA_EINVAL). A NULL weight gives BRA_EINVAL.
 *
 * Rounding: the attention output and the term are added in fp32 and rounded
 * once for bf16 regions of at most 8 x 8 tokens with at most 64 routed keys
 * per query (the term is fused into the attention kernel); otherwise
 * (fp32, larger regions, more keys) a second kernel adds the term to the
 * stored attention output, which for bf16 rounds twice.
 */

/* bra_attend_lce - bra_attend plus the local context term:
 * O = attention(Q, K, V; idx) + lce(V). Same arguments, checks and
 * streams as bra_attend, plus weight and bias. */
bra_status bra_attend_lce(const void* Q, const void* K, const void* V,
                          const int32_t* idx, const void* weight, const void* bias, void* O,
                          int B, int H, int W, int C, int heads, int S, int topk,
                          bra_dtype dtype, hipStream_t stream);

/* bra_forward_lce - the whole module output of explainer pseudocode steps
 * 1 and 3-7: bra_forward plus the local context term. Same arguments,
 * checks and streams as bra_forward, plus weight and bias, and a workspace
 * as in bra_forward_ws, except that NULL/0 asks for a stream-ordered
 * allocation as bra_forward makes; its routing table is bra_route's, bit
 * for bit. */
bra_status bra_forward_lce(const void* Q, const void* K, const void* V,
                           const void* weight, const void* bias, void* O,
                           int B, int H, int W, int C, int heads, int S, int topk,
                           bra_dtype dtype, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/*
 * Backward of the token attention, routing held fixed (the pages report
 * training throughput: explainer Part 7 and paper summary Appendix B; the
 * forward is explainer Part 2.2 step 4, pseudocode steps 6-7). The top-k
 * indices are not differentiable, so the region pooling receives no gradient.
 * For every image, region i and head m, with P = softmax(scale q k_g^T):
 *
 *   dV_g += P^T dO,  dZ = P * (dO V_g^T - rowsum(dO * O)),
 *   dQ = scale dZ K_g,  dK_g += scale dZ^T Q
 *
 * where K_g, V_g are the tokens of regions idx[b][i][.] and a token's dK, dV
 * sum over every query region routed to its region.
 *
 *   Q, K, V  : the forward inputs; O: the forward output (bra_attend /
 *              bra_forward with the same idx); dO: dL/dO. All [B, H, W, C]
 *              in `dtype`, 16-byte aligned, read only.
 *   idx      : the routing table of the forward, [B, S*S, topk] int32, with
 *              distinct entries per row (as bra_route writes them). A row
 *              with an entry outside [0, S*S), or with a repeated entry,
 *              makes that region's dQ NaN and its queries contribute
 *              nothing to dK, dV.
 *   dQ, dK, dV : outputs [B, H, W, C] in `dtype`, 16-byte aligned, not
 *              overlapping each other, the inputs or idx (BRA_EINVAL). Every
 *              element is written (tokens no region routes to get 0 in dK
 *              and dV).
 *   workspace  : bra_backward_workspace_bytes(...) bytes, 256-byte aligned,
 *              not overlapping any tensor argument, or NULL/0 for a
 *              stream-ordered allocation as in bra_forward.
 *
 * Deterministic: no atomics touch the gradients; fp32 accumulation.
 */
size_t bra_backward_workspace_bytes(int B, int H, int W, int C, int heads, int S, int topk);

bra_status bra_attend_backward(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                               const int32_t* idx, void* dQ, void* dK, void* dV,
                               int B, int H, int W, int C, int heads, int S, int topk,
                               bra_dtype dtype, void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

/*
 * The linear projection in front of the routing, with the region pooling
 * fused into its epilogue (explainer Part 2.2 steps 2-3 and pseudocode steps
 * 2-3; Part 3's 3HWC^2 projection term):
 *
 *   [Q | K | V] = X Wqkv^T + bqkv   (linear_qkv(x).chunk(3, dim=-1))
 *
 *   X      : [B, H, W, C] block input in `dtype`, 16-byte aligned.
 *   Wqkv   : [3C][C] in `dtype` (a torch Linear weight: row = output
 *            feature; Q's C features first, then K's, then V's), 16-byte
 *            aligned. bqkv: [3C] in `dtype` or NULL.
 *   Q, K, V: [B, H, W, C] outputs in `dtype`, 16-byte aligned, rounded once
 *            from fp32 accumulation.
 * Supported: C a multiple of 32, C <= 256 for bf16 and <= 128 for fp32
 * (BRA_EUNSUPPORTED otherwise).
 * Outputs may not overlap each other, X or the weights (BRA_EINVAL).
 */

/* bra_qkv_pool - Q, K, V and the region means Qr, Kr ([B, S*S, C] fp32,
 * 16-byte aligned, not overlapping) of the ROUNDED Q and K, i.e. what bra_route pools from the
 * stored Q and K (up to fp32 summation order), without reading them again. */
bra_status bra_qkv_pool(const void* X, const void* Wqkv, const void* bqkv, void* Q, void* K, void* V,
                        float* Qr, float* Kr, int B, int H, int W, int C, int S,
                        bra_dtype dtype, hipStream_t stream);

/* bra_forward_qkv - the module from its input: bra_qkv_pool into Q, K, V
 * (kept for the caller, e.g. for the backward) and the workspace's region
 * means, routing from those means, then attention into O. Workspace as in
 * bra_forward_lce (bra_workspace_bytes bytes, or NULL/0 for a stream-ordered
 * allocation); streams as bra_forward. */
bra_status bra_forward_qkv(const void* X, const void* Wqkv, const void* bqkv, void* Q, void* K, void* V, void* O,
                           int B, int H, int W, int C, int heads, int S, int topk,
                           bra_dtype dtype, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* BRA_H_ */
