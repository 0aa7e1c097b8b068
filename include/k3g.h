/*
 * k3g.h -- C ABI of libk3g, the MI355X (gfx950) routed-expert MXFP4 library.
 *
 * Sources of the operations (pages, with their sections):
 *   [KIC-README]  "kimi-k3-in-c" README (spark.entire.vc tools page)
 *   [KIC-ARTICLE] "kimi-k3-in-c: 2.78 trillion parameters, one CPU, 8 GB of RAM"
 *   [COLIBRI-K3]  "Kimi K3 engine (c/kimi_k3.c)" (colibri docs)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor pointer is a DEVICE pointer (HBM of the current HIP device)
 *    unless its comment says host. The caller owns all memory: weights,
 *    inputs, outputs and workspace. The compute calls allocate nothing and
 *    keep no state between calls. Three exceptions, each stated where it is
 *    declared: the expert cache object (k3g_cache_create allocates it on the
 *    host, and k3g_cache_prepare its pinned host staging on first use, both
 *    freed by k3g_cache_destroy); the static device scratch array of
 *    k3g_moe_layer_static (held by every GPU the library runs on); and the
 *    measurement hooks, which allocate nothing either.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Every call only enqueues work on `stream` and returns without
 *    synchronising. Results are valid once the stream reaches that point.
 *  - Arguments are validated on the host before anything is enqueued. A call
 *    that fails validation returns a negative k3g_status and enqueues
 *    nothing. Asynchronous device faults surface at the caller's next sync.
 *  - Preconditions that cannot be checked without a device sync are stated
 *    next to each call (e.g. idx values in [0, n_experts)).
 *  - Re-entrant. Calls that overlap on the device (other streams) must use
 *    distinct workspaces and outputs.
 *  - No dimension has a default: a zero or negative size where a positive
 *    one is needed is K3G_EINVAL ([KIC-README] "2. The config reader that
 *    refuses to guess": an absent field is an error, never a default).
 *  - An empty batch (n_tokens = 0) is not an error: the routing, layer,
 *    layer-stage and block calls check their other scalar arguments, then
 *    return K3G_OK with nothing enqueued; their data pointers and workspace
 *    may then be null (a torch tensor with no elements has none).
 *
 * MXFP4 matrix layout ([COLIBRI-K3] "Weights"; [KIC-ARTICLE] "Reduction one")
 * --------------------------------------------------------------------------
 *  W [rows x in], in a multiple of 32, is two row-major byte arrays:
 *    packed [rows][in/2]: e2m1 codes, two per byte, the LOW nibble is the even
 *                         column; bit 3 of a code is its sign;
 *    scales [rows][in/32]: one ue8m0 byte s per 32 columns;
 *  element value w = e2m1(code) * 2^(s-127); a group whose scale byte is 255
 *  contributes nothing. The weights are read in this form; nothing expands
 *  them to floats in HBM.
 */
#ifndef K3G_H
#define K3G_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    K3G_OK = 0,
    K3G_EINVAL = -1,       /* null pointer, bad size, bad enum, overlapping in/out */
    K3G_EALIGN = -2,       /* a pointer misses its required alignment            */
    K3G_ENOSPACE = -3,     /* workspace smaller than k3g_workspace_bytes()        */
    K3G_EHIP = -4,         /* a HIP launch or runtime call failed                 */
    K3G_EUNSUPPORTED = -5  /* shape beyond what the kernels handle, or not gfx950 */
} k3g_status;

/* EXACT: fp32 activations, exact e2m1 products, fp32 accumulation.
 * IDOT:  activations quantised per 32-group to int8, integer group dots
 *        ([COLIBRI-K3] "Streaming design", K3_IDOT), on the bf16 matrix cores
 *        by default (K3G_IDOT_BF16) or on the int8 ones (K3G_IDOT_INT8), with
 *        the same results bit for bit. The IDOT kernels need latent and inter
 *        to be multiples of 128 and the scale tensors 4-byte aligned
 *        (K3G_EUNSUPPORTED / K3G_EALIGN otherwise). */
typedef enum { K3G_EXACT = 0, K3G_IDOT = 1 } k3g_mode;

/* OR-ed into `mode` of the EXACT calls: decode the nibbles through the
 * byte-pair table held in LDS, the pages' decode ([KIC-ARTICLE] "Reduction
 * one", K3_E2M1_PAIR), instead of gfx950's FP4 -> FP32 convert instruction
 * (the default). Both give the same values: e2m1 codes are exact in either. */
#define K3G_DECODE_LUT 0x100

/* OR-ed into K3G_IDOT (the default form; the flag names it): the group dots
 * on the bf16 matrix cores. The int8 activations are widened to bf16 and the
 * e2m1 values carry their group's power-of-two scale (both exact), so each
 * group's fp32 result is exactly I * 2^(s-128) and the per-group epilogue is
 * one fma instead of a convert, a multiply and an fma. Results are identical
 * to the int8 form bit for bit; the workspace holds bf16 copies of xq and hq. */
#define K3G_IDOT_BF16 0x200

/* OR-ed into K3G_IDOT: the group dots on the int8 matrix cores
 * (v_mfma_i32_32x32x32_i8, int32 group sums, then a convert, a multiply and an
 * fma per result and group). K3G_IDOT_BF16 and K3G_IDOT_INT8 together are
 * K3G_EINVAL. */
#define K3G_IDOT_INT8 0x1000

/* Which kernels an EXACT layer runs on. With neither flag: the FP4 matrix
 * cores (below) for more than one token when the shape and the bank fit them,
 * the vector kernels otherwise (one token: the vector form is as fast and
 * needs no split of x). K3G_DECODE_MFMA asks for the matrix cores at any
 * token count, K3G_DECODE_VECTOR (or K3G_DECODE_LUT) for the vector kernels;
 * the two together are K3G_EINVAL. */
#define K3G_DECODE_VECTOR 0x800

/* OR-ed into K3G_EXACT: run the layer on the FP4 matrix cores instead of the
 * vector kernels. The products use v_mfma_scale_f32_16x16x128_f8f6f4 on the
 * stored nibbles and scales, with x and h written as sums of 16 e2m1 vectors
 * (one ue8m0 scale per 32 entries each, entries below 2^-127 dropped); every
 * product is exact and sums are fp32, as in the vector form, so both meet the
 * same bound. With more than one token each workgroup takes one expert's
 * sorted pairs 2, 4 or 8 at a time (by the average pairs per expert: below
 * 3, below 6, else), so each weight row is read once per pass.
 * Needs latent and inter multiples of 512 (at most 4096) and a bank with
 * 16-byte aligned scale tensors and stride; otherwise the vector kernels run. */
#define K3G_DECODE_MFMA 0x400

typedef struct {
    const uint8_t *packed; /* [rows][in/2], 16-byte aligned */
    const uint8_t *scales; /* [rows][in/32]                 */
    int32_t rows, in;
} k3g_mxfp4;

/* One routed expert: w1 (gate) and w3 (up) [inter x latent], w2 (down)
 * [latent x inter]. Which of w1/w3 is the gate is not stated on the pages;
 * w1 = gate is this library's reading. */
typedef struct {
    k3g_mxfp4 w1, w3, w2;
} k3g_expert;

/* A bank of experts resident in HBM. Expert e's six tensors are at
 * base + e*stride + off[i], i = w1 packed, w1 scales, w3 packed, w3 scales,
 * w2 packed, w2 scales (the pages store an expert's six tensors back to back,
 * [COLIBRI-K3] "Streaming design"). k3g_bank_layout() gives the packing this
 * library recommends; any offsets with 16-byte aligned packed tensors work. */
typedef struct {
    const uint8_t *base;
    int64_t stride;
    int32_t n_experts, latent, inter;
    int64_t off[6];
} k3g_expert_bank;

/* Dense bf16 weights of the LatentMoE block ([COLIBRI-K3] "Architecture
 * notes"): down [latent x hidden], up [hidden x latent], gamma [latent]
 * (fp32), shared experts w1/w3 [sh_inter x hidden] and w2 [hidden x sh_inter],
 * router [n_experts x hidden] fp32 and bias [n_experts] fp32. bf16 tensors
 * are uint16 bit patterns, row-major, 16-byte aligned. */
typedef struct {
    const float *w_router, *bias;
    const uint16_t *w_down, *w_up;
    const float *gamma;
    const uint16_t *sh_w1[2], *sh_w3[2], *sh_w2[2];
    int32_t n_shared, hidden, sh_inter;
    float rms_eps;
    k3g_expert_bank bank;
} k3g_block_weights;

/* Operation codes for the workspace queries. */
typedef enum {
    K3G_OP_EXPERT_GLU = 1,
    K3G_OP_MOE_ROUTE = 2,
    K3G_OP_MOE_LAYER = 3,
    K3G_OP_LATENT_BLOCK = 4
} k3g_op;

/* Sizes that fix a workspace. Fields an op does not use are ignored:
 * EXPERT_GLU uses latent, inter, mode; MOE_ROUTE uses n_tokens, n_experts;
 * MOE_LAYER adds top_k, latent, inter, mode; LATENT_BLOCK uses all. */
typedef struct {
    int32_t n_tokens, top_k, n_experts, latent, inter, hidden, sh_inter, mode;
} k3g_shape;

/* Byte offsets of the regions of a workspace, for the stage-by-stage checks
 * of a test (0 = region absent; every region is 256-byte aligned). P =
 * n_tokens * top_k pairs, sorted by (expert, token).
 *   logits  double [T][n_experts]        router logits; from 129 tokens up, where
 *           the product's K range is split across workgroups, the
 *           splits' partial sums follow in the same region
 *   counts  int32 [n_experts]            pairs per expert
 *   offsets int32 [n_experts+1]          exclusive prefix sum of counts
 *   perm    int32 [P]                    sorted position -> pair id t*top_k+k
 *   inv     int32 [P]                    pair id -> sorted position
 *   active  int32 [n_experts+1]          [0] = number of experts with pairs, then their ids ascending
 *   xq, xs  int8 [T][latent], float [T][latent/32]   IDOT activations
 *   h       float [P][inter]             SiTU output per sorted pair (EXACT only)
 *   hq, hs  int8 [P][inter], float [P][inter/32]      IDOT h, quantised by the
 *           up kernel (no fp32 h in IDOT; hq absent in the bf16 form, where
 *           hqb holds the same values)
 *   ypair   float [P][latent]            expert output per sorted pair, unweighted
 *   idx, wts int32/float [T][top_k]      block routing
 *   lat, agg, nrm  float [T][latent]     block stages
 *   shh     float [T][sh_inter]          block shared-expert SiTU output
 *   layer   the MoE layer's own workspace inside the block's
 *   xqb, hqb  uint16 (bf16) copies of xq and hq (the bf16 IDOT form only)
 *   xp, hp    layer with K3G_DECODE_MFMA: each token's x and each pair's h as
 *             16 e2m1 pieces, 1280 bytes per 128 entries (operand B of the
 *             instruction and its block scales)
 *   passes  int32 [1 + 2 * n]            K3G_DECODE_MFMA with more than one
 *             token: [0] = n, then (active slot, pass index) per pass, every
 *             expert's sorted pairs taken a few at a time
 *   dxh, dxl, dxs  block: the hidden state, the normalised aggregate and the
 *             shared experts' h as three bf16 pieces each (6 bytes per entry,
 *             tokens padded to a multiple of 64) for the dense products on the
 *             bf16 matrix cores; 0 where a product's shape keeps it on the
 *             fp32 fma kernels
 *   dpart   float  block: the dense products' K-slice partial sums */
typedef struct {
    size_t total;
    size_t logits, counts, offsets, perm, inv, active;
    size_t xq, xs, h, hq, hs, ypair;
    size_t idx, wts, lat, agg, nrm, shh, layer;
    size_t xqb, hqb;
    size_t xp, hp;
    size_t passes;
    size_t dxh, dxl, dxs, dpart;
} k3g_ws_layout;

/* Human-readable name of a status code (static storage). */
const char *k3g_status_string(int status);

/* Library version string and the device architecture it was built for. */
const char *k3g_version(void);

/* The recommended bank packing for experts of the given shape: six tensors
 * back to back, each 256-byte aligned. Writes off[6] and *stride (host
 * pointers). Returns K3G_OK or K3G_EINVAL. */
int k3g_bank_layout(int latent, int inter, int64_t off[6], int64_t *stride);

/* Workspace size in bytes for `op` at these sizes (0 when the arguments are
 * invalid), and the region offsets within it (host pointers). */
size_t k3g_workspace_bytes(int op, const k3g_shape *shape);
int k3g_workspace_layout(k3g_ws_layout *out, int op, const k3g_shape *shape);

/* ---- the hot path ------------------------------------------------------ */

/* y[r] = sum_g [s_rg != 255] 2^(s_rg-127) * sum_{j in g} e2m1(n_rj) * x_j
 * for one activation vector (batch 1): the pages' k3_matmul_mxfp4, same
 * argument order ([KIC-ARTICLE] "Reduction one"). y fp32 [rows], x fp32 [in].
 * group must be 32; in a positive multiple of 32; rows >= 1; packed 16-byte
 * aligned; x 16-byte and y 4-byte aligned; y must not overlap x. fp32
 * accumulation. */
int k3g_mxfp4_gemv(float *y, const float *x, const uint8_t *packed,
                   const uint8_t *scales, int in, int rows, int group, void *stream);

/* The same product with the nibbles decoded through the LDS byte-pair table
 * (see K3G_DECODE_LUT); same arguments, same results. */
int k3g_mxfp4_gemv_lut(float *y, const float *x, const uint8_t *packed,
                       const uint8_t *scales, int in, int rows, int group, void *stream);

/* The pages' Vulkan-tier format ([COLIBRI-K3] "Vulkan tier": e2m1 nibbles
 * uploaded as stored, ue8m0 exponents expanded to f32 per-32-group scales at
 * upload). k3g_mxfp4_scales_to_f32 expands n scale bytes: out = 2^(s-127)
 * exactly (s = 0 gives the subnormal 2^-127), 255 (skip) gives 0; out fp32 [n],
 * 4-byte aligned, not overlapping scales. k3g_mxfp4_gemv_f32s is
 * k3g_mxfp4_gemv with such scales (fp32 [rows][in/32], 4-byte aligned): each
 * group sum times its f32 scale. With finite x the results equal
 * k3g_mxfp4_gemv's bit for bit (both scalings are exact powers of two); a
 * skipped group contributes 0 * its sum, so a non-finite x in it propagates,
 * where the ue8m0 form drops the group. The f32 scales cost 3 more bytes per
 * group (20 instead of 17). */
int k3g_mxfp4_scales_to_f32(float *out, const uint8_t *scales, int64_t n, void *stream);
int k3g_mxfp4_gemv_f32s(float *y, const float *x, const uint8_t *packed, const float *scales,
                        int in, int rows, int group, void *stream);

/* One expert on one token: g = w1 x, u = w3 x, h = 4 tanh(g/4) sigmoid(g)
 * 25 tanh(u/25) (SiTU-GLU, [COLIBRI-K3] "Architecture notes"), y = w2 h.
 * y, x fp32 [latent], 16-byte aligned. In IDOT mode x and h are quantised per
 * 32-group to int8 first. ws: k3g_workspace_bytes(K3G_OP_EXPERT_GLU, ...) bytes,
 * 256-byte aligned. K3G_DECODE_LUT and the IDOT form flags apply; K3G_DECODE_MFMA
 * (a layer form) returns K3G_EUNSUPPORTED. */
int k3g_expert_glu(float *y, const float *x, const k3g_expert *e, int mode,
                   void *ws, size_t ws_bytes, void *stream);

/* Stable LatentMoE routing ([COLIBRI-K3] "Architecture notes"; [KIC-README]
 * "Three invariants", 3): logit = W_router x (double accumulation),
 * score = sigmoid(logit), biased = score + bias; the top_k experts by biased
 * score, largest first, equal scores to the lower id; wts = scores of the
 * selected experts / their sum. idx int32 [T][top_k], wts fp32 [T][top_k],
 * x fp32 [T][in], w_router fp32 [n_experts][in], bias fp32 [n_experts].
 * 1 <= top_k <= min(n_experts, 64); n_experts <= 4096. */
int k3g_moe_route(int32_t *idx, float *wts, const float *x, const float *w_router,
                  const float *bias, int n_tokens, int in, int n_experts, int top_k,
                  void *ws, size_t ws_bytes, void *stream);

/* The same routing with K3_TOPP ([COLIBRI-K3] "Streaming design" and its table
 * of environment variables: keep routed experts up to cumulative weight p,
 * drop the low-weight tail of the top-k, renormalise). This library's reading
 * of the steps the pages leave open: the top_k entries are ranked by weight,
 * largest first, equal weights in selection order; an entry is kept while the
 * weight ranked before it (summed in rank order, double) is below top_p, so
 * the entry that reaches top_p is kept; kept weights are the kept raw scores
 * renormalised over the kept set. idx and wts keep their [T][top_k] shape and
 * route order: a dropped entry is idx -1, wts 0 (k3g_moe_layer skips it, so
 * its expert is never read). top_p = 0 is k3g_moe_route; top_p outside
 * [0, 1] or NaN -> K3G_EINVAL. Same workspace as k3g_moe_route. */
int k3g_moe_route_topp(int32_t *idx, float *wts, const float *x, const float *w_router,
                       const float *bias, int n_tokens, int in, int n_experts, int top_k,
                       float top_p, void *ws, size_t ws_bytes, void *stream);

/* The MoE layer for given routing: y[t] = sum_k wts[t][k] * E_{idx[t][k]}(x_t)
 * with each expert a SiTU-GLU. Pairs are sorted by expert id so each selected
 * expert's weights stream from HBM once for all of its tokens ([COLIBRI-K3]
 * "Chunked prefill": each unique expert of a chunk is loaded once); the
 * weighted combine runs in k order per token. y, x fp32 [T][latent]; idx,
 * wts [T][top_k] as k3g_moe_route or k3g_moe_route_topp writes them: an idx
 * of -1 is a dropped entry and adds nothing (its expert is not read).
 * Precondition: every other idx value in [0, bank->n_experts) (not checked on
 * the device; the kernels drop any id outside it as they drop -1). */
int k3g_moe_layer(float *y, const float *x, const int32_t *idx, const float *wts,
                  const k3g_expert_bank *bank, int n_tokens, int top_k, int mode,
                  void *ws, size_t ws_bytes, void *stream);

/* The layer's stages, in the order k3g_moe_layer runs them. Each stage is
 * one kernel launch (stages a mode does not have enqueue nothing), so a
 * caller can place events between them to time each kernel:
 *   BUCKET   stable sort of the pairs by expert (counts, offsets, perm, inv, active)
 *   QUANT_X  IDOT: x -> xq, xs; K3G_DECODE_MFMA: x -> xp
 *   UP       per expert and row: g = w1 a, u = w3 a, h = SiTU(g, u) (IDOT:
 *            written quantised per 32-group, as the down product takes it)
 *   QUANT_H  enqueues nothing in every mode: the IDOT up-projection writes
 *            h quantised (hq or hqb, and hs) and the K3G_DECODE_MFMA one its
 *            pieces (hp) themselves; the stage is kept so that stage numbers
 *            stay fixed
 *   (BUCKET enqueues nothing for one token in EXACT mode: the up-projection
 *   ranks the route entries and writes the bucket itself.)
 *   DOWN     per expert and row: ypair = w2 h
 *   COMBINE  y[t] = sum_k wts[t][k] * ypair[inv[t*top_k+k]]
 * Arguments as k3g_moe_layer; every stage validates them the same way and
 * reads what the earlier stages left in ws. */
typedef enum {
    K3G_STAGE_BUCKET = 0,
    K3G_STAGE_QUANT_X = 1,
    K3G_STAGE_UP = 2,
    K3G_STAGE_QUANT_H = 3,
    K3G_STAGE_DOWN = 4,
    K3G_STAGE_COMBINE = 5
} k3g_stage;

int k3g_moe_layer_stage(int stage, float *y, const float *x, const int32_t *idx, const float *wts,
                        const k3g_expert_bank *bank, int n_tokens, int top_k, int mode,
                        void *ws, size_t ws_bytes, void *stream);

/* The full LatentMoE block ([COLIBRI-K3] "Architecture notes"): route on x,
 * lat = W_down x, agg = layer(lat), n = RMSNorm(agg) * gamma (eps =
 * w->rms_eps, 1e-5 in [KIC-README]'s config), out = W_up n +
 * sum_s W2_s SiTU(W1_s x, W3_s x) for the n_shared (0..2) shared experts,
 * added unweighted. out, x fp32 [T][hidden]; x 16-byte aligned. Every
 * product of a bf16 weight and an fp32 activation is exact and sums are fp32:
 * with hidden, latent and sh_inter multiples of 64 and the dense weights
 * 16-byte aligned the products run on the bf16 matrix cores, each activation
 * split exactly into three bf16 pieces (sums over K slices added in a fixed
 * order, so results do not depend on timing); otherwise on fp32 fma kernels.
 * top_k and the bank as for k3g_moe_layer; ws:
 * k3g_workspace_bytes(K3G_OP_LATENT_BLOCK, ...) with hidden and sh_inter set. */
int k3g_latent_moe_block(float *out, const float *x, const k3g_block_weights *w,
                         int n_tokens, int top_k, int mode, void *ws, size_t ws_bytes,
                         void *stream);

/* ---- the layer without a caller workspace --------------------------------- */

/* Bytes of the library's static scratch array (64 MiB). */
#define K3G_STATIC_SCRATCH_BYTES (64u << 20)

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops that forbid hipMalloc): k3g_moe_layer with its
 * workspace in a file-scope device array of K3G_STATIC_SCRATCH_BYTES that the
 * library holds on every GPU it runs on until the process ends. Same
 * arguments, kernels and results as k3g_moe_layer, without ws and ws_bytes;
 * allocates nothing. A shape whose k3g_workspace_bytes(K3G_OP_MOE_LAYER, ...)
 * exceeds the array returns K3G_ENOSPACE with nothing enqueued (at top_k 16:
 * 64 decode tokens in every mode). Every call on one GPU shares that GPU's
 * array: calls that overlap on the device (other streams, or other threads)
 * race, and the array keeps whatever the last call left in it (no call reads
 * what an earlier one left). The first call on a device looks up the array's
 * address there (that device current) and keeps it. */
int k3g_moe_layer_static(float *y, const float *x, const int32_t *idx, const float *wts,
                         const k3g_expert_bank *bank, int n_tokens, int top_k, int mode,
                         void *stream);
size_t k3g_static_scratch_bytes(void);

/* ---- the routed-expert cache: host memory -> HBM (streaming tier) -------- */

/* The pages stream experts from storage through an LRU of expert slots
 * ([KIC-ARTICLE] "The cache the project exists for"; [COLIBRI-K3] "Streaming
 * design"). Here the storage is host memory and the slots are an expert bank
 * in HBM (`arena`, arena->n_experts slots, any layout k3g_moe_layer accepts):
 * the cache rewrites a step's expert ids into slot ids, and k3g_moe_layer runs
 * on the arena with them. Policy: LRU with pinning; a miss takes the first
 * empty slot, else the least recently used slot that the step neither uses nor
 * fills and whose expert is not pinned (linear scan, equal ages to the lower
 * slot); slots taken by a step's prefetch are in flight (neither empty nor
 * evictable) until their copies are issued; misses are fetched in ascending
 * expert id (host-address) order; a request histogram per expert. All state
 * is host-side; the object is not thread-safe. */
typedef struct k3g_cache k3g_cache;

typedef struct {
    uint64_t steps, hits, misses, evictions, bytes_copied;
} k3g_cache_stats;

/* host_bank: host pointer (pinned memory copies fastest) holding n_total
 * experts at host_bank + e*arena->stride, each laid out as in the arena
 * (may be NULL for plan-only use); the arena's tensors must stay valid while
 * the cache lives. */
int k3g_cache_create(k3g_cache **out, const uint8_t *host_bank, int32_t n_total,
                     const k3g_expert_bank *arena);
void k3g_cache_destroy(k3g_cache *c);

/* Pin (1) or unpin (0) an expert: a pinned expert, once loaded, is never
 * evicted. */
int k3g_cache_pin(k3g_cache *c, int32_t expert, int pinned);

/* The policy alone (host pointers, no device work): for one step's routing
 * idx [T][top_k] (-1 = dropped entry) writes idx_slot [T][top_k] (slot ids,
 * -1 kept) and the copies the step needs, copy_expert/copy_slot [<= n_slots]
 * (may be NULL), *n_copies. The new slots stay in flight until
 * k3g_cache_complete (or the next plan). K3G_ENOSPACE, with nothing changed,
 * when the step's experts do not fit the unpinned slots. */
int k3g_cache_plan(k3g_cache *c, int32_t *idx_slot, int32_t *copy_expert, int32_t *copy_slot,
                   int32_t *n_copies, const int32_t *idx, int n_tokens, int top_k);
int k3g_cache_complete(k3g_cache *c);

/* Plan one step and enqueue it: idx is the step's routing on the host,
 * idx_slot a device int32 [T][top_k] that receives the slot ids. The copies
 * (one hipMemcpyAsync of arena->stride bytes per missing expert, then idx_slot)
 * go on copy_stream after everything already on `stream`; `stream` then waits
 * for them, so a k3g_moe_layer enqueued next on `stream` with idx_slot and the
 * arena sees the step's experts. Pinned host staging is allocated on first use
 * and kept by the cache. */
int k3g_cache_prepare(k3g_cache *c, int32_t *idx_slot, const int32_t *idx, int n_tokens, int top_k,
                      void *copy_stream, void *stream);

/* One decode token through the layer on the arena, with the expert copies
 * overlapped with the products, one expert at a time ([COLIBRI-K3] "Streaming
 * design", K3_PIPE: expert j's products run while expert j+1 is read). The
 * step is planned as k3g_cache_prepare plans it. On copy_stream, after the
 * work already on `stream`: each missing expert's copy (host-address order),
 * each followed by an event. On `stream`: the pairs whose experts are
 * resident first, in one up-projection (with SiTU) and one down-projection
 * launch over a pair table copied ahead of the experts, then each missing
 * expert's pair once its copy has landed (its own up and down launch), then
 * the weighted combine in k order; in IDOT mode x is quantised first. The result equals k3g_moe_layer on the arena
 * with the step's slot ids bit for bit.
 *   y, x: device float [latent] (16-byte aligned); idx: host int32 [top_k],
 *   expert ids (-1 = a dropped entry, K3_TOPP); wts: device float [top_k].
 *   mode: K3G_EXACT on the vector kernels (K3G_DECODE_VECTOR and
 *   K3G_DECODE_LUT allowed), or K3G_IDOT in either form (widths multiples of
 *   128); K3G_DECODE_MFMA is K3G_EUNSUPPORTED.
 *   ws: a k3g_moe_layer workspace for one token, top_k, the arena's shape and
 *   the same mode (256-byte aligned, ws_bytes >= k3g_workspace_bytes).
 * The host staging of the cache is reused: the call waits for the previous
 * step's host-to-device copy of it before planning. 1 <= top_k <= 64;
 * K3G_ENOSPACE as k3g_cache_plan, with nothing enqueued. */
int k3g_cache_decode_step(k3g_cache *c, float *y, const float *x, const int32_t *idx, const float *wts, int top_k,
                          int mode, void *ws, size_t ws_bytes, void *copy_stream, void *stream);

/* Counters, and optionally the expert -> slot map (int32 [n_total], -1 = not
 * resident) and the request histogram (uint64 [n_total]). */
int k3g_cache_query(const k3g_cache *c, k3g_cache_stats *stats, int32_t *slot_of, uint64_t *hist);

/* ---- stage hooks used by the bit-exact checks ----------------------------- */

/* Per row and 32-group: s = max|x|/127 (fp32), q = rint(x/s) clamped to
 * [-127, 127] with fp32 division and ties to even; max|x| = 0 gives s = 0,
 * q = 0. q int8 [n_rows][in], s fp32 [n_rows][in/32]. */
int k3g_quantize_i8_groups(int8_t *q, float *s, const float *x, int n_rows, int in,
                           void *stream);

/* Integer group sums of the IDOT product, computed on the matrix cores:
 * sums[t][r][g] = sum_{j in g} q[t][j] * 2*e2m1(n_rj), int32 [T][rows][in/32].
 * q int8 [T][in]. */
int k3g_mxfp4_idot_groupsums(int32_t *sums, const int8_t *q, const uint8_t *packed,
                             int in, int rows, int n_tokens, void *stream);

/* ---- measurement hooks (not part of the method) ---------------------------
 * What the chip sustains, as roofline denominators beside the datasheet peaks.
 * Each launches one kernel on `stream`; the caller times it. sink: a device
 * uint32 the kernel may store to (rarely; keeps the work from being removed).
 *
 * k3g_probe_mfma_rate: 2048 workgroups of 4 wavefronts, each wavefront
 * issuing `iters` rounds of 4 independent matrix products of one kind on
 * register operands, no memory traffic. kind 0: v_mfma_i32_32x32x32_i8
 * (65,536 ops each), 1: v_mfma_f32_16x16x32_bf16 (16,384 flops),
 * 2: v_mfma_scale_f32_16x16x128_f8f6f4 on fp4 (65,536 flops),
 * 3: v_mfma_f64_16x16x4_f64 (2,048 flops). Ops per launch =
 * 2048 * 4 * iters * 4 * ops-per-instruction. K3G_EINVAL for a kind outside
 * 0..3, iters < 1 or a null sink.
 * k3g_probe_read_rate: reads `bytes` (a multiple of 16, buf 16-byte aligned)
 * once with 16-byte loads, each wavefront taking 16 KB chunks in turn over
 * 8,192 workgroups (any tail smaller than a chunk grid-strided). K3G_EINVAL
 * otherwise. */
int k3g_probe_mfma_rate(int kind, int iters, uint32_t *sink, void *stream);
int k3g_probe_read_rate(const void *buf, size_t bytes, uint32_t *sink, void *stream);

/* k3g_probe_handoff: the cost of handing data from every workgroup of a launch
 * to one consumer. n_wg workgroups of 64 threads each store one float to
 * buf[i]; mode 0: nothing more (a launch of that grid); mode 1: a second,
 * dependent launch of one workgroup sums buf[0..n_wg) into buf[n_wg]; mode 2:
 * in the same launch, each workgroup releases at agent scope and adds one to
 * *counter, and the workgroup that adds last acquires, sums into buf[n_wg] and
 * sets *counter back to zero. buf float [n_wg + 1]; counter a device uint32
 * that is zero before the first mode-2 call (each call leaves it at zero).
 * 1 <= n_wg <= 65536; K3G_EINVAL otherwise. */
int k3g_probe_handoff(int mode, int n_wg, float *buf, uint32_t *counter, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* K3G_H */
