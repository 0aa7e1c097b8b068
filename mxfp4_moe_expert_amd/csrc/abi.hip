// abi.hip -- the extern "C" entry points of libk3g: validation, workspace
// layout, and the launch sequence of each operation. No entry point
// allocates, synchronises or copies to the host.
#include <stdio.h>
#include <string.h>

#include <algorithm>

#include "k3g_common.h"

namespace k3g {
// launchers (gemv.hip, route.hip, idot.hip)
int launch_gemv(float *y, const float *x, const uint8_t *packed, const uint8_t *scales, int in, int rows, bool lut,
                hipStream_t st);
int launch_moe_up_exact(float *h, const float *x, const BankDev &bank, const int32_t *active, const int32_t *offsets,
                        const int32_t *perm, int top_k, int latent, int inter, int max_slots, int n_pairs, bool lut,
                        const Route1 &rt, hipStream_t st);
int launch_moe_down_exact(float *ypair, const float *h, const BankDev &bank, const int32_t *active,
                          const int32_t *offsets, const int32_t *perm, int latent, int inter, int max_slots,
                          bool multi_pairs, bool lut, hipStream_t st);
int launch_combine(float *y, const float *ypair, const float *wts, const int32_t *inv, int n_tokens, int top_k,
                   int latent, hipStream_t st);
int launch_logits(double *logits, const float *x, const float *W, int T, int in, int E, hipStream_t st);
int logits_planes(int T, int E);
int launch_topk(int32_t *idx, float *wts, const double *logits, const float *bias, int T, int E, int K,
                double top_p, hipStream_t st);
int launch_bucket(int32_t *counts, int32_t *offsets, int32_t *perm, int32_t *inv, int32_t *active, const int32_t *idx,
                  int T, int K, int E, hipStream_t st, int32_t *passes = nullptr, int npp = 0);
int launch_quant_i8(int8_t *q, float *s, const float *x, int n_rows, int in, uint16_t *qb, hipStream_t st);
int launch_idot_groupsums(int32_t *sums, const int8_t *q, const uint8_t *packed, int in, int rows, int n_tokens,
                          hipStream_t st);
int launch_moe_up_idot(int8_t *hq, uint16_t *hqb, float *hs, const int8_t *xq, const uint16_t *xqb, const float *xs,
                       const BankDev &bank, const int32_t *active, const int32_t *offsets, const int32_t *perm,
                       int top_k, int latent, int inter, int max_slots, hipStream_t st);
int launch_moe_down_idot(float *ypair, const int8_t *hq, const uint16_t *hqb, const float *hs, const BankDev &bank, const int32_t *active,
                         const int32_t *offsets, const int32_t *perm, int latent, int inter, int max_slots,
                         hipStream_t st);
struct DenseSeg {
    const uint16_t *w;
    const float *x;
    int K;
};
int launch_dense(float *out, const DenseSeg *segs, int n_seg, int T, int N, hipStream_t st);
int launch_scales_f32(float *out, const uint8_t *s, int64_t n, hipStream_t st);
int launch_gemv_f32s(float *y, const float *x, const uint8_t *packed, const float *scales, int in, int rows,
                     hipStream_t st);
int launch_split(uint8_t *dst, const float *src, int n_vec, int len, int src_stride, hipStream_t st);
int launch_moe_up_f4(float *h, uint8_t *hp, const uint8_t *xp, const BankDev &bank, const Route1 &rt, int top_k,
                     int latent, int inter, int max_slots, hipStream_t st);
int launch_moe_down_f4(float *ypair, const uint8_t *hp, const BankDev &bank, const int32_t *active,
                       const int32_t *offsets, int latent, int inter, int max_slots, hipStream_t st);
int f4_pairs_per_pass(int n_pairs, int n_experts);
int launch_moe_up_f4m(float *h, uint8_t *hp, const uint8_t *xp, const BankDev &bank, const int32_t *active,
                      const int32_t *offsets, const int32_t *perm, const int32_t *passes, int npp, int top_k,
                      int latent, int inter, int n_pairs, int max_slots, hipStream_t st);
int launch_moe_down_f4m(float *ypair, const uint8_t *hp, const BankDev &bank, const int32_t *active,
                        const int32_t *offsets, const int32_t *passes, int npp, int latent, int inter, int n_pairs,
                        int max_slots, hipStream_t st);
bool f4_shape_ok(int latent, int inter);
bool f4_bank_ok(const BankDev &b);
int launch_dense_glu(float *h, const uint16_t *w1, const uint16_t *w3, const float *x, int T, int K, int N,
                     hipStream_t st);
int launch_rmsnorm(float *n, const float *a, const float *gamma, int T, int len, float eps, hipStream_t st);
int dense_t64(int T);
bool dense_mfma_ok(int T, int N, const int *K, int n_seg);
int dense_slices(int T, int N, int K_total, bool glu);
int launch_split3(uint8_t *xb, const float *x, int T, int K, int ld, hipStream_t st);
int launch_combine_norm(float *agg, float *nrm, uint8_t *xb, const float *ypair, const float *wts,
                        const int32_t *inv, const float *gamma, int T, int top_k, int len, float eps,
                        hipStream_t st);
int launch_dense_mfma(float *out, uint8_t *xb_out, float *part, const uint16_t *const *w, const uint8_t *const *xb,
                      const int *K, int n_seg, const uint16_t *w3, int T, int N, hipStream_t st, uint8_t *xp_out = nullptr);
}  // namespace k3g

using namespace k3g;

namespace {

constexpr int kMaxExperts = 2048;
constexpr int kMaxTopK = 64;

inline bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

inline bool overlap(const void *a, size_t na, const void *b, size_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

// The library is built for gfx950 only; refuse other devices once per device.
int check_device() {
    static int cached[64];  // 0 unknown, 1 ok, -1 not gfx950
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return K3G_EHIP;
    if (dev < 0 || dev >= 64) return K3G_EUNSUPPORTED;
    if (cached[dev] == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return K3G_EHIP;
        cached[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    }
    return cached[dev] == 1 ? K3G_OK : K3G_EUNSUPPORTED;
}

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

struct Carver {
    size_t cur = 0;
    size_t take(size_t bytes) {
        if (bytes == 0) return 0;
        cur = align_up(cur, 256);
        const size_t at = cur;
        cur += bytes;
        return at;
    }
};

constexpr int kFormFlags = K3G_DECODE_LUT | K3G_IDOT_BF16 | K3G_IDOT_INT8 | K3G_DECODE_MFMA | K3G_DECODE_VECTOR;
inline int base_mode(int mode) { return mode & ~kFormFlags; }
inline bool mode_ok(int mode) {
    if (mode & ~(kFormFlags | 0xFF)) return false;
    if ((mode & (K3G_IDOT_BF16 | K3G_IDOT_INT8)) && base_mode(mode) != K3G_IDOT) return false;
    if ((mode & K3G_IDOT_BF16) && (mode & K3G_IDOT_INT8)) return false;
    if ((mode & (K3G_DECODE_LUT | K3G_DECODE_MFMA | K3G_DECODE_VECTOR)) && base_mode(mode) != K3G_EXACT) return false;
    if ((mode & K3G_DECODE_MFMA) && (mode & (K3G_DECODE_LUT | K3G_DECODE_VECTOR))) return false;
    return base_mode(mode) == K3G_EXACT || base_mode(mode) == K3G_IDOT;
}
inline bool lut_of(int mode) { return (mode & K3G_DECODE_LUT) != 0; }
// EXACT layers run on the FP4 matrix cores when the shape fits them (the
// bank's alignment is checked where the bank is known): always with
// K3G_DECODE_MFMA, by default with more than one token (the faster form
// there), never with K3G_DECODE_VECTOR or K3G_DECODE_LUT (the vector kernels).
inline bool f4_layer(int mode, int n_tokens, int latent, int inter) {
    if (base_mode(mode) != K3G_EXACT || n_tokens < 1 || !f4_shape_ok(latent, inter)) return false;
    if (mode & (K3G_DECODE_VECTOR | K3G_DECODE_LUT)) return false;
    return (mode & K3G_DECODE_MFMA) || n_tokens > 1;
}
// The block's dense products on the bf16 matrix cores (x as three exact bf16
// pieces): the down-projection and the shared GLUs read the pieces of the
// hidden state, the up-projection those of the normalised aggregate and of
// the shared h. Each product takes that form when its shape allows; the
// workspace is sized for two shared experts.
struct DensePlan {
    bool down = false, glu = false, up = false;
    size_t part_floats = 0;  // the largest product's slices
};
inline DensePlan dense_plan(int T, int hidden, int latent, int sh_inter, int n_shared) {
    DensePlan d;
    if (T < 1) return d;
    const int kd[1] = {hidden};
    d.down = dense_mfma_ok(T, latent, kd, 1);
    d.glu = d.down && n_shared > 0 && dense_mfma_ok(T, sh_inter, kd, 1) && sh_inter % 64 == 0;
    const int ku[3] = {latent, sh_inter, sh_inter};
    d.up = latent % 64 == 0 && (n_shared == 0 || d.glu) && dense_mfma_ok(T, hidden, ku, 1 + n_shared);
    const size_t Ts = (size_t)T;
    if (d.down) d.part_floats = std::max(d.part_floats, dense_slices(T, latent, hidden, false) * Ts * latent);
    if (d.glu) d.part_floats = std::max(d.part_floats, dense_slices(T, sh_inter, hidden, true) * 2 * Ts * sh_inter);
    if (d.up)
        d.part_floats = std::max(
            d.part_floats, dense_slices(T, hidden, latent + n_shared * sh_inter, false) * Ts * hidden);
    return d;
}

// The IDOT kernels stage a row's scale bytes four groups at a time as aligned
// dwords: both widths must be multiples of 128 columns. The bf16 form addresses
// a row of its activations by a 32-bit byte offset: T rows of x and T*top_k
// rows of h, 2 bytes per element.
inline int idot_shape_ok(int mode, int latent, int inter, int n_tokens = 1, int top_k = 1) {
    if ((mode & 0xFF) != K3G_IDOT) return K3G_OK;
    if (latent % 128 || inter % 128) return K3G_EUNSUPPORTED;
    const int64_t P = (int64_t)n_tokens * top_k;
    if (P * inter * 2 >= ((int64_t)1 << 32) || (int64_t)n_tokens * latent * 2 >= ((int64_t)1 << 32))
        return K3G_EUNSUPPORTED;
    return K3G_OK;
}
// IDOT runs on the bf16 matrix cores unless K3G_IDOT_INT8 asks for the int8 ones
inline bool bf16_of(int mode) { return base_mode(mode) == K3G_IDOT && !(mode & K3G_IDOT_INT8); }

bool shape_ok_layer(const k3g_shape &s) {
    return s.n_tokens >= 0 && s.top_k >= 1 && s.top_k <= kMaxTopK && s.n_experts >= 1 &&
           s.n_experts <= kMaxExperts && s.top_k <= s.n_experts && s.latent > 0 && s.inter > 0 &&
           s.latent % kGroup == 0 && s.inter % kGroup == 0 && mode_ok(s.mode);
}

// The logits, and after them the partial planes of a K-split logits product.
inline size_t logits_bytes(int T, int E) {
    const size_t n = sizeof(double) * (size_t)(T > 0 ? T : 0) * E;
    const int planes = T > 0 ? logits_planes(T, E) : 1;
    return planes > 1 ? n * (1 + planes) : n;
}

// Regions are laid out from offset 256 so that 0 can mean "absent".
int layout(k3g_ws_layout *o, int op, const k3g_shape &s) {
    memset(o, 0, sizeof *o);
    Carver c;
    c.cur = 256;
    const size_t T = (size_t)(s.n_tokens > 0 ? s.n_tokens : 0);
    switch (op) {
        case K3G_OP_EXPERT_GLU: {
            if (s.latent <= 0 || s.inter <= 0 || s.latent % kGroup || s.inter % kGroup || !mode_ok(s.mode))
                return K3G_EINVAL;
            if (base_mode(s.mode) == K3G_IDOT) {  // h only quantised (the up kernel writes it so)
                o->xq = c.take((size_t)s.latent);
                o->xs = c.take(sizeof(float) * (s.latent / kGroup));
                o->hs = c.take(sizeof(float) * (s.inter / kGroup));
                if (bf16_of(s.mode)) {
                    o->xqb = c.take(sizeof(uint16_t) * s.latent);
                    o->hqb = c.take(sizeof(uint16_t) * s.inter);
                } else {
                    o->hq = c.take((size_t)s.inter);
                }
            } else {
                o->h = c.take(sizeof(float) * s.inter);
            }
            break;
        }
        case K3G_OP_MOE_ROUTE: {
            if (s.n_tokens < 0 || s.n_experts < 1 || s.n_experts > kMaxExperts) return K3G_EINVAL;
            o->logits = c.take(logits_bytes(s.n_tokens, s.n_experts));
            break;
        }
        case K3G_OP_MOE_LAYER:
        case K3G_OP_LATENT_BLOCK: {
            if (!shape_ok_layer(s)) return K3G_EINVAL;
            const size_t P = T * s.top_k, E = s.n_experts;
            if (op == K3G_OP_LATENT_BLOCK) {
                if (s.hidden <= 0 || s.sh_inter <= 0) return K3G_EINVAL;
                o->logits = c.take(logits_bytes(s.n_tokens, s.n_experts));
                o->idx = c.take(sizeof(int32_t) * P);
                o->wts = c.take(sizeof(float) * P);
                o->lat = c.take(sizeof(float) * T * s.latent);
                o->agg = c.take(sizeof(float) * T * s.latent);
                o->nrm = c.take(sizeof(float) * T * s.latent);
                o->shh = c.take(sizeof(float) * 2 * (T ? T : 1) * s.sh_inter);  // [2][T][sh_inter]
                const DensePlan dp = dense_plan(s.n_tokens, s.hidden, s.latent, s.sh_inter, 2);
                const size_t t64 = (size_t)dense_t64(s.n_tokens);
                if (dp.down) o->dxh = c.take(t64 * s.hidden * 6);
                if (dp.up) o->dxl = c.take(t64 * s.latent * 6);
                if (dp.glu) o->dxs = c.take(2 * t64 * s.sh_inter * 6);
                if (dp.part_floats) o->dpart = c.take(sizeof(float) * dp.part_floats);
            }
            o->counts = c.take(sizeof(int32_t) * E);
            o->offsets = c.take(sizeof(int32_t) * (E + 1));
            o->perm = c.take(sizeof(int32_t) * (P ? P : 1));
            o->inv = c.take(sizeof(int32_t) * (P ? P : 1));
            o->active = c.take(sizeof(int32_t) * (E + 1));
            if (base_mode(s.mode) != K3G_IDOT) o->h = c.take(sizeof(float) * (P ? P : 1) * s.inter);
            o->ypair = c.take(sizeof(float) * (P ? P : 1) * s.latent);
            if (base_mode(s.mode) == K3G_IDOT) {  // h only quantised (the up kernel writes it so)
                o->xq = c.take((T ? T : 1) * (size_t)s.latent);
                o->xs = c.take(sizeof(float) * (T ? T : 1) * (s.latent / kGroup));
                o->hs = c.take(sizeof(float) * (P ? P : 1) * (s.inter / kGroup));
                if (bf16_of(s.mode)) {
                    o->xqb = c.take(sizeof(uint16_t) * (T ? T : 1) * s.latent);
                    o->hqb = c.take(sizeof(uint16_t) * (P ? P : 1) * s.inter);
                } else {
                    o->hq = c.take((P ? P : 1) * (size_t)s.inter);
                }
            }
            if (f4_layer(s.mode, s.n_tokens, s.latent, s.inter)) {  // 10 bytes per entry
                o->xp = c.take(T * (size_t)s.latent / 128 * 1280);
                o->hp = c.take(P * (size_t)s.inter / 128 * 1280);
                // the pass table: each expert with pairs takes ceil(pairs / npp)
                // passes, fewer than P / npp + 1 per expert in all
                if (s.n_tokens > 1) {
                    const size_t npp = (size_t)f4_pairs_per_pass((int)P, s.n_experts);
                    o->passes = c.take(sizeof(int32_t) * (1 + 2 * ((P + npp - 1) / npp + std::min(P, E))));
                }
            }
            o->layer = 0;
            break;
        }
        default:
            return K3G_EINVAL;
    }
    o->total = align_up(c.cur, 256);
    return K3G_OK;
}

inline hipStream_t S(void *stream) { return (hipStream_t)stream; }

BankDev bank_dev(const k3g_expert_bank &b) {
    BankDev d;
    d.base = b.base;
    d.stride = b.stride;
    for (int i = 0; i < 6; ++i) d.off[i] = b.off[i];
    return d;
}

#define K3G_TRY(expr)               \
    do {                            \
        const int rc_ = (expr);     \
        if (rc_ != K3G_OK) return rc_; \
    } while (0)

int mxfp4_ok(const uint8_t *packed, const uint8_t *scales, int in, int rows) {
    if (!packed || !scales || in <= 0 || rows < 1 || in % kGroup) return K3G_EINVAL;
    if (!aligned(packed, 16)) return K3G_EALIGN;
    if (in / kGroup > 256) return K3G_EUNSUPPORTED;  // x must fit a wavefront's registers
    return K3G_OK;
}

}  // namespace

namespace k3g {
// the device check, for the entry points of the other sources (cache.hip)
int device_ok() { return check_device(); }
}  // namespace k3g

extern "C" {

const char *k3g_status_string(int status) {
    switch (status) {
        case K3G_OK: return "ok";
        case K3G_EINVAL: return "invalid argument";
        case K3G_EALIGN: return "misaligned pointer";
        case K3G_ENOSPACE: return "workspace too small";
        case K3G_EHIP: return "HIP error";
        case K3G_EUNSUPPORTED: return "unsupported shape or device";
        default: return "unknown status";
    }
}

const char *k3g_version(void) { return "k3g 0.1 (gfx950)"; }

int k3g_bank_layout(int latent, int inter, int64_t off[6], int64_t *stride) {
    if (!off || !stride || latent <= 0 || inter <= 0 || latent % kGroup || inter % kGroup) return K3G_EINVAL;
    Carver c;
    const size_t up_p = (size_t)inter * latent / 2, up_s = (size_t)inter * (latent / kGroup);
    const size_t dn_p = (size_t)latent * inter / 2, dn_s = (size_t)latent * (inter / kGroup);
    off[0] = (int64_t)c.take(up_p);
    off[1] = (int64_t)c.take(up_s);
    off[2] = (int64_t)c.take(up_p);
    off[3] = (int64_t)c.take(up_s);
    off[4] = (int64_t)c.take(dn_p);
    off[5] = (int64_t)c.take(dn_s);
    *stride = (int64_t)align_up(c.cur, 256);
    return K3G_OK;
}

size_t k3g_workspace_bytes(int op, const k3g_shape *shape) {
    if (!shape) return 0;
    k3g_ws_layout o;
    return layout(&o, op, *shape) == K3G_OK ? o.total : 0;
}

int k3g_workspace_layout(k3g_ws_layout *out, int op, const k3g_shape *shape) {
    if (!out || !shape) return K3G_EINVAL;
    return layout(out, op, *shape);
}

static int gemv_entry(float *y, const float *x, const uint8_t *packed, const uint8_t *scales, int in, int rows,
                      int group, bool lut, void *stream) {
    if (!y || !x || group != kGroup) return K3G_EINVAL;
    K3G_TRY(mxfp4_ok(packed, scales, in, rows));
    if (!aligned(x, 16) || !aligned(y, 4)) return K3G_EALIGN;
    if (overlap(y, sizeof(float) * rows, x, sizeof(float) * in)) return K3G_EINVAL;
    if ((int64_t)rows * (in / 2) >= ((int64_t)1 << 31)) return K3G_EUNSUPPORTED;  // 32-bit buffer offsets
    K3G_TRY(check_device());
    return launch_gemv(y, x, packed, scales, in, rows, lut, S(stream));
}

int k3g_mxfp4_gemv(float *y, const float *x, const uint8_t *packed, const uint8_t *scales, int in, int rows,
                   int group, void *stream) {
    return gemv_entry(y, x, packed, scales, in, rows, group, false, stream);
}

int k3g_mxfp4_gemv_lut(float *y, const float *x, const uint8_t *packed, const uint8_t *scales, int in, int rows,
                       int group, void *stream) {
    return gemv_entry(y, x, packed, scales, in, rows, group, true, stream);
}

int k3g_mxfp4_scales_to_f32(float *out, const uint8_t *scales, int64_t n, void *stream) {
    if (!out || !scales || n < 0) return K3G_EINVAL;
    if (!aligned(out, 4)) return K3G_EALIGN;
    if (n > 0 && overlap(out, sizeof(float) * (size_t)n, scales, (size_t)n)) return K3G_EINVAL;
    K3G_TRY(check_device());
    return launch_scales_f32(out, scales, n, S(stream));
}

int k3g_mxfp4_gemv_f32s(float *y, const float *x, const uint8_t *packed, const float *scales, int in, int rows,
                        int group, void *stream) {
    if (!y || !x || group != kGroup) return K3G_EINVAL;
    K3G_TRY(mxfp4_ok(packed, (const uint8_t *)scales, in, rows));
    if (!aligned(x, 16) || !aligned(y, 4) || !aligned(scales, 4)) return K3G_EALIGN;
    if (overlap(y, sizeof(float) * rows, x, sizeof(float) * in)) return K3G_EINVAL;
    if ((int64_t)rows * (in / 2) >= ((int64_t)1 << 31) || (int64_t)rows * (in / kGroup) * 4 >= ((int64_t)1 << 31))
        return K3G_EUNSUPPORTED;  // 32-bit buffer offsets
    K3G_TRY(check_device());
    return launch_gemv_f32s(y, x, packed, scales, in, rows, S(stream));
}

int k3g_quantize_i8_groups(int8_t *q, float *s, const float *x, int n_rows, int in, void *stream) {
    if (!q || !s || !x || n_rows < 0 || in <= 0 || in % kGroup) return K3G_EINVAL;
    if (!aligned(x, 16) || !aligned(q, 16) || !aligned(s, 4)) return K3G_EALIGN;
    K3G_TRY(check_device());
    return launch_quant_i8(q, s, x, n_rows, in, nullptr, S(stream));
}

int k3g_mxfp4_idot_groupsums(int32_t *sums, const int8_t *q, const uint8_t *packed, int in, int rows, int n_tokens,
                             void *stream) {
    if (!sums || !q || !packed || in <= 0 || in % kGroup || rows < 1 || n_tokens < 0) return K3G_EINVAL;
    if (!aligned(packed, 16) || !aligned(q, 16) || !aligned(sums, 4)) return K3G_EALIGN;
    K3G_TRY(check_device());
    return launch_idot_groupsums(sums, q, packed, in, rows, n_tokens, S(stream));
}

int k3g_expert_glu(float *y, const float *x, const k3g_expert *e, int mode, void *ws, size_t ws_bytes,
                   void *stream) {
    if (!y || !x || !e || !ws) return K3G_EINVAL;
    // the matrix-core form is a layer form (its work is cut by pairs and
    // experts); one expert runs on the vector kernels, so the flag is refused
    if (mode & K3G_DECODE_MFMA) return K3G_EUNSUPPORTED;
    const int latent = e->w1.in, inter = e->w1.rows;
    if (e->w3.in != latent || e->w3.rows != inter || e->w2.in != inter || e->w2.rows != latent) return K3G_EINVAL;
    K3G_TRY(mxfp4_ok(e->w1.packed, e->w1.scales, latent, inter));
    K3G_TRY(mxfp4_ok(e->w3.packed, e->w3.scales, latent, inter));
    K3G_TRY(mxfp4_ok(e->w2.packed, e->w2.scales, inter, latent));
    if (!aligned(x, 16) || !aligned(y, 16) || !aligned(ws, 256)) return K3G_EALIGN;
    if (overlap(y, sizeof(float) * latent, x, sizeof(float) * latent)) return K3G_EINVAL;
    k3g_shape s = {1, 1, 1, latent, inter, 0, 0, mode};
    k3g_ws_layout L;
    K3G_TRY(layout(&L, K3G_OP_EXPERT_GLU, s));
    K3G_TRY(idot_shape_ok(mode, latent, inter));
    if ((mode & 0xFF) == K3G_IDOT &&
        (!aligned(e->w1.scales, 4) || !aligned(e->w3.scales, 4) || !aligned(e->w2.scales, 4)))
        return K3G_EALIGN;
    if (ws_bytes < L.total) return K3G_ENOSPACE;
    K3G_TRY(check_device());
    // the expert as a one-expert bank: offsets relative to w1's packed bytes
    BankDev b;
    b.base = e->w1.packed;
    b.stride = 0;
    b.off[W1P] = 0;
    b.off[W1S] = e->w1.scales - e->w1.packed;
    b.off[W3P] = e->w3.packed - e->w1.packed;
    b.off[W3S] = e->w3.scales - e->w1.packed;
    b.off[W2P] = e->w2.packed - e->w1.packed;
    b.off[W2S] = e->w2.scales - e->w1.packed;
    char *w = (char *)ws;
    float *h = L.h ? (float *)(w + L.h) : nullptr;
    hipStream_t st = S(stream);
    if (base_mode(mode) == K3G_EXACT) {
        K3G_TRY(launch_moe_up_exact(h, x, b, nullptr, nullptr, nullptr, 1, latent, inter, 1, 1, lut_of(mode), Route1{},
                                    st));
        return launch_moe_down_exact(y, h, b, nullptr, nullptr, nullptr, latent, inter, 1, false, lut_of(mode), st);
    }
    int8_t *xq = (int8_t *)(w + L.xq), *hq = L.hq ? (int8_t *)(w + L.hq) : nullptr;
    float *xs = (float *)(w + L.xs), *hs = (float *)(w + L.hs);
    uint16_t *xqb = L.xqb ? (uint16_t *)(w + L.xqb) : nullptr, *hqb = L.hqb ? (uint16_t *)(w + L.hqb) : nullptr;
    K3G_TRY(launch_quant_i8(xq, xs, x, 1, latent, xqb, st));
    K3G_TRY(launch_moe_up_idot(hq, hqb, hs, xq, xqb, xs, b, nullptr, nullptr, nullptr, 1, latent, inter, 1, st));
    return launch_moe_down_idot(y, hq, hqb, hs, b, nullptr, nullptr, nullptr, latent, inter, 1, st);
}

int k3g_moe_route(int32_t *idx, float *wts, const float *x, const float *w_router, const float *bias, int n_tokens,
                  int in, int n_experts, int top_k, void *ws, size_t ws_bytes, void *stream) {
    return k3g_moe_route_topp(idx, wts, x, w_router, bias, n_tokens, in, n_experts, top_k, 0.0f, ws, ws_bytes,
                              stream);
}

int k3g_moe_route_topp(int32_t *idx, float *wts, const float *x, const float *w_router, const float *bias,
                       int n_tokens, int in, int n_experts, int top_k, float top_p, void *ws, size_t ws_bytes,
                       void *stream) {
    if (!(top_p >= 0.0f && top_p <= 1.0f)) return K3G_EINVAL;  // NaN too
    if (n_tokens < 0 || in <= 0 || n_experts < 1 || n_experts > kMaxExperts || top_k < 1 || top_k > kMaxTopK ||
        top_k > n_experts)
        return K3G_EINVAL;
    if (n_tokens == 0) return K3G_OK;  // nothing to route; the pointers may be null
    if (!idx || !wts || !x || !w_router || !bias || !ws) return K3G_EINVAL;
    if (!aligned(x, 4) || !aligned(w_router, 4) || !aligned(ws, 256) || !aligned(idx, 4) || !aligned(wts, 4))
        return K3G_EALIGN;
    k3g_shape s = {n_tokens, top_k, n_experts, 0, 0, 0, 0, 0};
    k3g_ws_layout L;
    K3G_TRY(layout(&L, K3G_OP_MOE_ROUTE, s));
    if (ws_bytes < L.total) return K3G_ENOSPACE;
    K3G_TRY(check_device());
    double *logits = (double *)((char *)ws + L.logits);
    hipStream_t st = S(stream);
    K3G_TRY(launch_logits(logits, x, w_router, n_tokens, in, n_experts, st));
    return launch_topk(idx, wts, logits, bias, n_tokens, n_experts, top_k, (double)top_p, st);
}

static int layer_prepare(k3g_ws_layout *L, const float *y, const float *x, const int32_t *idx, const float *wts,
                         const k3g_expert_bank *bank, int n_tokens, int top_k, int mode, void *ws, size_t ws_bytes) {
    if (!bank || n_tokens < 0) return K3G_EINVAL;
    const int latent = bank->latent, inter = bank->inter, E = bank->n_experts;
    k3g_shape s = {n_tokens, top_k, E, latent, inter, 0, 0, mode};
    K3G_TRY(layout(L, K3G_OP_MOE_LAYER, s));
    if (n_tokens == 0) return K3G_OK;  // the stages launch nothing; the pointers may be null
    if (!y || !x || !idx || !wts || !bank->base || !ws) return K3G_EINVAL;
    if (ws_bytes < L->total) return K3G_ENOSPACE;
    if (!aligned(x, 16) || !aligned(y, 16) || !aligned(ws, 256) || !aligned(idx, 4) || !aligned(wts, 4))
        return K3G_EALIGN;
    if (latent / kGroup > 256 || inter / kGroup > 256) return K3G_EUNSUPPORTED;
    K3G_TRY(idot_shape_ok(mode, latent, inter, n_tokens, top_k));
    for (int i = 0; i < 6; i += 2)
        if (!aligned(bank->base + bank->off[i], 16) || bank->stride % 16) return K3G_EALIGN;
    for (int i = 1; i < 6; i += 2)
        if (!aligned(bank->base + bank->off[i], 4)) return K3G_EALIGN;
    if (n_tokens > 0 && overlap(y, sizeof(float) * n_tokens * latent, x, sizeof(float) * n_tokens * latent))
        return K3G_EINVAL;
    return check_device();
}

// One stage of the layer: exactly one kernel launch (none for stages the mode
// does not have).
static int layer_stage(int stage, const k3g_ws_layout &L, float *y, const float *x, const int32_t *idx,
                       const float *wts, const k3g_expert_bank *bank, int n_tokens, int top_k, int mode, void *ws,
                       hipStream_t st) {
    if (n_tokens == 0) return K3G_OK;
    const int latent = bank->latent, inter = bank->inter, E = bank->n_experts;
    char *w = (char *)ws;
    int32_t *counts = (int32_t *)(w + L.counts), *offsets = (int32_t *)(w + L.offsets);
    int32_t *perm = (int32_t *)(w + L.perm), *inv = (int32_t *)(w + L.inv), *active = (int32_t *)(w + L.active);
    float *h = L.h ? (float *)(w + L.h) : nullptr, *ypair = (float *)(w + L.ypair);
    int8_t *xq = (int8_t *)(w + L.xq), *hq = L.hq ? (int8_t *)(w + L.hq) : nullptr;
    float *xs = (float *)(w + L.xs), *hs = (float *)(w + L.hs);
    uint16_t *xqb = L.xqb ? (uint16_t *)(w + L.xqb) : nullptr, *hqb = L.hqb ? (uint16_t *)(w + L.hqb) : nullptr;
    const int P = n_tokens * top_k;
    const int max_slots = P < E ? P : E;
    const BankDev b = bank_dev(*bank);
    // One token in EXACT mode: the up-projection ranks the route entries itself
    // and writes the bucket, so the bucket stage launches nothing.
    const bool route1 = n_tokens == 1 && base_mode(mode) == K3G_EXACT;
    const Route1 r1 = route1 ? Route1{idx, counts, offsets, perm, inv, active, E} : Route1{};
    // on the FP4 matrix cores x and h are split into e2m1 pieces first; more
    // than one token: the bucket also writes the table of (expert, pairs) passes
    const bool f4 = f4_layer(mode, n_tokens, latent, inter) && f4_bank_ok(b) && L.xp && L.hp;
    const bool f4m = f4 && n_tokens > 1 && L.passes;
    uint8_t *xp = (uint8_t *)(w + L.xp), *hp = (uint8_t *)(w + L.hp);
    int32_t *passes = f4m ? (int32_t *)(w + L.passes) : nullptr;
    const int npp = f4_pairs_per_pass(P, E);
    if (f4 && n_tokens > 1 && !f4m) return K3G_EINVAL;  // a layout without the pass table
    switch (stage) {
        case K3G_STAGE_BUCKET:
            return route1 ? K3G_OK
                          : launch_bucket(counts, offsets, perm, inv, active, idx, n_tokens, top_k, E, st, passes, npp);
        case K3G_STAGE_QUANT_X:
            if (f4) return launch_split(xp, x, n_tokens, latent, latent, st);
            return base_mode(mode) == K3G_IDOT ? launch_quant_i8(xq, xs, x, n_tokens, latent, xqb, st) : K3G_OK;
        case K3G_STAGE_UP:
            if (f4m)
                return launch_moe_up_f4m(h, hp, xp, b, active, offsets, perm, passes, npp, top_k, latent, inter, P,
                                         max_slots, st);
            if (f4) return launch_moe_up_f4(h, hp, xp, b, r1, top_k, latent, inter, max_slots, st);
            return base_mode(mode) == K3G_IDOT
                       ? launch_moe_up_idot(hq, hqb, hs, xq, xqb, xs, b, active, offsets, perm, top_k, latent, inter,
                                            max_slots, st)
                       : launch_moe_up_exact(h, x, b, active, offsets, perm, top_k, latent, inter, max_slots, P,
                                             lut_of(mode), r1, st);
        case K3G_STAGE_QUANT_H:
            // nothing to launch: the FP4 matrix-core up-projection writes hp, and the
            // IDOT up-projection writes hq (or hqb) and hs, itself
            return K3G_OK;
        case K3G_STAGE_DOWN:
            if (f4m)
                return launch_moe_down_f4m(ypair, hp, b, active, offsets, passes, npp, latent, inter, P, max_slots,
                                           st);
            if (f4) return launch_moe_down_f4(ypair, hp, b, active, offsets, latent, inter, max_slots, st);
            return base_mode(mode) == K3G_IDOT
                       ? launch_moe_down_idot(ypair, hq, hqb, hs, b, active, offsets, perm, latent, inter, max_slots, st)
                       : launch_moe_down_exact(ypair, h, b, active, offsets, perm, latent, inter, max_slots,
                                               n_tokens > 1, lut_of(mode), st);
        case K3G_STAGE_COMBINE:
            return launch_combine(y, ypair, wts, inv, n_tokens, top_k, latent, st);
        default:
            return K3G_EINVAL;
    }
}

int k3g_moe_layer_stage(int stage, float *y, const float *x, const int32_t *idx, const float *wts,
                        const k3g_expert_bank *bank, int n_tokens, int top_k, int mode, void *ws, size_t ws_bytes,
                        void *stream) {
    if (stage < K3G_STAGE_BUCKET || stage > K3G_STAGE_COMBINE) return K3G_EINVAL;
    k3g_ws_layout L;
    K3G_TRY(layer_prepare(&L, y, x, idx, wts, bank, n_tokens, top_k, mode, ws, ws_bytes));
    return layer_stage(stage, L, y, x, idx, wts, bank, n_tokens, top_k, mode, ws, S(stream));
}

int k3g_moe_layer(float *y, const float *x, const int32_t *idx, const float *wts, const k3g_expert_bank *bank,
                  int n_tokens, int top_k, int mode, void *ws, size_t ws_bytes, void *stream) {
    k3g_ws_layout L;
    K3G_TRY(layer_prepare(&L, y, x, idx, wts, bank, n_tokens, top_k, mode, ws, ws_bytes));
    for (int stage = K3G_STAGE_BUCKET; stage <= K3G_STAGE_COMBINE; ++stage)
        K3G_TRY(layer_stage(stage, L, y, x, idx, wts, bank, n_tokens, top_k, mode, ws, S(stream)));
    return K3G_OK;
}

}  // extern "C"

extern "C" int k3g_latent_moe_block(float *out, const float *x, const k3g_block_weights *w, int n_tokens, int top_k,
                                    int mode, void *ws, size_t ws_bytes, void *stream) {
    if (!w || n_tokens < 0) return K3G_EINVAL;
    if (w->n_shared < 0 || w->n_shared > 2 || !(w->rms_eps >= 0.0f)) return K3G_EINVAL;
    if (n_tokens == 0) return K3G_OK;  // nothing to do; out, x and ws may be null
    if (!out || !x || !ws || !w->w_router || !w->bias || !w->w_down || !w->w_up || !w->gamma || !w->bank.base)
        return K3G_EINVAL;
    for (int i = 0; i < w->n_shared; ++i)
        if (!w->sh_w1[i] || !w->sh_w3[i] || !w->sh_w2[i]) return K3G_EINVAL;
    const k3g_expert_bank *bank = &w->bank;
    const int T = n_tokens, E = bank->n_experts, latent = bank->latent, inter = bank->inter;
    const int hidden = w->hidden, sh_inter = w->n_shared ? w->sh_inter : 32;
    k3g_shape s = {T, top_k, E, latent, inter, hidden, sh_inter, mode};
    k3g_ws_layout L;
    K3G_TRY(layout(&L, K3G_OP_LATENT_BLOCK, s));
    if (ws_bytes < L.total) return K3G_ENOSPACE;
    if (!aligned(x, 16) || !aligned(out, 4) || !aligned(ws, 256) || !aligned(w->w_router, 16)) return K3G_EALIGN;
    if (latent / kGroup > 256 || inter / kGroup > 256) return K3G_EUNSUPPORTED;
    K3G_TRY(idot_shape_ok(mode, latent, inter, T, top_k));
    for (int i = 0; i < 6; i += 2)
        if (!aligned(bank->base + bank->off[i], 16) || bank->stride % 16) return K3G_EALIGN;
    for (int i = 1; i < 6; i += 2)
        if (!aligned(bank->base + bank->off[i], 4)) return K3G_EALIGN;
    if (T > 0 && overlap(out, sizeof(float) * T * hidden, x, sizeof(float) * T * hidden)) return K3G_EINVAL;
    K3G_TRY(check_device());
    if (T == 0) return K3G_OK;
    char *b = (char *)ws;
    double *logits = (double *)(b + L.logits);
    int32_t *idx = (int32_t *)(b + L.idx);
    float *wts = (float *)(b + L.wts);
    float *lat = (float *)(b + L.lat), *agg = (float *)(b + L.agg), *nrm = (float *)(b + L.nrm);
    float *shh = (float *)(b + L.shh);
    hipStream_t st = S(stream);
    // routing on the hidden state
    K3G_TRY(launch_logits(logits, x, w->w_router, T, hidden, E, st));
    K3G_TRY(launch_topk(idx, wts, logits, w->bias, T, E, top_k, 0.0, st));
    // the dense products: bf16 matrix cores where the plan allows (and the
    // workspace has the regions), the fp32 fma kernels otherwise
    DensePlan dp = dense_plan(T, hidden, latent, sh_inter, w->n_shared);
    bool al = aligned(w->w_down, 16) && aligned(w->w_up, 16);
    for (int i = 0; i < w->n_shared; ++i)
        al = al && aligned(w->sh_w1[i], 16) && aligned(w->sh_w3[i], 16) && aligned(w->sh_w2[i], 16);
    dp.down = dp.down && al && L.dxh && L.dpart;
    dp.glu = dp.glu && dp.down && L.dxs;
    dp.up = dp.up && al && L.dxl && L.dpart && (w->n_shared == 0 || dp.glu);
    uint8_t *dxh = (uint8_t *)(b + L.dxh), *dxl = (uint8_t *)(b + L.dxl), *dxs = (uint8_t *)(b + L.dxs);
    float *dpart = (float *)(b + L.dpart);
    const size_t t64 = (size_t)dense_t64(T);
    // does the routed layer split lat into e2m1 pieces (FP4 matrix cores)?
    const bool f4x = dp.down && T > 1 && f4_layer(mode, T, latent, bank->inter) && f4_bank_ok(bank_dev(*bank)) &&
                     L.xp && L.hp && L.passes && latent % 128 == 0;
    uint8_t *xp = (uint8_t *)(b + L.xp);
    // down-projection into the latent space
    if (dp.down) {
        K3G_TRY(launch_split3(dxh, x, T, hidden, hidden, st));
        const uint16_t *wd[1] = {w->w_down};
        const uint8_t *xd[1] = {dxh};
        const int kd[1] = {hidden};
        // the FP4 layer's e2m1 pieces of lat from the same reduction (its
        // split stage then has nothing to do)
        K3G_TRY(launch_dense_mfma(lat, nullptr, dpart, wd, xd, kd, 1, nullptr, T, latent, st, f4x ? xp : nullptr));
    } else {
        const DenseSeg down = {w->w_down, x, hidden};
        K3G_TRY(launch_dense(lat, &down, 1, T, latent, st));
    }
    // the routed experts on the latent tokens; on the matrix-core path their
    // combine, the RMSNorm of the aggregate and the pieces of the normed
    // aggregate for the up-projection are one kernel
    const bool fused = dp.up && latent % 32 == 0 && latent <= 4096;
    const int last = fused ? K3G_STAGE_DOWN : K3G_STAGE_COMBINE;
    for (int stage = K3G_STAGE_BUCKET; stage <= last; ++stage)
        if (!(f4x && stage == K3G_STAGE_QUANT_X))
            K3G_TRY(layer_stage(stage, L, agg, lat, idx, wts, bank, T, top_k, mode, ws, st));
    if (fused) {
        K3G_TRY(launch_combine_norm(agg, nrm, dxl, (const float *)(b + L.ypair), wts, (const int32_t *)(b + L.inv),
                                    w->gamma, T, top_k, latent, w->rms_eps, st));
    } else {
        K3G_TRY(launch_rmsnorm(nrm, agg, w->gamma, T, latent, w->rms_eps, st));
    }
    // the shared experts and the up-projection
    if (dp.up) {
        if (!fused) K3G_TRY(launch_split3(dxl, nrm, T, latent, latent, st));
        const uint16_t *wu[3] = {w->w_up, nullptr, nullptr};
        const uint8_t *xu[3] = {dxl, nullptr, nullptr};
        int ku[3] = {latent, 0, 0};
        for (int i = 0; i < w->n_shared; ++i) {
            float *h = shh + (size_t)i * T * sh_inter;
            uint8_t *hp = dxs + (size_t)i * t64 * sh_inter * 6;
            const uint16_t *w1[1] = {w->sh_w1[i]};
            const uint8_t *x1[1] = {dxh};
            const int k1[1] = {hidden};
            K3G_TRY(launch_dense_mfma(h, hp, dpart, w1, x1, k1, 1, w->sh_w3[i], T, sh_inter, st));
            wu[1 + i] = w->sh_w2[i];
            xu[1 + i] = hp;
            ku[1 + i] = sh_inter;
        }
        return launch_dense_mfma(out, nullptr, dpart, wu, xu, ku, 1 + w->n_shared, nullptr, T, hidden, st);
    }
    DenseSeg segs[3] = {{w->w_up, nrm, latent}, {nullptr, nullptr, 0}, {nullptr, nullptr, 0}};
    for (int i = 0; i < w->n_shared; ++i) {
        float *h = shh + (size_t)i * T * sh_inter;
        K3G_TRY(launch_dense_glu(h, w->sh_w1[i], w->sh_w3[i], x, T, hidden, sh_inter, st));
        segs[1 + i] = {w->sh_w2[i], h, sh_inter};
    }
    return launch_dense(out, segs, 1 + w->n_shared, T, hidden, st);
}
