// cache.hip -- the routed-expert cache in HBM, fed from host memory.
//
// The pages stream experts from storage through an LRU of expert slots
// ("kimi-k3-in-c: 2.78 trillion parameters, one CPU, 8 GB of RAM", section
// "The cache the project exists for"; "Kimi K3 engine (c/kimi_k3.c)", section
// "Streaming design"): LRU with pinning, a victim found by a plain linear scan,
// a slot table of three states (an expert, empty, or in flight -- reserved by
// a batch prefetch whose read has not finished, so that one batch never hands
// the same slot to two reads), a request histogram for choosing what to pin,
// and a token's misses read as one batch in storage order, overlapped with
// compute. Here the storage is host memory (ideally pinned) and the slots are
// an expert bank in HBM: the cache rewrites a step's expert ids into slot ids,
// so the layer runs unchanged on the slot bank. All state is host-side; the
// copies go out on the caller's copy stream as hipMemcpyAsync, one per
// missing expert (six tensors back to back = one copy), in host-address order.
// The pages' loader threads that overlap expert j's products with expert
// j+1's read become, for a decode token, an event after each copy and the
// pair's two launches queued behind that event on the compute stream.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <new>
#include <vector>

#include "k3g_common.h"

namespace k3g {
// launchers (gemv.hip) and the device check (abi.hip)
int launch_moe_up_exact(float *h, const float *x, const BankDev &bank, const int32_t *active, const int32_t *offsets,
                        const int32_t *perm, int top_k, int latent, int inter, int max_slots, int n_pairs, bool lut,
                        const Route1 &rt, hipStream_t st);
int launch_moe_down_exact(float *ypair, const float *h, const BankDev &bank, const int32_t *active,
                          const int32_t *offsets, const int32_t *perm, int latent, int inter, int max_slots,
                          bool multi_pairs, bool lut, hipStream_t st);
int launch_combine(float *y, const float *ypair, const float *wts, const int32_t *inv, int n_tokens, int top_k,
                   int latent, hipStream_t st);
int launch_quant_i8(int8_t *q, float *s, const float *x, int n_rows, int in, uint16_t *qb, hipStream_t st);
int launch_moe_up_idot(int8_t *hq, uint16_t *hqb, float *hs, const int8_t *xq, const uint16_t *xqb, const float *xs,
                       const BankDev &bank, const int32_t *active, const int32_t *offsets, const int32_t *perm,
                       int top_k, int latent, int inter, int max_slots, hipStream_t st);
int launch_moe_down_idot(float *ypair, const int8_t *hq, const uint16_t *hqb, const float *hs, const BankDev &bank,
                         const int32_t *active, const int32_t *offsets, const int32_t *perm, int latent, int inter,
                         int max_slots, hipStream_t st);
int device_ok();
}  // namespace k3g

namespace {

constexpr int32_t kEmpty = -1;     // slot holds nothing, free to take
constexpr int32_t kInflight = -2;  // slot reserved by this batch's prefetch
constexpr int kPipeMax = 64;       // pairs of one decode step (the largest top_k)

inline bool is_aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

}  // namespace

struct k3g_cache {
    const uint8_t *host_bank = nullptr;
    int32_t n_total = 0;
    k3g_expert_bank arena{};
    int32_t n_slots = 0;
    std::vector<int32_t> slot_key;   // per slot: expert id, kEmpty or kInflight
    std::vector<int32_t> incoming;   // per slot in flight: the expert it receives
    std::vector<int64_t> last_use;   // per slot: step of its last use
    std::vector<int32_t> slot_of;    // per expert: its slot, or -1
    std::vector<uint8_t> pinned;     // per expert
    std::vector<uint64_t> hist;      // per expert: requests seen
    std::vector<int32_t> step_copies_e, step_copies_s;
    int64_t tick = 0;
    k3g_cache_stats stats{};
    hipEvent_t ev_prev = nullptr, ev_copy = nullptr;
    hipEvent_t ev_pipe[kPipeMax] = {};  // one per copy of a pipelined decode step
    hipEvent_t ev_meta = nullptr;       // its pair table has landed
    int32_t *idx_stage = nullptr;    // pinned host staging of the rewritten ids
    size_t idx_stage_n = 0;
};

extern "C" {

int k3g_cache_create(k3g_cache **out, const uint8_t *host_bank, int32_t n_total, const k3g_expert_bank *arena) {
    if (!out || !arena || n_total < 1 || arena->n_experts < 1 || arena->stride <= 0) return K3G_EINVAL;
    k3g_cache *c = new (std::nothrow) k3g_cache;
    if (!c) return K3G_ENOSPACE;
    c->host_bank = host_bank;
    c->n_total = n_total;
    c->arena = *arena;
    c->n_slots = arena->n_experts;
    c->slot_key.assign(c->n_slots, kEmpty);
    c->incoming.assign(c->n_slots, -1);
    c->last_use.assign(c->n_slots, -1);
    c->slot_of.assign(n_total, -1);
    c->pinned.assign(n_total, 0);
    c->hist.assign(n_total, 0);
    *out = c;
    return K3G_OK;
}

void k3g_cache_destroy(k3g_cache *c) {
    if (!c) return;
    if (c->ev_prev) (void)hipEventDestroy(c->ev_prev);
    if (c->ev_copy) (void)hipEventDestroy(c->ev_copy);
    for (hipEvent_t e : c->ev_pipe)
        if (e) (void)hipEventDestroy(e);
    if (c->ev_meta) (void)hipEventDestroy(c->ev_meta);
    if (c->idx_stage) (void)hipHostFree(c->idx_stage);
    delete c;
}

int k3g_cache_pin(k3g_cache *c, int32_t expert, int pinned) {
    if (!c || expert < 0 || expert >= c->n_total) return K3G_EINVAL;
    c->pinned[expert] = pinned ? 1 : 0;
    return K3G_OK;
}

int k3g_cache_plan(k3g_cache *c, int32_t *idx_slot, int32_t *copy_expert, int32_t *copy_slot, int32_t *n_copies,
                   const int32_t *idx, int n_tokens, int top_k) {
    if (!c || !n_copies || n_tokens < 0 || top_k < 1 || (n_tokens > 0 && (!idx || !idx_slot))) return K3G_EINVAL;
    // the previous batch's slots are filled by now (its copies were ordered
    // before the work that used them)
    (void)k3g_cache_complete(c);
    const int64_t P = (int64_t)n_tokens * top_k;
    for (int64_t p = 0; p < P; ++p)
        if (idx[p] < -1 || idx[p] >= c->n_total) return K3G_EINVAL;
    // the step's distinct experts (ids ascending = host-address order)
    std::vector<int32_t> want;
    want.reserve((size_t)std::min<int64_t>(P, c->n_total));
    for (int64_t p = 0; p < P; ++p)
        if (idx[p] >= 0) want.push_back(idx[p]);
    std::sort(want.begin(), want.end());
    want.erase(std::unique(want.begin(), want.end()), want.end());
    // the step must fit before anything changes: its misses need slots that are
    // empty or hold an unpinned expert the step does not use
    std::vector<uint8_t> in_use(c->n_slots, 0);
    int32_t hits = 0;
    for (int32_t e : want)
        if (c->slot_of[e] >= 0) {
            in_use[c->slot_of[e]] = 1;
            ++hits;
        }
    int64_t free_slots = 0;
    for (int32_t i = 0; i < c->n_slots; ++i) {
        const int32_t k = c->slot_key[i];
        free_slots += !in_use[i] && (k == kEmpty || (k >= 0 && !c->pinned[k]));
    }
    if ((int64_t)want.size() - hits > free_slots) return K3G_ENOSPACE;
    ++c->tick;
    for (int64_t p = 0; p < P; ++p)
        if (idx[p] >= 0) ++c->hist[idx[p]];
    // hits: refresh, and keep them out of this batch's victims
    for (int32_t e : want)
        if (c->slot_of[e] >= 0) c->last_use[c->slot_of[e]] = c->tick;
    // misses, in host-address order: an empty slot if there is one, else the
    // least recently used slot that this batch neither uses nor fills and
    // whose expert is not pinned (a linear scan; equal ages: the lower slot)
    int32_t nc = 0;
    for (int32_t e : want) {
        if (c->slot_of[e] >= 0) continue;
        int32_t s = -1;
        for (int32_t i = 0; i < c->n_slots && s < 0; ++i)
            if (c->slot_key[i] == kEmpty) s = i;
        if (s < 0)
            for (int32_t i = 0; i < c->n_slots; ++i) {
                const int32_t k = c->slot_key[i];
                if (in_use[i] || k == kInflight || (k >= 0 && c->pinned[k])) continue;
                if (s < 0 || c->last_use[i] < c->last_use[s]) s = i;
            }
        if (c->slot_key[s] >= 0) {
            c->slot_of[c->slot_key[s]] = -1;
            ++c->stats.evictions;
        }
        c->slot_key[s] = kInflight;
        c->incoming[s] = e;
        c->slot_of[e] = s;
        c->last_use[s] = c->tick;
        in_use[s] = 1;
        if (copy_expert) copy_expert[nc] = e;
        if (copy_slot) copy_slot[nc] = s;
        ++nc;
    }
    for (int64_t p = 0; p < P; ++p) idx_slot[p] = idx[p] >= 0 ? c->slot_of[idx[p]] : -1;
    *n_copies = nc;
    c->stats.steps += 1;
    c->stats.hits += hits;
    c->stats.misses += nc;
    c->stats.bytes_copied += (uint64_t)nc * (uint64_t)c->arena.stride;
    return K3G_OK;
}

int k3g_cache_complete(k3g_cache *c) {
    if (!c) return K3G_EINVAL;
    for (int32_t s = 0; s < c->n_slots; ++s)
        if (c->slot_key[s] == kInflight) {
            c->slot_key[s] = c->incoming[s];
            c->incoming[s] = -1;
        }
    return K3G_OK;
}

}  // extern "C"

namespace {

// The events, and the pinned staging of P ids: the previous step's copy of
// the staging must be done before it is written again.
int stage_for(k3g_cache *c, size_t P) {
    if (!c->ev_prev) {
        if (hipEventCreateWithFlags(&c->ev_prev, hipEventDisableTiming) != hipSuccess ||
            hipEventCreateWithFlags(&c->ev_copy, hipEventDisableTiming) != hipSuccess)
            return K3G_EHIP;
    }
    if (hipEventSynchronize(c->ev_copy) != hipSuccess) return K3G_EHIP;
    if (c->idx_stage_n < P) {
        if (c->idx_stage) (void)hipHostFree(c->idx_stage);
        c->idx_stage = nullptr;
        c->idx_stage_n = 0;
        if (hipHostMalloc((void **)&c->idx_stage, sizeof(int32_t) * P, hipHostMallocDefault) != hipSuccess)
            return K3G_ENOSPACE;
        c->idx_stage_n = P;
    }
    return K3G_OK;
}

}  // namespace

extern "C" {

int k3g_cache_prepare(k3g_cache *c, int32_t *idx_slot, const int32_t *idx, int n_tokens, int top_k,
                      void *copy_stream, void *stream) {
    if (!c || !c->host_bank || n_tokens < 0 || top_k < 1) return K3G_EINVAL;
    const size_t P = (size_t)n_tokens * top_k;
    if (P == 0) return K3G_OK;
    if (!idx || !idx_slot) return K3G_EINVAL;
    const int rs = stage_for(c, P);
    if (rs != K3G_OK) return rs;
    c->step_copies_e.resize((size_t)c->n_slots);
    c->step_copies_s.resize((size_t)c->n_slots);
    int32_t nc = 0;
    const int rc = k3g_cache_plan(c, c->idx_stage, c->step_copies_e.data(), c->step_copies_s.data(), &nc, idx,
                                  n_tokens, top_k);
    if (rc != K3G_OK) return rc;
    hipStream_t cs = (hipStream_t)copy_stream, st = (hipStream_t)stream;
    // the slots about to be overwritten may still be read by work already on
    // `stream`: the copies start after it
    if (hipEventRecord(c->ev_prev, st) != hipSuccess || hipStreamWaitEvent(cs, c->ev_prev, 0) != hipSuccess)
        return K3G_EHIP;
    const size_t stride = (size_t)c->arena.stride;
    for (int32_t i = 0; i < nc; ++i) {
        const uint8_t *src = c->host_bank + (size_t)c->step_copies_e[i] * stride;
        uint8_t *dst = const_cast<uint8_t *>(c->arena.base) + (size_t)c->step_copies_s[i] * stride;
        if (hipMemcpyAsync(dst, src, stride, hipMemcpyHostToDevice, cs) != hipSuccess) return K3G_EHIP;
    }
    if (hipMemcpyAsync(idx_slot, c->idx_stage, sizeof(int32_t) * P, hipMemcpyHostToDevice, cs) != hipSuccess)
        return K3G_EHIP;
    if (hipEventRecord(c->ev_copy, cs) != hipSuccess || hipStreamWaitEvent(st, c->ev_copy, 0) != hipSuccess)
        return K3G_EHIP;
    return k3g_cache_complete(c);
}

int k3g_cache_decode_step(k3g_cache *c, float *y, const float *x, const int32_t *idx, const float *wts, int top_k,
                          int mode, void *ws, size_t ws_bytes, void *copy_stream, void *stream) {
    using namespace k3g;
    if (!c || !c->host_bank || !y || !x || !idx || !wts || !ws || top_k < 1 || top_k > kPipeMax) return K3G_EINVAL;
    // EXACT on the vector kernels (the LDS table optional), or IDOT in either form;
    // the FP4 matrix-core form is a layer form and is refused
    if (mode & K3G_DECODE_MFMA) return K3G_EUNSUPPORTED;
    const bool idot = (mode & 0xFF) == K3G_IDOT;
    const k3g_expert_bank &A = c->arena;
    const int latent = A.latent, inter = A.inter;
    if (idot && (latent % 128 || inter % 128)) return K3G_EUNSUPPORTED;
    k3g_shape sh = {1, top_k, A.n_experts, latent, inter, 0, 0, mode};
    k3g_ws_layout L;
    int rc = k3g_workspace_layout(&L, K3G_OP_MOE_LAYER, &sh);
    if (rc != K3G_OK) return rc;
    if (ws_bytes < L.total) return K3G_ENOSPACE;
    if (!is_aligned(x, 16) || !is_aligned(y, 16) || !is_aligned(ws, 256) || !is_aligned(wts, 4)) return K3G_EALIGN;
    if ((uintptr_t)y < (uintptr_t)x + sizeof(float) * latent && (uintptr_t)x < (uintptr_t)y + sizeof(float) * latent)
        return K3G_EINVAL;
    if (!A.base) return K3G_EINVAL;
    if (latent / kGroup > 256 || inter / kGroup > 256) return K3G_EUNSUPPORTED;
    for (int i = 0; i < 6; i += 2)
        if (!is_aligned(A.base + A.off[i], 16) || A.stride % 16) return K3G_EALIGN;
    for (int i = 1; i < 6; i += 2)
        if (!is_aligned(A.base + A.off[i], 4)) return K3G_EALIGN;
    for (int k = 0; k < top_k; ++k)
        if (idx[k] < -1 || idx[k] >= c->n_total) return K3G_EINVAL;
    if ((rc = device_ok()) != K3G_OK) return rc;
    const int E = A.n_experts;
    // staging: inv [top_k], active [E + 1], offsets [E + 1], perm [top_k]
    if ((rc = stage_for(c, (size_t)(2 * top_k + 2 * (E + 1)))) != K3G_OK) return rc;
    for (int i = 0; i < kPipeMax; ++i)
        if (!c->ev_pipe[i] && hipEventCreateWithFlags(&c->ev_pipe[i], hipEventDisableTiming) != hipSuccess)
            return K3G_EHIP;
    if (!c->ev_meta && hipEventCreateWithFlags(&c->ev_meta, hipEventDisableTiming) != hipSuccess) return K3G_EHIP;

    // the plan: slot of each pair, and the copies (at most one per pair)
    int32_t slot[kPipeMax];
    c->step_copies_e.resize((size_t)c->n_slots);
    c->step_copies_s.resize((size_t)c->n_slots);
    int32_t nc = 0;
    if ((rc = k3g_cache_plan(c, slot, c->step_copies_e.data(), c->step_copies_s.data(), &nc, idx, 1, top_k)) !=
        K3G_OK)
        return rc;
    auto copy_of = [&](int k) {
        for (int32_t i = 0; i < nc; ++i)
            if (c->step_copies_s[i] == slot[k]) return i;
        return -1;
    };
    // The pair table. The resident experts' pairs come first, in slot order,
    // as one bucket (active slots, offsets by slot, perm = pair), so that one
    // up and one down launch take them all; then each copied expert's pairs
    // in copy order. inv: pair -> row of h and ypair (-1: dropped entry).
    int32_t *st_inv = c->idx_stage, *st_act = st_inv + top_k, *st_off = st_act + (E + 1), *st_perm = st_off + (E + 1);
    for (int s = 0; s <= E; ++s) st_off[s] = 0;
    int n_hit = 0;
    for (int k = 0; k < top_k; ++k)
        if (slot[k] >= 0 && copy_of(k) < 0) {
            ++st_off[slot[k] + 1];
            ++n_hit;
        }
    int n_hit_slots = 0;
    for (int s = 0; s < E; ++s) {
        if (st_off[s + 1] > 0) st_act[1 + n_hit_slots++] = s;
        st_off[s + 1] += st_off[s];
    }
    st_act[0] = n_hit_slots;
    int next = 0;
    for (int k = 0; k < top_k; ++k) {
        st_inv[k] = -1;
        if (slot[k] < 0 || copy_of(k) >= 0) continue;
        int at = next++;  // stable insertion by slot: equal slots keep k order
        while (at > 0 && slot[st_perm[at - 1]] > slot[k]) {
            st_perm[at] = st_perm[at - 1];
            --at;
        }
        st_perm[at] = k;
    }
    for (int pos = 0; pos < n_hit; ++pos) st_inv[st_perm[pos]] = pos;
    for (int32_t i = 0; i < nc; ++i)
        for (int k = 0; k < top_k; ++k)
            if (slot[k] == c->step_copies_s[i]) st_inv[k] = next++;

    char *w = (char *)ws;
    float *h = L.h ? (float *)(w + L.h) : nullptr, *ypair = (float *)(w + L.ypair);
    // IDOT: x quantised per 32-group (and its bf16 copy in that form); h only quantised
    int8_t *xq = idot ? (int8_t *)(w + L.xq) : nullptr, *hq = L.hq ? (int8_t *)(w + L.hq) : nullptr;
    float *xs = idot ? (float *)(w + L.xs) : nullptr, *hs = idot ? (float *)(w + L.hs) : nullptr;
    uint16_t *xqb = L.xqb ? (uint16_t *)(w + L.xqb) : nullptr, *hqb = L.hqb ? (uint16_t *)(w + L.hqb) : nullptr;
    int32_t *inv = (int32_t *)(w + L.inv), *active = (int32_t *)(w + L.active);
    int32_t *offsets = (int32_t *)(w + L.offsets), *perm = (int32_t *)(w + L.perm);
    const bool lut = (mode & K3G_DECODE_LUT) != 0;
    hipStream_t cs = (hipStream_t)copy_stream, st = (hipStream_t)stream;
    BankDev bank;
    bank.base = A.base;
    bank.stride = A.stride;
    for (int i = 0; i < 6; ++i) bank.off[i] = A.off[i];
    // one copied expert's pair: up-projection with SiTU, then down-projection, at its row
    auto pair = [&](int k) {
        BankDev b = bank;
        b.base = A.base + (size_t)slot[k] * A.stride;
        b.stride = 0;
        const size_t row = (size_t)st_inv[k];
        if (idot) {
            int8_t *hqk = hq ? hq + row * inter : nullptr;
            uint16_t *hqbk = hqb ? hqb + row * inter : nullptr;
            float *hsk = hs + row * (inter / kGroup);
            const int r = launch_moe_up_idot(hqk, hqbk, hsk, xq, xqb, xs, b, nullptr, nullptr, nullptr, 1, latent,
                                             inter, 1, st);
            if (r != K3G_OK) return r;
            return launch_moe_down_idot(ypair + row * latent, hqk, hqbk, hsk, b, nullptr, nullptr, nullptr, latent,
                                        inter, 1, st);
        }
        float *hk = h + row * inter;
        const int r = launch_moe_up_exact(hk, x, b, nullptr, nullptr, nullptr, 1, latent, inter, 1, 1, lut, Route1{},
                                          st);
        if (r != K3G_OK) return r;
        return launch_moe_down_exact(ypair + row * latent, hk, b, nullptr, nullptr, nullptr, latent, inter, 1, false,
                                     lut, st);
    };
    // the slots about to be overwritten may still be read by work already on
    // `stream`: the copy stream starts after it, with the pair table first
    if (hipEventRecord(c->ev_prev, st) != hipSuccess || hipStreamWaitEvent(cs, c->ev_prev, 0) != hipSuccess)
        return K3G_EHIP;
    const size_t stride = (size_t)A.stride;
    if (hipMemcpyAsync(inv, st_inv, sizeof(int32_t) * top_k, hipMemcpyHostToDevice, cs) != hipSuccess ||
        hipMemcpyAsync(active, st_act, sizeof(int32_t) * (E + 1), hipMemcpyHostToDevice, cs) != hipSuccess ||
        hipMemcpyAsync(offsets, st_off, sizeof(int32_t) * (E + 1), hipMemcpyHostToDevice, cs) != hipSuccess ||
        hipMemcpyAsync(perm, st_perm, sizeof(int32_t) * top_k, hipMemcpyHostToDevice, cs) != hipSuccess ||
        hipEventRecord(c->ev_meta, cs) != hipSuccess)
        return K3G_EHIP;
    for (int32_t i = 0; i < nc; ++i) {
        const uint8_t *src = c->host_bank + (size_t)c->step_copies_e[i] * stride;
        uint8_t *dst = const_cast<uint8_t *>(A.base) + (size_t)c->step_copies_s[i] * stride;
        if (hipMemcpyAsync(dst, src, stride, hipMemcpyHostToDevice, cs) != hipSuccess ||
            hipEventRecord(c->ev_pipe[i], cs) != hipSuccess)
            return K3G_EHIP;
    }
    if (idot && (rc = launch_quant_i8(xq, xs, x, 1, latent, xqb, st)) != K3G_OK) return rc;
    // the staging is read by the table's copies: the next step waits for them
    if (hipStreamWaitEvent(st, c->ev_meta, 0) != hipSuccess || hipEventRecord(c->ev_copy, st) != hipSuccess)
        return K3G_EHIP;
    // the resident experts' pairs in one up and one down launch, then each
    // copied expert's pair once its copy has landed
    if (n_hit > 0 && idot) {
        if ((rc = launch_moe_up_idot(hq, hqb, hs, xq, xqb, xs, bank, active, offsets, perm, top_k, latent, inter,
                                     n_hit_slots, st)) != K3G_OK ||
            (rc = launch_moe_down_idot(ypair, hq, hqb, hs, bank, active, offsets, perm, latent, inter, n_hit_slots,
                                       st)) != K3G_OK)
            return rc;
    } else if (n_hit > 0) {
        if ((rc = launch_moe_up_exact(h, x, bank, active, offsets, perm, top_k, latent, inter, n_hit_slots, n_hit,
                                      lut, Route1{}, st)) != K3G_OK ||
            (rc = launch_moe_down_exact(ypair, h, bank, active, offsets, perm, latent, inter, n_hit_slots, false, lut,
                                        st)) != K3G_OK)
            return rc;
    }
    for (int32_t i = 0; i < nc; ++i) {
        if (hipStreamWaitEvent(st, c->ev_pipe[i], 0) != hipSuccess) return K3G_EHIP;
        for (int k = 0; k < top_k; ++k)
            if (slot[k] == c->step_copies_s[i] && (rc = pair(k)) != K3G_OK) return rc;
    }
    if ((rc = launch_combine(y, ypair, wts, inv, 1, top_k, latent, st)) != K3G_OK) return rc;
    return k3g_cache_complete(c);
}

int k3g_cache_query(const k3g_cache *c, k3g_cache_stats *stats, int32_t *slot_of, uint64_t *hist) {
    if (!c) return K3G_EINVAL;
    if (stats) *stats = c->stats;
    if (slot_of) memcpy(slot_of, c->slot_of.data(), sizeof(int32_t) * c->n_total);
    if (hist) memcpy(hist, c->hist.data(), sizeof(uint64_t) * c->n_total);
    return K3G_OK;
}

}  // extern "C"
