// gemv.hip -- batch-1 and grouped EXACT MXFP4 products (gfx950).
//
// The pages' kernel ("kimi-k3-in-c: 2.78 trillion parameters, one CPU, 8 GB
// of RAM", section "Reduction one") walks each row group by group: decode 32
// nibbles through a byte-pair table, dot them with x, apply the group's one
// scale, skip scale 255. Here a wavefront owns a row at a time:
//   - each lane owns NG consecutive groups of the row, so one row is one
//     coalesced sweep of 16-byte loads (lane l reads bytes [16*NG*l, ...));
//   - x for the lane's columns stays in VGPRs for every row of a work item;
//   - the byte-pair table lives in LDS as f16 pairs, one copy per lane;
//   - the group sum is scaled once by 2^(s-127) (or dropped for s = 255);
//   - the lane partials are summed with DPP and readlane.
// A work item is a run of consecutive rows of one matrix (and, for the MoE
// kernels, one expert), so x is fetched once per item.
#include "k3g_common.h"

// Build-time knobs (defaults are the shipped configuration).
#ifndef K3G_GEMV_THREADS
#define K3G_GEMV_THREADS 256
#endif
#ifndef K3G_WAVES_PER_EU
#define K3G_WAVES_PER_EU 0  // 0: let the compiler choose the register budget
#endif
#if K3G_WAVES_PER_EU
#define K3G_OCC __attribute__((amdgpu_waves_per_eu(K3G_WAVES_PER_EU)))
#else
#define K3G_OCC
#endif
#ifndef K3G_PIPE
#define K3G_PIPE 3  // rows (per matrix) a wavefront keeps in flight
#endif
#ifndef K3G_ITEMS_TARGET
#define K3G_ITEMS_TARGET 2048  // work items a decode launch is cut into
#endif
// Several tokens: the pairs of an expert take turns over short runs of rows, so
// that the later passes find the rows in L2 (one pair per pass keeps the
// kernel at two wavefronts per SIMD; two per pass needs all 256 VGPRs).
#ifndef K3G_MULTI_ITEMS
#define K3G_MULTI_ITEMS 131072  // work items when several tokens share experts
#endif
#ifndef K3G_MULTI_NP
#define K3G_MULTI_NP 1          // pairs per pass over the rows when several tokens share experts
#endif

namespace k3g {

template <int NG>
struct RowData {
    uint4 w[NG];
    uint32_t s[NG];
};

// Loads are unconditional so that the compiler can count them: a lane past
// the last group reads group ngrp-1 again, and row_partial drops it (the
// lane's `valid` bits). The row pointers are wave-uniform (SGPRs); each lane
// adds its own constant byte offset, so no per-lane address arithmetic is
// repeated per row.
template <int NG>
struct LaneCols {
    uint32_t pk[NG];  // byte offset of the lane's group i in a packed row
    uint32_t sc[NG];  // its index in a row of scale bytes
    uint32_t sc2;     // NG = 2: even index of the lane's two scale bytes (one 16-bit load)
};

template <int NG>
__device__ inline LaneCols<NG> lane_cols(int lane, int ngrp) {
    LaneCols<NG> c;
#pragma unroll
    for (int i = 0; i < NG; ++i) {
        const int g = lane * NG + i;
        const int gc = g < ngrp ? g : ngrp - 1;
        c.pk[i] = (uint32_t)gc * 16u;
        c.sc[i] = (uint32_t)gc;
    }
    const int g2 = lane * NG;
    c.sc2 = (uint32_t)(g2 + 1 < ngrp ? g2 : (ngrp >= 2 ? ((ngrp - 2) & ~1) : 0));
    return c;
}

// One MXFP4 matrix as two buffer resources plus its row pitches.
struct MatRef {
    rsrc_t p, s;
    uint32_t pitch_p, pitch_s;
};

__device__ inline MatRef mat_ref(const uint8_t *packed, const uint8_t *scales, int rows, int in) {
    MatRef m;
    m.pitch_p = (uint32_t)in / 2;
    m.pitch_s = (uint32_t)in / kGroup;
    m.p = make_rsrc(packed, m.pitch_p * (uint32_t)rows);
    m.s = make_rsrc(scales, m.pitch_s * (uint32_t)rows);
    return m;
}

// F32S: the scales are fp32 per group (expanded at upload; m.pitch_s in bytes
// is 4 * groups), d.s holds their bits.
template <int NG, bool SC2 = false, bool F32S = false>
__device__ inline void load_row(RowData<NG> &d, const MatRef &m, int r, const LaneCols<NG> &c) {
    const uint32_t op = (uint32_t)r * m.pitch_p, os = (uint32_t)r * m.pitch_s;
#pragma unroll
    for (int i = 0; i < NG; ++i) d.w[i] = buf_load16(m.p, c.pk[i], op);
    if constexpr (F32S) {
#pragma unroll
        for (int i = 0; i < NG; ++i)
            d.s[i] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(m.s, (int)(4u * c.sc[i]), (int)os, 0);
    } else if constexpr (NG == 2 && SC2) {
        const uint32_t v = buf_load_u16(m.s, c.sc2, os);
        d.s[0] = v & 0xFFu;
        d.s[NG - 1] = v >> 8;
    } else {
#pragma unroll
        for (int i = 0; i < NG; ++i) d.s[i] = buf_load8(m.s, c.sc[i], os);
    }
}

// Decode: LUT = the byte-pair table in LDS; otherwise gfx950's FP4 convert.
template <int NG, bool LUT, bool F32S = false>
__device__ inline float row_partial(const RowData<NG> &d, const uint32_t *lut, uint32_t lane_off, const float *xr,
                                   uint32_t valid) {
    float p = 0.f;
#pragma unroll
    for (int i = 0; i < NG; ++i) {
        float sub;
        if constexpr (LUT) {
            sub = group_dot(lut, lane_off, d.w[i], xr + i * kGroup);
        } else {
            sub = group_dot_cvt(d.w[i], xr + i * kGroup);
            (void)lut;
            (void)lane_off;
        }
        // a group past the row's end is dropped by masking its bits (+0.0): a
        // select here would be turned into a branch around the whole group,
        // and the branches would cost the loads of the rows in flight
        const uint32_t keep = 0u - ((valid >> i) & 1u);
        const float scaled = F32S ? sub * __builtin_bit_cast(float, d.s[i]) : apply_scale(sub, d.s[i]);
        p += __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, scaled) & keep);
    }
    return p;
}

// Bit i set: group lane*NG+i exists in a row of ngrp groups.
template <int NG>
__device__ inline uint32_t valid_groups(int lane, int ngrp) {
    uint32_t v = 0;
#pragma unroll
    for (int i = 0; i < NG; ++i) v |= (lane * NG + i < ngrp ? 1u : 0u) << i;
    return v;
}

// x columns owned by this lane: groups [lane*NG, lane*NG+NG) of a row of width
// ngrp*32. A lane past the last group holds a copy of the last group (its
// products are dropped by row_partial).
template <int NG>
__device__ inline void load_x(float *xr, const float *x, int lane, int ngrp) {
#pragma unroll
    for (int i = 0; i < NG; ++i) {
        const int g = lane * NG + i;
        const int gc = g < ngrp ? g : ngrp - 1;
#pragma unroll
        for (int j = 0; j < kGroup; j += 4) {
            const float4 v = *(const float4 *)(x + (size_t)gc * kGroup + j);
            xr[i * kGroup + j + 0] = v.x;
            xr[i * kGroup + j + 1] = v.y;
            xr[i * kGroup + j + 2] = v.z;
            xr[i * kGroup + j + 3] = v.w;
        }
    }
}

// x shared by every wavefront of the workgroup: copied once into LDS (a
// float4 per thread per step), then each lane reads its groups from there
// instead of every wavefront fetching the whole of x from L2.
__device__ inline void stage_x(float *xs, const float *x, int len) {
    for (int i = 4 * threadIdx.x; i < len; i += 4 * blockDim.x) *(float4 *)(xs + i) = *(const float4 *)(x + i);
    __syncthreads();
}

template <int NG>
__device__ inline void load_x_lds(float *xr, const float *xs, int lane, int ngrp) {
#pragma unroll
    for (int i = 0; i < NG; ++i) {
        const int g = lane * NG + i;
        const int gc = g < ngrp ? g : ngrp - 1;
#pragma unroll
        for (int j = 0; j < kGroup; j += 4) {
            const float4 v = *(const float4 *)(xs + gc * kGroup + j);
            xr[i * kGroup + j + 0] = v.x;
            xr[i * kGroup + j + 1] = v.y;
            xr[i * kGroup + j + 2] = v.z;
            xr[i * kGroup + j + 3] = v.w;
        }
    }
}

// y[r] for r in [0, rows): one matrix, one x (staged in LDS). Items of rpi rows. F32S: the
// scales are fp32 per group (the pages' Vulkan-tier format).
template <int NG, bool LUT, bool F32S = false>
__global__ __launch_bounds__(K3G_GEMV_THREADS) K3G_OCC void gemv_kernel(float *__restrict__ y, const float *__restrict__ x,
                                                   const uint8_t *__restrict__ packed,
                                                   const uint8_t *__restrict__ scales, int in, int rows, int rpi) {
    uint32_t *lut = nullptr;
    if constexpr (LUT) {
        __shared__ uint32_t lut_lds[kLutWords];
        build_pair_lut(lut_lds);
        __syncthreads();
        lut = lut_lds;
    }
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int waves = blockDim.x / kWave;
    const uint32_t lane_off = uint32_t(lane) << 2;
    const int ngrp = in / kGroup;
    const uint32_t valid = valid_groups<NG>(lane, ngrp);
    const LaneCols<NG> cols = lane_cols<NG>(lane, ngrp);
    MatRef mat = mat_ref(packed, scales, rows, in);
    if constexpr (F32S) {
        mat.pitch_s = 4u * (uint32_t)ngrp;
        mat.s = make_rsrc(scales, mat.pitch_s * (uint32_t)rows);
    }
    const int n_items = (rows + rpi - 1) / rpi;
    int item = blockIdx.x * waves + wave;
    RowData<NG> buf[K3G_PIPE];
    // the first item's rows go out before x is staged, so the two waits overlap
    if (item < n_items) {
        const int r0 = item * rpi, r1 = min(rows, r0 + rpi);
#pragma unroll
        for (int st = 0; st < K3G_PIPE; ++st) {
            load_row<NG, false, F32S>(buf[st], mat, min(r0 + st, r1 - 1), cols);
            __builtin_amdgcn_sched_barrier(0);  // keep the loop's load order (see below)
        }
    }
    extern __shared__ float xs_lds[];  // [in]
    stage_x(xs_lds, x, in);
    float xr[NG * kGroup];
    load_x_lds<NG>(xr, xs_lds, lane, ngrp);
    for (bool first = true; item < n_items; item += gridDim.x * waves, first = false) {
        const int r0 = item * rpi;
        const int r1 = min(rows, r0 + rpi);
        auto R = [&](int r) { return min(r, r1 - 1); };
        if (!first) {
#pragma unroll
            for (int st = 0; st < K3G_PIPE; ++st) {
                load_row<NG, false, F32S>(buf[st], mat, R(r0 + st), cols);
                __builtin_amdgcn_sched_barrier(0);  // keep the loop's load order (see below)
            }
        }
        float acc = 0.f;  // lane k holds row (r - r0) % 64 == k until its block of 64 is stored
        // every work item has at least one row: a do-while keeps the loads of x
        // and of the first rows in one block (no preheader to sink x into)
        int r = r0;
        do {
#pragma unroll
            for (int st = 0; st < K3G_PIPE; ++st) {
                const int rr = r + st;
                if (rr < r1) {
                    const float sa = wave_sum(row_partial<NG, LUT, F32S>(buf[st], lut, lane_off, xr, valid));
                    const int k = (rr - r0) & (kWave - 1);
                    acc = lane == k ? sa : acc;
                    if (k == kWave - 1 || rr == r1 - 1) {
                        if (lane <= k) y[rr - k + lane] = acc;
                    }
                }
                load_row<NG, false, F32S>(buf[st], mat, R(rr + K3G_PIPE), cols);
            }
            r += K3G_PIPE;
        } while (r < r1);
    }
}


// Grouped SiTU-GLU up-projection. Work item = (slot, run of rpi rows); slot i
// is the i-th expert that has pairs (active[1+i]); its pairs are the sorted
// positions [offsets[e], offsets[e+1]), token = perm[pos] / top_k. For each
// pair and row r: g = w1[r].x, u = w3[r].x, h[pos][r] = SiTU(g, u).
// NP pairs share each pass over the rows (their x in registers), so an expert
// chosen by several tokens is streamed ceil(pairs / NP) times.
// With perm == nullptr the call is one expert (bank expert 0) on token 0.
template <int NG, bool LUT, int NP, bool SC2>
__global__ __launch_bounds__(K3G_GEMV_THREADS) K3G_OCC void moe_up_exact_kernel(
    float *__restrict__ h, const float *__restrict__ x, BankDev bank, const int32_t *__restrict__ active,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ perm, int top_k, int latent, int inter,
    int max_slots, int rpi, Route1 rt) {
    constexpr int PIPE = NP > 1 ? 2 : K3G_PIPE;  // rows in flight: two pairs need the registers
    uint32_t *lut = nullptr;
    if constexpr (LUT) {
        __shared__ uint32_t lut_lds[kLutWords];
        build_pair_lut(lut_lds);
        __syncthreads();
        lut = lut_lds;
    }
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int waves = blockDim.x / kWave;
    const uint32_t lane_off = uint32_t(lane) << 2;
    const int ngrp = latent / kGroup;
    const uint32_t valid = valid_groups<NG>(lane, ngrp);
    const LaneCols<NG> cols = lane_cols<NG>(lane, ngrp);
    const int chunks = (inter + rpi - 1) / rpi;
    // one token without a bucket: rank the route entries here (rt.idx set)
    Route1Lane r1 = {};
    if (rt.idx) {
        r1 = route1_lane(rt.idx, top_k, rt.n_experts, lane);
        if (blockIdx.x == 0 && wave == 0) route1_write_bucket(rt, r1, top_k, lane);
    }
    const int n_act = rt.idx ? __popcll(r1.firsts) : (perm ? active[0] : 1);
    const int n_items = max_slots * chunks;
    float xr[NP][NG * kGroup];
    for (int item = blockIdx.x * waves + wave; item < n_items; item += gridDim.x * waves) {
        const int slot = item / chunks;
        if (slot >= n_act) continue;
        const int chunk = item - slot * chunks;
        int e, p0, p1;
        if (rt.idx) {  // the lane holding the first entry of this slot's expert
            const uint64_t m = __ballot(r1.first && r1.slot == slot);
            const int L = __builtin_amdgcn_readfirstlane(__builtin_ctzll(m));
            e = __builtin_amdgcn_readlane(r1.e, L);
            p0 = __builtin_amdgcn_readlane(r1.pos, L);
            p1 = p0 + __builtin_amdgcn_readlane(r1.cnt, L);
        } else {
            e = perm ? active[1 + slot] : 0;
            p0 = perm ? offsets[e] : 0;
            p1 = perm ? offsets[e + 1] : 1;
        }
        const uint8_t *eb = bank.base + (int64_t)e * bank.stride;
        const MatRef m1 = mat_ref(eb + bank.off[W1P], eb + bank.off[W1S], inter, latent);
        const MatRef m3 = mat_ref(eb + bank.off[W3P], eb + bank.off[W3S], inter, latent);
        const int r0 = chunk * rpi;
        const int r1 = min(inter, r0 + rpi);
        auto R = [&](int r) { return min(r, r1 - 1); };
        for (int pos = p0; pos < p1; pos += NP) {
            // a pass of NP pairs; a missing last pair repeats the one before and is not stored
            int ps[NP];
#pragma unroll
            for (int q = 0; q < NP; ++q) {
                ps[q] = min(pos + q, p1 - 1);
                const int t = (perm && !rt.idx) ? perm[ps[q]] / top_k : 0;  // one token: token 0
                load_x<NG>(xr[q], x + (size_t)t * latent, lane, ngrp);
            }
            __builtin_amdgcn_sched_barrier(0);  // x before the rows: the oldest loads
            RowData<NG> b1[PIPE], b3[PIPE];
#pragma unroll
            for (int st = 0; st < PIPE; ++st) {
                load_row<NG, SC2>(b1[st], m1, R(r0 + st), cols);
                load_row<NG, SC2>(b3[st], m3, R(r0 + st), cols);
                // The rows go out in the order the loop below will refill them,
                // so that on every pass the row being summed is the oldest load
                // and the compiler's wait leaves the later rows in flight.
                __builtin_amdgcn_sched_barrier(0);
            }
            float gv[NP], uv[NP];  // lane k holds row k of the current block of 64
#pragma unroll
            for (int q = 0; q < NP; ++q) gv[q] = uv[q] = 0.f;
            // every work item has at least one row: a do-while keeps the loads of x
            // and of the first rows in one block (no preheader to sink x into)
            int r = r0;
            do {
#pragma unroll
                for (int st = 0; st < PIPE; ++st) {
                    const int rr = r + st;
                    if (rr < r1) {
                        const int k = (rr - r0) & (kWave - 1);
#pragma unroll
                        for (int q = 0; q < NP; ++q) {
                            const float g = wave_sum(row_partial<NG, LUT>(b1[st], lut, lane_off, xr[q], valid));
                            const float u = wave_sum(row_partial<NG, LUT>(b3[st], lut, lane_off, xr[q], valid));
                            gv[q] = lane == k ? g : gv[q];
                            uv[q] = lane == k ? u : uv[q];
                        }
                        if (k == kWave - 1 || rr == r1 - 1) {
                            // SiTU once per block, one row per lane
#pragma unroll
                            for (int q = 0; q < NP; ++q)
                                if (lane <= k && pos + q < p1) h[(size_t)ps[q] * inter + rr - k + lane] = situ(gv[q], uv[q]);
                        }
                    }
                    load_row<NG, SC2>(b1[st], m1, R(r + st + PIPE), cols);
                    load_row<NG, SC2>(b3[st], m3, R(r + st + PIPE), cols);
                }
                r += PIPE;
            } while (r < r1);
        }
    }
}

// Grouped down-projection: ypair[pos][r] = w2[r] . h[pos] for every pair of
// the slot's expert. Same items as the up kernel, over latent rows; NP pairs
// share each pass over the rows.
template <int NG, bool LUT, int NP, bool SC2>
__global__ __launch_bounds__(K3G_GEMV_THREADS) K3G_OCC void moe_down_exact_kernel(
    float *__restrict__ ypair, const float *__restrict__ h, BankDev bank, const int32_t *__restrict__ active,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ perm, int latent, int inter,
    int max_slots, int rpi) {
    constexpr int PIPE = NP > 1 ? 2 : K3G_PIPE;  // rows in flight: two pairs need the registers
    uint32_t *lut = nullptr;
    if constexpr (LUT) {
        __shared__ uint32_t lut_lds[kLutWords];
        build_pair_lut(lut_lds);
        __syncthreads();
        lut = lut_lds;
    }
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int waves = blockDim.x / kWave;
    const uint32_t lane_off = uint32_t(lane) << 2;
    const int ngrp = inter / kGroup;
    const uint32_t valid = valid_groups<NG>(lane, ngrp);
    const LaneCols<NG> cols = lane_cols<NG>(lane, ngrp);
    const int chunks = (latent + rpi - 1) / rpi;
    const int n_act = perm ? active[0] : 1;
    const int n_items = max_slots * chunks;
    float xr[NP][NG * kGroup];
    for (int item = blockIdx.x * waves + wave; item < n_items; item += gridDim.x * waves) {
        const int slot = item / chunks;
        if (slot >= n_act) continue;
        const int chunk = item - slot * chunks;
        const int e = perm ? active[1 + slot] : 0;
        const int p0 = perm ? offsets[e] : 0;
        const int p1 = perm ? offsets[e + 1] : 1;
        const uint8_t *eb = bank.base + (int64_t)e * bank.stride;
        const MatRef m2 = mat_ref(eb + bank.off[W2P], eb + bank.off[W2S], latent, inter);
        const int r0 = chunk * rpi;
        const int r1 = min(latent, r0 + rpi);
        auto R = [&](int r) { return min(r, r1 - 1); };
        for (int pos = p0; pos < p1; pos += NP) {
            int ps[NP];
#pragma unroll
            for (int q = 0; q < NP; ++q) {
                ps[q] = min(pos + q, p1 - 1);
                load_x<NG>(xr[q], h + (size_t)ps[q] * inter, lane, ngrp);
            }
            __builtin_amdgcn_sched_barrier(0);  // h before the rows: the oldest loads
            RowData<NG> buf[PIPE];
#pragma unroll
            for (int st = 0; st < PIPE; ++st) {
                load_row<NG, SC2>(buf[st], m2, R(r0 + st), cols);
                __builtin_amdgcn_sched_barrier(0);  // the loop's load order
            }
            float acc[NP];  // lane k holds row k of the current block of 64
#pragma unroll
            for (int q = 0; q < NP; ++q) acc[q] = 0.f;
            // every work item has at least one row: a do-while keeps the loads of x
            // and of the first rows in one block (no preheader to sink x into)
            int r = r0;
            do {
#pragma unroll
                for (int st = 0; st < PIPE; ++st) {
                    const int rr = r + st;
                    if (rr < r1) {
                        const int k = (rr - r0) & (kWave - 1);
#pragma unroll
                        for (int q = 0; q < NP; ++q) {
                            const float sa = wave_sum(row_partial<NG, LUT>(buf[st], lut, lane_off, xr[q], valid));
                            acc[q] = lane == k ? sa : acc[q];
                        }
                        if (k == kWave - 1 || rr == r1 - 1) {
#pragma unroll
                            for (int q = 0; q < NP; ++q)
                                if (lane <= k && pos + q < p1) ypair[(size_t)ps[q] * latent + rr - k + lane] = acc[q];
                        }
                    }
                    load_row<NG, SC2>(buf[st], m2, R(r + st + PIPE), cols);
                }
                r += PIPE;
            } while (r < r1);
        }
    }
}

// y[t][i] = sum_k wts[t][k] * ypair[inv[t*top_k+k]][i], k in route order.
__global__ __launch_bounds__(256) void combine_kernel(float *__restrict__ y, const float *__restrict__ ypair,
                                                      const float *__restrict__ wts, const int32_t *__restrict__ inv,
                                                      int n_tokens, int top_k, int latent) {
    const int t = blockIdx.y;
    const int i = (blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (t >= n_tokens || i >= latent) return;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    // in blocks of 16 pairs: all loads of a block are issued before the sums
    for (int k0 = 0; k0 < top_k; k0 += 16) {
        float w[16];
        float4 v[16];
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
            const int k = k0 + kk < top_k ? k0 + kk : top_k - 1;
            const int pos = inv ? inv[t * top_k + k] : t * top_k + k;
            // a pair past top_k, or a dropped out-of-range expert id, adds nothing
            const bool live = k0 + kk < top_k && pos >= 0;
            const float wv = wts[t * top_k + k];
            const float4 yv = *(const float4 *)(ypair + (size_t)(pos >= 0 ? pos : 0) * latent + i);
            w[kk] = live ? wv : 0.0f;
            v[kk] = live ? yv : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
            acc.x = __builtin_fmaf(w[kk], v[kk].x, acc.x);
            acc.y = __builtin_fmaf(w[kk], v[kk].y, acc.y);
            acc.z = __builtin_fmaf(w[kk], v[kk].z, acc.z);
            acc.w = __builtin_fmaf(w[kk], v[kk].w, acc.w);
        }
    }
    *(float4 *)(y + (size_t)t * latent + i) = acc;
}

// ---- host launchers ---------------------------------------------------------

static int pick_ng(int ngrp) {
    if (ngrp <= 64) return 1;
    if (ngrp <= 128) return 2;
    if (ngrp <= 256) return 4;
    return 0;
}

// The LUT forms hold 64 KB of static LDS; with x in LDS beside it they are
// above the 64 KB a kernel gets without asking.
template <typename K>
static bool allow_lds(K *kernel, bool lut, size_t dyn) {
    return !lut || dyn == 0 ||
           hipFuncSetAttribute((const void *)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn) == hipSuccess;
}

static int grid_for(int items, int waves_per_block) {
    // enough blocks to cover the items once, capped at 4 blocks per CU
    const int need = (items + waves_per_block - 1) / waves_per_block;
    return need < 1024 ? (need < 1 ? 1 : need) : 1024;
}

int launch_gemv(float *y, const float *x, const uint8_t *packed, const uint8_t *scales, int in, int rows, bool lut,
                hipStream_t st) {
    const int ngrp = in / kGroup;
    const int ng = pick_ng(ngrp);
    // rows per item: aim for ~2048 items so every SIMD of the chip has work
    // rows per item: ~2048 items, at least one pipeline's worth of rows
    int rpi = rows / 2048;
    if (rpi < K3G_PIPE) rpi = K3G_PIPE;
    const size_t xb = sizeof(float) * (size_t)in;  // x in LDS
    const int items = (rows + rpi - 1) / rpi;
    const dim3 grid(grid_for(items, K3G_GEMV_THREADS / kWave)), block(K3G_GEMV_THREADS);
    switch (ng) {
        case 1: if (!allow_lds(gemv_kernel<1, true>, lut, xb)) return K3G_EHIP; if (lut) gemv_kernel<1, true><<<grid, block, xb, st>>>(y, x, packed, scales, in, rows, rpi); else gemv_kernel<1, false><<<grid, block, xb, st>>>(y, x, packed, scales, in, rows, rpi); break;
        case 2: if (!allow_lds(gemv_kernel<2, true>, lut, xb)) return K3G_EHIP; if (lut) gemv_kernel<2, true><<<grid, block, xb, st>>>(y, x, packed, scales, in, rows, rpi); else gemv_kernel<2, false><<<grid, block, xb, st>>>(y, x, packed, scales, in, rows, rpi); break;
        case 4: if (!allow_lds(gemv_kernel<4, true>, lut, xb)) return K3G_EHIP; if (lut) gemv_kernel<4, true><<<grid, block, xb, st>>>(y, x, packed, scales, in, rows, rpi); else gemv_kernel<4, false><<<grid, block, xb, st>>>(y, x, packed, scales, in, rows, rpi); break;
        default: return K3G_EUNSUPPORTED;
    }
    return hipGetLastError() == hipSuccess ? K3G_OK : K3G_EHIP;
}

// ue8m0 -> fp32 per group, as the pages' Vulkan tier does at upload: 2^(s-127)
// exactly (s = 0 is the subnormal 2^-127), 255 (skip) -> 0.
__global__ __launch_bounds__(256) void scales_f32_kernel(float *__restrict__ out, const uint8_t *__restrict__ s,
                                                         int64_t n) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const uint32_t b = s[i];
        const uint32_t bits = b == 255u ? 0u : (b == 0u ? 0x00400000u : b << 23);
        out[i] = __builtin_bit_cast(float, bits);
    }
}

int launch_scales_f32(float *out, const uint8_t *s, int64_t n, hipStream_t st) {
    if (n == 0) return K3G_OK;
    const int64_t blocks = (n + 255) / 256;
    scales_f32_kernel<<<(unsigned)(blocks < 65536 ? blocks : 65536), 256, 0, st>>>(out, s, n);
    return hipGetLastError() == hipSuccess ? K3G_OK : K3G_EHIP;
}

int launch_gemv_f32s(float *y, const float *x, const uint8_t *packed, const float *scales, int in, int rows,
                     hipStream_t st) {
    const int ngrp = in / kGroup;
    const int ng = pick_ng(ngrp);
    // rows per item: ~2048 items, at least one pipeline's worth of rows
    int rpi = rows / 2048;
    if (rpi < K3G_PIPE) rpi = K3G_PIPE;
    const size_t xb = sizeof(float) * (size_t)in;  // x in LDS
    const int items = (rows + rpi - 1) / rpi;
    const dim3 grid(grid_for(items, K3G_GEMV_THREADS / kWave)), block(K3G_GEMV_THREADS);
    const uint8_t *sc = (const uint8_t *)scales;
    switch (ng) {
        case 1: gemv_kernel<1, false, true><<<grid, block, xb, st>>>(y, x, packed, sc, in, rows, rpi); break;
        case 2: gemv_kernel<2, false, true><<<grid, block, xb, st>>>(y, x, packed, sc, in, rows, rpi); break;
        case 4: gemv_kernel<4, false, true><<<grid, block, xb, st>>>(y, x, packed, sc, in, rows, rpi); break;
        default: return K3G_EUNSUPPORTED;
    }
    return hipGetLastError() == hipSuccess ? K3G_OK : K3G_EHIP;
}

// Rows per work item: about `target` items in all, at least one pipeline's
// worth of rows each (a single expert is cut finer than a decode step's 16).
static int rows_per_item(int max_slots, int rows, int target) {
    int rpi = (int)(((int64_t)max_slots * rows + target - 1) / target);
    if (rpi < K3G_PIPE) rpi = K3G_PIPE;
    return rpi > rows ? rows : rpi;
}

// One token: every slot has exactly one pair (top-k picks distinct experts), and
// ~2048 items. More tokens: pairs go two to a pass and the rows are cut finer
// (more slots share the chip).
int launch_moe_up_exact(float *h, const float *x, const BankDev &bank, const int32_t *active, const int32_t *offsets,
                        const int32_t *perm, int top_k, int latent, int inter, int max_slots, int n_pairs, bool lut,
                        const Route1 &rt, hipStream_t st) {
    const int ng = pick_ng(latent / kGroup);
    const bool multi = n_pairs > top_k && ng <= 2;
    const int rpi = rows_per_item(max_slots, inter, multi ? K3G_MULTI_ITEMS : K3G_ITEMS_TARGET);
    const int items = max_slots * ((inter + rpi - 1) / rpi);
    const dim3 grid(grid_for(items, K3G_GEMV_THREADS / kWave)), block(K3G_GEMV_THREADS);
    // a lane's two scale bytes as one 16-bit load when every scale row starts at an even address
    const bool sc2 = ng == 2 && (latent / kGroup) % 2 == 0 && bank.stride % 2 == 0 &&
                     ((uintptr_t)bank.base + bank.off[W1S]) % 2 == 0 && ((uintptr_t)bank.base + bank.off[W3S]) % 2 == 0;
#define K3G_UP(NG_, LUT_, NP_)                                                                                     \
    do {                                                                                                           \
        if (NG_ == 2 && sc2)                                                                                       \
            moe_up_exact_kernel<NG_, LUT_, NP_, true><<<grid, block, 0, st>>>(h, x, bank, active, offsets, perm,   \
                                                                             top_k, latent, inter, max_slots, rpi, rt); \
        else                                                                                                       \
            moe_up_exact_kernel<NG_, LUT_, NP_, false><<<grid, block, 0, st>>>(h, x, bank, active, offsets, perm,  \
                                                                              top_k, latent, inter, max_slots, rpi, rt); \
    } while (0)
    switch (ng * 4 + (multi ? 2 : 0) + (lut ? 1 : 0)) {
        case 4: K3G_UP(1, false, 1); break;
        case 5: K3G_UP(1, true, 1); break;
        case 6: K3G_UP(1, false, K3G_MULTI_NP); break;
        case 7: K3G_UP(1, true, K3G_MULTI_NP); break;
        case 8: K3G_UP(2, false, 1); break;
        case 9: K3G_UP(2, true, 1); break;
        case 10: K3G_UP(2, false, K3G_MULTI_NP); break;
        case 11: K3G_UP(2, true, K3G_MULTI_NP); break;
        case 16: K3G_UP(4, false, 1); break;
        case 17: K3G_UP(4, true, 1); break;
        default: return K3G_EUNSUPPORTED;
    }
#undef K3G_UP
    return hipGetLastError() == hipSuccess ? K3G_OK : K3G_EHIP;
}

int launch_moe_down_exact(float *ypair, const float *h, const BankDev &bank, const int32_t *active,
                          const int32_t *offsets, const int32_t *perm, int latent, int inter, int max_slots,
                          bool multi_pairs, bool lut, hipStream_t st) {
    const int ng = pick_ng(inter / kGroup);
    const bool multi = multi_pairs && ng <= 2;
    const int rpi = rows_per_item(max_slots, latent, multi ? K3G_MULTI_ITEMS : K3G_ITEMS_TARGET);
    const int items = max_slots * ((latent + rpi - 1) / rpi);
    const dim3 grid(grid_for(items, K3G_GEMV_THREADS / kWave)), block(K3G_GEMV_THREADS);
    const bool sc2 = ng == 2 && (inter / kGroup) % 2 == 0 && bank.stride % 2 == 0 &&
                     ((uintptr_t)bank.base + bank.off[W2S]) % 2 == 0;
#define K3G_DN(NG_, LUT_, NP_)                                                                                      \
    do {                                                                                                            \
        if (NG_ == 2 && sc2)                                                                                        \
            moe_down_exact_kernel<NG_, LUT_, NP_, true><<<grid, block, 0, st>>>(ypair, h, bank, active, offsets,    \
                                                                               perm, latent, inter, max_slots, rpi); \
        else                                                                                                        \
            moe_down_exact_kernel<NG_, LUT_, NP_, false><<<grid, block, 0, st>>>(ypair, h, bank, active, offsets,   \
                                                                                perm, latent, inter, max_slots, rpi); \
    } while (0)
    switch (ng * 4 + (multi ? 2 : 0) + (lut ? 1 : 0)) {
        case 4: K3G_DN(1, false, 1); break;
        case 5: K3G_DN(1, true, 1); break;
        case 6: K3G_DN(1, false, K3G_MULTI_NP); break;
        case 7: K3G_DN(1, true, K3G_MULTI_NP); break;
        case 8: K3G_DN(2, false, 1); break;
        case 9: K3G_DN(2, true, 1); break;
        case 10: K3G_DN(2, false, K3G_MULTI_NP); break;
        case 11: K3G_DN(2, true, K3G_MULTI_NP); break;
        case 16: K3G_DN(4, false, 1); break;
        case 17: K3G_DN(4, true, 1); break;
        default: return K3G_EUNSUPPORTED;
    }
#undef K3G_DN
    return hipGetLastError() == hipSuccess ? K3G_OK : K3G_EHIP;
}

int launch_combine(float *y, const float *ypair, const float *wts, const int32_t *inv, int n_tokens, int top_k,
                   int latent, hipStream_t st) {
    if (n_tokens == 0) return K3G_OK;
    const dim3 block(256);
    const dim3 grid((latent / 4 + 255) / 256, n_tokens);
    combine_kernel<<<grid, block, 0, st>>>(y, ypair, wts, inv, n_tokens, top_k, latent);
    return hipGetLastError() == hipSuccess ? K3G_OK : K3G_EHIP;
}

}  // namespace k3g
