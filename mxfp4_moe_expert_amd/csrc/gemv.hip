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

namespace k3g {

template <int NG>
struct RowData {
    uint4 w[NG];
    uint32_t s[NG];
};

// Loads are unconditional so that the compiler can count them: a lane past
// the last group reads group ngrp-1 again, and row_partial drops it (the
// lane's `valid` bits).
template <int NG>
__device__ inline void load_row(RowData<NG> &d, const uint8_t *prow, const uint8_t *srow, int lane, int ngrp) {
#pragma unroll
    for (int i = 0; i < NG; ++i) {
        const int g = lane * NG + i;
        const int gc = g < ngrp ? g : ngrp - 1;
        d.w[i] = load16(prow + (size_t)gc * 16);
        d.s[i] = srow[gc];
    }
}

template <int NG>
__device__ inline float row_partial(const RowData<NG> &d, const uint32_t *lut, uint32_t lane_off, const float *xr,
                                   uint32_t valid) {
    float p = 0.f;
#pragma unroll
    for (int i = 0; i < NG; ++i) {
        const float sub = group_dot(lut, lane_off, d.w[i], xr + i * kGroup);
        p += ((valid >> i) & 1u) ? apply_scale(sub, d.s[i]) : 0.0f;
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

// y[r] for r in [0, rows): one matrix, one x. Items of rpi rows.
template <int NG>
__global__ __launch_bounds__(256) void gemv_kernel(float *__restrict__ y, const float *__restrict__ x,
                                                   const uint8_t *__restrict__ packed,
                                                   const uint8_t *__restrict__ scales, int in, int rows, int rpi) {
    __shared__ uint32_t lut[kLutWords];
    build_pair_lut(lut);
    __syncthreads();
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int waves = blockDim.x / kWave;
    const uint32_t lane_off = uint32_t(lane) << 2;
    const int ngrp = in / kGroup;
    const size_t rowbytes = (size_t)in / 2;
    const uint32_t valid = valid_groups<NG>(lane, ngrp);
    float xr[NG * kGroup];
    load_x<NG>(xr, x, lane, ngrp);
    const int n_items = (rows + rpi - 1) / rpi;
    for (int item = blockIdx.x * waves + wave; item < n_items; item += gridDim.x * waves) {
        const int r0 = item * rpi;
        const int r1 = min(rows, r0 + rpi);
        auto P = [&](int r) { return packed + (size_t)min(r, r1 - 1) * rowbytes; };
        auto Q = [&](int r) { return scales + (size_t)min(r, r1 - 1) * ngrp; };
        RowData<NG> a, b;
        load_row<NG>(a, P(r0), Q(r0), lane, ngrp);
        load_row<NG>(b, P(r0 + 1), Q(r0 + 1), lane, ngrp);
        for (int r = r0; r < r1; r += 2) {
            const float sa = wave_sum(row_partial<NG>(a, lut, lane_off, xr, valid));
            load_row<NG>(a, P(r + 2), Q(r + 2), lane, ngrp);
            if (lane == 0) y[r] = sa;
            if (r + 1 < r1) {
                const float sb = wave_sum(row_partial<NG>(b, lut, lane_off, xr, valid));
                if (lane == 0) y[r + 1] = sb;
            }
            load_row<NG>(b, P(r + 3), Q(r + 3), lane, ngrp);
        }
    }
}

// Grouped SiTU-GLU up-projection. Work item = (slot, run of rpi rows); slot i
// is the i-th expert that has pairs (active[1+i]); its pairs are the sorted
// positions [offsets[e], offsets[e+1]), token = perm[pos] / top_k. For each
// pair and row r: g = w1[r].x, u = w3[r].x, h[pos][r] = SiTU(g, u).
// With perm == nullptr the call is one expert (bank expert 0) on token 0.
template <int NG>
__global__ __launch_bounds__(256) void moe_up_exact_kernel(
    float *__restrict__ h, const float *__restrict__ x, BankDev bank, const int32_t *__restrict__ active,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ perm, int top_k, int latent, int inter,
    int max_slots, int rpi) {
    __shared__ uint32_t lut[kLutWords];
    build_pair_lut(lut);
    __syncthreads();
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int waves = blockDim.x / kWave;
    const uint32_t lane_off = uint32_t(lane) << 2;
    const int ngrp = latent / kGroup;
    const size_t rowbytes = (size_t)latent / 2;
    const uint32_t valid = valid_groups<NG>(lane, ngrp);
    const int chunks = (inter + rpi - 1) / rpi;
    const int n_act = perm ? active[0] : 1;
    const int n_items = max_slots * chunks;
    float xr[NG * kGroup];
    for (int item = blockIdx.x * waves + wave; item < n_items; item += gridDim.x * waves) {
        const int slot = item / chunks;
        if (slot >= n_act) continue;
        const int chunk = item - slot * chunks;
        const int e = perm ? active[1 + slot] : 0;
        const int p0 = perm ? offsets[e] : 0;
        const int p1 = perm ? offsets[e + 1] : 1;
        const uint8_t *eb = bank.base + (int64_t)e * bank.stride;
        const uint8_t *w1p = eb + bank.off[W1P], *w1s = eb + bank.off[W1S];
        const uint8_t *w3p = eb + bank.off[W3P], *w3s = eb + bank.off[W3S];
        const int r0 = chunk * rpi;
        const int r1 = min(inter, r0 + rpi);
        auto P1 = [&](int r) { return w1p + (size_t)min(r, r1 - 1) * rowbytes; };
        auto S1 = [&](int r) { return w1s + (size_t)min(r, r1 - 1) * ngrp; };
        auto P3 = [&](int r) { return w3p + (size_t)min(r, r1 - 1) * rowbytes; };
        auto S3 = [&](int r) { return w3s + (size_t)min(r, r1 - 1) * ngrp; };
        for (int pos = p0; pos < p1; ++pos) {
            const int t = perm ? perm[pos] / top_k : 0;
            load_x<NG>(xr, x + (size_t)t * latent, lane, ngrp);
            RowData<NG> a1, a3, b1, b3;
            load_row<NG>(a1, P1(r0), S1(r0), lane, ngrp);
            load_row<NG>(a3, P3(r0), S3(r0), lane, ngrp);
            load_row<NG>(b1, P1(r0 + 1), S1(r0 + 1), lane, ngrp);
            load_row<NG>(b3, P3(r0 + 1), S3(r0 + 1), lane, ngrp);
            for (int r = r0; r < r1; r += 2) {
                const float ga = wave_sum(row_partial<NG>(a1, lut, lane_off, xr, valid));
                const float ua = wave_sum(row_partial<NG>(a3, lut, lane_off, xr, valid));
                load_row<NG>(a1, P1(r + 2), S1(r + 2), lane, ngrp);
                load_row<NG>(a3, P3(r + 2), S3(r + 2), lane, ngrp);
                if (lane == 0) h[(size_t)pos * inter + r] = situ(ga, ua);
                if (r + 1 < r1) {
                    const float gb = wave_sum(row_partial<NG>(b1, lut, lane_off, xr, valid));
                    const float ub = wave_sum(row_partial<NG>(b3, lut, lane_off, xr, valid));
                    if (lane == 0) h[(size_t)pos * inter + r + 1] = situ(gb, ub);
                }
                load_row<NG>(b1, P1(r + 3), S1(r + 3), lane, ngrp);
                load_row<NG>(b3, P3(r + 3), S3(r + 3), lane, ngrp);
            }
        }
    }
}

// Grouped down-projection: ypair[pos][r] = w2[r] . h[pos] for every pair of
// the slot's expert. Same items as the up kernel, over latent rows.
template <int NG>
__global__ __launch_bounds__(256) void moe_down_exact_kernel(
    float *__restrict__ ypair, const float *__restrict__ h, BankDev bank, const int32_t *__restrict__ active,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ perm, int latent, int inter,
    int max_slots, int rpi) {
    __shared__ uint32_t lut[kLutWords];
    build_pair_lut(lut);
    __syncthreads();
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int waves = blockDim.x / kWave;
    const uint32_t lane_off = uint32_t(lane) << 2;
    const int ngrp = inter / kGroup;
    const size_t rowbytes = (size_t)inter / 2;
    const uint32_t valid = valid_groups<NG>(lane, ngrp);
    const int chunks = (latent + rpi - 1) / rpi;
    const int n_act = perm ? active[0] : 1;
    const int n_items = max_slots * chunks;
    float xr[NG * kGroup];
    for (int item = blockIdx.x * waves + wave; item < n_items; item += gridDim.x * waves) {
        const int slot = item / chunks;
        if (slot >= n_act) continue;
        const int chunk = item - slot * chunks;
        const int e = perm ? active[1 + slot] : 0;
        const int p0 = perm ? offsets[e] : 0;
        const int p1 = perm ? offsets[e + 1] : 1;
        const uint8_t *eb = bank.base + (int64_t)e * bank.stride;
        const uint8_t *w2p = eb + bank.off[W2P], *w2s = eb + bank.off[W2S];
        const int r0 = chunk * rpi;
        const int r1 = min(latent, r0 + rpi);
        auto P2 = [&](int r) { return w2p + (size_t)min(r, r1 - 1) * rowbytes; };
        auto S2 = [&](int r) { return w2s + (size_t)min(r, r1 - 1) * ngrp; };
        for (int pos = p0; pos < p1; ++pos) {
            load_x<NG>(xr, h + (size_t)pos * inter, lane, ngrp);
            RowData<NG> a, b;
            load_row<NG>(a, P2(r0), S2(r0), lane, ngrp);
            load_row<NG>(b, P2(r0 + 1), S2(r0 + 1), lane, ngrp);
            for (int r = r0; r < r1; r += 2) {
                const float sa = wave_sum(row_partial<NG>(a, lut, lane_off, xr, valid));
                load_row<NG>(a, P2(r + 2), S2(r + 2), lane, ngrp);
                if (lane == 0) ypair[(size_t)pos * latent + r] = sa;
                if (r + 1 < r1) {
                    const float sb = wave_sum(row_partial<NG>(b, lut, lane_off, xr, valid));
                    if (lane == 0) ypair[(size_t)pos * latent + r + 1] = sb;
                }
                load_row<NG>(b, P2(r + 3), S2(r + 3), lane, ngrp);
            }
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

static int grid_for(int items, int waves_per_block) {
    // enough blocks to cover the items once, capped at 4 blocks per CU
    const int need = (items + waves_per_block - 1) / waves_per_block;
    return need < 1024 ? (need < 1 ? 1 : need) : 1024;
}

int launch_gemv(float *y, const float *x, const uint8_t *packed, const uint8_t *scales, int in, int rows,
                hipStream_t st) {
    const int ngrp = in / kGroup;
    const int ng = pick_ng(ngrp);
    // rows per item: aim for ~2048 items so every SIMD of the chip has work
    int rpi = rows / 2048;
    if (rpi < 2) rpi = 2;
    const int items = (rows + rpi - 1) / rpi;
    const dim3 grid(grid_for(items, 4)), block(256);
    switch (ng) {
        case 1: gemv_kernel<1><<<grid, block, 0, st>>>(y, x, packed, scales, in, rows, rpi); break;
        case 2: gemv_kernel<2><<<grid, block, 0, st>>>(y, x, packed, scales, in, rows, rpi); break;
        case 4: gemv_kernel<4><<<grid, block, 0, st>>>(y, x, packed, scales, in, rows, rpi); break;
        default: return K3G_EUNSUPPORTED;
    }
    return hipGetLastError() == hipSuccess ? K3G_OK : K3G_EHIP;
}

int launch_moe_up_exact(float *h, const float *x, const BankDev &bank, const int32_t *active, const int32_t *offsets,
                        const int32_t *perm, int top_k, int latent, int inter, int max_slots, int n_pairs,
                        hipStream_t st) {
    const int ng = pick_ng(latent / kGroup);
    // rows per item: about 2048 items in all when each expert has one pair
    int rpi = (int)(((int64_t)max_slots * inter + 2047) / 2048);
    if (rpi < 8) rpi = 8;
    if (rpi > inter) rpi = inter;
    (void)n_pairs;
    const int items = max_slots * ((inter + rpi - 1) / rpi);
    const dim3 grid(grid_for(items, 4)), block(256);
    switch (ng) {
        case 1: moe_up_exact_kernel<1><<<grid, block, 0, st>>>(h, x, bank, active, offsets, perm, top_k, latent, inter, max_slots, rpi); break;
        case 2: moe_up_exact_kernel<2><<<grid, block, 0, st>>>(h, x, bank, active, offsets, perm, top_k, latent, inter, max_slots, rpi); break;
        case 4: moe_up_exact_kernel<4><<<grid, block, 0, st>>>(h, x, bank, active, offsets, perm, top_k, latent, inter, max_slots, rpi); break;
        default: return K3G_EUNSUPPORTED;
    }
    return hipGetLastError() == hipSuccess ? K3G_OK : K3G_EHIP;
}

int launch_moe_down_exact(float *ypair, const float *h, const BankDev &bank, const int32_t *active,
                          const int32_t *offsets, const int32_t *perm, int latent, int inter, int max_slots,
                          hipStream_t st) {
    const int ng = pick_ng(inter / kGroup);
    int rpi = (int)(((int64_t)max_slots * latent + 2047) / 2048);
    if (rpi < 8) rpi = 8;
    if (rpi > latent) rpi = latent;
    const int items = max_slots * ((latent + rpi - 1) / rpi);
    const dim3 grid(grid_for(items, 4)), block(256);
    switch (ng) {
        case 1: moe_down_exact_kernel<1><<<grid, block, 0, st>>>(ypair, h, bank, active, offsets, perm, latent, inter, max_slots, rpi); break;
        case 2: moe_down_exact_kernel<2><<<grid, block, 0, st>>>(ypair, h, bank, active, offsets, perm, latent, inter, max_slots, rpi); break;
        case 4: moe_down_exact_kernel<4><<<grid, block, 0, st>>>(ypair, h, bank, active, offsets, perm, latent, inter, max_slots, rpi); break;
        default: return K3G_EUNSUPPORTED;
    }
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
