// idot.hip -- the IDOT path: int8 activations against doubled e2m1 values on
// the matrix cores (gfx950).
//
// "Kimi K3 engine (c/kimi_k3.c)", section "Streaming design" (K3_IDOT): the
// expert products take per-32-group int8-quantised activations and integer
// dots against the e2m1 values doubled, which are exact int8 (-12..12). Each
// group dot is an exact int32; the float scales come after:
//   y[r] = sum_g [s_rg != 255] I_rg * s_x[g] * 2^(s_rg - 128),
// where 2^(s-128) = 2^(s-127)/2 undoes the doubling.
#include "k3g_common.h"

namespace k3g {

// ---- activation quantisation: one thread per (row, group) --------------------
// s = max|x|/127 in fp32 (correctly rounded division), q = rint(x/s) clamped
// to +-127 (ties to even); an all-zero group gives s = 0 and q = 0.
__global__ __launch_bounds__(256) void quant_i8_kernel(int8_t *__restrict__ q, float *__restrict__ s,
                                                       const float *__restrict__ x, int n_rows, int in) {
    const int ngrp = in / kGroup;
    const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (id >= (int64_t)n_rows * ngrp) return;
    const float *xg = x + id * kGroup;
    float v[kGroup];
#pragma unroll
    for (int j = 0; j < kGroup; j += 4) {
        const float4 f = *(const float4 *)(xg + j);
        v[j] = f.x; v[j + 1] = f.y; v[j + 2] = f.z; v[j + 3] = f.w;
    }
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < kGroup; ++j) amax = fmaxf(amax, fabsf(v[j]));
    uint32_t packed[kGroup / 4];
    if (amax == 0.f) {
        s[id] = 0.f;
#pragma unroll
        for (int j = 0; j < kGroup / 4; ++j) packed[j] = 0u;
    } else {
        const float sc = amax / 127.0f;
        s[id] = sc;
#pragma unroll
        for (int j = 0; j < kGroup / 4; ++j) {
            uint32_t w = 0;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const float r = fminf(fmaxf(rintf(v[4 * j + b] / sc), -127.f), 127.f);
                w |= (uint32_t)((int32_t)r & 0xff) << (8 * b);
            }
            packed[j] = w;
        }
    }
    uint4 *dst = (uint4 *)(q + id * kGroup);
    dst[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    dst[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
}

int launch_quant_i8(int8_t *q, float *s, const float *x, int n_rows, int in, hipStream_t st) {
    const int64_t n = (int64_t)n_rows * (in / kGroup);
    if (n == 0) return K3G_OK;
    const int blocks = (int)((n + 255) / 256);
    quant_i8_kernel<<<blocks, 256, 0, st>>>(q, s, x, n_rows, in);
    return hipGetLastError() == hipSuccess ? K3G_OK : K3G_EHIP;
}

}  // namespace k3g

namespace k3g {

// ---- decode: 8 packed bytes -> 16 doubled e2m1 values as int8 ----------------
// Magnitude code m = nibble & 7 -> 2*e2m1 = {0,1,2,3,4,6,8,12}; sign = bit 3.
// v_perm_b32 looks the magnitudes up in an 8-byte table (selectors 0..7), a
// second table holds the negatives, and a third perm turns the sign bits into
// a 0x00/0xFF byte mask (selector 12 -> 0x00, 13 -> 0xFF).
__device__ inline uint32_t dbl_e2m1_x4(uint32_t n /* 4 nibbles, one per byte */) {
    const uint32_t mag = n & 0x07070707u;
    const uint32_t pos = __builtin_amdgcn_perm(0x0C080604u, 0x03020100u, mag);
    const uint32_t neg = __builtin_amdgcn_perm(0xF4F8FAFCu, 0xFDFEFF00u, mag);
    const uint32_t sel = ((n >> 3) & 0x01010101u) | 0x0C0C0C0Cu;
    const uint32_t msk = __builtin_amdgcn_perm(0u, 0u, sel);
    return (neg & msk) | (pos & ~msk);
}

// Packed bytes b0..b3 (column pairs 2j, 2j+1) -> 8 int8 in column order:
// out0 = [d(b0.lo), d(b0.hi), d(b1.lo), d(b1.hi)], out1 = the same for b2, b3.
__device__ inline void decode8(uint32_t w, uint32_t &out0, uint32_t &out1) {
    const uint32_t lo = dbl_e2m1_x4(w & 0x0F0F0F0Fu);
    const uint32_t hi = dbl_e2m1_x4((w >> 4) & 0x0F0F0F0Fu);
    out0 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
    out1 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
}

// B operand of one group for this lane: weight row n = lane%32, columns
// 16h..16h+15 of the group (h = lane/32) = packed bytes 8h..8h+7.
__device__ inline int4_t decode_b(uint2 pk) {
    uint32_t a, b, c, d;
    decode8(pk.x, a, b);
    decode8(pk.y, c, d);
    int4_t r;
    r[0] = (int)a; r[1] = (int)b; r[2] = (int)c; r[3] = (int)d;
    return r;
}

// One 32x32x32 int8 product: rows = 32 tokens (A), columns = 32 weight rows
// (B), k = the group's 32 columns. Lane l of the result holds column l%32 and
// rows 8*(v/4) + 4*(l/32) + v%4 for v = 0..15.
__device__ inline int16_t_v mfma_group(int4_t a, int4_t b) {
    int16_t_v z = {};
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, z, 0, 0, 0);
}

__device__ inline int out_row(int lane, int v) { return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3); }

// ---- the integer group sums, as a stage hook ----------------------------------
// sums[t][r][g] for a tile of 32 tokens x 32 rows per wavefront and group.
__global__ __launch_bounds__(256) void idot_groupsums_kernel(int32_t *__restrict__ sums, const int8_t *__restrict__ q,
                                                             const uint8_t *__restrict__ packed, int in, int rows,
                                                             int n_tokens) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane((blockIdx.x * blockDim.x + threadIdx.x) / kWave);
    const int ngrp = in / kGroup;
    const int row_tiles = (rows + 31) / 32, tok_tiles = (n_tokens + 31) / 32;
    const int n_items = row_tiles * tok_tiles;
    const int half = lane >> 5;
    const rsrc_t rp = make_rsrc(packed, (uint32_t)rows * (uint32_t)(in / 2));
    for (int item = wave; item < n_items; item += gridDim.x * blockDim.x / kWave) {
        const int rt = item % row_tiles, tt = item / row_tiles;
        const int row = min(rt * 32 + (lane & 31), rows - 1);
        const int tok = min(tt * 32 + (lane & 31), n_tokens - 1);
        for (int g = 0; g < ngrp; ++g) {
            const uint32_t off = (uint32_t)row * (uint32_t)(in / 2) + (uint32_t)(g * 16 + half * 8);
            const auto raw = __builtin_amdgcn_raw_buffer_load_b64(rp, (int)off, 0, 0);
            const int4_t b = decode_b(make_uint2(raw[0], raw[1]));
            const int4_t a = *(const int4_t *)(q + (size_t)tok * in + g * kGroup + half * 16);
            const int16_t_v I = mfma_group(a, b);
            const int r_out = rt * 32 + (lane & 31);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int t_out = tt * 32 + out_row(lane, v);
                if (r_out < rows && t_out < n_tokens) sums[((size_t)t_out * rows + r_out) * ngrp + g] = I[v];
            }
        }
    }
}

int launch_idot_groupsums(int32_t *sums, const int8_t *q, const uint8_t *packed, int in, int rows, int n_tokens,
                          hipStream_t st) {
    if (n_tokens == 0) return K3G_OK;
    const int items = ((rows + 31) / 32) * ((n_tokens + 31) / 32);
    const int blocks = (items + 3) / 4 < 2048 ? (items + 3) / 4 : 2048;
    idot_groupsums_kernel<<<blocks, 256, 0, st>>>(sums, q, packed, in, rows, n_tokens);
    return hipGetLastError() == hipSuccess ? K3G_OK : K3G_EHIP;
}

// ---- the grouped IDOT expert kernels ---------------------------------------------
// Work item = (slot, block of weight rows); the wavefront loops over its
// expert's pairs in chunks of up to 32*IT_NT tokens. Per group and token tile
// one MFMA gives the int32 group dots I for 32 weight rows; the epilogue adds
// float(I) * (s_x[token][g] * 2^(s_rg - 128)) in fp32 (nothing for s_rg = 255).
// UP: the 32 MFMA columns are 16 rows of w1 and the same 16 rows of w3, so one
//     product yields g and u; h = SiTU(g, u) is written to h[pos][row].
// DOWN: 32 rows of w2 on the quantised h of each pair -> ypair[pos][row].
// Each lane keeps pointers to its own weight row (w1 or w3 for UP). Token
// scales of 8 groups at a time are staged in LDS.
constexpr int IT_NT = 4;  // token tiles (of 32) per chunk
constexpr int IT_KC = 8;  // groups whose token scales are staged together

template <bool UP>
__global__ __launch_bounds__(256) void moe_idot_kernel(float *__restrict__ out, const int8_t *__restrict__ aq,
                                                      const float *__restrict__ as, BankDev bank,
                                                      const int32_t *__restrict__ active,
                                                      const int32_t *__restrict__ offsets,
                                                      const int32_t *__restrict__ perm, int top_k, int n_in, int n_out,
                                                      int max_slots) {
    __shared__ float ts_lds[4][IT_KC][IT_NT * 32];
    const int lane = threadIdx.x & (kWave - 1);
    const int wl = threadIdx.x / kWave;
    const int wave = __builtin_amdgcn_readfirstlane(blockIdx.x * (blockDim.x / kWave) + wl);
    const int n_waves = gridDim.x * blockDim.x / kWave;
    const int half = lane >> 5;
    const int col = lane & 31;                 // MFMA column of this lane
    const int ngrp = n_in / kGroup;
    constexpr int ROWS = UP ? 16 : 32;        // weight rows per item
    const int row_tiles = (n_out + ROWS - 1) / ROWS;
    const int n_act = perm ? active[0] : 1;
    const int n_items = max_slots * row_tiles;
    float(*ts)[IT_NT * 32] = ts_lds[wl];
    // which matrix and row this lane's column is
    const int mat_p = UP ? (col < 16 ? W1P : W3P) : W2P;
    const int mat_s = UP ? (col < 16 ? W1S : W3S) : W2S;
    for (int item = wave; item < n_items; item += n_waves) {
        const int slot = item / row_tiles;
        if (slot >= n_act) continue;
        const int rt = item - slot * row_tiles;
        const int e = perm ? active[1 + slot] : 0;
        const int p0 = perm ? offsets[e] : 0;
        const int p1 = perm ? offsets[e + 1] : 1;
        const uint8_t *eb = bank.base + (int64_t)e * bank.stride;
        const int rr = rt * ROWS + (UP ? (col & 15) : col);
        const int row = min(rr, n_out - 1);
        const uint8_t *wrow = eb + bank.off[mat_p] + (size_t)row * (n_in / 2) + half * 8;
        const uint8_t *srow = eb + bank.off[mat_s] + (size_t)row * ngrp;
        for (int c0 = p0; c0 < p1; c0 += IT_NT * 32) {
            const int n_tok = min(p1 - c0, IT_NT * 32);
            const int n_tiles = (n_tok + 31) / 32;
            const int8_t *arow[IT_NT];
#pragma unroll
            for (int tt = 0; tt < IT_NT; ++tt) {
                const int pos = c0 + min(tt * 32 + col, n_tok - 1);
                const int ar = UP ? (perm ? perm[pos] / top_k : 0) : pos;
                arow[tt] = aq + (size_t)ar * n_in + half * 16;
            }
            int srow_a[2];
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int pos = c0 + min(2 * lane + k, n_tok - 1);
                srow_a[k] = (UP ? (perm ? perm[pos] / top_k : 0) : pos) * ngrp;
            }
            float acc[IT_NT][16];
#pragma unroll
            for (int tt = 0; tt < IT_NT; ++tt)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[tt][v] = 0.f;
            // group 0's operands
            auto ld_b = [&](int g, uint2 &pk, uint32_t &sc) {
                pk = *(const uint2 *)(wrow + g * 16);
                sc = srow[g];
            };
            uint2 pk_n;
            uint32_t sc_n;
            int4_t a_n[IT_NT];
            ld_b(0, pk_n, sc_n);
#pragma unroll
            for (int tt = 0; tt < IT_NT; ++tt) a_n[tt] = *(const int4_t *)(arow[tt]);
            for (int g0 = 0; g0 < ngrp; g0 += IT_KC) {
                const int kc = min(IT_KC, ngrp - g0);
                // stage the token scales of groups g0..g0+kc-1
                __builtin_amdgcn_wave_barrier();
                for (int j = 0; j < kc; ++j) {
                    ts[j][2 * lane] = as[srow_a[0] + g0 + j];
                    ts[j][2 * lane + 1] = as[srow_a[1] + g0 + j];
                }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                for (int j = 0; j < kc; ++j) {
                    const int g = g0 + j;
                    const uint2 pk = pk_n;
                    const uint32_t sc = sc_n;
                    int4_t a[IT_NT];
#pragma unroll
                    for (int tt = 0; tt < IT_NT; ++tt) a[tt] = a_n[tt];
                    // prefetch group g+1 (the last group reloads itself)
                    const int gn = g + 1 < ngrp ? g + 1 : g;
                    ld_b(gn, pk_n, sc_n);
#pragma unroll
                    for (int tt = 0; tt < IT_NT; ++tt) a_n[tt] = *(const int4_t *)(arow[tt] + gn * kGroup);
                    const int4_t b = decode_b(pk);
                    const float ws = sc == 255u ? 0.0f : __builtin_ldexpf(1.0f, (int)sc - 128);
#pragma unroll
                    for (int tt = 0; tt < IT_NT; ++tt) {
                        if (tt < n_tiles) {
                            const int16_t_v I = mfma_group(a[tt], b);
#pragma unroll
                            for (int v = 0; v < 16; ++v) {
                                const float sx = ts[j][tt * 32 + out_row(lane, v)];
                                acc[tt][v] = __builtin_fmaf((float)I[v], sx * ws, acc[tt][v]);
                            }
                        }
                    }
                }
            }
#pragma unroll
            for (int tt = 0; tt < IT_NT; ++tt) {
                if (tt < n_tiles) {
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int i = tt * 32 + out_row(lane, v);
                        float val = acc[tt][v];
                        if (UP) {
                            // lane col (< 16) holds g of row rr, lane col+16 holds u of the same row
                            const float other = __shfl_xor(val, 16, kWave);
                            val = situ(val, other);
                        }
                        const bool mine = UP ? (col < 16) : true;
                        if (mine && i < n_tok && rr < n_out) out[(size_t)(c0 + i) * n_out + rr] = val;
                    }
                }
            }
        }
    }
}

int launch_moe_up_idot(float *h, const int8_t *xq, const float *xs, const BankDev &bank, const int32_t *active,
                       const int32_t *offsets, const int32_t *perm, int top_k, int latent, int inter, int max_slots,
                       hipStream_t st) {
    const int items = max_slots * ((inter + 15) / 16);
    const int blocks = (items + 3) / 4 < 8192 ? (items + 3) / 4 : 8192;
    moe_idot_kernel<true><<<blocks, 256, 0, st>>>(h, xq, xs, bank, active, offsets, perm, top_k, latent, inter,
                                                  max_slots);
    return hipGetLastError() == hipSuccess ? K3G_OK : K3G_EHIP;
}

int launch_moe_down_idot(float *ypair, const int8_t *hq, const float *hs, const BankDev &bank, const int32_t *active,
                         const int32_t *offsets, const int32_t *perm, int latent, int inter, int max_slots,
                         hipStream_t st) {
    const int items = max_slots * ((latent + 31) / 32);
    const int blocks = (items + 3) / 4 < 8192 ? (items + 3) / 4 : 8192;
    moe_idot_kernel<false><<<blocks, 256, 0, st>>>(ypair, hq, hs, bank, active, offsets, perm, 1, inter, latent,
                                                   max_slots);
    return hipGetLastError() == hipSuccess ? K3G_OK : K3G_EHIP;
}

}  // namespace k3g
