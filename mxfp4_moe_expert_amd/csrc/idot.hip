// idot.hip -- the IDOT path: int8 activations against doubled e2m1 values on
// the matrix cores (gfx950).
//
// "Kimi K3 engine (c/kimi_k3.c)", section "Streaming design" (K3_IDOT): the
// expert products take per-32-group int8-quantised activations and integer
// dots against the e2m1 values doubled, which are exact int8 (-12..12). Each
// group dot is an exact int32; the float scales come after:
//   y[r] = sum_g [s_rg != 255] I_rg * s_x[g] * 2^(s_rg - 128),
// where 2^(s-128) = 2^(s-127)/2 undoes the doubling.
#include <type_traits>

#include "k3g_common.h"

namespace k3g {

// ---- activation quantisation: one thread per (row, group) --------------------
// s = max|x|/127 in fp32 (correctly rounded division), q = rint(x/s) clamped
// to +-127 (ties to even); an all-zero group gives s = 0 and q = 0.
// qb (optional): the same q as bf16 bit patterns (exact), for the bf16 MFMA form.
__global__ __launch_bounds__(256) void quant_i8_kernel(int8_t *__restrict__ q, float *__restrict__ s,
                                                       const float *__restrict__ x, int n_rows, int in,
                                                       uint16_t *__restrict__ qb) {
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
    if (qb) {
        // an int8 value has at most 8 significant bits: its fp32 form truncated to bf16 is exact
        uint32_t hb[kGroup / 2];
#pragma unroll
        for (int j = 0; j < kGroup / 2; ++j) {
            const int b0 = (int8_t)(packed[j / 2] >> (16 * (j & 1)));
            const int b1 = (int8_t)(packed[j / 2] >> (16 * (j & 1) + 8));
            hb[j] = (__builtin_bit_cast(uint32_t, (float)b0) >> 16) | (__builtin_bit_cast(uint32_t, (float)b1) & 0xFFFF0000u);
        }
        uint4 *db = (uint4 *)(qb + id * kGroup);
#pragma unroll
        for (int j = 0; j < 4; ++j) db[j] = make_uint4(hb[4 * j], hb[4 * j + 1], hb[4 * j + 2], hb[4 * j + 3]);
    }
}

int launch_quant_i8(int8_t *q, float *s, const float *x, int n_rows, int in, uint16_t *qb, hipStream_t st) {
    const int64_t n = (int64_t)n_rows * (in / kGroup);
    if (n == 0) return K3G_OK;
    const int blocks = (int)((n + 255) / 256);
    quant_i8_kernel<<<blocks, 256, 0, st>>>(q, s, x, n_rows, in, qb);
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
// Work item = (slot, block of weight rows), one per workgroup of IX_WAVES
// wavefronts; the workgroup loops over its expert's pairs in chunks of up to
// 32*IX_NT tokens. Each wavefront owns 32 weight rows (operand A) and meets
// every token tile of the chunk (operand B, 32 tokens); lane l of a result
// holds token l%32 and rows 8*(v/4) + 4*(l/32) + v%4.
// One v_mfma_i32_32x32x32_i8 per group and tile on the int8 activations and
// the doubled e2m1 values gives the int32 group dots I; the epilogue adds
// float(I) * (s_x[token][g] * 2^(s_rg - 128)). A scale byte of 255 contributes
// nothing. (The bf16 matrix-core form of the same products, whose epilogue is
// one fma per result, lives in idot_bf16.hip.)
// UP: a wavefront's 32 rows are 16 rows of w1 (result slots 0..7) and the same
//     16 rows of w3 (slots 8..15): g and u of a row meet in one lane and
//     h = SiTU(g, u) goes to h[pos][row].
// DOWN: 32 rows of w2 per wavefront on the quantised h of each pair.
//
// Operands reach LDS without passing through registers (global_load_lds:
// lane l's 16 or 4 bytes land at the instruction's LDS base + 16*l or 4*l),
// in blocks of GB groups, double-buffered: the next block is requested before
// the current one is computed. Every load instruction reads rows of a block
// whole (a run of lanes per row), and each row in LDS is padded by one 16-byte
// chunk, so that the 16 rows a fragment read touches in one cycle start in
// distinct banks and every fragment address is a per-lane base plus a constant:
//   tokens  [token m][chunks of the block + 1]
//   weights [row r][GB + 1 chunks] per wavefront
//   s_x     [group j][token m]
//   2^(s-128) (int8 form) [wavefront][group][row], written from registers.
constexpr int IX_WAVES = 8;
constexpr int IX_NT = 3;     // token tiles (of 32) per chunk

typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Written as inline assembly on purpose: the compiler would otherwise wait for
// every outstanding global-to-LDS load before the next LDS read, whatever its
// address, and the next block's loads could never overlap the current block's
// products. The kernel waits for them itself (s_waitcnt vmcnt(0)) before the
// barrier that hands the buffer over. M0 holds the wavefront's LDS base.
__device__ inline uint32_t lds_base(void *lds) {
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) void *)lds);
}
__device__ inline void lds_load16(const void *src, void *lds) {
    __asm__ volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "s"(lds_base(lds))
                     : "m0", "memory");
}
__device__ inline void lds_load4(const void *src, void *lds) {
    __asm__ volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" : : "v"(src), "s"(lds_base(lds))
                     : "m0", "memory");
}

template <bool UP>
__global__ __launch_bounds__(IX_WAVES * 64, 1) void moe_idot_kernel(
    float *__restrict__ out, int8_t *__restrict__ hq_out, float *__restrict__ hs_out, const int8_t *__restrict__ aq,
    const float *__restrict__ as, BankDev bank, const int32_t *__restrict__ active,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ perm, int top_k, int n_in, int n_out,
    int max_slots) {
    constexpr int GB = 4;                     // groups per block
    constexpr int GBYTES = 32;                // token bytes per group
    constexpr int TCHD = GB * GBYTES / 16;    // token chunks of a block: 8
    constexpr int TCH = TCHD + 1;             // token row in LDS: the chunks + pad
    constexpr int TPITCH = 16 * TCH;
    constexpr int WCH = GB + 1;               // weight row in LDS: GB chunks + pad
    constexpr int WPITCH = 16 * WCH;
    constexpr int NTOK = IX_NT * 32;
    constexpr int TLD = (NTOK * TCH + 64 * IX_WAVES - 1) / (64 * IX_WAVES);  // token loads per wavefront
    constexpr int WLD = (32 * WCH + 63) / 64;                                 // weight loads per wavefront
    constexpr int SXI = NTOK * GB / 64;                                       // scale load instructions
    static_assert(SXI <= IX_WAVES && NTOK * GB % 64 == 0, "one scale load per wavefront at most");
    __shared__ __attribute__((aligned(16))) char tok_lds[2][NTOK * TPITCH];
    __shared__ __attribute__((aligned(16))) char w_lds[2][IX_WAVES][WLD * 1024];
    __shared__ __attribute__((aligned(16))) float sx_lds[2][GB][NTOK];
    __shared__ __attribute__((aligned(16))) uint32_t sc_lds[2][IX_WAVES][64];   // a row's 4 scale bytes (x2)
    __shared__ __attribute__((aligned(16))) float ws_lds[IX_WAVES][GB][32];
    __shared__ int row_lds[NTOK];
    __shared__ float amax_lds[IX_WAVES][NTOK];  // UP: per wavefront and token, max |h| over its 16 rows
    const int tid = threadIdx.x, lane = tid & 63, wl = tid >> 6;
    const int half = lane >> 5, col = lane & 31;
    const int ngrp = n_in / kGroup;
    const int n_blocks = ngrp / GB;  // the launchers require in % 128 == 0
    constexpr int ROWS = UP ? 16 : 32;  // weight rows per wavefront (UP: of w1 and of w3 each)
    constexpr int WG_ROWS = ROWS * IX_WAVES;
    const int row_blocks = (n_out + WG_ROWS - 1) / WG_ROWS;
    const int n_act = perm ? active[0] : 1;
    const int n_items = max_slots * row_blocks;
    const uint32_t pitch = (uint32_t)(n_in / 2);
    for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
        const int slot = item / row_blocks;
        if (slot >= n_act) continue;
        const int rb = item - slot * row_blocks;
        const int e = perm ? active[1 + slot] : 0;
        const int p0 = perm ? offsets[e] : 0;
        const int p1 = perm ? offsets[e + 1] : 1;
        const uint8_t *eb = bank.base + (int64_t)e * bank.stride;
        const int rbase = rb * WG_ROWS + wl * ROWS;  // first row of this wavefront
        // the two matrices of this kernel's operand A (UP: w1 and w3; DOWN: w2 twice),
        // as wave-uniform pointers; a lane's row is an offset below 2^31 plus bit 31
        // for the second matrix
        const uint8_t *pa0 = eb + bank.off[UP ? W1P : W2P], *pa1 = eb + bank.off[UP ? W3P : W2P];
        const uint8_t *ps0 = eb + bank.off[UP ? W1S : W2S], *ps1 = eb + bank.off[UP ? W3S : W2S];
        auto row_of = [&](int r) {  // operand-A row r (0..31) of this wavefront
            return min(rbase + (UP ? (r & 15) : r), n_out - 1);
        };
        auto sel = [](uint32_t o, const uint8_t *p0, const uint8_t *p1) {
            return ((o >> 31) ? p1 : p0) + (o & 0x7FFFFFFFu);
        };
        // scale loads: lane l fetches the 4 scale bytes of a block of row l%32 (a dword:
        // rows are ngrp bytes apart and ngrp is a multiple of 4)
        const uint32_t ssrc = (uint32_t)row_of(col) * (uint32_t)ngrp | ((UP && col >= 16) ? 0x80000000u : 0u);
        // weight loads of this lane: LDS slot idx = 64*i + lane -> (row, chunk)
        uint32_t wsrc[WLD];
        int wch[WLD];
#pragma unroll
        for (int i = 0; i < WLD; ++i) {
            const int idx = 64 * i + lane;
            const int r = min(idx / WCH, 31);
            wch[i] = idx < 32 * WCH ? min(idx % WCH, GB - 1) : -1;  // the pad chunk repeats the last one
            wsrc[i] = (uint32_t)row_of(r) * pitch | ((UP && r >= 16) ? 0x80000000u : 0u);
        }
        for (int c0 = p0; c0 < p1; c0 += NTOK) {
            const int n_tok = min(p1 - c0, NTOK);
            const int n_tiles = __builtin_amdgcn_readfirstlane((n_tok + 31) / 32);
            __syncthreads();  // the previous chunk is done with the LDS
            if (tid < NTOK) {
                const int pos = c0 + min(tid, n_tok - 1);
                row_lds[tid] = UP ? (perm ? perm[pos] / top_k : 0) : pos;
            }
            __syncthreads();
            // token loads of this lane: slot idx = 64*(wl + 8i) + lane -> (token, chunk)
            const char *tbase = (const char *)aq;
            const uint32_t trow = (uint32_t)n_in;
            uint32_t tsrc[TLD];
            int tch[TLD];
#pragma unroll
            for (int i = 0; i < TLD; ++i) {
                const int idx = 64 * (wl + IX_WAVES * i) + lane;
                const int m = min(idx / TCH, NTOK - 1);
                tch[i] = idx < NTOK * TCH ? min(idx % TCH, TCHD - 1) : -1;
                tsrc[i] = (uint32_t)row_lds[m] * trow;
            }
            // scale load of wavefront wl (if wl < SXI): slot idx -> (group j = idx / NTOK, token idx % NTOK)
            const int sx_idx = 64 * wl + lane;
            const int sx_j = min(sx_idx / NTOK, GB - 1);
            const uint32_t xsrc = (uint32_t)row_lds[sx_idx % NTOK] * (uint32_t)ngrp;
            auto fetch = [&](int blk, int buf) {
                const int g0 = blk * GB;
                lds_load4(sel(ssrc, ps0, ps1) + g0, &sc_lds[buf][wl][0]);
#pragma unroll
                for (int i = 0; i < WLD; ++i) {
                    if (64 * i < 32 * WCH) {
                        if (wch[i] >= 0) lds_load16(sel(wsrc[i], pa0, pa1) + (uint32_t)(g0 + wch[i]) * 16u, &w_lds[buf][wl][i * 1024]);
                    }
                }
#pragma unroll
                for (int i = 0; i < TLD; ++i) {
                    const int d = wl + IX_WAVES * i;       // instruction: LDS bytes [1024 d, 1024 d + 1024)
                    if (64 * d < n_tiles * 32 * TCH) {     // tokens the chunk uses (whole rows or more)
                        const int c = tch[i];
                        if (c >= 0) lds_load16(tbase + tsrc[i] + (uint32_t)g0 * GBYTES + c * 16, &tok_lds[buf][d * 1024]);
                    }
                }
                if (wl < SXI) lds_load4(as + xsrc + g0 + sx_j, &sx_lds[buf][0][0] + 64 * wl);
            };
            // int8 form: 2^(s-128) of the block's groups for the rows' epilogues, from the
            // staged scale bytes into this wavefront's own table (so no workgroup barrier)
            auto row_scales = [&](int buf) {
                {
                    if (half == 0) {
                        const uint32_t sw = sc_lds[buf][wl][col];
#pragma unroll
                        for (int j = 0; j < GB; ++j) {
                            const uint32_t sb = (sw >> (8 * j)) & 0xFFu;
                            ws_lds[wl][j][col] = sb == 255u ? 0.0f : __builtin_ldexpf(1.0f, (int)sb - 128);
                        }
                    }
                    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                    __builtin_amdgcn_wave_barrier();
                    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                }
            };
            auto lds_loads_done = [] { __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory"); };

            auto run_chunk = [&](auto ntl_c) {
                constexpr int NTL = decltype(ntl_c)::value;
                float acc[NTL][16];
#pragma unroll
                for (int tt = 0; tt < NTL; ++tt)
#pragma unroll
                    for (int v = 0; v < 16; ++v) acc[tt][v] = 0.f;
                // one group j of the block in buffer buf
                auto group = [&](int buf, int j) {
                    // this lane's half of group j of its row (the whole 16 bytes are read)
                    const int4_t wq = *(const int4_t *)&w_lds[buf][wl][col * WPITCH + 16 * j];
                    const uint32_t wlo = (uint32_t)(half ? wq[2] : wq[0]), whi = (uint32_t)(half ? wq[3] : wq[1]);
                    auto tok_frag = [&](int tt, int c) {
                        return *(const int4_t *)&tok_lds[buf][(32 * tt + col) * TPITCH + 16 * c];
                    };
                    auto sx_of = [&](int tt) { return sx_lds[buf][j][32 * tt + col]; };
                    {
                        const int4_t a = decode_b(make_uint2(wlo, whi));
                        int16_t_v cur = mfma_group(a, tok_frag(0, 2 * j + half));
                        // row scales of result slots 4q..4q+3: rows 8q + 4*half + 0..3
                        float ws[16];
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const float4 w4 = *(const float4 *)&ws_lds[wl][j][8 * q + 4 * half];
                            ws[4 * q + 0] = w4.x; ws[4 * q + 1] = w4.y; ws[4 * q + 2] = w4.z; ws[4 * q + 3] = w4.w;
                        }
#pragma unroll
                        for (int tt = 0; tt < NTL; ++tt) {
                            int16_t_v nxt;
                            if (tt + 1 < NTL) nxt = mfma_group(a, tok_frag(tt + 1, 2 * j + half));
                            const float sx = sx_of(tt);
#pragma unroll
                            for (int v = 0; v < 16; ++v)
                                acc[tt][v] = __builtin_fmaf((float)cur[v], sx * ws[v], acc[tt][v]);
                            if (tt + 1 < NTL) cur = nxt;
                        }
                    }
                };
                fetch(0, 0);
                lds_loads_done();
                __syncthreads();
                for (int blk = 0; blk < n_blocks; ++blk) {
                    const int buf = blk & 1;
                    if (blk + 1 < n_blocks) fetch(blk + 1, buf ^ 1);
                    row_scales(buf);
#pragma unroll 1
                    for (int j = 0; j < GB; ++j) group(buf, j);
                    lds_loads_done();
                    __syncthreads();
                }
                // results: lane holds token col of each tile, rows 8q + 4*half + 0..3 in slots 4q..4q+3
                if constexpr (UP) {
                    // h = SiTU(g, u) of the wavefront's 16 rows, quantised per 32-group of h:
                    // the two wavefronts wl and wl^1 hold the halves of one group, so the
                    // group's maximum meets through LDS
                    float hv[NTL][8];
                    float m[NTL];
#pragma unroll
                    for (int tt = 0; tt < NTL; ++tt) {
                        m[tt] = 0.f;
#pragma unroll
                        for (int q = 0; q < 2; ++q)
#pragma unroll
                            for (int b = 0; b < 4; ++b) {
                                hv[tt][4 * q + b] = situ(acc[tt][4 * q + b], acc[tt][8 + 4 * q + b]);
                                m[tt] = __builtin_fmaxf(m[tt], __builtin_fabsf(hv[tt][4 * q + b]));
                            }
                        m[tt] = __builtin_fmaxf(m[tt], __shfl_xor(m[tt], 32));
                        if (half == 0) amax_lds[wl][32 * tt + col] = m[tt];
                    }
                    __syncthreads();
                    const int ngo = n_out / kGroup;
#pragma unroll
                    for (int tt = 0; tt < NTL; ++tt) {
                        const int i = tt * 32 + col;
                        const float sc = idot_group_scale(__builtin_fmaxf(m[tt], amax_lds[wl ^ 1][i]));
                        if (i < n_tok) {
                            const size_t pos = (size_t)(c0 + i);
#pragma unroll
                            for (int q = 0; q < 2; ++q) {
                                const int q0 = idot_quant(hv[tt][4 * q + 0], sc), q1 = idot_quant(hv[tt][4 * q + 1], sc);
                                const int q2 = idot_quant(hv[tt][4 * q + 2], sc), q3 = idot_quant(hv[tt][4 * q + 3], sc);
                                *(uint32_t *)(hq_out + pos * n_out + rbase + 8 * q + 4 * half) =
                                    (uint32_t)(q0 & 0xff) | ((uint32_t)(q1 & 0xff) << 8) |
                                    ((uint32_t)(q2 & 0xff) << 16) | ((uint32_t)q3 << 24);
                            }
                            if (half == 0 && (wl & 1) == 0) hs_out[pos * ngo + rbase / kGroup] = sc;
                        }
                    }
                } else {
#pragma unroll
                    for (int tt = 0; tt < NTL; ++tt) {
                        const int i = tt * 32 + col;
                        if (i < n_tok) {
                            float *dst = out + (size_t)(c0 + i) * n_out + rbase + 4 * half;
#pragma unroll
                            for (int q = 0; q < 4; ++q) {
                                const int r0 = rbase + 8 * q + 4 * half;
                                if (r0 + 3 < n_out && ((uintptr_t)(dst + 8 * q) & 15) == 0) {
                                    *(float4 *)(dst + 8 * q) =
                                        make_float4(acc[tt][4 * q], acc[tt][4 * q + 1], acc[tt][4 * q + 2], acc[tt][4 * q + 3]);
                                } else {
#pragma unroll
                                    for (int b = 0; b < 4; ++b)
                                        if (r0 + b < n_out) dst[8 * q + b] = acc[tt][4 * q + b];
                                }
                            }
                        }
                    }
                }
            };
            static_assert(IX_NT == 3, "one instantiation per tile count");
            switch (n_tiles) {
                case 1: run_chunk(std::integral_constant<int, 1>{}); break;
                case 2: run_chunk(std::integral_constant<int, 2>{}); break;
                default: run_chunk(std::integral_constant<int, 3>{}); break;
            }
        }
    }
}

int launch_idot_bf16(bool up, float *out, int8_t *hq, uint16_t *hqb, float *hs, const uint16_t *aqb, const float *as,
                     const BankDev &bank, const int32_t *active, const int32_t *offsets, const int32_t *perm,
                     int top_k, int n_in, int n_out, int max_slots, hipStream_t st);

// UP: the SiTU output of every pair, quantised per 32-group of h as the down
// product takes it: hq int8 [P][inter] (int8 form) or hqb its bf16 copy (bf16
// form), and hs fp32 [P][inter/32]. No fp32 h is written.
int launch_moe_up_idot(int8_t *hq, uint16_t *hqb, float *hs, const int8_t *xq, const uint16_t *xqb, const float *xs,
                       const BankDev &bank, const int32_t *active, const int32_t *offsets, const int32_t *perm,
                       int top_k, int latent, int inter, int max_slots, hipStream_t st) {
    if (xqb)
        return launch_idot_bf16(true, nullptr, nullptr, hqb, hs, xqb, xs, bank, active, offsets, perm, top_k, latent,
                                inter, max_slots, st);
    const int items = max_slots * ((inter + 16 * IX_WAVES - 1) / (16 * IX_WAVES));
    const int blocks = items < 16384 ? items : 16384;
    moe_idot_kernel<true><<<blocks, IX_WAVES * 64, 0, st>>>(nullptr, hq, hs, xq, xs, bank, active, offsets, perm,
                                                            top_k, latent, inter, max_slots);
    return hipGetLastError() == hipSuccess ? K3G_OK : K3G_EHIP;
}

int launch_moe_down_idot(float *ypair, const int8_t *hq, const uint16_t *hqb, const float *hs, const BankDev &bank,
                         const int32_t *active, const int32_t *offsets, const int32_t *perm, int latent, int inter,
                         int max_slots, hipStream_t st) {
    if (hqb)
        return launch_idot_bf16(false, ypair, nullptr, nullptr, nullptr, hqb, hs, bank, active, offsets, perm, 1, inter,
                                latent, max_slots, st);
    const int items = max_slots * ((latent + 32 * IX_WAVES - 1) / (32 * IX_WAVES));
    const int blocks = items < 16384 ? items : 16384;
    moe_idot_kernel<false><<<blocks, IX_WAVES * 64, 0, st>>>(ypair, nullptr, nullptr, hq, hs, bank, active, offsets,
                                                             perm, 1, inter, latent, max_slots);
    return hipGetLastError() == hipSuccess ? K3G_OK : K3G_EHIP;
}

}  // namespace k3g
