// idot_bf16.hip -- the grouped IDOT expert products on the bf16 matrix cores
// (gfx950), one 16x16x32 product per 32-column group.
//
// "Kimi K3 engine (c/kimi_k3.c)", section "Streaming design" (K3_IDOT): the
// activations are quantised per 32-group to int8 and dotted with the e2m1
// values doubled (exact int8); each group's integer dot I is scaled after the
// fact:  y[r] = sum_g [s_rg != 255] I_rg * s_x[g] * 2^(s_rg - 128).
//
// Here the int8 activations arrive widened to bf16 (exact) and the e2m1 codes
// are widened by v_cvt_scalef32_pk_bf16_fp4 with the group's 2^(s-127) folded
// in (exact: two significant bits times a power of two). Every product and
// partial sum of a group is then an integer below 2^16 times 2^(s-128), so
// the fp32 result of one v_mfma_f32_16x16x32_bf16 over the group's 32 columns
// is I * 2^(s-128) exactly, and the epilogue of a group is one fma with s_x.
// The results equal the int8 matrix-core form bit for bit.
//
// Work decomposition (one workgroup of 8 wavefronts per item):
//   item = (expert slot, block of output rows); the items of one XCD form a
//   contiguous run, so the row blocks of an expert share that XCD's L2 for
//   the expert's token rows.
//   Each wavefront owns 64 rows of operand A, as four tiles of 16:
//     UP:   w1 rows r..r+15, w1 r+16..r+31, w3 r..r+15, w3 r+16..r+31,
//           so g and u of a row meet in the same lane (h = SiTU(g, u));
//     DOWN: w2 rows r..r+63.
//   Operand B is up to 128 tokens (8 tiles of 16) of the expert, all of them
//   in one pass when the expert has no more, so its weights are read once.
// The K loop runs over blocks of two groups. Global-to-LDS loads
// (global_load_lds) bring weights, scale bytes, tokens and token scales
// without passing through registers. Tokens and their scales go through a
// 4-stage ring of blocks, each requested three blocks before it is used;
// the weights through a ring of two stages of four groups (two blocks), each
// requested two blocks before its first use. LDS layouts:
//   weights [wavefront][tile 0..3][row 0..15][4 chunks of 16 bytes] per stage:
//           one load per tile, the four consecutive lanes of a row reading its
//           64 contiguous bytes (the L2 serves 64-byte row pieces far faster
//           than 32-byte ones or rows in consecutive lanes); row r's chunk c
//           sits in slot c ^ ((r / 4) % 4), so the fragment reads of one
//           group (lane (i, q): dword q of row i) fall in 64 distinct banks.
//           Each wavefront loads and reads only its own rows.
//   scales  [tile][row 0..15][4 dwords]: the scale bytes of 16 groups, loaded
//           once per 8 blocks into one of two windows; the tiles ordered
//           (matrix, wavefront, tile within the matrix)
//   tokens  [token 0..127][8 chunks + 1 pad] (conflict-free 16-byte reads)
//   s_x     [token 0..127][group 0..1]
#include <type_traits>

#include "k3g_common.h"

namespace k3g {

namespace ib {

constexpr int NW = 8;             // wavefronts per workgroup
constexpr int GB = 2;             // groups per block (token stage)
constexpr int S = 4;              // token stages in the ring
constexpr int WGS = 4;            // groups per weight stage (two blocks)
constexpr int TMAX = 8;           // token tiles (of 16) per pass
constexpr int NTOK = 16 * TMAX;   // tokens per pass
constexpr int WG_AR = NW * 64;    // operand-A rows per workgroup
constexpr int TCH = 4 * GB + 1;   // 16-byte chunks per token row in LDS (with the pad)
constexpr int W_BYTES = WG_AR * WGS * 16;    // 32 KB per weight stage
constexpr int T_BYTES = NTOK * TCH * 16;     // 18 KB
constexpr int SWG = 16;                      // groups per window of staged scale bytes
constexpr int SW_BYTES = WG_AR * SWG;        // 8 KB: 4 dwords of scale bytes per A row
constexpr int SW_LD = SW_BYTES / 256 / NW;   // scale-window loads per wavefront: 4
constexpr int SX_BYTES = NTOK * GB * 4;      // 1 KB

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

struct Lds {
    char w[2][W_BYTES];
    char t[S][T_BYTES];
    uint32_t ws[2][WG_AR * SWG / 4];
    float sx[S][NTOK * GB];
    int rows[NTOK];
};

// 4 packed bytes (8 e2m1 codes, column order) -> 8 bf16 scaled by 2^(e-127),
// e = the exponent field of `scale`.
__device__ inline bf16x8_t fp4x8_bf16(uint32_t w, float scale) {
    const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0);
    const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1);
    const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2);
    const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3);
    return bf16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// Number of token-load instructions of a pass with NT tiles, and how many of
// them fall on wavefront wl (instruction n goes to wavefront n % NW).
constexpr int tok_instr(int nt) { return (nt * 16 * TCH + 63) / 64; }
constexpr int sx_instr(int nt) { return (nt * 16 * GB + 63) / 64; }
// The fewest token and token-scale loads any wavefront issues per block (the
// vmcnt bound; the weight and scale-window loads only add to what is in flight).
constexpr int min_tok_loads(int nt) { return tok_instr(nt) / NW + (sx_instr(nt) >= NW ? 1 : 0); }

}  // namespace ib

template <bool UP>
__global__ __launch_bounds__(ib::NW * 64, 1) void moe_idot_bf16_kernel(
    float *__restrict__ out, int8_t *__restrict__ hq_out, uint16_t *__restrict__ hqb_out, float *__restrict__ hs_out,
    const uint16_t *__restrict__ aqb, const float *__restrict__ as, BankDev bank,
    const int32_t *__restrict__ active, const int32_t *__restrict__ offsets, const int32_t *__restrict__ perm,
    int top_k, int n_in, int n_out, int max_slots, int row_blocks) {
    using namespace ib;
    __shared__ __attribute__((aligned(16))) Lds L;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wl = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, quad = lane >> 4;

    // blockIdx -> item: workgroups are handed to the 8 XCDs in turn, so XCD x
    // runs blocks x, x+8, ...; give it the contiguous items [x*q + min(x, r), ...).
    const int n_items = max_slots * row_blocks;
    const int xcd = blockIdx.x & 7, kk = blockIdx.x >> 3;
    const int item = xcd * (n_items >> 3) + min(xcd, n_items & 7) + kk;
    if (item >= n_items) return;
    const int slot = item / row_blocks, rb = item - slot * row_blocks;
    const int n_act = perm ? active[0] : 1;
    if (slot >= n_act) return;
    const int e = perm ? active[1 + slot] : 0;
    const int p0 = perm ? offsets[e] : 0;
    const int p1 = perm ? offsets[e + 1] : 1;
    const uint8_t *eb = bank.base + (int64_t)e * bank.stride;
    const int ngrp = n_in / kGroup;
    const int n_blocks = ngrp / GB;
    const uint32_t pitch = (uint32_t)n_in / 2;

    // The (up to) two matrices of operand A, as wave-uniform base pointers:
    // UP: w1 and w3; DOWN: w2 twice. Every load instruction below reads one of
    // them, so its base goes in SGPRs and each lane adds a 32-bit offset.
    const uint8_t *pk[2] = {eb + bank.off[UP ? W1P : W2P], eb + bank.off[UP ? W3P : W2P]};
    const uint8_t *sc[2] = {eb + bank.off[UP ? W1S : W2S], eb + bank.off[UP ? W3S : W2S]};
    // row (in its matrix) of wavefront w's tile k, row i; the matrix is k >> 1
    auto arow = [&](int w, int k, int i) {
        const int r = UP ? rb * (WG_AR / 2) + w * 32 + (k & 1) * 16 + i : rb * WG_AR + w * 64 + k * 16 + i;
        return (uint32_t)min(r, n_out - 1);
    };
    // weight loads: this wavefront's tile k, one instruction per weight stage;
    // lane 4r + c reads chunk c ^ ((r / 4) % 4) of row r. n_out is a multiple of
    // 128, so a wavefront's rows are all inside the matrix or all past it: the
    // latter read the matrix's first rows instead (their results are dropped).
    const int w_row0 = (UP ? rb * (WG_AR / 2) + wl * 32 : rb * WG_AR + wl * 64) < n_out ? 0 : -1;
    const uint8_t *w_tile[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t r = w_row0 < 0 ? (uint32_t)(UP ? (k & 1) * 16 : k * 16) : arow(wl, k, 0);
        w_tile[k] = pk[k >> 1] + (size_t)r * pitch;
    }
    const uint32_t w_off = (uint32_t)(lane >> 2) * pitch + 16u * (uint32_t)((lane & 3) ^ ((lane >> 4) & 3));
    // scale bytes, staged per window of 16 groups: tile slot ((k>>1)*NW + w)*2 + (k&1)
    // holds wavefront w's tile k, 16 rows x 4 dwords; instruction n = wl + NW*m fills
    // tile slot n (one matrix: n >> 4 = m >> 1), lane -> (row lane/4, dword lane%4)
    auto s_off = [&](int m) {
        const int n = wl + NW * m;
        const int s_w = (n & 15) >> 1, s_k = ((n >> 4) << 1) | (n & 1);
        return arow(s_w, s_k, lane >> 2) * (uint32_t)ngrp;
    };
    const int n_dw = ngrp / 4;  // scale dwords per row
    const uint32_t lds_w = lds_addr(&L.w[0][0]) + 4096u * (uint32_t)wl, lds_t = lds_addr(&L.t[0][0]);
    const uint32_t lds_ws = lds_addr(&L.ws[0][0]), lds_sx = lds_addr(&L.sx[0][0]);
    const uint32_t tok_row_bytes = (uint32_t)n_in * 2u;

    for (int c0 = p0; c0 < p1; c0 += NTOK) {
        const int n_tok = min(p1 - c0, NTOK);
        const int n_tiles = __builtin_amdgcn_readfirstlane((n_tok + 15) >> 4);
        __syncthreads();  // the previous pass is done with the LDS
        if (tid < NTOK) {
            const int pos = c0 + min(tid, n_tok - 1);
            L.rows[tid] = UP ? (perm ? perm[pos] / top_k : 0) : pos;
        }
        __syncthreads();

        auto run = [&](auto nt_c) {
            constexpr int NT = decltype(nt_c)::value;
            constexpr int TI = tok_instr(NT), SI = sx_instr(NT);
            constexpr int TPW = (TI + NW - 1) / NW;  // token loads per wavefront, at most
            // waiting for block b (its tokens, and the weight stage it reads) leaves
            // at least the token loads of blocks b+1 and b+2 in flight: weight stage
            // c is requested at block 2c - 2 before the tokens of block 2c + 1
            constexpr int VM = (S - 2) * min_tok_loads(NT);
            // token loads of this lane: instruction n = wl + NW*m, slot 64n + lane -> (token, chunk)
            uint32_t t_off[TPW];
#pragma unroll
            for (int m = 0; m < TPW; ++m) {
                const int s = 64 * (wl + NW * m) + lane;
                const int tk = min(s / TCH, NT * 16 - 1);
                const int ch = min(s % TCH, 4 * GB - 1);  // the pad slot repeats the last chunk
                t_off[m] = (uint32_t)L.rows[tk] * tok_row_bytes + 16u * (uint32_t)ch;
            }
            // token-scale loads (wavefronts 0..SI-1): slot -> (token, group)
            uint32_t x_off;
            {
                const int s = 64 * wl + lane;
                const int tk = min(s / GB, NT * 16 - 1);
                x_off = ((uint32_t)L.rows[tk] * (uint32_t)ngrp + (uint32_t)(s % GB)) * 4u;
            }
            // The token loads of one block, as NPART parts of one instruction
            // each (or none): tokens, token scales, and every eighth block the
            // scale window. Block b requests block b+3 right after its barrier,
            // and an even block b the weight stage b/2 + 1 before that.
            constexpr int NPART = TPW + 1 + SW_LD;
            constexpr int NSPREAD = TPW + 1;  // the parts every block has
            auto fetch_part = [&](int blk, int part) {
                const int buf = blk % S;
                const int g0 = blk * GB;
                if (part < TPW) {
                    const int m = part;
                    if (wl + NW * m < TI)
                        dma16((const char *)aqb + 64 * g0, t_off[m], lds_t + buf * T_BYTES + 1024 * (wl + NW * m));
                } else if (part == TPW) {
                    if (wl < SI) dma4(as + g0, x_off, lds_sx + buf * SX_BYTES + 256 * wl);
                } else if ((blk & 7) == 0) {  // the scale window of groups [g0, g0 + 16)
                    const int m = part - (TPW + 1);
                    const int wdw = g0 / 4, wb = (blk >> 3) & 1;
                    dma4(sc[m >> 1], s_off(m) + 4u * (uint32_t)min(wdw + (lane & 3), n_dw - 1),
                         lds_ws + wb * SW_BYTES + 256 * (wl + NW * m));
                }
            };
            auto fetch = [&](int blk) {
#pragma unroll
                for (int part = 0; part < NPART; ++part) fetch_part(blk, part);
            };
            // weight stage c: groups [4c, 4c + 4) of the wavefront's 4 tiles
            auto fetch_w = [&](int c) {
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    dma16(w_tile[k] + 64 * c, w_off, lds_w + (c & 1) * W_BYTES + 1024 * k);
            };

            f32x4_t acc[4][NT];
#pragma unroll
            for (int k = 0; k < 4; ++k)
#pragma unroll
                for (int tt = 0; tt < NT; ++tt) acc[k][tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

            fetch_w(0);  // n_blocks is even: at least one weight stage
#pragma unroll
            for (int b = 0; b < S - 1; ++b)
                if (b < n_blocks) fetch(b);
            for (int blk = 0; blk < n_blocks; ++blk) {
                if (blk + S - 2 < n_blocks) wait_vm<VM>();
                else wait_vm<0>();
                __syncthreads();  // block blk is in LDS for all; block blk-1's buffer is free
                if (!(blk & 1) && blk + 2 < n_blocks) fetch_w((blk >> 1) + 1);
                const bool more = blk + S - 1 < n_blocks;  // a stage to request during this block
                if (more) {
#pragma unroll
                    for (int part = 0; part < NSPREAD; ++part) fetch_part(blk + S - 1, part);
                    if (((blk + S - 1) & 7) == 0) {
#pragma unroll
                        for (int part = NSPREAD; part < NPART; ++part) fetch_part(blk + S - 1, part);
                    }
                }
                const int buf = blk % S;
                const int gsel = (blk * GB) & 3;            // byte of group 2*blk in its dword
                const int sdw = (blk & 7) >> 1;              // that dword in the window
                const uint32_t *wq = (const uint32_t *)&L.w[(blk >> 1) & 1][4096 * wl];
                const uint32_t *wsd = &L.ws[(blk >> 3) & 1][0];
                const char *tb = &L.t[buf][0];
                const float *sxb = &L.sx[buf][0];
#pragma unroll
                for (int j = 0; j < GB; ++j) {
                    bf16x8_t a[4];
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const int jj = 2 * (blk & 1) + j;  // the group in the weight stage
                        const uint32_t w = wq[(k * 16 + col) * 16 + 4 * (jj ^ ((col >> 2) & 3)) + quad];
                        const uint32_t sd = wsd[(((((k >> 1) * NW + wl) << 1) + (k & 1)) * 16 + col) * 4 + sdw];
                        const uint32_t sb = (sd >> (8 * (gsel + j))) & 0xFFu;
                        const bool skip = sb == 255u;
                        const float scale = __builtin_bit_cast(float, (skip ? 127u : sb) << 23);
                        a[k] = fp4x8_bf16(skip ? 0u : w, scale);
                    }
                    auto rd_b = [&](int tt) {
                        return *(const bf16x8_t *)(tb + ((16 * tt + col) * TCH + 4 * j + quad) * 16);
                    };
                    auto rd_s = [&](int tt) { return sxb[(16 * tt + col) * GB + j]; };
                    // software pipeline over the token tiles: operands two tiles
                    // ahead, products one tile ahead of their epilogue
                    bf16x8_t bq[2];
                    float sv[2];  // s_x of tile tt in sv[tt & 1], read one tile ahead
                    sv[0] = rd_s(0);
                    bq[0] = rd_b(0);
                    if (NT > 1) bq[1] = rd_b(1);
                    f32x4_t d[2][4];  // products of tile tt in d[tt & 1] (static once unrolled)
                    const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int k = 0; k < 4; ++k) d[0][k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[k], bq[0], z, 0, 0, 0);
#pragma unroll
                    for (int tt = 0; tt < NT; ++tt) {
                        if (tt + 1 < NT) {
                            const bf16x8_t bn = bq[(tt + 1) & 1];
                            if (tt + 2 < NT) bq[tt & 1] = rd_b(tt + 2);
                            sv[(tt + 1) & 1] = rd_s(tt + 1);
#pragma unroll
                            for (int k = 0; k < 4; ++k)
                                d[(tt + 1) & 1][k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[k], bn, z, 0, 0, 0);
                        }
                        const float sc = sv[tt & 1];
#pragma unroll
                        for (int k = 0; k < 4; ++k)
#pragma unroll
                            for (int v = 0; v < 4; ++v) acc[k][tt][v] = __builtin_fmaf(d[tt & 1][k][v], sc, acc[k][tt][v]);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            }
            // results: lane holds token col of each tile and rows 4*quad + v of each A tile;
            // n_out is a multiple of 128: a wavefront's rows are all inside the matrix or
            // all past it (the last row block of a width that is an odd multiple of 128)
            if constexpr (UP) {
                // h = SiTU(g, u) of the wavefront's 32 rows (one 32-group of h) for each
                // token, quantised here: the group's maximum over the 8 values of each of
                // the 4 lanes that hold the token, then q and s of the group
                const int hrow = rb * (WG_AR / 2) + wl * 32;  // the group's first row
                const bool rows_in = hrow < n_out;
                const int ngo = n_out / kGroup;
#pragma unroll
                for (int tt = 0; tt < NT; ++tt) {
                    const int i = 16 * tt + col;
                    float hv[2][4];
                    float amax = 0.f;
#pragma unroll
                    for (int k = 0; k < 2; ++k)
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            hv[k][v] = situ(acc[k][tt][v], acc[k + 2][tt][v]);
                            amax = __builtin_fmaxf(amax, __builtin_fabsf(hv[k][v]));
                        }
                    amax = __builtin_fmaxf(amax, __shfl_xor(amax, 16));
                    amax = __builtin_fmaxf(amax, __shfl_xor(amax, 32));
                    const float sc = idot_group_scale(amax);
                    if (i < n_tok && rows_in) {
                        const size_t pos = (size_t)(c0 + i);
#pragma unroll
                        for (int k = 0; k < 2; ++k) {
                            const size_t at = pos * n_out + hrow + 16 * k + 4 * quad;
                            const int q0 = idot_quant(hv[k][0], sc), q1 = idot_quant(hv[k][1], sc);
                            const int q2 = idot_quant(hv[k][2], sc), q3 = idot_quant(hv[k][3], sc);
                            if (hqb_out) {
                                *(uint2 *)(hqb_out + at) = make_uint2(i8_bf16_bits(q0) | (i8_bf16_bits(q1) << 16),
                                                                      i8_bf16_bits(q2) | (i8_bf16_bits(q3) << 16));
                            } else {
                                *(uint32_t *)(hq_out + at) = (uint32_t)(q0 & 0xff) | ((uint32_t)(q1 & 0xff) << 8) |
                                                             ((uint32_t)(q2 & 0xff) << 16) | ((uint32_t)q3 << 24);
                            }
                        }
                        if (quad == 0) hs_out[pos * ngo + hrow / kGroup] = sc;
                    }
                }
            } else {
#pragma unroll
                for (int tt = 0; tt < NT; ++tt) {
                    const int i = 16 * tt + col;
                    float *dst = out + (size_t)(c0 + min(i, n_tok - 1)) * n_out;
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const int r0 = rb * WG_AR + wl * 64 + 16 * k + 4 * quad;
                        if (i < n_tok && r0 < n_out)
                            *(float4 *)(dst + r0) = make_float4(acc[k][tt][0], acc[k][tt][1], acc[k][tt][2], acc[k][tt][3]);
                    }
                }
            }
        };
        switch (n_tiles) {
            case 1: run(std::integral_constant<int, 1>{}); break;
            case 2: run(std::integral_constant<int, 2>{}); break;
            case 3: run(std::integral_constant<int, 3>{}); break;
            case 4: run(std::integral_constant<int, 4>{}); break;
            case 5: run(std::integral_constant<int, 5>{}); break;
            case 6: run(std::integral_constant<int, 6>{}); break;
            case 7: run(std::integral_constant<int, 7>{}); break;
            default: run(std::integral_constant<int, 8>{}); break;
        }
    }
}

// UP: h = SiTU(w1 . x, w3 . x) for every pair of every active expert, written
// quantised per 32-group (hq int8, or hqb as bf16, and hs [pair][inter/32]);
// DOWN: ypair[pos][r] = w2[r] . h[pos]. Operands as the IDOT stages leave them:
// bf16 copies of the int8 activations and their fp32 group scales.
int launch_idot_bf16(bool up, float *out, int8_t *hq, uint16_t *hqb, float *hs, const uint16_t *aqb, const float *as,
                     const BankDev &bank, const int32_t *active, const int32_t *offsets, const int32_t *perm,
                     int top_k, int n_in, int n_out, int max_slots, hipStream_t st) {
    const int per_block = up ? ib::WG_AR / 2 : ib::WG_AR;
    const int row_blocks = (n_out + per_block - 1) / per_block;
    const int64_t items = (int64_t)max_slots * row_blocks;
    if (items == 0) return K3G_OK;
    if (items > (int64_t)1 << 30) return K3G_EUNSUPPORTED;
    const dim3 grid((unsigned)items), block(ib::NW * 64);
    if (up)
        moe_idot_bf16_kernel<true><<<grid, block, 0, st>>>(nullptr, hq, hqb, hs, aqb, as, bank, active, offsets, perm,
                                                           top_k, n_in, n_out, max_slots, row_blocks);
    else
        moe_idot_bf16_kernel<false><<<grid, block, 0, st>>>(out, nullptr, nullptr, nullptr, aqb, as, bank, active,
                                                            offsets, perm, top_k, n_in, n_out, max_slots, row_blocks);
    return hipGetLastError() == hipSuccess ? K3G_OK : K3G_EHIP;
}

}  // namespace k3g
