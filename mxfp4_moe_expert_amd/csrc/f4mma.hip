// f4mma.hip -- the expert products on gfx950's block-scaled FP4 matrix cores:
// one token (moe_f4_kernel), and more tokens in passes of 2, 4 or 8 of an
// expert's sorted pairs (moe_f4m_kernel, moe_f4q_kernel, moe_f4s_kernel).
//
// The product is the pages' exact one ("kimi-k3-in-c: 2.78 trillion
// parameters, one CPU, 8 GB of RAM", section "Reduction one"): per row, every
// 32-group's e2m1 values dotted with fp32 x, times 2^(s-127), groups with
// s = 255 left out, fp32 accumulation. The convert-and-FMA form of it spends
// about 1.5 vector instructions per weight, which on this chip takes longer
// than streaming the weights from HBM. Here the weights go to
// v_mfma_scale_f32_16x16x128_f8f6f4 as they are stored: the nibbles are
// operand A and the group's ue8m0 byte is A's block scale, so decoding costs
// nothing. The matrix cores take no fp32 operand, so x is first written as a
// sum of 16 e2m1 vectors ("pieces") with one ue8m0 scale per 32 entries each.
// Piece 0 rounds x to e2m1 on the power-of-two grid that puts the group's
// largest |x| in (3, 6]; every later piece rounds what is left on a grid four
// times finer than the one before. Each step is exact in fp32, and what is
// left never exceeds half a grid unit of the step before, so it always fits
// the next grid (at most 4 of its units) and shrinks at least four-fold per
// piece: after 16 pieces it is below 2^-30 of the group's largest entry (in
// practice zero: an fp32 entry has 24 bits). Grids stop at 2^-126, so entries
// below 2^-127 are dropped. The 16 pieces are the 16
// columns of operand B; every product e2m1 * e2m1 * 2^a * 2^b is exact, the
// matrix cores add in fp32, and the 16 column sums are added at the end
// (fp32, by DPP).
//
// Layout of one vector's pieces (n = 32 * ngrp entries, ngrp a multiple of 4),
// in chunks of 128 entries (one k-step of the instruction), 1280 bytes each:
//   bytes [0, 1024):    lane l = p + 16*q holds, at 16*l, the 32 nibbles of
//                       piece p for group 4*i + q (entry 2b in the low nibble
//                       of byte b) -- exactly operand B of the instruction;
//   bytes [1024, 1280): lane l's uint32 at 1024 + 4*l, low byte the ue8m0
//                       scale of that piece and group -- B's block scale.
// Operand A uses the same k order: lane l = r + 16*q of a 16-row tile loads
// the 16 bytes of group 4*i + q of row r, so one instruction reads 64
// contiguous bytes of each of 16 rows.
//
// With more tokens every pair is its own 16 columns (its token's x pieces for
// the up-projection, its own h pieces for the down-projection), so an A
// fragment feeds one product per pair of a pass. The passes come from the
// bucket's table (the pages sort a chunk's pairs by expert so that each
// selected expert is read once: "Kimi K3 engine (c/kimi_k3.c)", section
// "Chunked prefill"); here an expert is read once per pass.
#include <atomic>

#include "k3g_common.h"

// Build-time knob (the default is the shipped configuration): blocks of four
// chunks in the product kernels' load ring; all but one are in flight while
// the oldest is multiplied.
#ifndef K3G_F4_NBUF
#define K3G_F4_NBUF 6
#endif
// Consecutive passes per XCD group in the four-pair kernel's item order (0:
// plain order; the up-projection's own), and in the eight-pair kernel's.
#ifndef K3G_F4Q_GROUP
#define K3G_F4Q_GROUP 4
#endif
#ifndef K3G_F4Q_GROUP_UP
#define K3G_F4Q_GROUP_UP 8
#endif
#ifndef K3G_F4_FRIENDLY
#define K3G_F4_FRIENDLY 1
#endif
#ifndef K3G_F4S_GROUP
#define K3G_F4S_GROUP 4
#endif

namespace k3g {

typedef int v8i_t __attribute__((ext_vector_type(8)));

namespace f4 {
constexpr int kChunkBytes = 1280;  // pieces + scales of 128 entries
constexpr int kWaves = 4;          // wavefronts per workgroup
constexpr int kRows = 32;          // rows a wavefront owns (two 16-row tiles)
constexpr int kPieces = 16;
}  // namespace f4

// ---- pieces -----------------------------------------------------------------

// The 16 pieces of one 32-entry group whose entry e = lane & 31 is r (both
// halves of the wavefront may hold groups): written at `out` (the group's
// chunk) as column group q when `store`. The rounding to e2m1 is gfx950's
// scaled convert (to nearest, ties to the even code, r / 2^x with a
// power-of-two scale; the way back gives the value times 2^x exactly).
__device__ inline void split_group(float r, uint8_t *out, int q, bool store) {
    const int e = threadIdx.x & 31;
    float m = __builtin_fabsf(r);
#pragma unroll
    for (int s = 1; s < 32; s <<= 1) m = fmaxf(m, __shfl_xor(m, s, 32));
    // piece 0's grid: the smallest x with m <= 6 * 2^x. With m = M * 2^E, M in
    // [1, 2): E - 2 when M <= 1.5, else E - 1 (m / 2^x then lies in (3, 6]).
    // Grids stop at 2^-126 (a normal fp32 scale): entries below 2^-127 are
    // dropped.
    const uint32_t mb = __builtin_bit_cast(uint32_t, m);
    const int x0 = int(mb >> 23) - 129 + ((mb & 0x7FFFFFu) > 0x400000u ? 1 : 0);
    // lane e keeps dword e >> 3 of pieces (e & 7) and (e & 7) + 8, so that the
    // 16 pieces go out in two 128-byte stores a half-wavefront, and lane e < 16
    // writes piece e's scale
    uint32_t keep0 = 0, keep1 = 0;
#pragma unroll
    for (int p = 0; p < f4::kPieces; ++p) {
        const int x = max(x0 - 2 * p, -126);
        const float sc = __builtin_bit_cast(float, (uint32_t)(x + 127) << 23);
        const uint32_t nib = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, r, 0.0f, sc, 0) & 15u;
        r -= __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(nib, sc, 0)[0];  // exact: both are multiples of r's last bit
        // eight nibbles per dword: every lane of an aligned group of 8 collects
        // entries 8d..8d+7 (quad swaps, then the half-row mirror)
        uint32_t w = nib << (4 * (e & 7));
        w |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)w, 0xB1, 0xF, 0xF, false);
        w |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)w, 0x4E, 0xF, 0xF, false);
        w |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)w, 0x141, 0xF, 0xF, false);
        if ((e & 7) == (p & 7)) {
            if (p < 8)
                keep0 = w;
            else
                keep1 = w;
        }
    }
    if (store) {
        *(uint32_t *)(out + 16 * ((e & 7) + 16 * q) + 4 * (e >> 3)) = keep0;
        *(uint32_t *)(out + 16 * ((e & 7) + 8 + 16 * q) + 4 * (e >> 3)) = keep1;
        if (e < 16) *(uint32_t *)(out + 1024 + 4 * (e + 16 * q)) = (uint32_t)(max(x0 - 2 * e, -126) + 127);
    }
}

// Pieces of n_vec vectors of ngrp groups each: src fp32 rows of src_stride
// floats, dst rows of (ngrp/4)*1280 bytes. One half-wavefront per group.
__global__ __launch_bounds__(256) void split_kernel(uint8_t *__restrict__ dst, const float *__restrict__ src,
                                                    int n_vec, int ngrp, int src_stride) {
    const int G = blockIdx.x * 8 + (threadIdx.x >> 5);
    const bool live = G < n_vec * ngrp;
    const int Gc = live ? G : 0;
    const int v = Gc / ngrp, g = Gc - v * ngrp;
    const float r = src[(size_t)v * src_stride + g * kGroup + (threadIdx.x & 31)];
    split_group(r, dst + (size_t)v * (ngrp / 4) * f4::kChunkBytes + (g >> 2) * f4::kChunkBytes, g & 3, live);
}

// The sum of S partial products [S][T][len] (slices added in order, as the
// dense products' reduction does) into out [T][len], and its pieces, as
// split_kernel writes them, into dst. One half-wavefront per 32-entry group.
__global__ __launch_bounds__(256) void reduce_split_kernel(float *__restrict__ out, uint8_t *__restrict__ dst,
                                                           const float *__restrict__ part, int S, int T, int ngrp) {
    const int64_t gid = (int64_t)blockIdx.x * 8 + threadIdx.x / 32;
    const bool live = gid < (int64_t)T * ngrp;
    const int t = live ? (int)(gid / ngrp) : 0, g = live ? (int)(gid - (int64_t)t * ngrp) : 0;
    const int len = ngrp * kGroup;
    const int n = g * kGroup + (threadIdx.x & 31);
    float v = 0.f;
    for (int s = 0; s < S; ++s) v += part[((size_t)s * T + t) * len + n];
    if (live) out[(size_t)t * len + n] = v;
    split_group(v, dst + (size_t)t * (ngrp / 4) * f4::kChunkBytes + (g >> 2) * f4::kChunkBytes, g & 3, live);
}

int launch_reduce_split(float *out, uint8_t *dst, const float *part, int S, int T, int len, hipStream_t st) {
    const int ngrp = len / kGroup;
    const int64_t groups = (int64_t)T * ngrp;
    if (groups == 0) return K3G_OK;
    if (len % 128) return K3G_EUNSUPPORTED;
    reduce_split_kernel<<<(unsigned)((groups + 7) / 8), 256, 0, st>>>(out, dst, part, S, T, ngrp);
    return hipGetLastError() == hipSuccess ? K3G_OK : K3G_EHIP;
}

int launch_split(uint8_t *dst, const float *src, int n_vec, int len, int src_stride, hipStream_t st) {
    const int ngrp = len / kGroup;
    const int groups = n_vec * ngrp;
    if (groups == 0) return K3G_OK;
    split_kernel<<<(groups + 7) / 8, 256, 0, st>>>(dst, src, n_vec, ngrp, src_stride);
    return hipGetLastError() == hipSuccess ? K3G_OK : K3G_EHIP;
}

// ---- the products -------------------------------------------------------------

// A wavefront with no rows (its first row past the output) still runs the
// same straight-line code and barriers: it reads the expert's first rows and
// stores nothing. (Its loads stay in range: a load past a buffer's range
// returns at once, possibly before older loads, and the counted waits here
// assume loads complete in the order they were issued.)

// Workgroup b runs on XCD b % 8 (the dispatcher deals workgroups round the
// XCDs). In a grid of whole rounds of 8 groups of gi consecutive items, group
// g goes to XCD g % 8: workgroup b takes item xcd_item(b, gi). Items past the
// end exit.
__device__ inline int xcd_item(int b, int gi) {
    const int x = b % 8, loc = b / 8;
    return (x + 8 * (loc / gi)) * gi + loc % gi;
}

// UP:   tiles (w1, rows r0..r0+15), (w3, r0..r0+15), (w1, r0+16..), (w3, r0+16..);
//       h[pos][r] = SiTU(g, u) for the 32 rows, and the 16 pieces of this
//       32-entry group of h (the down-projection's operand B) into hp[pos].
// DOWN: tiles (w2, rows r0..r0+15), (w2, r0+16..); ypair[pos][r] for the 32 rows.
// A wavefront walks its tiles one after another (a tile's 16 rows are
// contiguous in memory) in blocks of four chunks: a block's loads (four
// 16-byte loads of nibbles a lane and one 16-byte load of the rows' scale
// dwords) go out together into a ring of NBUF blocks, and NBUF - 1 blocks are
// in flight while the oldest is multiplied.
// A workgroup's wavefronts own consecutive 32-row blocks of one slot (DOWN) or
// of any slots (UP: B is x for all of them). One token: every slot has one
// pair, or several equal ones when the route repeats an expert.
template <bool UP, int NCK>
__global__ __launch_bounds__(f4::kWaves * kWave, 2) void moe_f4_kernel(
    float *__restrict__ out, const uint8_t *__restrict__ pieces, uint8_t *__restrict__ hp, BankDev bank, Route1 rt,
    const int32_t *__restrict__ active, const int32_t *__restrict__ offsets, int top_k, int latent, int inter,
    int max_slots) {
    constexpr int TILES = UP ? 4 : 2;
    constexpr int NS = TILES * NCK;  // steps: (tile, chunk)
    constexpr int CPB = 4;                // chunks per block
    constexpr int NB = TILES * NCK / CPB;  // blocks
    constexpr int NBUF = K3G_F4_NBUF;      // ring of blocks
    constexpr int ngrp = 4 * NCK;
    extern __shared__ uint4 lds_b[];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int n_out = UP ? inter : latent;
    const int blocks_per_slot = n_out / f4::kRows;

    // which slot and rows this wavefront owns
    int slot, blk32;
    if (UP) {
        const int item = blockIdx.x * f4::kWaves + wave;
        slot = item / blocks_per_slot;
        blk32 = item - slot * blocks_per_slot;
    } else {
        const int wgs = (blocks_per_slot + f4::kWaves - 1) / f4::kWaves;
        slot = blockIdx.x / wgs;
        blk32 = (blockIdx.x - slot * wgs) * f4::kWaves + wave;
    }
    int e = 0, p0 = 0, p1 = 0, n_act;
    Route1Lane r1 = {};
    if (UP) {
        r1 = route1_lane(rt.idx, top_k, rt.n_experts, lane);
        n_act = __popcll(r1.firsts);
        const uint64_t m = __ballot(r1.first && r1.slot == slot);
        if (m) {
            const int L = __builtin_amdgcn_readfirstlane(__builtin_ctzll(m));
            e = __builtin_amdgcn_readlane(r1.e, L);
            p0 = __builtin_amdgcn_readlane(r1.pos, L);
            p1 = p0 + __builtin_amdgcn_readlane(r1.cnt, L);
        }
    } else {
        n_act = active[0];
        if (slot < n_act) {
            e = active[1 + slot];
            p0 = offsets[e];
            p1 = offsets[e + 1];
        }
    }
    if (!UP && slot >= n_act) return;  // whole workgroup: DOWN's workgroups hold one slot
    const bool live = slot < n_act && slot < max_slots && blk32 < blocks_per_slot && p1 > p0;

    // the wavefront's tiles: buffer resources, and this lane's row offsets
    const uint8_t *eb = bank.base + (int64_t)e * bank.stride;
    constexpr uint32_t pitch_p = 16u * ngrp, pitch_s = ngrp;
    const int r0 = (live ? blk32 : 0) * f4::kRows;
    rsrc_t rp[TILES], rs[TILES];
    uint32_t vp[TILES], vs[TILES];
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
        const int mp = UP ? ((t & 1) ? W3P : W1P) : W2P;
        const uint32_t rt = (uint32_t)(r0 + 16 * (UP ? t >> 1 : t));
        const uint32_t row = rt + (uint32_t)(lane & 15);
        rp[t] = make_rsrc(eb + bank.off[mp], pitch_p * (uint32_t)n_out);
        rs[t] = make_rsrc(eb + bank.off[mp + 1], pitch_s * (uint32_t)n_out);
        vp[t] = K3G_F4_FRIENDLY ? (rt + (uint32_t)(lane >> 2)) * pitch_p + 16u * (uint32_t)(lane & 3)
                                : row * pitch_p + 16u * (uint32_t)(lane >> 4);
        vs[t] = row * pitch_s;
    }
    // block k: tile k / (NCK/4), chunks 4*(k % (NCK/4)) .. +3
    uint4 A[NBUF][CPB], S[NBUF];
    auto load_block = [&](int k) {
        const int t = k / (NCK / CPB), c0 = CPB * (k % (NCK / CPB)), b = k % NBUF;
#pragma unroll
        for (int c = 0; c < CPB; ++c) A[b][c] = buf_load16(rp[t], vp[t], (uint32_t)(c0 + c) * 64u);
        S[b] = buf_load16(rs[t], vs[t], (uint32_t)c0 * 4u);
    };
    // the bucket: wavefront 0 of workgroup b writes counts and offsets
    // [64b, 64b + 64) (workgroup 0 also perm, inv, active)
    if (UP && wave == 0)
        for (int part = blockIdx.x; part * kWave <= rt.n_experts; part += gridDim.x)
            route1_write_bucket_part(rt, r1, top_k, lane, part);
    // B: this workgroup's vector of pieces into LDS (no registers); then the
    // first NBUF - 1 blocks of weights. The wait before the barrier leaves
    // exactly those in flight (vmcnt counts the bucket's stores, the DMA and
    // the weight loads in the order they were issued).
    {
        const int pos_b = UP ? 0 : p0;
        const uint8_t *src = pieces + (size_t)pos_b * NCK * f4::kChunkBytes;
        const uint32_t lb = lds_addr(lds_b);
        constexpr int units = NCK * f4::kChunkBytes / 1024;  // 1 KB per wavefront instruction
        for (int u = wave; u < units; u += f4::kWaves) dma16(src, 1024u * u + 16u * lane, lb + 1024u * u);
    }
    __asm__ volatile("" ::: "memory");  // the weight loads stay after the DMA
    __builtin_amdgcn_sched_barrier(0);
    constexpr int PRO = NBUF - 1 < NB ? NBUF - 1 : NB;  // blocks loaded ahead
#pragma unroll
    for (int k = 0; k < PRO; ++k) load_block(k);
    wait_vm<PRO * (CPB + 1)>();
    __syncthreads();

    const uint32_t qsh = 8u * (uint32_t)(lane >> 4);
    // two accumulators per tile (even and odd chunks), so that consecutive
    // products do not wait for each other
    float4_t acc[TILES][2];
#pragma unroll
    for (int t = 0; t < TILES; ++t) acc[t][0] = acc[t][1] = float4_t{0.f, 0.f, 0.f, 0.f};
    // B of block k, read from LDS one block ahead
    uint4 Bv[2][CPB];
    uint32_t Bs[2][CPB];
    auto read_b = [&](int k) {
        const int c0 = CPB * (k % (NCK / CPB));
        // every tile reads B again from LDS: without this the compiler keeps the
        // first tile's reads of all chunks in registers for the later tiles
        if (c0 == 0) __asm__ volatile("" ::: "memory");
#pragma unroll
        for (int c = 0; c < CPB; ++c) {
            const int i = c0 + c;
            Bv[k & 1][c] = lds_b[i * (f4::kChunkBytes / 16) + lane];
            Bs[k & 1][c] = ((const uint32_t *)lds_b)[(i * f4::kChunkBytes + 1024) / 4 + lane];
        }
    };
    auto compute = [&](int k) {
        const int t = k / (NCK / CPB), b = k % NBUF;
#pragma unroll
        for (int c = 0; c < CPB; ++c) {
            const uint4 bv = Bv[k & 1][c];
            const v8i_t B = {(int)bv.x, (int)bv.y, (int)bv.z, (int)bv.w, 0, 0, 0, 0};
            const uint32_t sd = c == 0 ? S[b].x : c == 1 ? S[b].y : c == 2 ? S[b].z : S[b].w;
            const uint32_t sa = __builtin_amdgcn_ubfe(sd, qsh, 8);
            // scale 255: the group is left out (its data zeroed, its scale made finite)
            const uint32_t keep = sa == 255u ? 0u : ~0u;
            const uint4 a = K3G_F4_FRIENDLY ? to_operand(A[b][c], 4 * (4 * (lane & 15) + (lane >> 4))) : A[b][c];
            const v8i_t Av = {(int)(a.x & keep), (int)(a.y & keep), (int)(a.z & keep), (int)(a.w & keep), 0, 0, 0, 0};
            float4_t &ac = acc[t][c & 1];
            ac = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(Av, B, ac, 4, 4, 0, (int)(sa & keep), 0,
                                                                  (int)Bs[k & 1][c]);
        }
    };
    read_b(0);
#pragma unroll
    for (int k = 0; k < NB; ++k) {
        if (k + NBUF - 1 < NB) load_block(k + NBUF - 1);
        if (k + 1 < NB) read_b(k + 1);
        __builtin_amdgcn_sched_barrier(0);
        compute(k);
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int t = 0; t < TILES; ++t) acc[t][0] += acc[t][1];
    // (no early exit for a dead wavefront here: a branch around the epilogue
    // would let the compiler sink every product into it, after all the loads)

    // sum the 16 piece columns: lanes 16w..16w+15 hold one row block's columns
#pragma unroll
    for (int t = 0; t < TILES; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            float sm = acc[t][0][v];
            sm += dpp<0xB1>(sm);
            sm += dpp<0x4E>(sm);
            sm += dpp<0x141>(sm);
            sm += dpp<0x140>(sm);
            acc[t][0][v] = sm;
        }
    // lane (q = lane & 15) < 8 holds row 16*ts + 4*(lane >> 4) + v, ts = q >> 2, v = q & 3
    const int q = lane & 15, ts = (q >> 2) & 1, v = q & 3;
    auto sel = [&](const float4_t &x0, const float4_t &x1) {
        const float4_t &x = ts ? x1 : x0;
        return v == 0 ? x[0] : v == 1 ? x[1] : v == 2 ? x[2] : x[3];
    };
    const int row = r0 + 16 * ts + 4 * (lane >> 4) + v;
    if constexpr (UP) {
        const float g = sel(acc[0][0], acc[2][0]);
        const float u = sel(acc[1][0], acc[3][0]);
        const float hv = situ(g, u);
        if (live && q < 8)
            for (int p = p0; p < p1; ++p) out[(size_t)p * n_out + row] = hv;
        // the pieces of this group of h: entry j (row r0 + j) from lane
        // 16*((j%16)/4) + 4*(j/16) + j%4 into lanes j and 32 + j
        const int j = lane & 31;
        const float hj = __shfl(hv, 16 * ((j & 15) >> 2) + 4 * (j >> 4) + (j & 3));
        const int g32 = r0 / kGroup;  // the group's index in a row of h
        const size_t hstride = (size_t)(inter / 128) * f4::kChunkBytes;
        uint8_t *dst = hp + (size_t)p0 * hstride + (g32 >> 2) * f4::kChunkBytes;
        split_group(hj, dst, g32 & 3, live && lane < 32);
        for (int p = p0 + 1; p < p1; ++p)  // a repeated expert: equal pairs, equal pieces
            split_group(hj, dst + (size_t)(p - p0) * hstride, g32 & 3, live && lane < 32);
    } else {
        const float y = sel(acc[0][0], acc[1][0]);
        if (live && q < 8)
            for (int p = p0; p < p1; ++p) out[(size_t)p * n_out + row] = y;
    }
}

// More tokens: workgroup w takes the pass k = w / row_blocks of the work
// table the bucket wrote (passes[0] = count, then (slot, pass index) pairs):
// the slot's sorted pairs [p0, p1), up to NPP of them, and 128 rows
// (4 wavefronts x 32). The pairs' B operands (x's pieces per token for UP,
// h's pieces per pair for DOWN) sit in LDS; every A fragment of the weights
// feeds one product per pair, so the weights stream once per pass. A pass
// with fewer than NPP pairs repeats its last pair (products not stored).
template <bool UP, int NCK, int NPP>
__global__ __launch_bounds__(f4::kWaves * kWave, 2) void moe_f4m_kernel(
    float *__restrict__ out, const uint8_t *__restrict__ pieces, uint8_t *__restrict__ hp, BankDev bank,
    const int32_t *__restrict__ active, const int32_t *__restrict__ offsets, const int32_t *__restrict__ perm,
    const int32_t *__restrict__ passes, int top_k, int latent, int inter) {
    constexpr int TILES = UP ? 4 : 2;
    constexpr int CPB = 4;                 // chunks per block
    constexpr int NB = TILES * NCK / CPB;  // blocks
    constexpr int NBUF = 4;                // ring of blocks
    constexpr int ngrp = 4 * NCK;
    constexpr int VEC = NCK * f4::kChunkBytes;  // one vector's pieces
    extern __shared__ uint4 lds_b[];
    const int lane = threadIdx.x & (kWave - 1);
    const int psrc = 4 * (4 * (lane & 15) + (lane >> 4));  // row-friendly loads: see to_operand
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int n_out = UP ? inter : latent;
    const int row_blocks = (n_out / f4::kRows + f4::kWaves - 1) / f4::kWaves;
    // (plain order: about one pair per expert leaves nothing for XCD groups of
    // passes to share; they measured slower here)
    const int item = (int)blockIdx.x;
    const int k = item / row_blocks;
    if (k >= passes[0]) return;  // whole workgroup
    const int slot = passes[1 + 2 * k], pass = passes[2 + 2 * k];
    const int e = active[1 + slot];
    const int p0 = offsets[e] + pass * NPP;
    const int np = min(NPP, offsets[e + 1] - p0);
    const int blk32 = (item - k * row_blocks) * f4::kWaves + wave;
    const bool live = blk32 < n_out / f4::kRows;

    // the wavefront's tiles: buffer resources, and this lane's row offsets
    const uint8_t *eb = bank.base + (int64_t)e * bank.stride;
    constexpr uint32_t pitch_p = 16u * ngrp, pitch_s = ngrp;
    const int r0 = (live ? blk32 : 0) * f4::kRows;
    rsrc_t rp[TILES], rs[TILES];
    uint32_t vp[TILES], vs[TILES];
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
        const int mp = UP ? ((t & 1) ? W3P : W1P) : W2P;
        const uint32_t rt = (uint32_t)(r0 + 16 * (UP ? t >> 1 : t));
        const uint32_t row = rt + (uint32_t)(lane & 15);
        rp[t] = make_rsrc(eb + bank.off[mp], pitch_p * (uint32_t)n_out);
        rs[t] = make_rsrc(eb + bank.off[mp + 1], pitch_s * (uint32_t)n_out);
        vp[t] = K3G_F4_FRIENDLY ? (rt + (uint32_t)(lane >> 2)) * pitch_p + 16u * (uint32_t)(lane & 3)
                                : row * pitch_p + 16u * (uint32_t)(lane >> 4);
        vs[t] = row * pitch_s;
    }
    uint4 A[NBUF][CPB];
    auto load_block = [&](int kb) {
        const int t = kb / (NCK / CPB), c0 = CPB * (kb % (NCK / CPB)), b = kb % NBUF;
#pragma unroll
        for (int c = 0; c < CPB; ++c) A[b][c] = buf_load16(rp[t], vp[t], (uint32_t)(c0 + c) * 64u);
    };
    // the rows' scale bytes in windows, once, as the four-pair kernel takes
    // them (chunk i's byte for lane (r, q) comes by one ds_bpermute)
    constexpr int NSW = (NCK + 15) / 16;
    uint4 SW[NSW][TILES];
    // B: the pass's NPP vectors of pieces into LDS, then the first weight blocks
    {
        const uint32_t lb = lds_addr(lds_b);
        constexpr int units = VEC / 1024;  // 1 KB per wavefront instruction
#pragma unroll
        for (int q = 0; q < NPP; ++q) {
            const int pq = p0 + min(q, np - 1);
            const int v = UP ? perm[pq] / top_k : pq;  // UP: the pair's token; DOWN: the pair's h
            const uint8_t *src = pieces + (size_t)v * VEC;
            for (int u = wave; u < units; u += f4::kWaves)
                dma16(src, 1024u * u + 16u * lane, lb + (uint32_t)(q * VEC) + 1024u * u);
        }
    }
    __asm__ volatile("" ::: "memory");  // the weight loads stay after the DMA
    __builtin_amdgcn_sched_barrier(0);
    constexpr int PRO = NBUF - 1 < NB ? NBUF - 1 : NB;
#pragma unroll
    for (int j = 0; j < NSW; ++j) {
        const uint32_t off = (uint32_t)min(16 * ((lane >> 4) + 4 * j), ngrp - 16);
#pragma unroll
        for (int t = 0; t < TILES; ++t) SW[j][t] = buf_load16(rs[t], vs[t] + off, 0u);
    }
#pragma unroll
    for (int kb = 0; kb < PRO; ++kb) load_block(kb);
    wait_vm<PRO * CPB>();
    __syncthreads();

    const uint32_t qsh = 8u * (uint32_t)(lane >> 4);
    float4_t acc[NPP][TILES];
#pragma unroll
    for (int q = 0; q < NPP; ++q)
#pragma unroll
        for (int t = 0; t < TILES; ++t) acc[q][t] = float4_t{0.f, 0.f, 0.f, 0.f};
    // the lane's LDS index, opaque to the compiler: every read is then one base
    // register plus an immediate offset (known, the compiler rebuilds each
    // address from the previous one and keeps them all live)
    int li = lane;
    __asm__ volatile("" : "+v"(li));
    const uint4 *bq[NPP];
    const uint32_t *sq[NPP];
#pragma unroll
    for (int q = 0; q < NPP; ++q) {
        bq[q] = lds_b + q * (VEC / 16) + li;
        sq[q] = (const uint32_t *)lds_b + (q * VEC + 1024) / 4 + li;
    }
    // B of block kb for every pair, read from LDS one block ahead
    uint4 Bv[2][NPP][CPB];
    uint32_t Bs[2][NPP][CPB];
    auto read_b = [&](int kb) {
        const int c0 = CPB * (kb % (NCK / CPB));
        // every tile reads B again: without this the compiler keeps the first
        // tile's reads of all chunks in registers for the later tiles
        if (c0 == 0) __asm__ volatile("" ::: "memory");
#pragma unroll
        for (int q = 0; q < NPP; ++q)
#pragma unroll
            for (int c = 0; c < CPB; ++c) {
                Bv[kb & 1][q][c] = bq[q][(c0 + c) * (f4::kChunkBytes / 16)];
                Bs[kb & 1][q][c] = sq[q][(c0 + c) * (f4::kChunkBytes / 4)];
            }
    };
    auto compute = [&](int kb) {
        const int t = kb / (NCK / CPB), b = kb % NBUF, c0 = CPB * (kb % (NCK / CPB));
#pragma unroll
        for (int c = 0; c < CPB; ++c) {
            const int i = c0 + c;
            const uint4 w = SW[i / 16][t];
            const uint32_t d = i % 4 == 0 ? w.x : i % 4 == 1 ? w.y : i % 4 == 2 ? w.z : w.w;
            const uint32_t sd = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * ((lane & 15) + 16 * ((i / 4) % 4)), (int)d);
            const uint32_t sa = __builtin_amdgcn_ubfe(sd, qsh, 8);
            const uint32_t keep = sa == 255u ? 0u : ~0u;  // scale 255: the group is left out
            const uint4 a = K3G_F4_FRIENDLY ? to_operand(A[b][c], psrc) : A[b][c];
            const v8i_t Av = {(int)(a.x & keep), (int)(a.y & keep), (int)(a.z & keep), (int)(a.w & keep), 0, 0, 0, 0};
#pragma unroll
            for (int q = 0; q < NPP; ++q) {
                const uint4 bv = Bv[kb & 1][q][c];
                const v8i_t B = {(int)bv.x, (int)bv.y, (int)bv.z, (int)bv.w, 0, 0, 0, 0};
                acc[q][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(Av, B, acc[q][t], 4, 4, 0,
                                                                             (int)(sa & keep), 0, (int)Bs[kb & 1][q][c]);
            }
        }
    };
    read_b(0);
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) {
        if (kb + NBUF - 1 < NB) load_block(kb + NBUF - 1);
        if (kb + 1 < NB) read_b(kb + 1);
        __builtin_amdgcn_sched_barrier(0);
        compute(kb);
        __builtin_amdgcn_sched_barrier(0);
    }
    // every product is done here: left free, the compiler sinks a later pair's
    // products into the epilogue past the earlier pairs' stores, holding their
    // operands live all the way
#pragma unroll
    for (int q = 0; q < NPP; ++q)
#pragma unroll
        for (int t = 0; t < TILES; ++t) __asm__ volatile("" : "+v"(acc[q][t]));
    // (no early exit for a dead wavefront here: a branch around the epilogue
    // would let the compiler sink every product into it, after all the loads)

    // per pair: sum the 16 piece columns (lanes 16w..16w+15 hold one row
    // block's columns), then lane q < 8 of each 16 holds row 16*ts + 4*(lane >> 4) + v
    const int qd = lane & 15, ts = (qd >> 2) & 1, v = qd & 3;
    const int row = r0 + 16 * ts + 4 * (lane >> 4) + v;
    float hvs[NPP];  // UP: this lane's h of each pair
#pragma unroll
    for (int q = 0; q < NPP; ++q) {
#pragma unroll
        for (int t = 0; t < TILES; ++t)
#pragma unroll
            for (int vv = 0; vv < 4; ++vv) {
                float sm = acc[q][t][vv];
                sm += dpp<0xB1>(sm);
                sm += dpp<0x4E>(sm);
                sm += dpp<0x141>(sm);
                sm += dpp<0x140>(sm);
                acc[q][t][vv] = sm;
            }
        auto sel = [&](const float4_t &x0, const float4_t &x1) {
            const float4_t &x = ts ? x1 : x0;
            return v == 0 ? x[0] : v == 1 ? x[1] : v == 2 ? x[2] : x[3];
        };
        const bool store = live && q < np;
        const int pq = p0 + q;
        if constexpr (UP) {
            const float hv = situ(sel(acc[q][0], acc[q][2]), sel(acc[q][1], acc[q][3]));
            if (store && qd < 8) out[(size_t)pq * n_out + row] = hv;
            hvs[q] = hv;
        } else {
            const float y = sel(acc[q][0], acc[q][1]);
            if (store && qd < 8) out[(size_t)pq * n_out + row] = y;
        }
    }
    if constexpr (UP) {
        // each pair's group of h as pieces for the down-projection, two pairs
        // a call: pair q in lanes 0..31, q + 1 in lanes 32..63
        const int j = lane & 31;
        const int src = 16 * ((j & 15) >> 2) + 4 * (j >> 4) + (j & 3);
        const int g32 = r0 / kGroup;
        const size_t hstride = (size_t)(inter / 128) * f4::kChunkBytes;
        const int hi = lane >> 5;
#pragma unroll
        for (int q = 0; q < NPP; q += 2) {
            const float h0 = __shfl(hvs[q], src), h1 = __shfl(hvs[q + 1], src);
            const int qq = q + hi;
            const bool store = live && qq < np;
            split_group(hi ? h1 : h0, hp + (size_t)(store ? p0 + qq : 0) * hstride + (g32 >> 2) * f4::kChunkBytes,
                        g32 & 3, store);
        }
    }
}

// Denser routing (several pairs per expert): four pairs a pass and eight
// wavefronts a workgroup sharing them (their 4 x 1280 bytes per chunk stay in
// LDS, up to 160 KB), each wavefront owning four row tiles (UP: w1 and w3 of
// 32 rows; DOWN: 64 rows). The loop runs chunk by chunk over all four tiles,
// so each B fragment read from LDS feeds four products and each A fragment
// four (one per pair): 16 products per chunk for 4 A and 4 B fragments.
// Operand A streams through a 3-deep ring of 2-chunk blocks; an item's scale
// bytes come in two 16-byte loads a tile, handed to the lanes chunk by chunk
// by ds_bpermute; B of the next chunk is read while this chunk's products
// issue.
//
// The grid is persistent: one workgroup per CU (the LDS holds one), walking
// the items (pass, row block), row blocks fastest, gridDim apart. When an
// item's products are done, the next item's B (into the LDS, once every
// wavefront has read its last chunk) and its first weight blocks are
// requested before this item's epilogue, so the epilogue's vector work and
// stores and the next item's first loads overlap instead of leaving the
// CU's memory pipe idle between workgroups.
template <bool UP, int NCK>
__global__ __launch_bounds__(8 * kWave, 1) void moe_f4q_kernel(
    float *__restrict__ out, const uint8_t *__restrict__ pieces, uint8_t *__restrict__ hp, BankDev bank,
    const int32_t *__restrict__ active, const int32_t *__restrict__ offsets, const int32_t *__restrict__ perm,
    const int32_t *__restrict__ passes, int top_k, int latent, int inter) {
    constexpr int NPP = 4, WAVES = 8, TILES = 4;
    constexpr int CPB = 2, NB = NCK / CPB, NBUF = 3;
    static_assert(NB % 2 == 0, "a scale load covers two blocks");
    constexpr int ROWS_W = UP ? 32 : 64;
    constexpr int ngrp = 4 * NCK;
    constexpr int VEC = NCK * f4::kChunkBytes;
    extern __shared__ uint4 lds_b[];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int n_out = UP ? inter : latent;
    // (row blocks fastest: the workgroups running at once cover every row
    // block of a few passes; an order with the passes fastest, for L2 sharing
    // between the passes of one expert, measured slower: all of them then
    // read the same rows of different experts)
    const int row_blocks = (n_out + WAVES * ROWS_W - 1) / (WAVES * ROWS_W);
    const int n_items = passes[0] * row_blocks;
    // XCD-aware order: workgroup w runs on XCD w % 8 (the dispatcher deals
    // workgroups round the XCDs); the items come in groups of G consecutive
    // passes (all their row blocks), group g on XCD g % 8, so the row blocks
    // of a pass share its B, and the passes of one expert its weights,
    // through that XCD's L2
    constexpr int G = UP ? K3G_F4Q_GROUP_UP : K3G_F4Q_GROUP;
    const bool xcd = G > 0 && gridDim.x % 8 == 0;
    const int per = xcd ? (int)gridDim.x / 8 : (int)gridDim.x;
    const int gi = G * row_blocks;
    // Where a group's items divide evenly among the XCD's workgroups, each
    // takes a run of ipw consecutive items (row blocks of one pass, mostly),
    // and loads the pass's B once for the run.
    const bool runs = xcd && gi % per == 0;
    const int ipw = runs ? gi / per : 1;
    auto item_at = [&](int L) {  // the workgroup's L-th item (its own sequence)
        if (!xcd) return L;
        const int x = (int)blockIdx.x % 8;
        if (runs) return (x + 8 * (L / ipw)) * gi + ((int)blockIdx.x / 8) * ipw + L % ipw;
        return (x + 8 * (L / gi)) * gi + L % gi;
    };
    const int step_loc = runs ? 1 : per;
    int loc = !xcd ? (int)blockIdx.x : runs ? 0 : (int)blockIdx.x / 8;
    int item = item_at(loc);
    if (item >= n_items) return;  // whole workgroup

    // the current item
    int p0 = 0, np = 0, r0 = 0;
    bool live = false;
    constexpr uint32_t pitch_p = 16u * ngrp, pitch_s = ngrp;
    rsrc_t rp[TILES], rs[TILES];
    uint32_t vp[TILES], vs[TILES];
    auto setup = [&](int it) {
        const int k = it / row_blocks;
        const int slot = passes[1 + 2 * k], pass = passes[2 + 2 * k];
        const int e = active[1 + slot];
        p0 = offsets[e] + pass * NPP;
        np = min(NPP, offsets[e + 1] - p0);
        r0 = ((it - k * row_blocks) * WAVES + wave) * ROWS_W;
        live = r0 < n_out;
        const uint8_t *eb = bank.base + (int64_t)e * bank.stride;
#pragma unroll
        for (int t = 0; t < TILES; ++t) {
            const int mp = UP ? ((t & 1) ? W3P : W1P) : W2P;
            const uint32_t rt = (uint32_t)((live ? r0 : 0) + 16 * (UP ? t >> 1 : t));
            const uint32_t row = rt + (uint32_t)(lane & 15);
            rp[t] = make_rsrc(eb + bank.off[mp], pitch_p * (uint32_t)n_out);
            rs[t] = make_rsrc(eb + bank.off[mp + 1], pitch_s * (uint32_t)n_out);
            vp[t] = K3G_F4_FRIENDLY ? (rt + (uint32_t)(lane >> 2)) * pitch_p + 16u * (uint32_t)(lane & 3)
                                    : row * pitch_p + 16u * (uint32_t)(lane >> 4);
            vs[t] = row * pitch_s;
        }
    };
    uint4 A[NBUF][TILES][CPB];
    auto load_block = [&](int kb) {
        const int b = kb % NBUF;
#pragma unroll
        for (int t = 0; t < TILES; ++t)
#pragma unroll
            for (int c = 0; c < CPB; ++c)
                A[b][t][c] = buf_load16(rp[t], vp[t], (uint32_t)(CPB * kb + c) * 64u);
    };
    // The item's scale bytes, once: lane (r, q) of a tile holds bytes
    // [16 (q + 4j), +16) of row r in SW[j] (4 lanes, 64 bytes a row per load;
    // a window past the row's last byte -- never read -- is moved back into
    // it, so no load leaves the matrix). Chunk i's group q of row r, byte
    // 4i + q, then sits in lane (r, (i / 4) % 4), window i / 16, dword i % 4,
    // byte q: one ds_bpermute a tile and chunk brings it to lane (r, q).
    constexpr int NSW = (NCK + 15) / 16;
    uint4 SW[NSW][TILES];
    auto load_sw = [&]() {
#pragma unroll
        for (int j = 0; j < NSW; ++j) {
            const uint32_t off = (uint32_t)min(16 * ((lane >> 4) + 4 * j), ngrp - 16);
#pragma unroll
            for (int t = 0; t < TILES; ++t) SW[j][t] = buf_load16(rs[t], vs[t] + off, 0u);
        }
    };
    // B: the item's four vectors of pieces into LDS (a short pass repeats its
    // last pair)
    auto load_b = [&]() {
        const uint32_t lb = lds_addr(lds_b);
        constexpr int units = VEC / 1024;
#pragma unroll
        for (int q = 0; q < NPP; ++q) {
            const int pq = p0 + min(q, np - 1);
            const int vec = UP ? perm[pq] / top_k : pq;
            const uint8_t *src = pieces + (size_t)vec * VEC;
            for (int u = wave; u < units; u += WAVES)
                dma16(src, 1024u * u + 16u * lane, lb + (uint32_t)(q * VEC) + 1024u * u);
        }
    };
    constexpr int PRO = NBUF - 1 < NB ? NBUF - 1 : NB;
    auto prologue = [&](bool with_b) {
        if (with_b) load_b();
        __asm__ volatile("" ::: "memory");  // the weight loads stay after the DMA
        __builtin_amdgcn_sched_barrier(0);
        load_sw();
#pragma unroll
        for (int kb = 0; kb < PRO; ++kb) load_block(kb);
    };
    setup(item);
    prologue(true);
    wait_vm<0>();
    __syncthreads();

    const uint32_t qsh = 8u * (uint32_t)(lane >> 4);
    int li = lane;
    __asm__ volatile("" : "+v"(li));
    const uint4 *bq = lds_b + li;
    const uint32_t *sq = (const uint32_t *)lds_b + 256 + li;
    const int qd = lane & 15, v = qd & 3;
    const int psrc = 4 * (4 * (lane & 15) + (lane >> 4));  // byte address of the lane loaded for (r, q)
    while (true) {
        float4_t acc[NPP][TILES];
#pragma unroll
        for (int q = 0; q < NPP; ++q)
#pragma unroll
            for (int t = 0; t < TILES; ++t) acc[q][t] = float4_t{0.f, 0.f, 0.f, 0.f};
        uint4 Bv[2][NPP];
        uint32_t Bs[2][NPP];
        // chunk i's scale dword per tile (byte q is lane (r, q)'s), brought in at
        // the chunk's start (two of them, held a chunk ahead, spill registers)
        uint32_t Sd[1][TILES];
        auto read_b = [&](int i) {
#pragma unroll
            for (int q = 0; q < NPP; ++q) {
                Bv[i & 1][q] = bq[(q * VEC + i * f4::kChunkBytes) / 16];
                Bs[i & 1][q] = sq[(q * VEC + i * f4::kChunkBytes) / 4];
            }
        };
        auto read_s = [&](int i) {
            const int src = 4 * ((lane & 15) + 16 * ((i / 4) % 4));  // byte address of the source lane
#pragma unroll
            for (int t = 0; t < TILES; ++t) {
                const uint4 w = SW[i / 16][t];
                const uint32_t d = i % 4 == 0 ? w.x : i % 4 == 1 ? w.y : i % 4 == 2 ? w.z : w.w;
                Sd[0][t] = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)d);
            }
        };
        read_b(0);
#pragma unroll
        for (int i = 0; i < NCK; ++i) {
            const int kb = i / CPB, c = i % CPB, b = kb % NBUF;
            if (c == 0 && kb + NBUF - 1 < NB) load_block(kb + NBUF - 1);
            if (i + 1 < NCK) read_b(i + 1);
            read_s(i);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int t = 0; t < TILES; ++t) {
                const uint32_t sa = __builtin_amdgcn_ubfe(Sd[0][t], qsh, 8);
                const uint32_t keep = sa == 255u ? 0u : ~0u;  // scale 255: the group is left out
                const uint4 a = K3G_F4_FRIENDLY ? to_operand(A[b][t][c], psrc) : A[b][t][c];
                const v8i_t Av = {(int)(a.x & keep), (int)(a.y & keep), (int)(a.z & keep), (int)(a.w & keep), 0, 0, 0, 0};
#pragma unroll
                for (int q = 0; q < NPP; ++q) {
                    const uint4 bv = Bv[i & 1][q];
                    const v8i_t B = {(int)bv.x, (int)bv.y, (int)bv.z, (int)bv.w, 0, 0, 0, 0};
                    acc[q][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(Av, B, acc[q][t], 4, 4, 0,
                                                                                 (int)(sa & keep), 0, (int)Bs[i & 1][q]);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int q = 0; q < NPP; ++q)
#pragma unroll
            for (int t = 0; t < TILES; ++t) __asm__ volatile("" : "+v"(acc[q][t]));

        // this item's epilogue inputs; then the next item's first loads
        const int cp0 = p0, cnp = np, cr0 = r0;
        const bool clive = live;
        const int next = item_at(loc + step_loc);
        const bool more = next < n_items;
        const bool same_b = next / row_blocks == item / row_blocks;  // the same pass: B stays
        __syncthreads();  // every wavefront has read its last chunk of B
        if (more) {
            setup(next);
            prologue(!same_b);
        }
        __builtin_amdgcn_sched_barrier(0);

        // per pair: sum the 16 piece columns, then lane qd = lane & 15 holds row
        // tile ts = qd >> 2, row 4 * (lane >> 4) + (qd & 3) (UP: g and u of the
        // wavefront's two row tiles, lanes qd < 8)
        float hvs[NPP];  // UP: this lane's h of each pair
#pragma unroll
        for (int q = 0; q < NPP; ++q) {
#pragma unroll
            for (int t = 0; t < TILES; ++t)
#pragma unroll
                for (int vv = 0; vv < 4; ++vv) {
                    float sm = acc[q][t][vv];
                    sm += dpp<0xB1>(sm);
                    sm += dpp<0x4E>(sm);
                    sm += dpp<0x141>(sm);
                    sm += dpp<0x140>(sm);
                    acc[q][t][vv] = sm;
                }
            // values, not references: a lane-dependent choice of an array element
            // by reference puts the accumulators on the stack
            float pv[TILES];
#pragma unroll
            for (int t = 0; t < TILES; ++t) {
                const float4_t x = acc[q][t];
                pv[t] = v == 0 ? x[0] : v == 1 ? x[1] : v == 2 ? x[2] : x[3];
            }
            const bool store = clive && q < cnp;
            const int pq = cp0 + q;
            if constexpr (UP) {
                const int ts = (qd >> 2) & 1;
                const int row = cr0 + 16 * ts + 4 * (lane >> 4) + v;
                const float g = ts ? pv[2] : pv[0], u = ts ? pv[3] : pv[1];
                const float hv = situ(g, u);
                if (store && qd < 8) out[(size_t)pq * n_out + row] = hv;
                hvs[q] = hv;
            } else {
                const int ts = qd >> 2;
                const int row = cr0 + 16 * ts + 4 * (lane >> 4) + v;
                const float y = ts == 0 ? pv[0] : ts == 1 ? pv[1] : ts == 2 ? pv[2] : pv[3];
                if (store) out[(size_t)pq * n_out + row] = y;
            }
        }
        if constexpr (UP) {
            // each pair's group of h (the wavefront's 32 rows) as pieces for the
            // down-projection, two pairs a call: pair q in lanes 0..31, q + 1 in
            // lanes 32..63 (entry e of the group in lane e of its half)
            const int j = lane & 31;
            const int src = 16 * ((j & 15) >> 2) + 4 * (j >> 4) + (j & 3);
            const int g32 = cr0 / kGroup;
            const size_t hstride = (size_t)(inter / 128) * f4::kChunkBytes;
            const int hi = lane >> 5;
#pragma unroll
            for (int q = 0; q < NPP; q += 2) {
                const float h0 = __shfl(hvs[q], src), h1 = __shfl(hvs[q + 1], src);
                const int qq = q + hi;
                const bool store = clive && qq < cnp;
                split_group(hi ? h1 : h0, hp + (size_t)(store ? cp0 + qq : 0) * hstride + (g32 >> 2) * f4::kChunkBytes,
                            g32 & 3, store);
            }
        }
        if (!more) break;
        // the next item's B and first blocks (and this epilogue's stores)
        wait_vm<0>();
        __syncthreads();
        item = next;
        loc += step_loc;
    }
}

// Dense routing (many pairs per expert): eight pairs a pass, so an expert's
// weights stream once per eight pairs. Their pieces do not fit in LDS whole
// (8 x 1280 bytes per chunk), so they stream through it chunk by chunk in a
// ring of 3 buffers, two chunks ahead: wavefront w brings pair w's 1 KB of
// pieces and 256 bytes of scales of each chunk (two DMA instructions, the same
// count in every wavefront, so the waits are exact). Eight wavefronts, four
// row tiles each (UP: w1 and w3 of 32 rows; DOWN: 64 rows); operand A in a
// 4-deep ring of single chunks (row-friendly loads); the rows' scale bytes in
// windows loaded once an item, as the four-pair kernel takes them; per chunk
// each B fragment feeds four products and each A fragment eight.
template <bool UP, int NCK>
__global__ __launch_bounds__(8 * kWave, 1) void moe_f4s_kernel(
    float *__restrict__ out, const uint8_t *__restrict__ pieces, uint8_t *__restrict__ hp, BankDev bank,
    const int32_t *__restrict__ active, const int32_t *__restrict__ offsets, const int32_t *__restrict__ perm,
    const int32_t *__restrict__ passes, int top_k, int latent, int inter) {
    constexpr int NPP = 8, WAVES = 8, TILES = 4, NBUF = 4, NBB = 3;
    constexpr int ROWS_W = UP ? 32 : 64;
    constexpr int ngrp = 4 * NCK;
    constexpr int VEC = NCK * f4::kChunkBytes;
    constexpr int BBUF = NPP * f4::kChunkBytes;  // one chunk of all pairs: 10 KB
    __shared__ __attribute__((aligned(16))) uint8_t lds_b[NBB * BBUF];
    const int lane = threadIdx.x & (kWave - 1);
    const int psrc = 4 * (4 * (lane & 15) + (lane >> 4));  // row-friendly loads: see to_operand
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int n_out = UP ? inter : latent;
    const int row_blocks = (n_out + WAVES * ROWS_W - 1) / (WAVES * ROWS_W);
    // workgroup = (pass, row block), row blocks fastest within groups of
    // K3G_F4S_GROUP consecutive passes, each group on one XCD: the row blocks
    // of a pass share its B, and the passes of one expert its weights, through
    // that XCD's L2 (the launch rounds the grid to whole rounds of 8 groups)
    const int item = xcd_item((int)blockIdx.x, K3G_F4S_GROUP * row_blocks);
    const int k = item / row_blocks;
    if (k >= passes[0]) return;  // whole workgroup
    const int slot = passes[1 + 2 * k], pass = passes[2 + 2 * k];
    const int e = active[1 + slot];
    const int p0 = offsets[e] + pass * NPP;
    const int np = min(NPP, offsets[e + 1] - p0);
    const int r0 = ((item - k * row_blocks) * WAVES + wave) * ROWS_W;
    const bool live = r0 < n_out;

    const uint8_t *eb = bank.base + (int64_t)e * bank.stride;
    constexpr uint32_t pitch_p = 16u * ngrp, pitch_s = ngrp;
    rsrc_t rp[TILES], rs[TILES];
    uint32_t vp[TILES], vs[TILES];
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
        const int mp = UP ? ((t & 1) ? W3P : W1P) : W2P;
        const uint32_t rt = (uint32_t)((live ? r0 : 0) + 16 * (UP ? t >> 1 : t));
        const uint32_t row = rt + (uint32_t)(lane & 15);
        rp[t] = make_rsrc(eb + bank.off[mp], pitch_p * (uint32_t)n_out);
        rs[t] = make_rsrc(eb + bank.off[mp + 1], pitch_s * (uint32_t)n_out);
        vp[t] = K3G_F4_FRIENDLY ? (rt + (uint32_t)(lane >> 2)) * pitch_p + 16u * (uint32_t)(lane & 3)
                                : row * pitch_p + 16u * (uint32_t)(lane >> 4);
        vs[t] = row * pitch_s;
    }
    uint4 A[NBUF][TILES];
    auto load_a = [&](int i) {
        const int b = i % NBUF;
#pragma unroll
        for (int t = 0; t < TILES; ++t) A[b][t] = buf_load16(rp[t], vp[t], (uint32_t)i * 64u);
    };
    // the item's scale bytes, once, as the four-pair kernel takes them: lane
    // (r, q) of a tile holds bytes [16 (q + 4j), +16) of row r in SW[j]; chunk
    // i's byte for lane (r, q) comes by one ds_bpermute a tile
    constexpr int NSW = (NCK + 15) / 16;
    uint4 SW[NSW][TILES];
    // this wavefront's pair (the pass's last pair again past its end)
    const int pw = p0 + min(wave, np - 1);
    const uint8_t *src = pieces + (size_t)(UP ? perm[pw] / top_k : pw) * VEC;
    const uint32_t lb = lds_addr(lds_b);
    auto dma_b = [&](int i) {
        const uint32_t dst = lb + (uint32_t)((i % NBB) * BBUF + wave * f4::kChunkBytes);
        const uint8_t *s = src + (size_t)i * f4::kChunkBytes;
        dma16(s, 16u * lane, dst);
        dma4(s + 1024, 4u * lane, dst + 1024);
    };
    constexpr int VM_A = TILES;  // vector loads of one chunk of A
    // prologue: B of chunks 0 and 1, the scale windows, then A of chunks 0 .. NBUF-2
    dma_b(0);
    if (NCK > 1) dma_b(1);
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < NSW; ++j) {
        const uint32_t off = (uint32_t)min(16 * ((lane >> 4) + 4 * j), ngrp - 16);
#pragma unroll
        for (int t = 0; t < TILES; ++t) SW[j][t] = buf_load16(rs[t], vs[t] + off, 0u);
    }
#pragma unroll
    for (int i = 0; i < NBUF - 1; ++i)
        if (i < NCK) load_a(i);
    wait_vm<(NBUF - 1) * VM_A>();
    __syncthreads();

    const uint32_t qsh = 8u * (uint32_t)(lane >> 4);
    float4_t acc[NPP][TILES];
#pragma unroll
    for (int q = 0; q < NPP; ++q)
#pragma unroll
        for (int t = 0; t < TILES; ++t) acc[q][t] = float4_t{0.f, 0.f, 0.f, 0.f};
    int li = lane;
    __asm__ volatile("" : "+v"(li));
#pragma unroll
    for (int i = 0; i < NCK; ++i) {
        const int b = i % NBUF;
        // requests: B two chunks ahead, then A NBUF-1 chunks ahead
        if (i + 2 < NCK) dma_b(i + 2);
        __asm__ volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        if (i + NBUF - 1 < NCK) load_a(i + NBUF - 1);
        __builtin_amdgcn_sched_barrier(0);
        const uint4 *bq = (const uint4 *)(lds_b + (i % NBB) * BBUF) + li;
        const uint32_t *sq = (const uint32_t *)(lds_b + (i % NBB) * BBUF + 1024) + li;
        uint32_t sa[TILES];
        v8i_t Av[TILES];
        const int ssrc = 4 * ((lane & 15) + 16 * ((i / 4) % 4));  // byte address of the source lane
#pragma unroll
        for (int t = 0; t < TILES; ++t) {
            const uint4 w = SW[i / 16][t];
            const uint32_t d = i % 4 == 0 ? w.x : i % 4 == 1 ? w.y : i % 4 == 2 ? w.z : w.w;
            sa[t] = __builtin_amdgcn_ubfe((uint32_t)__builtin_amdgcn_ds_bpermute(ssrc, (int)d), qsh, 8);
            const uint32_t keep = sa[t] == 255u ? 0u : ~0u;  // scale 255: the group is left out
            const uint4 a = K3G_F4_FRIENDLY ? to_operand(A[b][t], psrc) : A[b][t];
            Av[t] = v8i_t{(int)(a.x & keep), (int)(a.y & keep), (int)(a.z & keep), (int)(a.w & keep), 0, 0, 0, 0};
            sa[t] &= keep;
        }
#pragma unroll
        for (int q = 0; q < NPP; ++q) {
            const uint4 bv = bq[q * (f4::kChunkBytes / 16)];
            const uint32_t bs = sq[q * (f4::kChunkBytes / 4)];
            const v8i_t B = {(int)bv.x, (int)bv.y, (int)bv.z, (int)bv.w, 0, 0, 0, 0};
#pragma unroll
            for (int t = 0; t < TILES; ++t)
                acc[q][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(Av[t], B, acc[q][t], 4, 4, 0, (int)sa[t],
                                                                             0, (int)bs);
        }
        __builtin_amdgcn_sched_barrier(0);
        // chunk i+1's B is in LDS for every wavefront, and every wavefront is
        // done with buffer i % 3 before chunk i+3 is brought into it. Issued
        // after chunk i+1's B: A of chunk i+NBUF-2, B of chunk i+2, A of chunk
        // i+NBUF-1 (when they exist)
        if (i + 1 < NCK) {
            if (i + NBUF - 1 < NCK) wait_vm<2 * VM_A + 2>();
            else wait_vm<0>();
            __syncthreads();
        }
    }
#pragma unroll
    for (int q = 0; q < NPP; ++q)
#pragma unroll
        for (int t = 0; t < TILES; ++t) __asm__ volatile("" : "+v"(acc[q][t]));

    // per pair, as in the four-pair kernel
    const int qd = lane & 15, v = qd & 3;
    float hvs[NPP];  // UP: this lane's h of each pair
#pragma unroll
    for (int q = 0; q < NPP; ++q) {
#pragma unroll
        for (int t = 0; t < TILES; ++t)
#pragma unroll
            for (int vv = 0; vv < 4; ++vv) {
                float sm = acc[q][t][vv];
                sm += dpp<0xB1>(sm);
                sm += dpp<0x4E>(sm);
                sm += dpp<0x141>(sm);
                sm += dpp<0x140>(sm);
                acc[q][t][vv] = sm;
            }
        float pv[TILES];  // values: a lane-dependent choice by reference would go through scratch
#pragma unroll
        for (int t = 0; t < TILES; ++t) {
            const float4_t x = acc[q][t];
            pv[t] = v == 0 ? x[0] : v == 1 ? x[1] : v == 2 ? x[2] : x[3];
        }
        const bool store = live && q < np;
        const int pq = p0 + q;
        if constexpr (UP) {
            const int ts = (qd >> 2) & 1;
            const int row = r0 + 16 * ts + 4 * (lane >> 4) + v;
            const float hv = situ(ts ? pv[2] : pv[0], ts ? pv[3] : pv[1]);
            if (store && qd < 8) out[(size_t)pq * n_out + row] = hv;
            hvs[q] = hv;
        } else {
            const int ts = qd >> 2;
            const int row = r0 + 16 * ts + 4 * (lane >> 4) + v;
            const float y = ts == 0 ? pv[0] : ts == 1 ? pv[1] : ts == 2 ? pv[2] : pv[3];
            if (store) out[(size_t)pq * n_out + row] = y;
        }
    }
    if constexpr (UP) {
        // each pair's group of h as pieces for the down-projection, two pairs
        // a call: pair q in lanes 0..31, q + 1 in lanes 32..63
        const int j = lane & 31;
        const int src = 16 * ((j & 15) >> 2) + 4 * (j >> 4) + (j & 3);
        const int g32 = r0 / kGroup;
        const size_t hstride = (size_t)(inter / 128) * f4::kChunkBytes;
        const int hi = lane >> 5;
#pragma unroll
        for (int q = 0; q < NPP; q += 2) {
            const float h0 = __shfl(hvs[q], src), h1 = __shfl(hvs[q + 1], src);
            const int qq = q + hi;
            const bool store = live && qq < np;
            split_group(hi ? h1 : h0, hp + (size_t)(store ? p0 + qq : 0) * hstride + (g32 >> 2) * f4::kChunkBytes,
                        g32 & 3, store);
        }
    }
}

// The matrix-core path takes whole 4-chunk blocks (512 entries; a row's
// scale bytes in 16-byte loads), whole 32-row blocks and whole 4-chunk groups
// of h's pieces: in and out sizes multiples of 512, at most 4096 (B -- a
// vector's pieces, 40 bytes per entry -- in LDS); scale tensors and bank
// stride 16-byte aligned. (Other shapes and banks use the vector kernels.)
// The current device's compute units (cached per device; 0 on error).
static int cu_count() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    if (cached[dev] <= 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cached[dev] = n;
    }
    return cached[dev];
}

bool f4_shape_ok(int latent, int inter) {
    auto ok = [](int n) { return n % 512 == 0 && n >= 512 && n <= 4096; };
    return ok(latent) && ok(inter);
}

bool f4_bank_ok(const BankDev &b) {
    if (b.stride % 16) return false;
    for (int i = 1; i < 6; i += 2)
        if (((uintptr_t)b.base + b.off[i]) % 16) return false;
    return true;
}

template <bool UP, int NCK>
static int launch_f4(float *out, const uint8_t *pieces, uint8_t *hp, const BankDev &bank, const Route1 &rt,
                     const int32_t *active, const int32_t *offsets, int top_k, int latent, int inter, int max_slots,
                     hipStream_t st) {
    const int n_out = UP ? inter : latent;
    const int bps = n_out / f4::kRows;
    const int grid = UP ? (max_slots * bps + f4::kWaves - 1) / f4::kWaves
                        : max_slots * ((bps + f4::kWaves - 1) / f4::kWaves);
    if (grid == 0) return K3G_OK;
    const size_t lds = (size_t)NCK * f4::kChunkBytes;
    moe_f4_kernel<UP, NCK><<<grid, f4::kWaves * kWave, lds, st>>>(out, pieces, hp, bank, rt, active, offsets, top_k,
                                                                  latent, inter, max_slots);
    return hipGetLastError() == hipSuccess ? K3G_OK : K3G_EHIP;
}

// NCK = a row's chunks of 128 entries (n/128: 4, 8, ..., 32).
template <bool UP>
static int launch_f4_n(int n_in, float *out, const uint8_t *pieces, uint8_t *hp, const BankDev &bank,
                       const Route1 &rt, const int32_t *active, const int32_t *offsets, int top_k, int latent,
                       int inter, int max_slots, hipStream_t st) {
    switch (n_in / 128) {
#define K3G_F4(C)                                                                                              \
    case C:                                                                                                    \
        return launch_f4<UP, C>(out, pieces, hp, bank, rt, active, offsets, top_k, latent, inter, max_slots, st);
        K3G_F4(4) K3G_F4(8) K3G_F4(12) K3G_F4(16) K3G_F4(20) K3G_F4(24) K3G_F4(28) K3G_F4(32)
#undef K3G_F4
        default: return K3G_EUNSUPPORTED;
    }
}

// More tokens: the bucket's pass table drives the grid (an upper bound on the
// passes: every slot's last pass may be short). Pairs a pass by the average
// pairs per expert: two below 3 (the 4-wavefront kernel), four below 6 (the
// 8-wavefront kernel with the pairs resident in LDS), else eight (the
// 8-wavefront kernel with the pairs streamed through LDS).
int f4_pairs_per_pass(int n_pairs, int n_experts) {
    return n_pairs >= 6 * n_experts ? 8 : n_pairs >= 3 * n_experts ? 4 : 2;
}

template <bool UP, int NCK>
static int launch_f4m(int npp, float *out, const uint8_t *pieces, uint8_t *hp, const BankDev &bank,
                      const int32_t *active, const int32_t *offsets, const int32_t *perm, const int32_t *passes,
                      int top_k, int latent, int inter, int n_pairs, int max_slots, hipStream_t st) {
    const int n_out = UP ? inter : latent;
    const int rows_wg = npp >= 4 ? 8 * (UP ? 32 : 64) : f4::kWaves * f4::kRows;
    const int row_blocks = (n_out + rows_wg - 1) / rows_wg;
    const int64_t max_passes = (int64_t)(n_pairs + npp - 1) / npp + max_slots;
    const int64_t grid = max_passes * row_blocks;
    if (grid == 0) return K3G_OK;
    if (grid > 0x7fffffff) return K3G_EUNSUPPORTED;
    // the eight-pair kernel: whole rounds of 8 XCD groups
    const int64_t round8 = 8 * (int64_t)K3G_F4S_GROUP * row_blocks;
    const int64_t gridx = (grid + round8 - 1) / round8 * round8;
    if (gridx > 0x7fffffff) return K3G_EUNSUPPORTED;
    const size_t lds = (size_t)npp * NCK * f4::kChunkBytes;  // above the 64 KB default from 26 chunks on
    if (npp == 8) {
        moe_f4s_kernel<UP, NCK><<<(unsigned)gridx, 8 * kWave, 0, st>>>(out, pieces, hp, bank, active, offsets, perm,
                                                                     passes, top_k, latent, inter);
    } else if (npp == 4) {
        if (lds > 65536 && hipFuncSetAttribute((const void *)moe_f4q_kernel<UP, NCK>,
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
            return K3G_EHIP;
        const int n_cu = cu_count();  // persistent: one workgroup per CU
        if (n_cu <= 0) return K3G_EHIP;
        const int64_t g8 = (grid + 7) / 8 * 8;  // whole rounds of the 8 XCDs
        const int64_t pgrid = g8 < n_cu ? g8 : n_cu;
        moe_f4q_kernel<UP, NCK><<<(unsigned)pgrid, 8 * kWave, lds, st>>>(out, pieces, hp, bank, active, offsets, perm,
                                                                       passes, top_k, latent, inter);
    } else if (npp == 2) {
        if (lds > 65536 &&
            hipFuncSetAttribute((const void *)moe_f4m_kernel<UP, NCK, 2>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)lds) != hipSuccess)
            return K3G_EHIP;
        moe_f4m_kernel<UP, NCK, 2><<<(unsigned)grid, f4::kWaves * kWave, lds, st>>>(
            out, pieces, hp, bank, active, offsets, perm, passes, top_k, latent, inter);
    } else {
        return K3G_EINVAL;
    }
    return hipGetLastError() == hipSuccess ? K3G_OK : K3G_EHIP;
}

template <bool UP>
static int launch_f4m_n(int n_in, int npp, float *out, const uint8_t *pieces, uint8_t *hp, const BankDev &bank,
                        const int32_t *active, const int32_t *offsets, const int32_t *perm, const int32_t *passes,
                        int top_k, int latent, int inter, int n_pairs, int max_slots, hipStream_t st) {
    switch (n_in / 128) {
#define K3G_F4M(C)                                                                                                 \
    case C:                                                                                                        \
        return launch_f4m<UP, C>(npp, out, pieces, hp, bank, active, offsets, perm, passes, top_k, latent, inter,   \
                                 n_pairs, max_slots, st);
        K3G_F4M(4) K3G_F4M(8) K3G_F4M(12) K3G_F4M(16) K3G_F4M(20) K3G_F4M(24) K3G_F4M(28) K3G_F4M(32)
#undef K3G_F4M
        default: return K3G_EUNSUPPORTED;
    }
}

int launch_moe_up_f4m(float *h, uint8_t *hp, const uint8_t *xp, const BankDev &bank, const int32_t *active,
                      const int32_t *offsets, const int32_t *perm, const int32_t *passes, int npp, int top_k,
                      int latent, int inter, int n_pairs, int max_slots, hipStream_t st) {
    return launch_f4m_n<true>(latent, npp, h, xp, hp, bank, active, offsets, perm, passes, top_k, latent, inter,
                              n_pairs, max_slots, st);
}

int launch_moe_down_f4m(float *ypair, const uint8_t *hp, const BankDev &bank, const int32_t *active,
                        const int32_t *offsets, const int32_t *passes, int npp, int latent, int inter, int n_pairs,
                        int max_slots, hipStream_t st) {
    return launch_f4m_n<false>(inter, npp, ypair, hp, nullptr, bank, active, offsets, nullptr, passes, 1, latent,
                               inter, n_pairs, max_slots, st);
}

// The up-projection also writes the pieces of h (hp) for the down-projection.
int launch_moe_up_f4(float *h, uint8_t *hp, const uint8_t *xp, const BankDev &bank, const Route1 &rt, int top_k,
                     int latent, int inter, int max_slots, hipStream_t st) {
    return launch_f4_n<true>(latent, h, xp, hp, bank, rt, nullptr, nullptr, top_k, latent, inter, max_slots, st);
}

int launch_moe_down_f4(float *ypair, const uint8_t *hp, const BankDev &bank, const int32_t *active,
                       const int32_t *offsets, int latent, int inter, int max_slots, hipStream_t st) {
    return launch_f4_n<false>(inter, ypair, hp, nullptr, bank, Route1{}, active, offsets, 1, latent, inter,
                              max_slots, st);
}

}  // namespace k3g
