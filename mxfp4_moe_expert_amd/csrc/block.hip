// block.hip -- the dense parts of the LatentMoE block (gfx950).
//
// "Kimi K3 engine (c/kimi_k3.c)", "Architecture notes", Stable LatentMoE: the
// token is projected 7168 -> 3584, the routed experts run in that latent
// space, the aggregate is RMSNorm-ed and projected back 3584 -> 7168, and two
// full-width shared SiTU-GLU experts (inter 6144) are added. "kimi-k3-in-c"
// README, config struct: rms_eps 1e-5, the shared experts added unweighted.
//
// The dense weights are bf16 (widened exactly to fp32); activations stay fp32
// and every product accumulates in fp32, so nothing is rounded to bf16.
#include <algorithm>

#include "k3g_common.h"

namespace k3g {

// ---- dense products: out[t][n] (+)= sum over segments s of W_s[n][:] . x_s[t][:]
// A tile of 64 tokens x 64 outputs per workgroup (each thread 4 x 4), K in
// chunks of 32 staged through LDS. Up to three (W, x) segments accumulate into
// the same registers, so out = W_up n + W2_0 h_0 + W2_1 h_1 is one kernel.
// GLU: two weight matrices on one x, and the epilogue writes SiTU(g, u).
struct DenseSeg {
    const uint16_t *w;  // bf16 bits [N][K]
    const float *x;     // [T][K]
    int K;
};

constexpr int DT = 64, DK = 32;

__device__ inline float bf16f(uint16_t b) { return __builtin_bit_cast(float, (uint32_t)b << 16); }

template <bool GLU>
__global__ __launch_bounds__(256) void dense_kernel(float *__restrict__ out, DenseSeg s0, DenseSeg s1, DenseSeg s2,
                                                    int n_seg, int T, int N) {
    __shared__ float xs[DK][DT + 4];
    __shared__ float wa[DK][DT + 4];
    __shared__ float wb[GLU ? DK : 1][DT + 4];
    const int t0 = blockIdx.y * DT, n0 = blockIdx.x * DT;
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    float acc[4][4], acc3[GLU ? 4 : 1][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            acc[i][j] = 0.f;
            if (GLU) acc3[i][j] = 0.f;
        }
    for (int si = 0; si < (GLU ? 1 : n_seg); ++si) {
        const DenseSeg sg = si == 0 ? s0 : (si == 1 ? s1 : s2);
        for (int k0 = 0; k0 < sg.K; k0 += DK) {
#pragma unroll
            for (int l = 0; l < (DT * DK) / 256; ++l) {
                const int id = threadIdx.x + l * 256;
                const int r = id / DK, kk = id % DK;
                const int k = k0 + kk;
                xs[kk][r] = (t0 + r < T && k < sg.K) ? sg.x[(size_t)(t0 + r) * sg.K + k] : 0.f;
                wa[kk][r] = (n0 + r < N && k < sg.K) ? bf16f(sg.w[(size_t)(n0 + r) * sg.K + k]) : 0.f;
                if (GLU) wb[kk][r] = (n0 + r < N && k < sg.K) ? bf16f(s1.w[(size_t)(n0 + r) * sg.K + k]) : 0.f;
            }
            __syncthreads();
#pragma unroll 8
            for (int kk = 0; kk < DK; ++kk) {
                float a[4], b[4], c[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) a[i] = xs[kk][ty * 4 + i];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    b[j] = wa[kk][tx * 4 + j];
                    if (GLU) c[j] = wb[kk][tx * 4 + j];
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
                        if (GLU) acc3[i][j] = __builtin_fmaf(a[i], c[j], acc3[i][j]);
                    }
            }
            __syncthreads();
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int t = t0 + ty * 4 + i, n = n0 + tx * 4 + j;
            if (t < T && n < N) out[(size_t)t * N + n] = GLU ? situ(acc[i][j], acc3[i][j]) : acc[i][j];
        }
}

int launch_dense(float *out, const DenseSeg *segs, int n_seg, int T, int N, hipStream_t st) {
    if (T == 0) return K3G_OK;
    const DenseSeg z = {nullptr, nullptr, 0};
    const dim3 grid((N + DT - 1) / DT, (T + DT - 1) / DT);
    dense_kernel<false><<<grid, 256, 0, st>>>(out, segs[0], n_seg > 1 ? segs[1] : z, n_seg > 2 ? segs[2] : z,
                                              n_seg, T, N);
    return hipGetLastError() == hipSuccess ? K3G_OK : K3G_EHIP;
}

// h = SiTU(W1 x, W3 x) for the shared experts.
int launch_dense_glu(float *h, const uint16_t *w1, const uint16_t *w3, const float *x, int T, int K, int N,
                     hipStream_t st) {
    if (T == 0) return K3G_OK;
    const DenseSeg a = {w1, x, K}, b = {w3, x, K}, z = {nullptr, nullptr, 0};
    const dim3 grid((N + DT - 1) / DT, (T + DT - 1) / DT);
    dense_kernel<true><<<grid, 256, 0, st>>>(h, a, b, z, 1, T, N);
    return hipGetLastError() == hipSuccess ? K3G_OK : K3G_EHIP;
}

// ---- RMSNorm over the aggregate: n = a / sqrt(mean(a^2) + eps) * gamma ---------
__global__ __launch_bounds__(256) void rmsnorm_kernel(float *__restrict__ n, const float *__restrict__ a,
                                                      const float *__restrict__ gamma, int len, float eps) {
    __shared__ float part[4];
    const int t = blockIdx.x;
    const float *at = a + (size_t)t * len;
    float ss = 0.f;
    for (int i = threadIdx.x; i < len; i += blockDim.x) ss = __builtin_fmaf(at[i], at[i], ss);
    ss = wave_sum(ss);
    if ((threadIdx.x & (kWave - 1)) == 0) part[threadIdx.x / kWave] = ss;
    __syncthreads();
    const float tot = (part[0] + part[1]) + (part[2] + part[3]);
    const float rms = sqrtf(tot / (float)len + eps);
    for (int i = threadIdx.x; i < len; i += blockDim.x) n[(size_t)t * len + i] = at[i] / rms * gamma[i];
}

int launch_rmsnorm(float *n, const float *a, const float *gamma, int T, int len, float eps, hipStream_t st) {
    if (T == 0) return K3G_OK;
    rmsnorm_kernel<<<T, 256, 0, st>>>(n, a, gamma, len, eps);
    return hipGetLastError() == hipSuccess ? K3G_OK : K3G_EHIP;
}

// ---- dense products on the bf16 matrix cores ------------------------------------------
//
// out[t][n] = sum_s W_s[n][:] . x_s[t][:] with W bf16 and x fp32. Each entry of
// x is written exactly as three bf16 pieces, x = x0 + x1 + x2: x0 is x cut to
// its top 8 significant bits, x1 the top 8 bits of what is left and x2 the
// rest (at most 8 bits, so exact while |x| >= 2^-100 keeps the pieces normal).
// Every product w * x_i (8 x 8 bits) is exact in fp32 and
// v_mfma_f32_16x16x32_bf16 sums them in fp32, so the result meets the same
// bound as the fp32 fma form, with the matrix cores doing three products per
// weight instead of the vector unit doing one.
//
// Pieces in HBM, in the order the products read them (operand B of
// 16x16x32: lane l = token l%16, entries 8*(l/16)..+7 of a 32-entry step):
//   [token tile of 16][step of 32][piece 0..2][lane 0..63][8 bf16]
// so one step of one token tile is 3 KB, and the token count is padded to a
// multiple of 64 with zero pieces.
//
// The product splits K over S slices (S chosen so that the grid fills the
// chip): each workgroup sums one slice of 256 rows (GLU: 128 rows of both
// W1 and W3) x 64 tokens into fp32 partials [S][G][T][N]; the reduction adds
// the slices in order (the result does not depend on timing) and applies the
// epilogue. Per workgroup: 4 wavefronts, each owning 64 operand-A rows as four
// tiles of 16 (GLU: W1 rows r..r+31 and W3 rows r..r+31) loaded straight into
// registers through a 3-deep ring of 64-entry blocks; operand B (4 token tiles
// x 2 steps x 3 pieces, 24 KB per block) goes global -> LDS by DMA into two
// buffers, one block ahead.

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

namespace dm {
constexpr int kTok = 64;        // token padding (and the small tile's tokens)
constexpr int kKB = 64;         // entries per block (two steps)
constexpr int kStepBytes = 3 * 1024;           // one token tile, one step, three pieces
#ifndef K3G_DENSE_NBUF
#define K3G_DENSE_NBUF 3
#endif
constexpr int kNBUF = K3G_DENSE_NBUF;  // operand-A ring depth (blocks), small tile
constexpr int kMaxSeg = 3;
// Two tiles: W = 4 wavefronts x (64 rows, 64 tokens), two workgroups a CU;
// W = 8 wavefronts x (64 rows, 128 tokens), one workgroup a CU (96 KB of
// LDS), which loads half the bytes per product: the weights once per 128
// tokens, the activations' pieces once per 512 rows.
constexpr int block_b(int W) { return W * 2 * kStepBytes; }  // one block of operand B
}  // namespace dm

struct DenseMSeg {
    const uint16_t *w;   // bf16 [N][K]
    const uint8_t *xb;   // pieces of x [T64 / 16][K / 32][3][64][16 B]
    int K;               // multiple of 64
};

struct DenseMArgs {
    DenseMSeg seg[dm::kMaxSeg];
    const uint16_t *w3;  // GLU: the second matrix (same K and x as seg[0])
    float *part;         // [S][G][T][N]
    int n_seg, N, T, S, nkb;  // nkb: blocks over all segments
    int kb_start[dm::kMaxSeg + 1];
    int row_blocks, tok_blocks, n_items;
};

__device__ inline uint32_t f32_bits(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ inline float bits_f32(uint32_t b) { return __builtin_bit_cast(float, b); }

// x -> three bf16 pieces (bit patterns): cut to the top 8 significant bits
// twice, the remainder being exact in bf16.
__device__ inline void bf16x3(float x, uint32_t &p0, uint32_t &p1, uint32_t &p2) {
    const uint32_t b0 = f32_bits(x) & 0xFFFF0000u;
    const float r1 = x - bits_f32(b0);
    const uint32_t b1 = f32_bits(r1) & 0xFFFF0000u;
    const float r2 = r1 - bits_f32(b1);
    p0 = b0 >> 16;
    p1 = b1 >> 16;
    p2 = f32_bits(r2) >> 16;
}

// Write the pieces of 8 consecutive entries (k = 8c..8c+7) of token t.
__device__ inline void store_pieces8(uint8_t *xb, int nks, int t, int c, const float *v) {
    uint32_t q[3][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        uint32_t a0, a1, a2, b0, b1, b2;
        bf16x3(v[2 * j], a0, a1, a2);
        bf16x3(v[2 * j + 1], b0, b1, b2);
        q[0][j] = a0 | (b0 << 16);
        q[1][j] = a1 | (b1 << 16);
        q[2][j] = a2 | (b2 << 16);
    }
    const int tt = t >> 4, s = c >> 2, lane = (t & 15) + 16 * (c & 3);
    uint8_t *dst = xb + ((size_t)tt * nks + s) * dm::kStepBytes + 16 * lane;
#pragma unroll
    for (int p = 0; p < 3; ++p) *(uint4 *)(dst + 1024 * p) = make_uint4(q[p][0], q[p][1], q[p][2], q[p][3]);
}

// x [T][K] (row stride ld) -> pieces for T64 tokens (zero past T).
__global__ __launch_bounds__(256) void split3_kernel(uint8_t *__restrict__ xb, const float *__restrict__ x, int T,
                                                     int T64, int K, int ld) {
    const int nc = K / 8;
    const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (id >= (int64_t)T64 * nc) return;
    const int t = (int)(id / nc), c = (int)(id - (int64_t)t * nc);
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (t < T) {
        const float4 a = *(const float4 *)(x + (size_t)t * ld + 8 * c);
        const float4 b = *(const float4 *)(x + (size_t)t * ld + 8 * c + 4);
        v[0] = a.x, v[1] = a.y, v[2] = a.z, v[3] = a.w, v[4] = b.x, v[5] = b.y, v[6] = b.z, v[7] = b.w;
    }
    store_pieces8(xb, K / 32, t, c, v);
}

int dense_t64(int T);

// ---- combine, RMSNorm and the up-projection's pieces in one pass ------------------
// agg[t] = sum over k of wts[t][k] * ypair[inv[t][k]] (the layer's combine: fma
// in k order, a dropped pair adding nothing), n[t] = agg[t] / sqrt(mean(agg^2)
// + eps) * gamma as rmsnorm_kernel, and the three bf16 pieces of n (zero for
// the padding tokens T..T64-1). One workgroup a token; thread c takes entries
// 8c..8c+7 (len a multiple of 8, at most 4096).
__global__ __launch_bounds__(512) void combine_norm_kernel(float *__restrict__ agg, float *__restrict__ nrm,
                                                           uint8_t *__restrict__ xb, const float *__restrict__ ypair,
                                                           const float *__restrict__ wts,
                                                           const int32_t *__restrict__ inv,
                                                           const float *__restrict__ gamma, int T, int top_k,
                                                           int len, float eps) {
    __shared__ float part[8];
    const int t = blockIdx.x, c = threadIdx.x;
    const int nc = len / 8;
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (t >= T) {  // padding token: zero pieces
        if (c < nc) store_pieces8(xb, len / 32, t, c, v);
        return;
    }
    if (c < nc) {
        for (int k0 = 0; k0 < top_k; k0 += 8) {
            float w[8];
            float4 a[8], b[8];
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {  // a block's loads go out before its sums
                const int k = min(k0 + kk, top_k - 1);
                const int pos = inv[t * top_k + k];
                const bool live = k0 + kk < top_k && pos >= 0;
                const float *src = ypair + (size_t)(pos >= 0 ? pos : 0) * len + 8 * c;
                const float4 a0 = *(const float4 *)src, b0 = *(const float4 *)(src + 4);
                w[kk] = live ? wts[t * top_k + k] : 0.0f;
                a[kk] = live ? a0 : make_float4(0.f, 0.f, 0.f, 0.f);
                b[kk] = live ? b0 : make_float4(0.f, 0.f, 0.f, 0.f);
            }
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                v[0] = __builtin_fmaf(w[kk], a[kk].x, v[0]);
                v[1] = __builtin_fmaf(w[kk], a[kk].y, v[1]);
                v[2] = __builtin_fmaf(w[kk], a[kk].z, v[2]);
                v[3] = __builtin_fmaf(w[kk], a[kk].w, v[3]);
                v[4] = __builtin_fmaf(w[kk], b[kk].x, v[4]);
                v[5] = __builtin_fmaf(w[kk], b[kk].y, v[5]);
                v[6] = __builtin_fmaf(w[kk], b[kk].z, v[6]);
                v[7] = __builtin_fmaf(w[kk], b[kk].w, v[7]);
            }
        }
        float *dst = agg + (size_t)t * len + 8 * c;
        *(float4 *)dst = make_float4(v[0], v[1], v[2], v[3]);
        *(float4 *)(dst + 4) = make_float4(v[4], v[5], v[6], v[7]);
    }
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) ss = __builtin_fmaf(v[j], v[j], ss);
    ss = wave_sum(ss);
    if ((c & (kWave - 1)) == 0) part[c / kWave] = ss;
    __syncthreads();
    const float tot = ((part[0] + part[1]) + (part[2] + part[3])) + ((part[4] + part[5]) + (part[6] + part[7]));
    const float rms = sqrtf(tot / (float)len + eps);
    if (c < nc) {
        float n[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) n[j] = v[j] / rms * gamma[8 * c + j];
        float *dst = nrm + (size_t)t * len + 8 * c;
        *(float4 *)dst = make_float4(n[0], n[1], n[2], n[3]);
        *(float4 *)(dst + 4) = make_float4(n[4], n[5], n[6], n[7]);
        store_pieces8(xb, len / 32, t, c, n);
    }
}

int launch_combine_norm(float *agg, float *nrm, uint8_t *xb, const float *ypair, const float *wts,
                        const int32_t *inv, const float *gamma, int T, int top_k, int len, float eps,
                        hipStream_t st) {
    if (T == 0) return K3G_OK;
    if (len % 32 || len > 4096 || top_k < 1) return K3G_EUNSUPPORTED;
    combine_norm_kernel<<<dense_t64(T), 512, 0, st>>>(agg, nrm, xb, ypair, wts, inv, gamma, T, top_k, len, eps);
    return hipGetLastError() == hipSuccess ? K3G_OK : K3G_EHIP;
}

// W wavefronts, each with 64 output rows (GLU: 32 of W1 and the same 32 of W3)
// and W token tiles of 16; the workgroup's W token tiles of operand B are
// staged in LDS, wavefront w bringing tile w.
template <bool GLU, int W>
__global__ __launch_bounds__(W * kWave, 8 / W) void dense_mfma_kernel(DenseMArgs a) {
    using namespace dm;
    constexpr int kBlockB = block_b(W);
    constexpr int NB = W == 8 ? 2 : kNBUF;  // the big tile: 128 accumulators, a 2-deep ring
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];  // 2 * kBlockB
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    // XCD-aware order: consecutive workgroups go round the 8 XCDs, so item
    // w = (XCD, position) keeps each XCD on a contiguous run of items. Items
    // run token blocks fastest, then row blocks, then K slices: the token
    // blocks of one (row block, slice) share its weights, and an XCD's row
    // blocks share one or two slices of operand B, through that XCD's L2
    const int per_xcd = (int)(gridDim.x / 8);
    const int item = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
    if (item >= a.n_items) return;  // whole workgroup
    const int tb = item % a.tok_blocks;
    const int rest = item / a.tok_blocks;
    const int rb = rest % a.row_blocks, sl = rest / a.row_blocks;
    const int kb0 = (int)((int64_t)a.nkb * sl / a.S), kb1 = (int)((int64_t)a.nkb * (sl + 1) / a.S);
    constexpr int ROWS_W = GLU ? 32 : 64;  // output rows per wavefront
    const int r0 = (rb * W + wave) * ROWS_W;

    // operand A: four tiles of 16 rows; lane (i = l%16, q = l/16) reads 16 B at
    // entry 8q of a step for row i of its tile
    rsrc_t ra[kMaxSeg], ra3;
#pragma unroll
    for (int s = 0; s < kMaxSeg; ++s)
        ra[s] = make_rsrc(s < a.n_seg ? a.seg[s].w : a.seg[0].w,
                          (uint32_t)((s < a.n_seg ? (uint64_t)a.seg[s].K : 0) * 2 * (uint64_t)a.N));
    ra3 = make_rsrc(GLU ? a.w3 : a.seg[0].w, GLU ? (uint32_t)((uint64_t)a.seg[0].K * 2 * a.N) : 0u);
    auto seg_of = [&](int kb) { return kb >= a.kb_start[2] ? 2 : kb >= a.kb_start[1] ? 1 : 0; };
    uint4 A[NB][4][2];
    // Block kb of A into ring slot `slot`. Issued on every step, also where
    // there is no block left to fetch (then block kb is the current one,
    // loaded again into the free slot): the compiler's waits for a slot then
    // count the same loads on every path, instead of waiting, on the path that
    // issues them, for the loads just issued. (No load here may be past the
    // range: such a load can return before older ones, and the counted waits
    // assume loads complete in the order they were issued.)
    auto load_a = [&](int kb, int slot) {
        const int s = seg_of(kb);
        const uint32_t K2 = 2u * (uint32_t)a.seg[s].K;
        const uint32_t soff = 128u * (uint32_t)(kb - a.kb_start[s]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // rows past N (the last row block) read row N - 1 and store nothing:
            // the wavefront's counted waits also cover the B tile it brings
            const int row = min(r0 + (GLU ? 16 * (i & 1) : 16 * i) + (lane & 15), a.N - 1);
            const uint32_t v = (uint32_t)row * K2 + 16u * (uint32_t)(lane >> 4);
            const rsrc_t r = (GLU && i >= 2) ? ra3 : (s == 0 ? ra[0] : s == 1 ? ra[1] : ra[2]);
#pragma unroll
            for (int h = 0; h < 2; ++h) A[slot][i][h] = buf_load16(r, v, soff + 64u * h);
        }
    };
    // operand B: wavefront w brings token tile w of the block (6 KB)
    const uint32_t lb = lds_addr(lds);
    auto dma_b = [&](int kb, int buf) {
        const int s = seg_of(kb);
        const int nks = a.seg[s].K / 32;
        const int ttg = tb * W + wave;
        const uint8_t *src = a.seg[s].xb + ((size_t)ttg * nks + 2 * (kb - a.kb_start[s])) * kStepBytes;
#pragma unroll
        for (int j = 0; j < 6; ++j)
            dma16(src, 1024u * j + 16u * lane, lb + (uint32_t)(buf * kBlockB + wave * 2 * kStepBytes + 1024 * j));
    };

    float4_t acc[4][W];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int t = 0; t < W; ++t) acc[i][t] = float4_t{0.f, 0.f, 0.f, 0.f};

    int li = lane;
    __asm__ volatile("" : "+v"(li));
    // B fragments two-deep: the next (step, token tile)'s three are read from
    // LDS while this one's twelve products issue
    auto compute = [&](int slot, int buf) {
        const uint4 *bb = (const uint4 *)(lds + buf * kBlockB) + li;
        __asm__ volatile("" ::: "memory");
        bf16x8_t B[2][3];
        auto read_b = [&](int it) {  // it = W * step + token tile
            const int st = it / W, t = it % W;
#pragma unroll
            for (int p = 0; p < 3; ++p) B[it & 1][p] = __builtin_bit_cast(bf16x8_t, bb[((t * 2 + st) * 3 + p) * 64]);
        };
        read_b(0);
#pragma unroll
        for (int it = 0; it < 2 * W; ++it) {
            const int st = it / W, t = it % W;
            if (it + 1 < 2 * W) read_b(it + 1);
            __builtin_amdgcn_sched_barrier(0);  // the reads go out ahead of the products
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bf16x8_t Av = __builtin_bit_cast(bf16x8_t, A[slot][i][st]);
#pragma unroll
                for (int p = 0; p < 3; ++p)
                    acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Av, B[it & 1][p], acc[i][t], 0, 0, 0);
            }
        }
    };

    // prologue: B of the first block, A of the first two
    if (kb0 < kb1) {
        dma_b(kb0, 0);
        __asm__ volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < NB - 1; ++j) load_a(min(kb0 + j, kb1 - 1), j);
        wait_vm<0>();
        __syncthreads();
    }
    // one block: B of the next into the other LDS buffer, A of the one after
    // next into the ring, this block's products; then the next block's B is
    // in LDS (vmcnt: only the 8 A loads, issued after the DMA, may still be in
    // flight), and every wavefront is done with this buffer before it is
    // filled again
    auto step = [&](int k, int j) {  // j = (k - kb0) % NB
        const int buf = (k - kb0) & 1;
        if (k + 1 < kb1) dma_b(k + 1, buf ^ 1);
        __asm__ volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        const bool na = k + NB - 1 < kb1;
        load_a(na ? k + NB - 1 : k, (j + NB - 1) % NB);
        __builtin_amdgcn_sched_barrier(0);
        compute(j, buf);
        __builtin_amdgcn_sched_barrier(0);
        // (where there is no block left to fetch, the compiler may drop the
        // extra A loads, whose values are never read: then nothing but the
        // DMA may be counted)
        if (na)
            wait_vm<8>();
        else
            wait_vm<0>();
        __syncthreads();
    };
    // whole rounds of the ring (every ring slot static, no branch inside),
    // then the last one or two blocks
    const int nblk = kb1 - kb0, nround = nblk / NB;
    for (int rd = 0; rd < nround; ++rd) {
        const int kb = kb0 + rd * NB;
#pragma unroll
        for (int j = 0; j < NB; ++j) step(kb + j, j);
    }
    const int kt = kb0 + nround * NB;
#pragma unroll
    for (int j = 0; j < NB - 1; ++j)
        if (kt + j < kb1) step(kt + j, j);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int t = 0; t < W; ++t) __asm__ volatile("" : "+v"(acc[i][t]));

    // lane l holds token 16t + l%16 and rows 4(l/16)..+3 of each tile
    const int tok0 = tb * 16 * W + (lane & 15);
    const int G = GLU ? 2 : 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int g = GLU ? i >> 1 : 0;
        const int n = r0 + (GLU ? 16 * (i & 1) : 16 * i) + 4 * (lane >> 4);
#pragma unroll
        for (int t = 0; t < W; ++t) {
            const int tok = tok0 + 16 * t;
            if (tok < a.T && n < a.N) {
                float *dst = a.part + (((size_t)sl * G + g) * a.T + tok) * a.N + n;
                *(float4 *)dst = make_float4(acc[i][t][0], acc[i][t][1], acc[i][t][2], acc[i][t][3]);
            }
        }
    }
}

// partials [S][G][T][N] -> out [T][N] (G = 1: the sum over slices; G = 2: SiTU
// of the two sums), slices added in order; optionally also the pieces of out
// for the next product (T64 tokens, zero past T). Thread: 8 entries of a token.
template <bool GLU>
__global__ __launch_bounds__(256) void dense_reduce_kernel(float *__restrict__ out, uint8_t *__restrict__ xb,
                                                           const float *__restrict__ part, int S, int T, int T64,
                                                           int N) {
    const int nc = N / 8;
    const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (id >= (int64_t)T64 * nc) return;
    const int t = (int)(id / nc), c = (int)(id - (int64_t)t * nc);
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (t < T) {
        const int G = GLU ? 2 : 1;
        float g[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, u[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int s = 0; s < S; ++s) {
            const float *pg = part + (((size_t)s * G) * T + t) * N + 8 * c;
            const float4 a0 = *(const float4 *)pg, a1 = *(const float4 *)(pg + 4);
            g[0] += a0.x, g[1] += a0.y, g[2] += a0.z, g[3] += a0.w;
            g[4] += a1.x, g[5] += a1.y, g[6] += a1.z, g[7] += a1.w;
            if (GLU) {
                const float *pu = pg + (size_t)T * N;
                const float4 b0 = *(const float4 *)pu, b1 = *(const float4 *)(pu + 4);
                u[0] += b0.x, u[1] += b0.y, u[2] += b0.z, u[3] += b0.w;
                u[4] += b1.x, u[5] += b1.y, u[6] += b1.z, u[7] += b1.w;
            }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = GLU ? situ(g[j], u[j]) : g[j];
        float *o = out + (size_t)t * N + 8 * c;
        *(float4 *)o = make_float4(v[0], v[1], v[2], v[3]);
        *(float4 *)(o + 4) = make_float4(v[4], v[5], v[6], v[7]);
    }
    if (xb) store_pieces8(xb, N / 32, t, c, v);
}

// ---- host side -------------------------------------------------------------------------

int dense_t64(int T) { return (T + dm::kTok - 1) / dm::kTok * dm::kTok; }

// The matrix-core form takes K multiples of 64 and N multiples of 16, with
// every 32-bit offset in range; otherwise the fp32 fma form runs.
bool dense_mfma_ok(int T, int N, const int *K, int n_seg) {
    if (T < 1 || N < 16 || N % 16) return false;
    const int64_t t64 = dense_t64(T);
    for (int s = 0; s < n_seg; ++s) {
        if (K[s] < 64 || K[s] % 64) return false;
        if ((int64_t)N * K[s] * 2 >= ((int64_t)1 << 31) || t64 * K[s] * 6 >= ((int64_t)1 << 31)) return false;
    }
    return true;
}

// The tile: 128 tokens a workgroup where the padded batch is a whole number
// of them, else 64.
static int dense_w(int T) { return dense_t64(T) % 128 == 0 ? 8 : 4; }

// Slices of K. A cost model in block-steps of the busiest CU, a block-step
// being one workgroup's block of the small tile (four wavefronts' products on
// one block of 64 entries): the items (tiles x slices) spread evenly over the
// chip's 256 CUs; the busiest runs ceil(items / 256) of them, each ceil(nkb /
// S) blocks plus about two for its prologue and partial stores. Small tile: a
// CU with one workgroup is counted as slow as with two (one wavefront a SIMD
// leaves the matrix cores half idle). Big tile: one workgroup a CU, each block
// four block-steps of work. The partials' round trip (written, then read by
// the reduction) adds about one block-step per 4 MB. At least 4 blocks a
// slice.
int dense_slices(int T, int N, int K_total, bool glu) {
    const int W = dense_w(T);
    const int rows_wg = W * (glu ? 32 : 64);
    const int64_t tiles = (int64_t)((N + rows_wg - 1) / rows_wg) * (dense_t64(T) / (16 * W));
    const int nkb = K_total / dm::kKB;
    const int max_s = nkb / 4 > 1 ? nkb / 4 : 1;
    const double part_bytes = 8.0 * (glu ? 2 : 1) * (double)dense_t64(T) * N;  // per slice, both ways
    int best = 1;
    double best_cost = 1e300;
    for (int s = 1; s <= max_s; ++s) {
        const int64_t rounds = (tiles * s + 255) / 256;
        const double work = W == 8 ? 4.0 * (double)rounds * ((nkb + s - 1) / s + 1)
                                   : (double)std::max<int64_t>(rounds, 2) * ((nkb + s - 1) / s + 2);
        const double cost = work + s * part_bytes / (4.0 * (1 << 20));
        if (cost < best_cost) best_cost = cost, best = s;
    }
    return best;
}

int launch_split3(uint8_t *xb, const float *x, int T, int K, int ld, hipStream_t st) {
    if (K % 64 || ld % 4 || ld < K || ((uintptr_t)x & 15)) return K3G_EUNSUPPORTED;
    const int64_t n = (int64_t)dense_t64(T) * (K / 8);
    if (n == 0) return K3G_OK;
    split3_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(xb, x, T, dense_t64(T), K, ld);
    return hipGetLastError() == hipSuccess ? K3G_OK : K3G_EHIP;
}

// out (+ pieces of out when xb_out) = sum over segments of W_s x_s; GLU (one
// segment, w3 given): out = SiTU(W1 x, W3 x). part holds S * G * T * N floats.
int launch_reduce_split(float *out, uint8_t *dst, const float *part, int S, int T, int len, hipStream_t st);

// xp_out (not with GLU or xb_out): also the e2m1 pieces of out, as the FP4
// layer's split writes them, from the same reduction.
int launch_dense_mfma(float *out, uint8_t *xb_out, float *part, const uint16_t *const *w, const uint8_t *const *xb,
                      const int *K, int n_seg, const uint16_t *w3, int T, int N, hipStream_t st, uint8_t *xp_out) {
    if (T == 0) return K3G_OK;
    if (n_seg < 1 || n_seg > dm::kMaxSeg || (w3 && n_seg != 1) || !dense_mfma_ok(T, N, K, n_seg) ||
        (xb_out && N % 64))  // the pieces feed a product whose K is this N
        return K3G_EUNSUPPORTED;
    const bool glu = w3 != nullptr;
    DenseMArgs a{};
    int kt = 0;
    for (int s = 0; s < dm::kMaxSeg; ++s) {
        a.kb_start[s] = kt / dm::kKB;
        if (s < n_seg) {
            a.seg[s] = DenseMSeg{w[s], xb[s], K[s]};
            kt += K[s];
        } else {
            a.kb_start[s] = 0x7fffffff;
        }
    }
    a.kb_start[dm::kMaxSeg] = 0x7fffffff;
    a.w3 = w3;
    a.part = part;
    a.n_seg = n_seg;
    a.N = N;
    a.T = T;
    a.nkb = kt / dm::kKB;
    a.S = dense_slices(T, N, kt, glu);
    const int W = dense_w(T);
    const int rows_wg = W * (glu ? 32 : 64);
    a.row_blocks = (N + rows_wg - 1) / rows_wg;
    a.tok_blocks = dense_t64(T) / (16 * W);
    const int64_t items = (int64_t)a.row_blocks * a.S * a.tok_blocks;
    if (items > (1 << 30)) return K3G_EUNSUPPORTED;
    a.n_items = (int)items;
    const unsigned grid = (unsigned)((items + 7) / 8 * 8);  // a whole number per XCD
    const size_t lds = 2 * (size_t)dm::block_b(W);
    if (W == 8) {
        // 96 KB of LDS: above the 64 KB a launch gets by default
        const void *f = glu ? (const void *)dense_mfma_kernel<true, 8> : (const void *)dense_mfma_kernel<false, 8>;
        if (hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
            return K3G_EHIP;
        if (glu) dense_mfma_kernel<true, 8><<<grid, 8 * kWave, lds, st>>>(a);
        else dense_mfma_kernel<false, 8><<<grid, 8 * kWave, lds, st>>>(a);
    } else {
        if (glu) dense_mfma_kernel<true, 4><<<grid, 4 * kWave, lds, st>>>(a);
        else dense_mfma_kernel<false, 4><<<grid, 4 * kWave, lds, st>>>(a);
    }
    if (hipGetLastError() != hipSuccess) return K3G_EHIP;
    const int64_t n = (int64_t)dense_t64(T) * (N / 8);
    if (xp_out && !glu && !xb_out) return launch_reduce_split(out, xp_out, part, a.S, T, N, st);
    if (glu) dense_reduce_kernel<true><<<(unsigned)((n + 255) / 256), 256, 0, st>>>(out, xb_out, part, a.S, T,
                                                                                   dense_t64(T), N);
    else dense_reduce_kernel<false><<<(unsigned)((n + 255) / 256), 256, 0, st>>>(out, xb_out, part, a.S, T,
                                                                                 dense_t64(T), N);
    return hipGetLastError() == hipSuccess ? K3G_OK : K3G_EHIP;
}

}  // namespace k3g
