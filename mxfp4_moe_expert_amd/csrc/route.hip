// route.hip -- Stable LatentMoE routing and the expert bucket (gfx950).
//
// Routing ("Kimi K3 engine (c/kimi_k3.c)", "Architecture notes"; "kimi-k3-in-c"
// README, "Three invariants", 3): sigmoid scores plus a score-correction bias,
// top-k on the biased scores, weights = the selected raw scores renormalised.
// Logits are accumulated in fp64: fp32 x fp32 products are exact there, so the
// only rounding is in the additions, and the selection agrees with a double
// reference unless two biased scores sit within ~1e-15 of each other.
//
// Bucket: pairs (t, k) sorted by (expert, token), so each selected expert's
// weights are streamed once for all its tokens ("Kimi K3 engine", "Chunked
// prefill": each unique expert of a chunk is loaded once). Stable and
// deterministic: no atomics decide an order.
#include "k3g_common.h"

// Up to this many tokens, top-k runs one workgroup per token; above it, one
// wavefront per token.
#ifndef K3G_TOPK_BLOCK_MAX_T
#define K3G_TOPK_BLOCK_MAX_T 256
#endif

namespace k3g {

// ---- logits, few tokens: one wavefront per expert row ------------------------
// The row is read once with 16-byte loads into registers (in <= 64*4*RW
// floats), then dotted with each token's x in fp64. Four wavefronts (four
// rows) per workgroup: a quarter of the workgroups to dispatch (0.5 us of a
// one-token step's 10 us of routing, against one row per workgroup).
constexpr int kLogitWaves = 4;

template <int RW>
__global__ __launch_bounds__(64 * kLogitWaves) void logits_rows_kernel(double *__restrict__ logits,
                                                                       const float *__restrict__ x,
                                                                       const float *__restrict__ W, int T, int in,
                                                                       int E) {
    const int lane = threadIdx.x & (kWave - 1);
    const int n4 = in / 4;
    for (int e = blockIdx.x * kLogitWaves + (int)(threadIdx.x / kWave); e < E; e += gridDim.x * kLogitWaves) {
        const float4 *w4 = (const float4 *)(W + (size_t)e * in);
        float4 wr[RW];
#pragma unroll
        for (int i = 0; i < RW; ++i) {
            const int j = lane + i * kWave;
            wr[i] = w4[j < n4 ? j : n4 - 1];
        }
        for (int t = 0; t < T; ++t) {
            const float4 *x4 = (const float4 *)(x + (size_t)t * in);
            float4 xr[RW];
#pragma unroll
            for (int i = 0; i < RW; ++i) {
                const int j = lane + i * kWave;
                xr[i] = x4[j < n4 ? j : n4 - 1];
            }
            double acc = 0.0;
#pragma unroll
            for (int i = 0; i < RW; ++i) {
                // a lane past the row's end holds a duplicate of its last chunk: drop it
                const double m = (lane + i * kWave < n4) ? 1.0 : 0.0;
                double part = (double)wr[i].x * (double)xr[i].x;
                part = __builtin_fma((double)wr[i].y, (double)xr[i].y, part);
                part = __builtin_fma((double)wr[i].z, (double)xr[i].z, part);
                part = __builtin_fma((double)wr[i].w, (double)xr[i].w, part);
                acc = __builtin_fma(m, part, acc);
            }
            acc = wave_sum_f64(acc);
            if (lane == 0) logits[(size_t)t * E + e] = acc;
        }
    }
}

// Any width: scalar loads, one wavefront per row.
__global__ __launch_bounds__(64) void logits_rows_any_kernel(double *__restrict__ logits, const float *__restrict__ x,
                                                             const float *__restrict__ W, int T, int in, int E) {
    const int lane = threadIdx.x;
    for (int e = blockIdx.x; e < E; e += gridDim.x) {
        const float *w = W + (size_t)e * in;
        for (int t = 0; t < T; ++t) {
            const float *xt = x + (size_t)t * in;
            double acc = 0.0;
            for (int i = lane; i < in; i += kWave) acc = __builtin_fma((double)w[i], (double)xt[i], acc);
            acc = wave_sum_f64(acc);
            if (lane == 0) logits[(size_t)t * E + e] = acc;
        }
    }
}

// ---- logits, more tokens: fp64 matrix cores ------------------------------------
// v_mfma_f64_16x16x4_f64 on the exact fp64 widenings of x and W. A workgroup
// owns a tile of 16*BM tokens x 16*BN experts; its SPLIT wavefronts each take
// a slice of the columns and the partial tiles are added in wavefront order
// through LDS, so the result does not depend on timing. Within a step of 16
// columns, lane quarter q supplies columns 4q..4q+3, one per MFMA (A and B use
// the same assignment, so every product meets its partner).
typedef double v4d __attribute__((ext_vector_type(4)));

template <int BM, int BN, int SPLIT, bool VEC>
__global__ __launch_bounds__(SPLIT * 64) void logits_mfma_kernel(double *__restrict__ logits,
                                                                 const float *__restrict__ x,
                                                                 const float *__restrict__ W, int T, int in, int E) {
    __shared__ double red[SPLIT][BM * BN][4][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int q = lane >> 4, r = lane & 15;
    const int t0 = blockIdx.y * 16 * BM, e0 = blockIdx.x * 16 * BN;
    const int nk = (in + 15) / 16;
    const int per = (nk + SPLIT - 1) / SPLIT;
    const int ka = wave * per, kb = min(nk, ka + per);
    const float *xr[BM], *wr[BN];
#pragma unroll
    for (int i = 0; i < BM; ++i) xr[i] = x + (size_t)min(t0 + 16 * i + r, T - 1) * in;
#pragma unroll
    for (int j = 0; j < BN; ++j) wr[j] = W + (size_t)min(e0 + 16 * j + r, E - 1) * in;
    v4d acc[BM][BN];
#pragma unroll
    for (int i = 0; i < BM; ++i)
#pragma unroll
        for (int j = 0; j < BN; ++j) acc[i][j] = v4d{0.0, 0.0, 0.0, 0.0};
    // NS steps of operands are loaded back to back, then consumed: one memory
    // latency per NS steps (steps past the slice read zeros)
    constexpr int NS = 8;
    for (int k0 = ka; k0 < kb; k0 += NS) {
        float a[NS][BM][4], b[NS][BN][4];
#pragma unroll
        for (int st = 0; st < NS; ++st) {
            const int k = (k0 + st) * 16 + 4 * q;
            const bool live = k0 + st < kb;
            if (VEC && live && k + 4 <= in) {
#pragma unroll
                for (int i = 0; i < BM; ++i) {
                    const float4 v = *(const float4 *)(xr[i] + k);
                    a[st][i][0] = v.x; a[st][i][1] = v.y; a[st][i][2] = v.z; a[st][i][3] = v.w;
                }
#pragma unroll
                for (int j = 0; j < BN; ++j) {
                    const float4 v = *(const float4 *)(wr[j] + k);
                    b[st][j][0] = v.x; b[st][j][1] = v.y; b[st][j][2] = v.z; b[st][j][3] = v.w;
                }
            } else {
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const bool in_k = live && k + s < in;
#pragma unroll
                    for (int i = 0; i < BM; ++i) a[st][i][s] = in_k ? xr[i][k + s] : 0.0f;
#pragma unroll
                    for (int j = 0; j < BN; ++j) b[st][j][s] = in_k ? wr[j][k + s] : 0.0f;
                }
            }
        }
#pragma unroll
        for (int st = 0; st < NS; ++st)
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int i = 0; i < BM; ++i)
#pragma unroll
                    for (int j = 0; j < BN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)a[st][i][s], (double)b[st][j][s],
                                                                        acc[i][j], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < BM; ++i)
#pragma unroll
        for (int j = 0; j < BN; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) red[wave][i * BN + j][v][lane] = acc[i][j][v];
    __syncthreads();
    // output element (block, v, lane): token 16*bi + lane/16 + 4*v, expert 16*bj + lane%16
    // (the fp64 16x16x4 result layout: item v of lane l is row l/16 + 4v, column l%16)
    for (int o = threadIdx.x; o < BM * BN * 256; o += SPLIT * 64) {
        const int blk = o >> 8, v = (o >> 6) & 3, ln = o & 63;
        double sum = red[0][blk][v][ln];
#pragma unroll
        for (int w = 1; w < SPLIT; ++w) sum += red[w][blk][v][ln];
        const int t = t0 + 16 * (blk / BN) + (ln >> 4) + 4 * v;
        const int e = e0 + 16 * (blk % BN) + (ln & 15);
        if (t < T && e < E) logits[(size_t)t * E + e] = sum;
    }
}

// ---- logits, many tokens: 64 x 64 tiles, K split across workgroups -----------
// The same products as logits_mfma_kernel on a tile of 64 tokens x 64 experts
// (16 accumulator tiles a wavefront: each operand load feeds four times the
// products of a 32 x 32 tile). Workgroup (x, y, z) takes K-split z of tile
// (x, y); its 8 wavefronts take consecutive slices of that split and add their
// tiles in a fixed order through LDS: wavefront w + 4 into w, then 0..3 in
// order. With KS splits the workgroup writes its sum to partial plane z and
// logits_sum_kernel adds the planes in order, so the result does not depend
// on timing.
constexpr int kLT = 4;                                      // 16-row tiles per side
constexpr size_t kLTLds = (size_t)4 * kLT * kLT * 4 * 64 * sizeof(double);  // 128 KB

template <bool VEC>
__global__ __launch_bounds__(512) void logits_tile_kernel(double *__restrict__ out, const float *__restrict__ x,
                                                          const float *__restrict__ W, int T, int in, int E,
                                                          int KS) {
    extern __shared__ double red_lt[];  // [4][kLT * kLT][4][64]
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int q = lane >> 4, r = lane & 15;
    const int t0 = blockIdx.y * 16 * kLT, e0 = blockIdx.x * 16 * kLT;
    const int nk = (in + 15) / 16;
    const int z = blockIdx.z;
    const int za = (int)((int64_t)nk * z / KS), zb = (int)((int64_t)nk * (z + 1) / KS);
    const int ka = za + (int)((int64_t)(zb - za) * wave / 8), kb = za + (int)((int64_t)(zb - za) * (wave + 1) / 8);
    const float *xr[kLT], *wr[kLT];
#pragma unroll
    for (int i = 0; i < kLT; ++i) xr[i] = x + (size_t)min(t0 + 16 * i + r, T - 1) * in;
#pragma unroll
    for (int j = 0; j < kLT; ++j) wr[j] = W + (size_t)min(e0 + 16 * j + r, E - 1) * in;
    v4d acc[kLT][kLT];
#pragma unroll
    for (int i = 0; i < kLT; ++i)
#pragma unroll
        for (int j = 0; j < kLT; ++j) acc[i][j] = v4d{0.0, 0.0, 0.0, 0.0};
    // NS steps of operands loaded back to back, then consumed (steps past the
    // slice read zeros)
    constexpr int NS = 2;
    for (int k0 = ka; k0 < kb; k0 += NS) {
        float a[NS][kLT][4], b[NS][kLT][4];
#pragma unroll
        for (int st = 0; st < NS; ++st) {
            const int k = (k0 + st) * 16 + 4 * q;
            const bool live = k0 + st < kb;
            if (VEC && live && k + 4 <= in) {
#pragma unroll
                for (int i = 0; i < kLT; ++i) {
                    const float4 v = *(const float4 *)(xr[i] + k);
                    a[st][i][0] = v.x; a[st][i][1] = v.y; a[st][i][2] = v.z; a[st][i][3] = v.w;
                }
#pragma unroll
                for (int j = 0; j < kLT; ++j) {
                    const float4 v = *(const float4 *)(wr[j] + k);
                    b[st][j][0] = v.x; b[st][j][1] = v.y; b[st][j][2] = v.z; b[st][j][3] = v.w;
                }
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const bool in_k = live && k + c < in;
#pragma unroll
                    for (int i = 0; i < kLT; ++i) a[st][i][c] = in_k ? xr[i][k + c] : 0.0f;
#pragma unroll
                    for (int j = 0; j < kLT; ++j) b[st][j][c] = in_k ? wr[j][k + c] : 0.0f;
                }
            }
        }
#pragma unroll
        for (int st = 0; st < NS; ++st)
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int i = 0; i < kLT; ++i)
#pragma unroll
                    for (int j = 0; j < kLT; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)a[st][i][c], (double)b[st][j][c],
                                                                        acc[i][j], 0, 0, 0);
    }
    // the 8 slices' tiles: w + 4 into w, then planes 0..3 in order
    auto plane = [&](int p, int blk, int v) -> double & { return red_lt[((p * kLT * kLT + blk) * 4 + v) * 64 + lane]; };
    if (wave >= 4) {
#pragma unroll
        for (int i = 0; i < kLT; ++i)
#pragma unroll
            for (int j = 0; j < kLT; ++j)
#pragma unroll
                for (int v = 0; v < 4; ++v) plane(wave - 4, i * kLT + j, v) = acc[i][j][v];
    }
    __syncthreads();
    if (wave < 4) {
#pragma unroll
        for (int i = 0; i < kLT; ++i)
#pragma unroll
            for (int j = 0; j < kLT; ++j)
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[i][j][v] += plane(wave, i * kLT + j, v);
    }
    __syncthreads();
    if (wave < 4) {
#pragma unroll
        for (int i = 0; i < kLT; ++i)
#pragma unroll
            for (int j = 0; j < kLT; ++j)
#pragma unroll
                for (int v = 0; v < 4; ++v) plane(wave, i * kLT + j, v) = acc[i][j][v];
    }
    __syncthreads();
    // output element (block, v, lane): token 16*bi + lane/16 + 4*v, expert 16*bj + lane%16
    double *dst = out + (size_t)z * T * E;
    for (int o = threadIdx.x; o < kLT * kLT * 256; o += 512) {
        const int blk = o >> 8, v = (o >> 6) & 3, ln = o & 63;
        const int base = (blk * 4 + v) * 64 + ln, pl = kLT * kLT * 4 * 64;
        const double sum = ((red_lt[base] + red_lt[pl + base]) + red_lt[2 * pl + base]) + red_lt[3 * pl + base];
        const int t = t0 + 16 * (blk / kLT) + (ln >> 4) + 4 * v;
        const int e = e0 + 16 * (blk % kLT) + (ln & 15);
        if (t < T && e < E) dst[(size_t)t * E + e] = sum;
    }
}

// logits = the KS partial planes added in order
__global__ __launch_bounds__(256) void logits_sum_kernel(double *__restrict__ logits, const double *__restrict__ part,
                                                         int64_t n, int KS) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    double s = part[i];
    for (int z = 1; z < KS; ++z) s += part[(size_t)z * n + i];
    logits[i] = s;
}

// ---- top-k: one wavefront per token, candidates in registers ---------------------
// The order is "larger biased score first, equal scores to the lower expert
// id". Round k picks, over all lanes, the best candidate that comes strictly
// after round k-1's winner, so nothing has to be marked as taken. The
// cross-lane arg-max uses DPP within each row of 16 lanes and readlane across
// the four rows: no LDS and no barriers.
__device__ inline bool before(double va, int ia, double vb, int ib) {
    // bitwise, not short-circuit: straight-line compares and selects, no branches
    return (va > vb) | ((va == vb) & (ia < ib));
}

template <int CTRL>
__device__ inline void dpp_best(double &v, int &i) {
    const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), CTRL, 0xF, 0xF, false);
    const int oi = __builtin_amdgcn_update_dpp(0, i, CTRL, 0xF, 0xF, false);
    const double ov = __hiloint2double(hi, lo);
    const bool take = before(ov, oi, v, i);
    v = take ? ov : v;
    i = take ? oi : i;
}

__device__ inline void wave_best(double &v, int &i) {
    dpp_best<0xB1>(v, i);   // quad_perm [1,0,3,2]
    dpp_best<0x4E>(v, i);   // quad_perm [2,3,0,1]
    dpp_best<0x141>(v, i);  // row_half_mirror
    dpp_best<0x140>(v, i);  // row_mirror: every lane of a row holds the row's best
    double bv = __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), 0),
                                 __builtin_amdgcn_readlane(__double2loint(v), 0));
    int bi = __builtin_amdgcn_readlane(i, 0);
#pragma unroll
    for (int r = 16; r < 64; r += 16) {
        const double rv = __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), r),
                                           __builtin_amdgcn_readlane(__double2loint(v), r));
        const int ri = __builtin_amdgcn_readlane(i, r);
        if (before(rv, ri, bv, bi)) {
            bv = rv;
            bi = ri;
        }
    }
    v = bv;
    i = bi;
}

__device__ inline double sigmoid64(double z) { return 1.0 / (1.0 + exp(-z)); }

// Compare-exchange of register slots a < b so that slot a holds the one that
// comes first in the selection order.
template <int NV>
__device__ inline void cex(double (&v)[NV], int (&id)[NV], int a, int b) {
    const bool sw = before(v[b], id[b], v[a], id[a]);
    const double va = v[a], vb = v[b];
    const int ia = id[a], ib = id[b];
    v[a] = sw ? vb : va;
    v[b] = sw ? va : vb;
    id[a] = sw ? ib : ia;
    id[b] = sw ? ia : ib;
}

__device__ inline double readlane_f64(double v, int l) {
    return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), l),
                            __builtin_amdgcn_readlane(__double2loint(v), l));
}

// One token's routing from its winners: lane k < K holds entry k (selection
// order) with its expert id and raw score. The weights are the raw scores
// renormalised over the selection (summed in selection order). With top_p > 0,
// K3_TOPP ("Kimi K3 engine (c/kimi_k3.c)", "Streaming design" and its table of
// environment variables): the entries are ranked by weight, largest first,
// equal weights in selection order; an entry is kept while the weight ranked
// before it (summed in rank order, double) is below top_p, so the entry that
// reaches top_p is kept; a dropped entry is written as idx -1, wts 0 and the
// kept weights are renormalised over the kept raw scores.
__device__ inline void write_routing(int32_t *idx, float *wts, int my_id, double my_sc, int K, int lane,
                                     double top_p) {
    double sum = 0.0;
    for (int k = 0; k < K; ++k) sum += readlane_f64(my_sc, k);
    bool keep = true;
    if (top_p > 0.0) {
        const double w = my_sc / sum;
        int rank = 0;
        for (int j = 0; j < K; ++j) {
            const double wj = readlane_f64(w, j);
            rank += (wj > w || (wj == w && j < lane)) ? 1 : 0;
        }
        double before = 0.0, mine = 0.0;
        for (int r = 0; r < K; ++r) {
            const uint64_t m = __ballot(lane < K && rank == r);
            const int L = __builtin_amdgcn_readfirstlane(m ? __builtin_ctzll(m) : 0);
            mine = lane == L ? before : mine;
            before += readlane_f64(w, L);
        }
        keep = mine < top_p;
    }
    double kept = 0.0;
    for (int k = 0; k < K; ++k) kept += readlane_f64(keep ? my_sc : 0.0, k);
    if (lane < K) {
        idx[lane] = keep ? my_id : -1;
        wts[lane] = keep ? (float)(my_sc / kept) : 0.0f;
    }
}

// Each lane first sorts its NV candidates (a bitonic network over register
// slots, all indices compile-time); then every round the lanes' heads compete
// and the winning lane shifts its list by one. No per-round scan, no LDS.
template <int NV>
__global__ __launch_bounds__(64) void topk_kernel(int32_t *__restrict__ idx, float *__restrict__ wts,
                                                  const double *__restrict__ logits, const float *__restrict__ bias,
                                                  int T, int E, int K, double top_p) {
    const int lane = threadIdx.x;
    for (int t = blockIdx.x; t < T; t += gridDim.x) {
        const double *lg = logits + (size_t)t * E;
        double v[NV];
        int id[NV];
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int e = lane + j * kWave;
            const int ec = e < E ? e : E - 1;
            const double b = sigmoid64(lg[ec]) + (double)bias[ec];
            v[j] = e < E ? b : -__builtin_inf();
            id[j] = e < E ? e : 0x7fffffff;
        }
#pragma unroll
        for (int k = 2; k <= NV; k <<= 1)
#pragma unroll
            for (int jj = k >> 1; jj > 0; jj >>= 1)
#pragma unroll
                for (int i = 0; i < NV; ++i) {
                    const int l = i ^ jj;
                    if (l > i) {
                        if ((i & k) == 0)
                            cex<NV>(v, id, i, l);
                        else
                            cex<NV>(v, id, l, i);
                    }
                }
        int my_id = 0;  // lane k keeps the k-th winner
        for (int k = 0; k < K; ++k) {
            double bv = v[0];
            int bi = id[0];
            wave_best(bv, bi);
            if (bi >= E) bi = 0;  // only with non-finite scores, outside the contract
            my_id = lane == k ? bi : my_id;
            const bool me = id[0] == bi;  // the winner sits at the head of its lane's list
#pragma unroll
            for (int j = 0; j < NV - 1; ++j) {
                v[j] = me ? v[j + 1] : v[j];
                id[j] = me ? id[j + 1] : id[j];
            }
            v[NV - 1] = me ? -__builtin_inf() : v[NV - 1];
            id[NV - 1] = me ? 0x7fffffff : id[NV - 1];
        }
        // weights: each lane's raw score (the value its key was built from)
        const double my_sc = lane < K ? sigmoid64(lg[my_id]) : 0.0;
        write_routing(idx + (size_t)t * K, wts + (size_t)t * K, my_id, my_sc, K, lane, top_p);
    }
}

// ---- top-k, few tokens: one workgroup per token ---------------------------------
// One candidate per thread. Each wavefront sorts its four rows of 16 lanes
// (a bitonic sort in the "flip" form: every compare-exchange leaves the better
// candidate in the lower lane, so all rows end sorted the same way), then
// merges rows 0+1 and 2+3 and the two results: its best 16, in order. The
// wavefronts' lists meet in LDS and are merged four at a time, twice. Almost
// every exchange is a DPP move; only the merges across 32 lanes go through the
// LDS crossbar. Needs top_k <= 16 and E <= 1024.
constexpr int TB_LIST = 16;         // candidates kept per list
constexpr int TB_MAX_WAVES = 16;    // E <= 1024

struct Cand {
    double v;
    int id;
};

template <int CTRL>
__device__ inline Cand dpp_cand(const Cand &c) {
    Cand o;
    const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(c.v), CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(c.v), CTRL, 0xF, 0xF, false);
    o.v = __hiloint2double(hi, lo);
    o.id = __builtin_amdgcn_update_dpp(0, c.id, CTRL, 0xF, 0xF, false);
    return o;
}

template <int PATTERN>
__device__ inline Cand swz_cand(const Cand &c) {
    Cand o;
    const int lo = __builtin_amdgcn_ds_swizzle(__double2loint(c.v), PATTERN);
    const int hi = __builtin_amdgcn_ds_swizzle(__double2hiint(c.v), PATTERN);
    o.v = __hiloint2double(hi, lo);
    o.id = __builtin_amdgcn_ds_swizzle(c.id, PATTERN);
    return o;
}

__device__ inline Cand shfl_cand(const Cand &c, int src) {
    Cand o;
    const int lo = __shfl(__double2loint(c.v), src, kWave);
    const int hi = __shfl(__double2hiint(c.v), src, kWave);
    o.v = __hiloint2double(hi, lo);
    o.id = __shfl(c.id, src, kWave);
    return o;
}

// The lower lane of a pair keeps the candidate that comes first.
__device__ inline void cx(Cand &c, const Cand &p, bool lower) {
    const bool p_first = before(p.v, p.id, c.v, c.id);
    const bool c_first = before(c.v, c.id, p.v, p.id);
    const bool take = lower ? p_first : c_first;
    c.v = take ? p.v : c.v;
    c.id = take ? p.id : c.id;
}

// Partner lane ^ 4 inside a row of 16: one of the two row rotations by 4 and
// by 12 supplies it, depending on the lane; `use4` says which (found once at
// start-up from the rotated lane ids, so the rotation direction is not assumed).
__device__ inline Cand xor4_cand(const Cand &c, bool use4) {
    const Cand a = dpp_cand<0x124>(c);  // row_ror:4
    const Cand b = dpp_cand<0x12C>(c);  // row_ror:12
    return use4 ? a : b;
}

// Half-cleaners 8, 4, 2, 1 inside each row of 16.
__device__ inline void clean16(Cand &c, int lane, bool use4) {
    cx(c, dpp_cand<0x128>(c), (lane & 8) == 0);  // row_ror:8 = lane ^ 8
    cx(c, xor4_cand(c, use4), (lane & 4) == 0);
    cx(c, dpp_cand<0x4E>(c), (lane & 2) == 0);   // quad_perm [2,3,0,1]
    cx(c, dpp_cand<0xB1>(c), (lane & 1) == 0);   // quad_perm [1,0,3,2]
}

// Sort every row of 16 lanes, best first.
__device__ inline void sort16(Cand &c, int lane, bool use4) {
    cx(c, dpp_cand<0xB1>(c), (lane & 1) == 0);   // k = 2
    cx(c, dpp_cand<0x1B>(c), (lane & 2) == 0);   // k = 4: mirror in 4 (quad_perm [3,2,1,0])
    cx(c, dpp_cand<0xB1>(c), (lane & 1) == 0);
    cx(c, dpp_cand<0x141>(c), (lane & 4) == 0);  // k = 8: row_half_mirror
    cx(c, dpp_cand<0x4E>(c), (lane & 2) == 0);
    cx(c, dpp_cand<0xB1>(c), (lane & 1) == 0);
    cx(c, dpp_cand<0x140>(c), (lane & 8) == 0);  // k = 16: row_mirror
    cx(c, xor4_cand(c, use4), (lane & 4) == 0);
    cx(c, dpp_cand<0x4E>(c), (lane & 2) == 0);
    cx(c, dpp_cand<0xB1>(c), (lane & 1) == 0);
}

// Rows 0..3 hold sorted lists; afterwards row 0 holds the best 16 of the four,
// sorted. Rows 0+1 and 2+3 merge by mirroring inside 32 lanes (swizzle with
// xor mask 31), then row 0 meets row 2 reversed.
__device__ inline void merge4(Cand &c, int lane, bool use4) {
    cx(c, swz_cand<0x7C1F>(c), (lane & 16) == 0);  // and 0x1F, or 0, xor 0x1F
    clean16(c, lane, use4);
    const Cand p = shfl_cand(c, 47 - (lane & 15));   // row 2, last to first
    cx(c, p, true);                                  // only row 0 is kept
    clean16(c, lane, use4);
}

__global__ __launch_bounds__(TB_MAX_WAVES * 64) void topk_block_kernel(int32_t *__restrict__ idx,
                                                                       float *__restrict__ wts,
                                                                       const double *__restrict__ logits,
                                                                       const float *__restrict__ bias, int T, int E,
                                                                       int K, double top_p) {
    __shared__ double sc_lds[TB_MAX_WAVES * 64];
    __shared__ double l1v[TB_MAX_WAVES * TB_LIST];
    __shared__ int l1i[TB_MAX_WAVES * TB_LIST];
    __shared__ double l2v[4 * TB_LIST];
    __shared__ int l2i[4 * TB_LIST];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int n_lists = (E + kWave - 1) / kWave;
    const bool use4 = __builtin_amdgcn_update_dpp(0, lane, 0x124, 0xF, 0xF, false) == (lane ^ 4);
    const Cand none = {-__builtin_inf(), 0x7fffffff};
    for (int t = blockIdx.x; t < T; t += gridDim.x) {
        const double *lg = logits + (size_t)t * E;
        Cand c = none;
        if (tid < E) {
            const double sc = sigmoid64(lg[tid]);
            sc_lds[tid] = sc;
            c.v = sc + (double)bias[tid];
            c.id = tid;
        }
        sort16(c, lane, use4);
        merge4(c, lane, use4);
        if (wave < n_lists && lane < TB_LIST) {
            l1v[wave * TB_LIST + lane] = c.v;
            l1i[wave * TB_LIST + lane] = c.id;
        }
        __syncthreads();
        if (wave < 4) {
            const int l = wave * 4 + lane / TB_LIST;
            Cand d = none;
            if (l < n_lists) {
                d.v = l1v[l * TB_LIST + (lane & 15)];
                d.id = l1i[l * TB_LIST + (lane & 15)];
            }
            merge4(d, lane, use4);
            if (lane < TB_LIST) {
                l2v[wave * TB_LIST + lane] = d.v;
                l2i[wave * TB_LIST + lane] = d.id;
            }
        }
        __syncthreads();
        if (wave == 0) {
            Cand d;
            d.v = l2v[lane];
            d.id = l2i[lane];
            merge4(d, lane, use4);
            const int my_id = d.id < E ? d.id : 0;  // not a real id only with non-finite scores
            // weights: the raw scores of the winners
            const double my_sc = lane < K ? sc_lds[my_id] : 0.0;
            write_routing(idx + (size_t)t * K, wts + (size_t)t * K, my_id, my_sc, K, lane, top_p);
        }
        __syncthreads();  // the LDS lists are reused by the next token
    }
}

// ---- bucket: stable counting sort of the T*K pairs by expert ---------------------
// One workgroup of NT threads. counts/offsets by an LDS histogram and scan;
// positions within an expert follow token order: tokens are taken up to 64 at
// a time, a 64-bit mask per expert marks which of them chose it, and a pair's
// rank is the popcount of the mask below its token.
template <int NT>
__device__ inline int block_excl_scan(int v, int *wsum) {
    // wavefront scans with shuffles, then a scan of the per-wavefront totals;
    // returns the exclusive prefix of v over the block.
    const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
    constexpr int nw = NT / kWave;
    int inc = v;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int o = __shfl_up(inc, d, kWave);
        if (lane >= d) inc += o;
    }
    if (nw == 1) return inc - v;
    if (lane == kWave - 1) wsum[w] = inc;
    __syncthreads();
    if (w == 0) {
        int t = lane < nw ? wsum[lane] : 0;
#pragma unroll
        for (int d = 1; d < nw; d <<= 1) {
            const int o = __shfl_up(t, d, kWave);
            if (lane >= d) t += o;
        }
        if (lane < nw) wsum[lane] = t;
    }
    __syncthreads();
    const int res = (w > 0 ? wsum[w - 1] : 0) + inc - v;
    __syncthreads();
    return res;
}

// With `passes` set (npp > 0), also the work table of the matrix-core layer:
// every slot's pairs in passes of npp, passes[0] = their number, then
// passes[1 + 2k], passes[2 + 2k] = (slot, pass index) in slot order.
template <int NT>
__global__ __launch_bounds__(NT) void bucket_kernel(int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
                                                    int32_t *__restrict__ perm, int32_t *__restrict__ inv,
                                                    int32_t *__restrict__ active, const int32_t *__restrict__ idx,
                                                    int T, int K, int E, int32_t *__restrict__ passes, int npp) {
    extern __shared__ int sm[];
    int *cnt = sm;                                        // [E]
    int *run = sm + E;                                    // [E]
    int *tmp = sm + 2 * E;                                // [NT / 64], then the repeat flag
    unsigned long long *mask = (unsigned long long *)(sm + 2 * E + 18);  // [E], 8-byte aligned
    const int tid = threadIdx.x;
    const int P = T * K;
    for (int e = tid; e < E; e += NT) { cnt[e] = 0; mask[e] = 0ull; }
    __syncthreads();
    // ids outside [0, E) break the caller's precondition; they are dropped here
    // (their pair gets inv = -1 and contributes nothing) rather than written
    // out of bounds.
    for (int p = tid; p < P; p += NT) {
        const int e = idx[p];
        if ((unsigned)e < (unsigned)E) atomicAdd(&cnt[e], 1);
        else inv[p] = -1;
    }
    __syncthreads();
    // each thread owns a run of ceil(E/NT) experts
    const int per = (E + NT - 1) / NT;
    const int e0 = tid * per;
    int local = 0, nz = 0;
    for (int e = e0; e < e0 + per && e < E; ++e) { local += cnt[e]; nz += cnt[e] > 0; }
    const int base = block_excl_scan<NT>(local, tmp);
    const int nzbase = block_excl_scan<NT>(nz, tmp);
    int acc = base, nacc = nzbase;
    for (int e = e0; e < e0 + per && e < E; ++e) {
        counts[e] = cnt[e];
        offsets[e] = acc;
        run[e] = acc;
        if (cnt[e] > 0) active[1 + nacc++] = e;
        acc += cnt[e];
    }
    if (tid == NT - 1) {
        offsets[E] = acc;  // the last thread's prefix + its own is the total
        active[0] = nacc;
    }
    if (passes) {  // uniform: every thread takes part in the scan
        int np = 0;
        for (int e = e0; e < e0 + per && e < E; ++e) np += (cnt[e] + npp - 1) / npp;
        const int pbase = block_excl_scan<NT>(np, tmp);
        int k = pbase, slot = nzbase;
        for (int e = e0; e < e0 + per && e < E; ++e) {
            if (cnt[e] == 0) continue;
            for (int j = 0; j * npp < cnt[e]; ++j, ++k) {
                passes[1 + 2 * k] = slot;
                passes[2 + 2 * k] = j;
            }
            ++slot;
        }
        if (tid == NT - 1) passes[0] = k;
    }
    __syncthreads();
    const int tpc = (NT / K) < 64 ? (NT / K) : 64;  // tokens per chunk
    // A pair's rank among its expert's pairs of the chunk is the number of
    // earlier tokens of the chunk that name the expert: one mask bit per token.
    // That count is a pair count only while no token names an expert twice, so
    // a chunk where one does (the OR finds its own bit already set) is placed
    // by one thread in (token, k) order instead.
    static_assert(NT / 64 <= 16, "the scan scratch holds 16 wavefront sums");
    int *dup = tmp + NT / 64;                             // [1], after the scan scratch
    if (tid == 0) *dup = 0;
    __syncthreads();
    for (int c0 = 0; c0 < T; c0 += tpc) {
        const int lt = tid / K, k = tid - lt * K;
        const int t = c0 + lt;
        int e = 0;
        const bool live = lt < tpc && t < T && (unsigned)(e = idx[t * K + k]) < (unsigned)E;
        if (live && (atomicOr(&mask[e], 1ull << lt) & (1ull << lt))) *dup = 1;
        __syncthreads();
        const bool serial = *dup != 0;
        if (!serial) {
            if (live) {
                const int rank = __popcll(mask[e] & ((1ull << lt) - 1ull));
                const int pos = run[e] + rank;
                perm[pos] = t * K + k;
                inv[t * K + k] = pos;
            }
        } else if (tid == 0) {
            const int t1 = c0 + tpc < T ? c0 + tpc : T;
            for (int q = c0 * K; q < t1 * K; ++q) {
                const int eq = idx[q];
                if ((unsigned)eq >= (unsigned)E) continue;
                const int pos = run[eq]++;
                perm[pos] = q;
                inv[q] = pos;
            }
        }
        __syncthreads();
        for (int ee = tid; ee < E; ee += NT) {
            if (!serial) run[ee] += __popcll(mask[ee]);
            mask[ee] = 0ull;
        }
        if (tid == 0) *dup = 0;
        __syncthreads();
    }
}

// ---- host launchers -----------------------------------------------------------

// K splits of the 64 x 64 logits tiles (more than 128 tokens): enough
// workgroups for the chip's 256 CUs, at most 8 (logits_planes, which sizes the
// workspace), and each wavefront at least two steps of 16 columns. With more
// than one split the partial planes follow the logits in the same workspace
// region.
int logits_planes(int T, int E) {
    if (T <= 128) return 1;
    const int64_t tiles = (int64_t)((E + 63) / 64) * ((T + 63) / 64);
    if (tiles >= 192) return 1;
    const int ks = (int)(256 / tiles);
    return ks < 8 ? (ks > 1 ? ks : 1) : 8;
}
int logits_splits(int T, int in, int E) {
    const int ks = logits_planes(T, E), nk = (in + 15) / 16;
    return ks < nk / 16 ? ks : (nk / 16 > 1 ? nk / 16 : 1);
}

int launch_logits(double *logits, const float *x, const float *W, int T, int in, int E, hipStream_t st) {
    if (T == 0) return K3G_OK;
    if (T <= 8) {
        const bool vec = in % 4 == 0 && ((uintptr_t)x % 16) == 0 && ((uintptr_t)W % 16) == 0;
        const int rw = (in / 4 + kWave - 1) / kWave;
        const int g4 = (E + kLogitWaves - 1) / kLogitWaves;
        if (vec && rw <= 8)
            logits_rows_kernel<8><<<g4, 64 * kLogitWaves, 0, st>>>(logits, x, W, T, in, E);
        else if (vec && rw <= 16)
            logits_rows_kernel<16><<<g4, 64 * kLogitWaves, 0, st>>>(logits, x, W, T, in, E);
        else if (vec && rw <= 32)
            logits_rows_kernel<32><<<g4, 64 * kLogitWaves, 0, st>>>(logits, x, W, T, in, E);
        else
            logits_rows_any_kernel<<<E, 64, 0, st>>>(logits, x, W, T, in, E);
    } else {
        const bool vec = in % 4 == 0 && ((uintptr_t)x % 16) == 0 && ((uintptr_t)W % 16) == 0;
        if (T <= 128) {
            // few token tiles: eight wavefronts share each tile's columns
            const dim3 grid((E + 31) / 32, (T + 15) / 16);
            if (vec) logits_mfma_kernel<1, 2, 8, true><<<grid, 512, 0, st>>>(logits, x, W, T, in, E);
            else logits_mfma_kernel<1, 2, 8, false><<<grid, 512, 0, st>>>(logits, x, W, T, in, E);
        } else {
            // 64 x 64 tiles; K split across workgroups while the tiles alone
            // would leave the chip short of workgroups
            const int KS = logits_splits(T, in, E);
            const dim3 grid((E + 63) / 64, (T + 63) / 64, KS);
            double *dst = KS > 1 ? logits + (size_t)T * E : logits;
            const void *f = vec ? (const void *)logits_tile_kernel<true> : (const void *)logits_tile_kernel<false>;
            if (hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLTLds) != hipSuccess)
                return K3G_EHIP;
            if (vec) logits_tile_kernel<true><<<grid, 512, kLTLds, st>>>(dst, x, W, T, in, E, KS);
            else logits_tile_kernel<false><<<grid, 512, kLTLds, st>>>(dst, x, W, T, in, E, KS);
            if (KS > 1) {
                if (hipGetLastError() != hipSuccess) return K3G_EHIP;
                const int64_t n = (int64_t)T * E;
                logits_sum_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(logits, dst, n, KS);
            }
        }
    }
    return hipGetLastError() == hipSuccess ? K3G_OK : K3G_EHIP;
}

int launch_topk(int32_t *idx, float *wts, const double *logits, const float *bias, int T, int E, int K,
                double top_p, hipStream_t st) {
    if (T == 0) return K3G_OK;
    const int blocks = T < 65536 ? T : 65536;
    const int nv = (E + kWave - 1) / kWave;
    if (K <= TB_LIST && nv <= TB_MAX_WAVES && T <= K3G_TOPK_BLOCK_MAX_T) {
        const int waves = nv < 4 ? 4 : nv;
        topk_block_kernel<<<blocks, waves * kWave, 0, st>>>(idx, wts, logits, bias, T, E, K, top_p);
    } else if (nv <= 16)
        topk_kernel<16><<<blocks, 64, 0, st>>>(idx, wts, logits, bias, T, E, K, top_p);
    else
        topk_kernel<32><<<blocks, 64, 0, st>>>(idx, wts, logits, bias, T, E, K, top_p);
    return hipGetLastError() == hipSuccess ? K3G_OK : K3G_EHIP;
}

size_t bucket_lds_bytes(int E) {
    // cnt, run [E]; the scan scratch [16] and the repeat flag; alignment; mask [E]
    return sizeof(int) * (size_t)(2 * E + 16 + 2) + sizeof(unsigned long long) * (size_t)E;
}

int launch_bucket(int32_t *counts, int32_t *offsets, int32_t *perm, int32_t *inv, int32_t *active, const int32_t *idx,
                  int T, int K, int E, hipStream_t st, int32_t *passes, int npp) {
    // one wavefront was measured slower for 16 pairs: its per-expert loops run 16x longer
    bucket_kernel<1024><<<1, 1024, bucket_lds_bytes(E), st>>>(counts, offsets, perm, inv, active, idx, T, K, E,
                                                              passes, npp);
    return hipGetLastError() == hipSuccess ? K3G_OK : K3G_EHIP;
}

}  // namespace k3g
