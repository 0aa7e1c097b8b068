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

namespace k3g {

// ---- logits, few tokens: one wavefront per expert row ------------------------
__global__ __launch_bounds__(256) void logits_rows_kernel(double *__restrict__ logits, const float *__restrict__ x,
                                                          const float *__restrict__ W, int T, int in, int E) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = (blockIdx.x * blockDim.x + threadIdx.x) / kWave;
    const int n_waves = gridDim.x * blockDim.x / kWave;
    for (int e = wave; e < E; e += n_waves) {
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

// ---- logits, many tokens: 64x64 register-tiled fp64 product -------------------
constexpr int LT = 64, LK = 16;
__global__ __launch_bounds__(256) void logits_tiled_kernel(double *__restrict__ logits, const float *__restrict__ x,
                                                           const float *__restrict__ W, int T, int in, int E) {
    __shared__ double xs[LK][LT + 1];
    __shared__ double ws[LK][LT + 1];
    const int t0 = blockIdx.y * LT, e0 = blockIdx.x * LT;
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    double acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.0;
    for (int k0 = 0; k0 < in; k0 += LK) {
#pragma unroll
        for (int l = 0; l < 4; ++l) {
            const int id = threadIdx.x + l * 256;
            const int r = id / LK, kk = id % LK;
            const int k = k0 + kk;
            xs[kk][r] = (t0 + r < T && k < in) ? (double)x[(size_t)(t0 + r) * in + k] : 0.0;
            ws[kk][r] = (e0 + r < E && k < in) ? (double)W[(size_t)(e0 + r) * in + k] : 0.0;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < LK; ++kk) {
            double a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = xs[kk][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = ws[kk][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fma(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int t = t0 + ty * 4 + i, e = e0 + tx * 4 + j;
            if (t < T && e < E) logits[(size_t)t * E + e] = acc[i][j];
        }
}

// ---- top-k: one wavefront per token --------------------------------------------
// Biased scores in LDS; k rounds of a wavefront arg-max where a larger score
// wins and equal scores go to the lower expert id; the winner is retired.
__device__ inline bool better(double va, int ia, double vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}

__global__ __launch_bounds__(64) void topk_kernel(int32_t *__restrict__ idx, float *__restrict__ wts,
                                                  const double *__restrict__ logits, const float *__restrict__ bias,
                                                  int T, int E, int K) {
    extern __shared__ double smem[];
    double *bs = smem;                   // biased score, -inf once taken
    double *sc = smem + E;               // raw sigmoid score
    int *sel = (int *)(smem + 2 * E);    // selected ids, k order
    const int lane = threadIdx.x;
    for (int t = blockIdx.x; t < T; t += gridDim.x) {
        for (int e = lane; e < E; e += kWave) {
            const double s = 1.0 / (1.0 + exp(-logits[(size_t)t * E + e]));
            sc[e] = s;
            bs[e] = s + (double)bias[e];
        }
        __syncthreads();
        double sum = 0.0;
        for (int k = 0; k < K; ++k) {
            double bv = -__builtin_inf();
            int bi = 0x7fffffff;
            for (int e = lane; e < E; e += kWave) {
                const double v = bs[e];
                if (better(v, e, bv, bi)) { bv = v; bi = e; }
            }
            for (int m = 32; m >= 1; m >>= 1) {
                const double ov = __shfl_xor(bv, m, kWave);
                const int oi = __shfl_xor(bi, m, kWave);
                if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
            }
            // every lane now holds the same winner; NaN logits (outside the
            // contract) could leave none, so stay in bounds
            if (bi >= E) bi = 0;
            sum += sc[bi];
            if (lane == 0) {
                idx[(size_t)t * K + k] = bi;
                sel[k] = bi;
            }
            __syncthreads();
            if ((bi & (kWave - 1)) == lane) bs[bi] = -__builtin_inf();
            __syncthreads();
        }
        if (lane < K) wts[(size_t)t * K + lane] = (float)(sc[sel[lane]] / sum);
        __syncthreads();
    }
}

// ---- bucket: stable counting sort of the T*K pairs by expert ---------------------
// One workgroup. counts/offsets by an LDS histogram and scan; positions within
// an expert follow token order: tokens are taken 64 at a time, a 64-bit mask
// per expert marks which of them chose it, and a pair's rank is the popcount of
// the mask below its token.
constexpr int BK_THREADS = 1024;

__device__ inline int block_excl_scan(int v, int *tmp) {
    // Hillis-Steele over BK_THREADS values in LDS; returns the exclusive prefix.
    const int tid = threadIdx.x;
    tmp[tid] = v;
    __syncthreads();
    for (int off = 1; off < BK_THREADS; off <<= 1) {
        const int a = tid >= off ? tmp[tid - off] : 0;
        __syncthreads();
        tmp[tid] += a;
        __syncthreads();
    }
    const int incl = tmp[tid];
    __syncthreads();
    return incl - v;
}

__global__ __launch_bounds__(BK_THREADS) void bucket_kernel(int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
                                                            int32_t *__restrict__ perm, int32_t *__restrict__ inv,
                                                            int32_t *__restrict__ active, const int32_t *__restrict__ idx,
                                                            int T, int K, int E) {
    extern __shared__ int sm[];
    int *cnt = sm;                                        // [E]
    int *run = sm + E;                                    // [E]
    int *tmp = sm + 2 * E;                                // [BK_THREADS]
    unsigned long long *mask = (unsigned long long *)(sm + 2 * E + BK_THREADS + ((2 * E + BK_THREADS) & 1));  // [E]
    const int tid = threadIdx.x;
    const int P = T * K;
    for (int e = tid; e < E; e += BK_THREADS) { cnt[e] = 0; mask[e] = 0ull; }
    __syncthreads();
    // ids outside [0, E) break the caller's precondition; they are dropped here
    // (their pair gets inv = -1 and contributes nothing) rather than written
    // out of bounds.
    for (int p = tid; p < P; p += BK_THREADS) {
        const int e = idx[p];
        if ((unsigned)e < (unsigned)E) atomicAdd(&cnt[e], 1);
        else inv[p] = -1;
    }
    __syncthreads();
    // each thread owns a run of ceil(E/BK_THREADS) experts
    const int per = (E + BK_THREADS - 1) / BK_THREADS;
    const int e0 = tid * per;
    int local = 0, nz = 0;
    for (int e = e0; e < e0 + per && e < E; ++e) { local += cnt[e]; nz += cnt[e] > 0; }
    const int base = block_excl_scan(local, tmp);
    const int nzbase = block_excl_scan(nz, tmp);
    int acc = base, nacc = nzbase;
    for (int e = e0; e < e0 + per && e < E; ++e) {
        counts[e] = cnt[e];
        offsets[e] = acc;
        run[e] = acc;
        if (cnt[e] > 0) active[1 + nacc++] = e;
        acc += cnt[e];
    }
    if (tid == BK_THREADS - 1) {
        offsets[E] = acc;  // the last thread's prefix + its own is the total
        active[0] = nacc;
    }
    __syncthreads();
    const int tpc = (BK_THREADS / K) < 64 ? (BK_THREADS / K) : 64;  // tokens per chunk
    for (int c0 = 0; c0 < T; c0 += tpc) {
        const int lt = tid / K, k = tid - lt * K;
        const int t = c0 + lt;
        int e = 0;
        const bool live = lt < tpc && t < T && (unsigned)(e = idx[t * K + k]) < (unsigned)E;
        if (live) atomicOr(&mask[e], 1ull << lt);
        __syncthreads();
        if (live) {
            const int rank = __popcll(mask[e] & ((1ull << lt) - 1ull));
            const int pos = run[e] + rank;
            perm[pos] = t * K + k;
            inv[t * K + k] = pos;
        }
        __syncthreads();
        for (int ee = tid; ee < E; ee += BK_THREADS) {
            run[ee] += __popcll(mask[ee]);
            mask[ee] = 0ull;
        }
        __syncthreads();
    }
}

// ---- host launchers -----------------------------------------------------------

int launch_logits(double *logits, const float *x, const float *W, int T, int in, int E, hipStream_t st) {
    if (T == 0) return K3G_OK;
    if (T <= 8) {
        const int blocks = (E + 3) / 4;
        logits_rows_kernel<<<blocks, 256, 0, st>>>(logits, x, W, T, in, E);
    } else {
        const dim3 grid((E + LT - 1) / LT, (T + LT - 1) / LT);
        logits_tiled_kernel<<<grid, 256, 0, st>>>(logits, x, W, T, in, E);
    }
    return hipGetLastError() == hipSuccess ? K3G_OK : K3G_EHIP;
}

int launch_topk(int32_t *idx, float *wts, const double *logits, const float *bias, int T, int E, int K,
                hipStream_t st) {
    if (T == 0) return K3G_OK;
    const int blocks = T < 8192 ? T : 8192;
    topk_kernel<<<blocks, 64, sizeof(double) * 2 * E + sizeof(int) * 64, st>>>(idx, wts, logits, bias, T, E, K);
    return hipGetLastError() == hipSuccess ? K3G_OK : K3G_EHIP;
}

size_t bucket_lds_bytes(int E) {
    return sizeof(int) * (size_t)(2 * E + BK_THREADS + 2) + sizeof(unsigned long long) * (size_t)E;
}

int launch_bucket(int32_t *counts, int32_t *offsets, int32_t *perm, int32_t *inv, int32_t *active, const int32_t *idx,
                  int T, int K, int E, hipStream_t st) {
    bucket_kernel<<<1, BK_THREADS, bucket_lds_bytes(E), st>>>(counts, offsets, perm, inv, active, idx, T, K, E);
    return hipGetLastError() == hipSuccess ? K3G_OK : K3G_EHIP;
}

}  // namespace k3g
