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

}  // namespace k3g
