// probe.hip -- measurement hooks: what this MI355X sustains, as denominators
// for the roofline beside the datasheet peaks. Not part of the method.
//
// k3g_probe_mfma_rate: every wavefront issues `iters` rounds of four
// independent matrix-core products of one kind (the kinds the path uses:
// int8 32x32x32, bf16 16x16x32, block-scaled FP4 16x16x128, fp64 16x16x4) on
// register operands; no memory traffic, four accumulators so that no product
// waits for the one before.
// k3g_probe_read_rate: a streaming read of a buffer, every byte once. Each
// wavefront takes 16 KB chunks in turn (sixteen 1 KB loads in flight, lane l
// reading bytes 16l..16l+15 of each KB) over 8192 workgroups: of the read
// orders tried on this chip (grid-stride with 4 or 8 loads in flight,
// wave-contiguous chunks of 8 or 16 KB, 1024..8192 workgroups) this one reads
// fastest, so it stands for what a streaming kernel can reach.
// Both store to `sink` only when a result takes one particular value, so
// the compiler must keep the work (the store itself is rare and harmless).
// k3g_probe_handoff: what handing data from every workgroup of a launch to
// one consumer costs, by the two ways a kernel can do it: a second,
// dependent launch, or inside the launch with an agent-scope release by each
// workgroup, a device counter, and an acquire by the workgroup that counts
// last (the pattern a one-launch expert or a fused route would need).
#include "k3g_common.h"
#include "k3g.h"

namespace k3g {

typedef int v4i_t __attribute__((ext_vector_type(4)));
typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef int v16i_t __attribute__((ext_vector_type(16)));
typedef double v4d_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int kProbeBlocks = 2048;  // 8 wavefronts per CU
constexpr int kProbeThreads = 256;

template <int KIND>
__global__ __launch_bounds__(kProbeThreads) void mfma_rate_kernel(uint32_t *sink, int iters) {
    const int t = (int)threadIdx.x;
    if constexpr (KIND == 0) {  // int8 32x32x32
        const v4i_t a = {t, t + 1, t + 2, t + 3}, b = {t ^ 5, t ^ 6, t ^ 7, t ^ 9};
        v16i_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
        for (int i = 0; i < iters; ++i) {
            c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c0, 0, 0, 0);
            c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, a, c1, 0, 0, 0);
            c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, c2, 0, 0, 0);
            c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, b, c3, 0, 0, 0);
        }
        if (c0[0] + c1[1] + c2[2] + c3[3] == 0x7fffffff) sink[0] = 1u;
    } else if constexpr (KIND == 1) {  // bf16 16x16x32
        bf16x8_t a, b;
        for (int j = 0; j < 8; ++j) {
            a[j] = (__bf16)(float)(t + j);
            b[j] = (__bf16)(float)(t - j);
        }
        float4_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
        for (int i = 0; i < iters; ++i) {
            c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c0, 0, 0, 0);
            c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b, a, c1, 0, 0, 0);
            c2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, a, c2, 0, 0, 0);
            c3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b, b, c3, 0, 0, 0);
        }
        if (c0[0] + c1[1] + c2[2] + c3[3] == -1.5f) sink[0] = 1u;
    } else if constexpr (KIND == 2) {  // FP4 16x16x128 with block scales
        const v8i_t a = {t, t * 3, t * 5, t * 7, 0, 0, 0, 0}, b = {t ^ 1, t ^ 2, t ^ 3, t ^ 4, 0, 0, 0, 0};
        float4_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
        for (int i = 0; i < iters; ++i) {
            c0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c0, 4, 4, 0, 127, 0, 127);
            c1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b, a, c1, 4, 4, 0, 127, 0, 127);
            c2 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, a, c2, 4, 4, 0, 127, 0, 127);
            c3 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b, b, c3, 4, 4, 0, 127, 0, 127);
        }
        if (c0[0] + c1[1] + c2[2] + c3[3] == -1.5f) sink[0] = 1u;
    } else {  // fp64 16x16x4
        const double a = (double)t, b = (double)(t + 1);
        v4d_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
        for (int i = 0; i < iters; ++i) {
            c0 = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c0, 0, 0, 0);
            c1 = __builtin_amdgcn_mfma_f64_16x16x4f64(b, a, c1, 0, 0, 0);
            c2 = __builtin_amdgcn_mfma_f64_16x16x4f64(a, a, c2, 0, 0, 0);
            c3 = __builtin_amdgcn_mfma_f64_16x16x4f64(b, b, c3, 0, 0, 0);
        }
        if (c0[0] + c1[1] + c2[2] + c3[3] == -1.5) sink[0] = 1u;
    }
}

constexpr int kReadBlocks = 8192;
constexpr int kReadChunk = 16;  // 1 KB loads per wavefront chunk

__global__ __launch_bounds__(kProbeThreads) void read_rate_kernel(const uint4 *__restrict__ buf, int64_t n16,
                                                                  uint32_t *sink) {
    constexpr int64_t chunk16 = 64 * kReadChunk;  // 16-byte units per chunk
    const int lane = (int)(threadIdx.x & 63);
    const int64_t n_waves = (int64_t)gridDim.x * (kProbeThreads / 64);
    const int64_t n_chunks = n16 / chunk16;
    uint32_t x = 0;
    for (int64_t c = (int64_t)blockIdx.x * (kProbeThreads / 64) + (threadIdx.x >> 6); c < n_chunks; c += n_waves) {
        const uint4 *p = buf + c * chunk16 + lane;
        uint4 v[kReadChunk];
#pragma unroll
        for (int j = 0; j < kReadChunk; ++j) v[j] = p[j * 64];
#pragma unroll
        for (int j = 0; j < kReadChunk; ++j) x ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
    }
    // the tail that fills no whole chunk, grid-strided
    for (int64_t i = n_chunks * chunk16 + (int64_t)blockIdx.x * kProbeThreads + threadIdx.x; i < n16;
         i += (int64_t)gridDim.x * kProbeThreads) {
        const uint4 v = buf[i];
        x ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (x == 0x9E3779B9u) sink[0] = x;  // rare, and harmless: every writer stores the same value
}

}  // namespace k3g

using namespace k3g;

namespace k3g {

// Each workgroup stores one value; with MODE 2 it then releases (agent scope)
// and counts itself, and the workgroup that counts last acquires, sums every
// value into buf[n] and sets the counter back to zero.
template <int MODE>
__global__ __launch_bounds__(64) void handoff_produce_kernel(float *buf, uint32_t *counter, int n) {
    const int lane = threadIdx.x;
    if (lane == 0) buf[blockIdx.x] = (float)blockIdx.x * 0.5f;
    if constexpr (MODE == 2) {
        __shared__ int last;
        if (lane == 0) {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            last = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                   (uint32_t)n - 1;
        }
        __syncthreads();
        if (!last) return;
        if (lane == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        float sum = 0.f;
        for (int i = lane; i < n; i += kWave) sum += buf[i];
        sum = wave_sum(sum);
        if (lane == 0) buf[n] = sum;
    }
}

// The dependent second launch: one workgroup sums the n values.
__global__ __launch_bounds__(64) void handoff_consume_kernel(float *buf, int n) {
    float sum = 0.f;
    for (int i = threadIdx.x; i < n; i += kWave) sum += buf[i];
    sum = wave_sum(sum);
    if (threadIdx.x == 0) buf[n] = sum;
}

}  // namespace k3g

extern "C" {

int k3g_probe_handoff(int mode, int n_wg, float *buf, uint32_t *counter, void *stream) {
    using namespace k3g;
    if (mode < 0 || mode > 2 || n_wg < 1 || n_wg > 65536 || !buf || (mode == 2 && !counter)) return K3G_EINVAL;
    hipStream_t st = (hipStream_t)stream;
    switch (mode) {
        case 0: handoff_produce_kernel<0><<<n_wg, 64, 0, st>>>(buf, counter, n_wg); break;
        case 1:
            handoff_produce_kernel<0><<<n_wg, 64, 0, st>>>(buf, counter, n_wg);
            handoff_consume_kernel<<<1, 64, 0, st>>>(buf, n_wg);
            break;
        default: handoff_produce_kernel<2><<<n_wg, 64, 0, st>>>(buf, counter, n_wg); break;
    }
    return hipGetLastError() == hipSuccess ? K3G_OK : K3G_EHIP;
}

int k3g_probe_mfma_rate(int kind, int iters, uint32_t *sink, void *stream) {
    if (!sink || kind < 0 || kind > 3 || iters < 1) return K3G_EINVAL;
    hipStream_t st = (hipStream_t)stream;
    switch (kind) {
        case 0: mfma_rate_kernel<0><<<kProbeBlocks, kProbeThreads, 0, st>>>(sink, iters); break;
        case 1: mfma_rate_kernel<1><<<kProbeBlocks, kProbeThreads, 0, st>>>(sink, iters); break;
        case 2: mfma_rate_kernel<2><<<kProbeBlocks, kProbeThreads, 0, st>>>(sink, iters); break;
        default: mfma_rate_kernel<3><<<kProbeBlocks, kProbeThreads, 0, st>>>(sink, iters); break;
    }
    return hipGetLastError() == hipSuccess ? K3G_OK : K3G_EHIP;
}

int k3g_probe_read_rate(const void *buf, size_t bytes, uint32_t *sink, void *stream) {
    if (!buf || !sink || bytes == 0 || bytes % 16 || ((uintptr_t)buf & 15)) return K3G_EINVAL;
    read_rate_kernel<<<kReadBlocks, kProbeThreads, 0, (hipStream_t)stream>>>((const uint4 *)buf,
                                                                              (int64_t)(bytes / 16), sink);
    return hipGetLastError() == hipSuccess ? K3G_OK : K3G_EHIP;
}

}  // extern "C"
