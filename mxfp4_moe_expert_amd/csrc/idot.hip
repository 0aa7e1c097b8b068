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
// The matrix-core kernels are not built yet: the IDOT entry points report
// K3G_EUNSUPPORTED until they are.
int launch_idot_groupsums(int32_t *, const int8_t *, const uint8_t *, int, int, int, hipStream_t) {
    return K3G_EUNSUPPORTED;
}
int launch_moe_up_idot(float *, const int8_t *, const float *, const BankDev &, const int32_t *, const int32_t *,
                       const int32_t *, int, int, int, int, hipStream_t) {
    return K3G_EUNSUPPORTED;
}
int launch_moe_down_idot(float *, const int8_t *, const float *, const BankDev &, const int32_t *, const int32_t *,
                         const int32_t *, int, int, int, hipStream_t) {
    return K3G_EUNSUPPORTED;
}
}  // namespace k3g
