// k3g_common.h -- device helpers shared by the libk3g kernels (gfx950 only).
//
// Format facts used here ("Kimi K3 engine (c/kimi_k3.c)", section "Weights";
// "kimi-k3-in-c: 2.78 trillion parameters, one CPU, 8 GB of RAM", section
// "Reduction one"): e2m1 codes two per byte, low nibble = even column, bit 3 =
// sign; one ue8m0 scale per 32 columns, w = v * 2^(s-127), scale 255 skips
// the group.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "k3g.h"

namespace k3g {

constexpr int kGroup = 32;          // columns per scale
constexpr int kWave = 64;           // CDNA wavefront
constexpr int kLutSlots = 64;       // LUT copies: one per lane, so no bank conflicts
constexpr int kLutWords = 256 * kLutSlots;  // 64 KB of LDS

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef int int4_t __attribute__((ext_vector_type(4)));
typedef int int16_t_v __attribute__((ext_vector_type(16)));

// Expert bank as the kernels see it: tensor i of expert e at base + e*stride + off[i].
struct BankDev {
    const uint8_t *base;
    int64_t stride;
    int64_t off[6];
};

enum { W1P = 0, W1S = 1, W3P = 2, W3S = 3, W2P = 4, W2S = 5 };

// One token's route entries handed to the decode up-projection, which ranks
// them in the bucket's order itself and writes the bucket from workgroup 0
// (idx null: the bucket was built by its own kernel).
struct Route1 {
    const int32_t *idx;                                // the token's K route entries
    int32_t *counts, *offsets, *perm, *inv, *active;  // the bucket's arrays
    int n_experts;
};

// Value of an e2m1 code from its bit fields: sign bit 3, exponent bits 2..1
// (bias 1), mantissa bit 0; exponent 0 is subnormal (0 or 0.5).
__host__ __device__ constexpr float e2m1_value(unsigned c) {
    const float mag = ((c >> 1) & 3u) == 0
                          ? 0.5f * float(c & 1u)
                          : float(1u << (((c >> 1) & 3u) - 1u)) * (1.0f + 0.5f * float(c & 1u));
    return (c & 8u) ? -mag : mag;
}

// The byte-pair LUT: byte -> two f16 values (low half = even column = low
// nibble, high half = odd column = high nibble). e2m1 values are exact in f16.
// Stored 64 times interleaved (word e*64 + lane) so that each lane reads its own
// bank: data-dependent indices never conflict.
__device__ inline void build_pair_lut(uint32_t *lut) {
    for (int i = threadIdx.x; i < kLutWords; i += blockDim.x) {
        const unsigned b = unsigned(i) >> 6;
        half2_t v;
        v.x = (_Float16)e2m1_value(b & 15u);
        v.y = (_Float16)e2m1_value(b >> 4);
        lut[i] = __builtin_bit_cast(uint32_t, v);
    }
}

// LDS byte address of byte k (0..3) of word w in this lane's LUT copy:
// (byte << 8) | (lane << 2), built with one v_perm_b32.
__device__ inline uint32_t lut_addr(uint32_t w, uint32_t lane_off, int k) {
    return __builtin_amdgcn_perm(w, lane_off, 0x0C0C0000u | ((4u + (uint32_t)k) << 8));
}

__device__ inline half2_t lut_read(const uint32_t *lut, uint32_t addr) {
    return __builtin_bit_cast(half2_t, *(const uint32_t *)((const char *)lut + addr));
}

// Sum of one group of 32 columns: 16 packed bytes (a uint4) against x[0..31].
// Two accumulators (even and odd columns), combined at the end. fp32 FMAs with
// the exact f16 weight widened inside the instruction (v_fma_mix_f32).
__device__ inline float group_dot(const uint32_t *lut, uint32_t lane_off, uint4 w, const float *xg) {
    float a0 = 0.f, a1 = 0.f;
    const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const half2_t v = lut_read(lut, lut_addr(d[q], lane_off, b));
            a0 = __builtin_fmaf((float)v.x, xg[q * 8 + b * 2], a0);
            a1 = __builtin_fmaf((float)v.y, xg[q * 8 + b * 2 + 1], a1);
        }
    }
    return a0 + a1;
}

// The same group sum with gfx950's scaled FP4 -> FP32 conversion instead of
// the LDS table: one v_cvt_scalef32_pk_f32_fp4 decodes the two nibbles of a
// byte (scale 1.0, so the values are the raw e2m1 ones).
template <int B>
__device__ inline void cvt_byte(uint32_t w, const float *xq, float &a0, float &a1) {
    const auto v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, B);
    a0 = __builtin_fmaf(v[0], xq[2 * B], a0);
    a1 = __builtin_fmaf(v[1], xq[2 * B + 1], a1);
}

__device__ inline float group_dot_cvt(uint4 w, const float *xg) {
    float a0 = 0.f, a1 = 0.f;
    const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        cvt_byte<0>(d[q], xg + q * 8, a0, a1);
        cvt_byte<1>(d[q], xg + q * 8, a0, a1);
        cvt_byte<2>(d[q], xg + q * 8, a0, a1);
        cvt_byte<3>(d[q], xg + q * 8, a0, a1);
    }
    return a0 + a1;
}

// Apply one group's ue8m0 scale: 2^(s-127) * sub, or nothing for s = 255.
__device__ inline float apply_scale(float sub, uint32_t s) {
    return s == 255u ? 0.0f : __builtin_ldexpf(sub, int(s) - 127);
}

// Full-wavefront sum, returned in every lane: DPP within each row of 16 lanes,
// then the four row sums read out of lanes 0, 16, 32, 48.
template <int CTRL>
__device__ inline float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

__device__ inline float wave_sum(float v) {
    v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp<0x141>(v);  // row_half_mirror
    v += dpp<0x140>(v);  // row_mirror
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
    return (r0 + r1) + (r2 + r3);
}

__device__ inline double wave_sum_f64(double v) {
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
    return v;
}

// e^x to about 2 ulp: v_exp_f32 (2^t, 1 ulp) at t = x*log2(e) rounded, times
// 1 + r*ln(2) for the part r of x*log2(e) that the rounding dropped (|r| is
// at most 2^-17 where the result is finite, so the factor is exact enough).
__device__ inline float exp_fast(float x) {
    constexpr float kL2E = 1.44269502f;        // log2(e) rounded to fp32
    constexpr float kL2E_LO = 1.92596299e-8f;  // log2(e) - kL2E
    const float t = x * kL2E;
    const float r = __builtin_fmaf(x, kL2E_LO, __builtin_fmaf(x, kL2E, -t));
    return __builtin_amdgcn_exp2f(t) * __builtin_fmaf(r, 0.693147182f, 1.0f);
}

// tanh(y): below |y| = 0.3 the odd Taylor series through y^9 (the next term
// is under 6e-8 of the value); above, 1 - 2/(e^{2|y|} + 1) with y's sign
// (v_rcp_f32, 1 ulp; the subtraction loses under 2 bits at |y| = 0.3).
__device__ inline float tanh_fast(float y) {
    const float a = __builtin_fabsf(y);
    const float s = y * y;
    float p = __builtin_fmaf(s, 62.0f / 2835.0f, -17.0f / 315.0f);
    p = __builtin_fmaf(s, p, 2.0f / 15.0f);
    p = __builtin_fmaf(s, p, -1.0f / 3.0f);
    const float small = __builtin_fmaf(y * s, p, y);
    const float big = __builtin_fmaf(-2.0f, __builtin_amdgcn_rcpf(exp_fast(2.0f * a) + 1.0f), 1.0f);
    return a < 0.3f ? small : __builtin_copysignf(big, y);
}

// SiTU-GLU ("Kimi K3 engine (c/kimi_k3.c)", "Architecture notes"):
// 4 tanh(g/4) sigmoid(g) * 25 tanh(u/25), in fp32 (a few ulp: exp and the
// reciprocal through the hardware approximations above; u/25 as u * 0.04).
__device__ inline float situ(float g, float u) {
    const float sig = __builtin_amdgcn_rcpf(1.0f + exp_fast(-g));
    return 4.0f * tanh_fast(g * 0.25f) * sig * (25.0f * tanh_fast(u * 0.04f));
}

// ---- IDOT quantisation of one value ("Kimi K3 engine (c/kimi_k3.c)", "Streaming
// design", K3_IDOT: per-32-group int8 activations) ---------------------------------
// With s = max|v|/127 of the value's 32-group (fp32, correctly rounded): q =
// rint(v / s) with the division correctly rounded and ties to even, clamped to
// +-127; a group whose maximum is 0 has s = 0 and q = 0.
__device__ inline float idot_group_scale(float amax) { return amax / 127.0f; }
__device__ inline int idot_quant(float v, float s) {
    return s == 0.0f ? 0 : (int)__builtin_fminf(__builtin_fmaxf(__builtin_rintf(v / s), -127.0f), 127.0f);
}
// An int8 value as bf16 bits: its fp32 form has at most 8 significant bits, so
// the top half of the fp32 bits is exact.
__device__ inline uint32_t i8_bf16_bits(int q) { return __builtin_bit_cast(uint32_t, (float)q) >> 16; }

// ---- one token: its route entries in the bucket's order -------------------------
// With a single token the bucket (pairs sorted by expert, then token) is a
// small permutation of the K route entries, which a wavefront can rank on its
// own; the decode up-projection does that instead of waiting for a separate
// bucket launch. Lane k holds entry k: its expert, whether the id is in range,
// its position among the sorted pairs, whether it is the first entry of its
// expert (duplicates share one slot), the slot of its expert (rank among the
// distinct experts) and the number of entries of its expert.
struct Route1Lane {
    int e, pos, slot, cnt;
    bool valid, first;
    uint64_t firsts;  // ballot of `first`: popcount = number of slots
};

__device__ inline Route1Lane route1_lane(const int32_t *idx, int K, int E, int lane) {
    Route1Lane r;
    r.e = lane < K ? idx[lane] : -1;
    r.valid = lane < K && (unsigned)r.e < (unsigned)E;
    r.pos = 0;
    r.cnt = 0;
    r.first = r.valid;
    for (int j = 0; j < K; ++j) {  // uniform loop: entry j's expert read from lane j
        const int ej = __builtin_amdgcn_readlane(r.e, j);
        if ((unsigned)ej < (unsigned)E) {
            r.pos += (ej < r.e || (ej == r.e && j < lane)) ? 1 : 0;
            r.cnt += ej == r.e ? 1 : 0;
            r.first = r.first && !(ej == r.e && j < lane);
        }
    }
    r.firsts = __ballot(r.first);
    r.slot = 0;
    for (int j = 0; j < K; ++j) {
        const int ej = __builtin_amdgcn_readlane(r.e, j);
        if ((r.firsts >> j) & 1ull) r.slot += ej < r.e ? 1 : 0;
    }
    return r;
}

// One slice of the bucket as the bucket kernel would write it: counts and
// offsets of experts [64*part, 64*part + 64), and for part 0 also perm, inv
// and active.
__device__ inline void route1_write_bucket_part(const Route1 &rt, const Route1Lane &r, int K, int lane, int part) {
    const int E = rt.n_experts;
    const int e = part * kWave + lane;
    int below = 0, c = 0;
    for (int j = 0; j < K; ++j) {
        const int ej = __builtin_amdgcn_readlane(r.e, j);
        if ((unsigned)ej < (unsigned)E) {
            below += ej < e ? 1 : 0;
            c += ej == e ? 1 : 0;
        }
    }
    if (e < E) rt.counts[e] = c;
    if (e <= E) rt.offsets[e] = below;
    if (part == 0) {
        if (r.valid) rt.perm[r.pos] = lane;
        if (lane < K) rt.inv[lane] = r.valid ? r.pos : -1;
        if (r.first) rt.active[1 + r.slot] = r.e;
        if (lane == 0) rt.active[0] = __popcll(r.firsts);
    }
}

// Workgroup 0's wavefront 0 writes the bucket as the bucket kernel would.
__device__ inline void route1_write_bucket(const Route1 &rt, const Route1Lane &r, int K, int lane) {
    const int E = rt.n_experts;
    for (int e0 = 0; e0 <= E; e0 += kWave) {
        const int e = e0 + lane;
        int below = 0, c = 0;
        for (int j = 0; j < K; ++j) {
            const int ej = __builtin_amdgcn_readlane(r.e, j);
            if ((unsigned)ej < (unsigned)E) {
                below += ej < e ? 1 : 0;
                c += ej == e ? 1 : 0;
            }
        }
        if (e < E) rt.counts[e] = c;
        if (e <= E) rt.offsets[e] = below;
    }
    if (r.valid) rt.perm[r.pos] = lane;
    if (lane < K) rt.inv[lane] = r.valid ? r.pos : -1;
    if (r.first) rt.active[1 + r.slot] = r.e;
    if (lane == 0) rt.active[0] = __popcll(r.firsts);
}

__device__ inline uint4 load16(const uint8_t *p) { return *(const uint4 *)p; }

// Buffer resources: a wave-uniform base and byte range in SGPRs. A buffer load
// adds a per-lane VGPR offset and a wave-uniform SGPR offset, so per-row address
// arithmetic stays on the scalar unit, and any byte past the range reads as 0.
// 0x00020000 is the resource word-3 value for raw (untyped) access on gfx9-class
// parts.
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ inline rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ inline uint4 buf_load16(rsrc_t r, uint32_t voff, uint32_t soff) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ inline uint32_t buf_load8(rsrc_t r, uint32_t voff, uint32_t soff) {
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, (int)voff, (int)soff, 0);
}

__device__ inline uint32_t buf_load_u16(rsrc_t r, uint32_t voff, uint32_t soff) {
    return (uint32_t)(uint16_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)voff, (int)soff, 0);
}

// ---- LDS DMA ----------------------------------------------------------------------

__device__ inline uint32_t lds_addr(const void *p) {
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void *)p);
}

// Global -> LDS without registers: lane l's 16 (or 4) bytes from base + voff
// land at `lds` + 16*l (or 4*l). `base` is wave-uniform (SGPRs). The loads are
// inline assembly so that the compiler does not wait for them before every
// LDS read; the kernel waits with s_waitcnt vmcnt itself.
__device__ inline void dma16(const void *base, uint32_t voff, uint32_t lds) {
    lds = __builtin_amdgcn_readfirstlane(lds);
    __asm__ volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(base), "s"(lds)
                     : "m0");
}
__device__ inline void dma4(const void *base, uint32_t voff, uint32_t lds) {
    lds = __builtin_amdgcn_readfirstlane(lds);
    __asm__ volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" : : "v"(voff), "s"(base), "s"(lds)
                     : "m0");
}

// Row-friendly operand loads: for a 16-row x 64-byte matrix-core operand
// (16 bytes a lane), lane 4r + q reads bytes [16q, 16q + 16) of row r, so
// each four lanes take 64 contiguous bytes of one row (the L2 serves that
// several times faster than 16 rows in consecutive lanes). The instruction
// wants row r, quarter q in lane r + 16q; ds_bpermute brings it from lane
// 4r + q, whose byte address is psrc = 4 * (4 * (lane % 16) + lane / 16).
__device__ inline uint4 to_operand(uint4 a, int psrc) {
    return make_uint4((uint32_t)__builtin_amdgcn_ds_bpermute(psrc, (int)a.x),
                      (uint32_t)__builtin_amdgcn_ds_bpermute(psrc, (int)a.y),
                      (uint32_t)__builtin_amdgcn_ds_bpermute(psrc, (int)a.z),
                      (uint32_t)__builtin_amdgcn_ds_bpermute(psrc, (int)a.w));
}

template <int N>
__device__ inline void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __asm__ volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

}  // namespace k3g
