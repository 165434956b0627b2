// Per-token symmetric int4 activation quantization (the W4A4 setting of the
// MosaicQuant summary's Experimental Results; a stage of the ZipperEngine
// pipeline in its Methodology 3), as a workgroup-level device function shared by
// the stand-alone quantization kernel and the GEMM that quantizes its own
// activations:
//   sx[m] = fp32(max_k |x[m][k]| / 7),  code = sx == 0 ? 0 : clamp(rint(x / sx), -7, 7)
// with the correctly rounded division's result, ties to even.
#pragma once

#include "mq_device.h"

namespace mq {

constexpr int kQaWords = 4;      // words kept in registers per thread
constexpr int kQaMaxWaves = 16;  // workgroups of up to 1024 threads

__device__ __forceinline__ void load8(const void* row, bool bf16, int64_t j, float (&v)[8],
                                      const float* __restrict__ colscale) {
#pragma clang fp contract(off)
    if (bf16) {
        const uint4 u = static_cast<const uint4*>(row)[j];
        const uint32_t p[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(p[i] << 16);
            v[2 * i + 1] = __uint_as_float(p[i] & 0xffff0000u);
        }
    } else {
        const float4 a = static_cast<const float4*>(row)[2 * j];
        const float4 b = static_cast<const float4*>(row)[2 * j + 1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
    // migrated activations: x^ = fp32(x * r_k), one rounding per element
    if (colscale) {
        const float4 a = reinterpret_cast<const float4*>(colscale)[2 * j];
        const float4 b = reinterpret_cast<const float4*>(colscale)[2 * j + 1];
        v[0] = v[0] * a.x; v[1] = v[1] * a.y; v[2] = v[2] * a.z; v[3] = v[3] * a.w;
        v[4] = v[4] * b.x; v[5] = v[5] * b.y; v[6] = v[6] * b.z; v[7] = v[7] * b.w;
    }
}

// Quantizes token m with the calling workgroup (nt threads, a multiple of 64, at
// most 64 * kQaMaxWaves; t = this thread). Each thread owns code words (8
// consecutive inputs each) and keeps the first kQaWords of them in registers
// between the exact max-reduction of |x| (order-free) and the quantization, so x
// is read once for K <= 8 * kQaWords * nt. Words are stored group-major
// ([K/128][M][64 B]), the layout the GEMM loads from. red: kQaMaxWaves floats of
// LDS. Contains workgroup barriers: every thread of the workgroup must call it.
__device__ __forceinline__ void quant_act_row(const void* __restrict__ x, int bf16, int64_t M, int64_t K,
                                              const float* __restrict__ colscale, uint8_t* __restrict__ xq,
                                              float* __restrict__ sx, int64_t m, int t, int nt, float* red) {
#pragma clang fp contract(off)
    const int64_t W = K / 8;
    const int nw = nt >> 6;
    const void* row = bf16 ? static_cast<const void*>(static_cast<const uint16_t*>(x) + m * K)
                           : static_cast<const void*>(static_cast<const float*>(x) + m * K);
    // The words kept in registers: every load is issued before the first is used
    // (a load under a per-word branch would be waited for before the next word's
    // went out). A word past the row reads the row's last word and is zeroed.
    float v[kQaWords][8];
    float a = 0.0f;
    if (bf16) {
        uint4 raw[kQaWords];
#pragma unroll
        for (int i = 0; i < kQaWords; ++i)
            raw[i] = static_cast<const uint4*>(row)[min(t + static_cast<int64_t>(nt) * i, W - 1)];
        __builtin_amdgcn_sched_barrier(0);   // all loads out before the first use
#pragma unroll
        for (int i = 0; i < kQaWords; ++i) {
            const uint32_t p[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[i][2 * e] = __uint_as_float(p[e] << 16);
                v[i][2 * e + 1] = __uint_as_float(p[e] & 0xffff0000u);
            }
        }
    } else {
        float4 ra[kQaWords], rb[kQaWords];
#pragma unroll
        for (int i = 0; i < kQaWords; ++i) {
            const int64_t jc = min(t + static_cast<int64_t>(nt) * i, W - 1);
            ra[i] = static_cast<const float4*>(row)[2 * jc];
            rb[i] = static_cast<const float4*>(row)[2 * jc + 1];
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < kQaWords; ++i) {
            v[i][0] = ra[i].x; v[i][1] = ra[i].y; v[i][2] = ra[i].z; v[i][3] = ra[i].w;
            v[i][4] = rb[i].x; v[i][5] = rb[i].y; v[i][6] = rb[i].z; v[i][7] = rb[i].w;
        }
    }
    // migrated activations: x^ = fp32(x * r_k), one rounding per element
    if (colscale) {
        float4 ca[kQaWords], cb[kQaWords];
#pragma unroll
        for (int i = 0; i < kQaWords; ++i) {
            const int64_t jc = min(t + static_cast<int64_t>(nt) * i, W - 1);
            ca[i] = reinterpret_cast<const float4*>(colscale)[2 * jc];
            cb[i] = reinterpret_cast<const float4*>(colscale)[2 * jc + 1];
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < kQaWords; ++i) {
            v[i][0] = v[i][0] * ca[i].x; v[i][1] = v[i][1] * ca[i].y;
            v[i][2] = v[i][2] * ca[i].z; v[i][3] = v[i][3] * ca[i].w;
            v[i][4] = v[i][4] * cb[i].x; v[i][5] = v[i][5] * cb[i].y;
            v[i][6] = v[i][6] * cb[i].z; v[i][7] = v[i][7] * cb[i].w;
        }
    }
#pragma unroll
    for (int i = 0; i < kQaWords; ++i) {
        const bool in = t + static_cast<int64_t>(nt) * i < W;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            v[i][e] = in ? v[i][e] : 0.0f;
            a = fmaxf(a, fabsf(v[i][e]));
        }
    }
    for (int64_t j = t + static_cast<int64_t>(nt) * kQaWords; j < W; j += nt) {
        float u[8];
        load8(row, bf16, j, u, colscale);
#pragma unroll
        for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf(u[e]));
    }
    for (int off = 32; off > 0; off >>= 1) a = fmaxf(a, __shfl_xor(a, off));
    if ((t & 63) == 0) red[t >> 6] = a;
    __syncthreads();
    a = red[0];
    for (int w = 1; w < nw; ++w) a = fmaxf(a, red[w]);
    const float s = a / 7.0f;
    const float rs = s == 0.0f ? 0.0f : 1.0f / s;
    if (t == 0) sx[m] = s;
    // group-major output: word j (inputs 8j..8j+7) is bytes 4(j%16).. of group j/16's chunk
    auto dst = [&](int64_t j) { return reinterpret_cast<uint32_t*>(xq + xq_row(j >> 4, M, m) + (j & 15) * 4); };
    // Branch-free codes for the values held in registers. A word with a quotient
    // within 4e-6 of a rounding boundary (or every word, when 1/s is not finite:
    // the products are then infinite or NaN and flag themselves) is marked in
    // `near` and recoded exactly from the values still in its registers (a value
    // that was not near a boundary gets the same code either way).
    uint32_t nib[kQaWords];
    uint32_t near = 0;
#pragma unroll
    for (int i = 0; i < kQaWords; ++i) {
        float worst = 0.0f;
        nib[i] = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            nib[i] |= (static_cast<uint32_t>(static_cast<int>(rtn_fast(v[i][e], rs, worst))) & 15u) << (4 * e);
        near |= static_cast<uint32_t>(!(worst < kFastMargin)) << i;
    }
    if (!(fabsf(rs) <= 3.0e38f)) near = (1u << kQaWords) - 1u;
    if (near) {
#pragma unroll
        for (int i = 0; i < kQaWords; ++i)
            if ((near >> i) & 1u) {
                nib[i] = 0;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    nib[i] |= (static_cast<uint32_t>(static_cast<int>(rtn_codef(v[i][e], s, rs))) & 15u) << (4 * e);
            }
    }
#pragma unroll
    for (int i = 0; i < kQaWords; ++i) {
        const int64_t j = t + static_cast<int64_t>(nt) * i;
        if (j < W) *dst(j) = code_word(nib[i]);
    }
    for (int64_t j = t + static_cast<int64_t>(nt) * kQaWords; j < W; j += nt) {
        float u[8];
        load8(row, bf16, j, u, colscale);
        uint32_t n8 = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) n8 |= (static_cast<uint32_t>(static_cast<int>(rtn_codef(u[e], s, rs))) & 15u) << (4 * e);
        *dst(j) = code_word(n8);
    }
}

}  // namespace mq
