// Offline and per-call preparation kernels of the MosaicQuant path (gfx950).
//
//   a0  k_hessian       diagonal-Hessian estimate h_k (Methodology 2)
//   a4  k_quant_act     per-token int4 activation quantization (W4A4)
//   a2  k_delta         Hessian-guided Delta-score of every residual block
//       k_rank / k_csr  global top-K selection and its CSR block lists
//   a1+a3 k_pack        dense 4-bit base + residual payload of chosen blocks
//
// Citations are to the MosaicQuant technical summary on gist.science
// ("MosaicQuant: Inlier-Outlier Disaggregation for Unified 4-Bit LLM
// Quantization"), sections Methodology 1-3 and Experimental Results.
//
// This file is compiled with -ffp-contract=off: every fp32/fp64 operation is
// rounded on its own, in the order written, so codes, scales and scores are
// bit-identical to the plain CPU definition.
#include "mq_device.h"
#include "mq_internal.h"

namespace mq {

// ---------------------------------------------------------------------------
// a0: h_k = fp32( sum_{m ascending} x_mk^2 / M ). A workgroup owns 64 channels:
// all 256 threads stage 128-token slabs of those channels in LDS (every load of
// a slab in flight at once), then one thread per channel adds its column in
// token order.
// ---------------------------------------------------------------------------
constexpr int kHCh = 64, kHRows = 128;

__global__ __launch_bounds__(256) void k_hessian(const void* __restrict__ x, int bf16, int64_t M,
                                                 int64_t K, float* __restrict__ h) {
    __shared__ float tile[kHRows][kHCh + 1];
    const int64_t k0 = static_cast<int64_t>(blockIdx.x) * kHCh;
    const int t = threadIdx.x;
    double acc = 0.0;
    for (int64_t m0 = 0; m0 < M; m0 += kHRows) {
        const int rows = static_cast<int>(M - m0 < kHRows ? M - m0 : kHRows);
        float v[kHRows * kHCh / 256];
#pragma unroll
        for (int i = 0; i < kHRows * kHCh / 256; ++i) {
            const int idx = t + 256 * i, r = idx / kHCh, c = idx % kHCh;
            v[i] = (r < rows && k0 + c < K) ? load_x(x, bf16, (m0 + r) * K + k0 + c) : 0.0f;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kHRows * kHCh / 256; ++i) {
            const int idx = t + 256 * i;
            tile[idx / kHCh][idx % kHCh] = v[i];
        }
        __syncthreads();
        if (t < kHCh)
            for (int r = 0; r < rows; ++r) {
                const double d = tile[r][t];
                acc = acc + d * d;
            }
    }
    if (t < kHCh && k0 + t < K) h[k0 + t] = static_cast<float>(acc / static_cast<double>(M));
}

// ---------------------------------------------------------------------------
// a4: per-token symmetric int4 quantization. One workgroup per token; each
// thread keeps its pairs of values in registers between the exact max-reduction
// of |x| (order-free) and the quantization, so x is read once. Codes are stored
// group-major ([K/128][M][64 B]), the layout the GEMM loads from.
// ---------------------------------------------------------------------------
constexpr int kQaRegs = 16;     // pairs kept in registers per thread (K <= 8192 read once)

__device__ __forceinline__ float2 load_pair(const void* x, bool bf16, int64_t j) {
    if (bf16) {
        const uint32_t u = static_cast<const uint32_t*>(x)[j];
        return make_float2(__uint_as_float(u << 16), __uint_as_float(u & 0xffff0000u));
    }
    return static_cast<const float2*>(x)[j];
}

__global__ __launch_bounds__(256) void k_quant_act(const void* __restrict__ x, int bf16, int64_t M, int64_t K,
                                                   uint8_t* __restrict__ xq, float* __restrict__ sx) {
    const int64_t m = blockIdx.x, P = K / 2;
    const void* row = bf16 ? static_cast<const void*>(static_cast<const uint16_t*>(x) + m * K)
                           : static_cast<const void*>(static_cast<const float*>(x) + m * K);
    const int t = threadIdx.x;
    __shared__ float red[4];
    float2 v[kQaRegs];
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < kQaRegs; ++i) {
        const int64_t j = t + 256 * i;
        v[i] = j < P ? load_pair(row, bf16, j) : make_float2(0.0f, 0.0f);
        a = fmaxf(a, fmaxf(fabsf(v[i].x), fabsf(v[i].y)));
    }
    for (int64_t j = t + 256 * kQaRegs; j < P; j += 256) {
        const float2 u = load_pair(row, bf16, j);
        a = fmaxf(a, fmaxf(fabsf(u.x), fabsf(u.y)));
    }
    for (int off = 32; off > 0; off >>= 1) a = fmaxf(a, __shfl_xor(a, off));
    if ((t & 63) == 0) red[t >> 6] = a;
    __syncthreads();
    a = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float s = a / 7.0f;
    const float rs = s == 0.0f ? 0.0f : 1.0f / s;
    if (t == 0) sx[m] = s;
    // group-major output: byte j of the row (inputs 2j, 2j+1) goes to group j/64
    auto code = [&](float v) { return static_cast<int>(rtn_codef(v, s, rs)) & 15; };
    auto dst = [&](int64_t j) { return xq + xq_row(j >> 6, M, m) + (j & 63); };
#pragma unroll
    for (int i = 0; i < kQaRegs; ++i) {
        const int64_t j = t + 256 * i;
        if (j < P) *dst(j) = static_cast<uint8_t>(code(v[i].x) | (code(v[i].y) << 4));
    }
    for (int64_t j = t + 256 * kQaRegs; j < P; j += 256) {
        const float2 u = load_pair(row, bf16, j);
        *dst(j) = static_cast<uint8_t>(code(u.x) | (code(u.y) << 4));
    }
}

// ---------------------------------------------------------------------------
// a2 (part 1): Delta-score. One workgroup per (block row, two groups); a lane
// owns one (group, row, block) chain: it loads the row's 64 weights of that block
// (sixteen 16-byte loads, all in flight together), takes the group max with its
// partner lane (exact), and adds its 64 terms h_k * (E^2 - E'^2) strictly in
// column order. Block score = sum over the block's rows in ascending order.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_delta(const float* __restrict__ w, const float* __restrict__ h,
                                               int64_t K, int bn, double* __restrict__ delta,
                                               int32_t* __restrict__ rank) {
    __shared__ float hs[2][kGroup];
    __shared__ double rowsum[2][2][128];
    const int64_t G = K / kGroup, nbc = K / kBk;
    const int t = threadIdx.x, gsel = t >> 7, row = (t & 127) >> 1, half = t & 1;
    const int64_t br = blockIdx.x, g = 2 * static_cast<int64_t>(blockIdx.y) + gsel;
    const bool valid = g < G;                        // uniform per wavefront
    hs[gsel][t & 127] = valid ? h[g * kGroup + (t & 127)] : 0.0f;
    __syncthreads();
    const float* hrow = hs[gsel] + half * kBk;
    for (int r0 = 0; r0 < bn; r0 += 64) {
        if (valid) {
            const float* src = w + (br * bn + r0 + row) * K + g * kGroup + half * kBk;
            float wv[kBk];
#pragma unroll
            for (int i = 0; i < kBk / 4; ++i) {
                const float4 u = *reinterpret_cast<const float4*>(src + 4 * i);
                wv[4 * i] = u.x; wv[4 * i + 1] = u.y; wv[4 * i + 2] = u.z; wv[4 * i + 3] = u.w;
            }
            float a = 0.0f;
#pragma unroll
            for (int i = 0; i < kBk; ++i) a = fmaxf(a, fabsf(wv[i]));
            a = fmaxf(a, __shfl_xor(a, 1));
            const GroupScale gs = group_scale(f16_bits_to_f32(f32_to_f16_bits(a / 7.0f)));
            double acc = 0.0;
#pragma unroll
            for (int i0 = 0; i0 < kBk; i0 += 8) {
                // bounded scheduling window: keeps the live range of the
                // per-element temporaries short (no spills)
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = i0; i < i0 + 8; ++i) {
                    const Elem o = quant_elem(wv[i], gs);
                    const double e = o.e, ep = o.ep;
                    const double reduction = e * e - ep * ep;
                    acc = acc + static_cast<double>(hrow[i]) * reduction;
                }
            }
            rowsum[gsel][half][r0 + row] = acc;
        }
    }
    __syncthreads();
    if (t < 4) {
        const int gs2 = t >> 1, hf = t & 1;
        const int64_t gg = 2 * static_cast<int64_t>(blockIdx.y) + gs2;
        if (gg < G) {
            double total = 0.0;
            for (int r = 0; r < bn; ++r) total = total + rowsum[gs2][hf][r];
            delta[br * nbc + 2 * gg + hf] = total;
            rank[br * nbc + 2 * gg + hf] = 0;     // counters for the ranking pass
        }
    }
}

// ---------------------------------------------------------------------------
// a2 (part 2): rank of every block under (Delta descending, id ascending),
// counted over a 2-D grid: workgroup (i, j) compares 256 blocks with a slice of
// 256 scores staged in LDS and adds its counts into rank[]. Exact for any ties.
// ---------------------------------------------------------------------------
constexpr int kRankSlice = 256;

__global__ __launch_bounds__(256) void k_rank(const double* __restrict__ delta, int64_t nb,
                                              int32_t* __restrict__ rank) {
    __shared__ __align__(16) double tile[kRankSlice];
    const int64_t b = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t j0 = static_cast<int64_t>(blockIdx.y) * kRankSlice;
    if (j0 + threadIdx.x < nb) tile[threadIdx.x] = delta[j0 + threadIdx.x];
    __syncthreads();
    if (b >= nb) return;
    const double d = delta[b];
    const int lim = static_cast<int>(nb - j0 < kRankSlice ? nb - j0 : kRankSlice);
    // entries of this slice that precede b in id order win ties
    const int64_t before64 = b - j0;
    const int before = before64 < 0 ? 0 : (before64 > kRankSlice ? kRankSlice : static_cast<int>(before64));
    int cnt = 0;
    if (lim == kRankSlice) {
#pragma unroll 8
        for (int i = 0; i < kRankSlice; i += 2) {
            const double2 o = *reinterpret_cast<const double2*>(tile + i);
            cnt += static_cast<int>(o.x > d) + (static_cast<int>(o.x == d) & static_cast<int>(i < before));
            cnt += static_cast<int>(o.y > d) + (static_cast<int>(o.y == d) & static_cast<int>(i + 1 < before));
        }
    } else {
        for (int i = 0; i < lim; ++i) {
            const double o = tile[i];
            cnt += static_cast<int>(o > d) + (static_cast<int>(o == d) & static_cast<int>(i < before));
        }
    }
    if (cnt) atomicAdd(rank + b, cnt);
}

// ---------------------------------------------------------------------------
// a2 (part 3): CSR of the chosen blocks (rank < k_blocks) in id order, i.e. block
// row, then column block ascending. One workgroup scans the flags.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void k_csr(const int32_t* __restrict__ rank, int64_t nb, int64_t nbc,
                                              int64_t nbr, int64_t k_blocks, int32_t* __restrict__ row_ptr,
                                              int32_t* __restrict__ col_idx) {
    __shared__ int wsum[16];
    __shared__ int carry_s;
    if (threadIdx.x == 0) carry_s = 0;
    __syncthreads();
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    // flags of the first 32 passes are loaded up front (independent loads)
    constexpr int kPre = 32;
    uint32_t pre = 0;
#pragma unroll
    for (int i = 0; i < kPre; ++i) {
        const int64_t id = static_cast<int64_t>(i) * blockDim.x + threadIdx.x;
        if (id < nb && rank[id] < k_blocks) pre |= 1u << i;
    }
    int pass = 0;
    for (int64_t base = 0; base < nb; base += blockDim.x, ++pass) {
        const int64_t id = base + threadIdx.x;
        const int f = id < nb ? (pass < kPre ? static_cast<int>((pre >> pass) & 1u) : (rank[id] < k_blocks)) : 0;
        // inclusive scan inside the wavefront
        int v = f;
        for (int off = 1; off < 64; off <<= 1) {
            const int u = __shfl_up(v, off);
            if (lane >= off) v += u;
        }
        if (lane == 63) wsum[wv] = v;
        __syncthreads();
        int before = carry_s;
        for (int i = 0; i < wv; ++i) before += wsum[i];
        const int excl = before + v - f;
        if (id < nb) {
            if (id % nbc == 0) row_ptr[id / nbc] = excl;
            // ranks form a permutation, so exactly k_blocks flags are set; the
            // bound only matters for non-finite scores (unsupported inputs)
            if (f && excl < k_blocks) col_idx[excl] = static_cast<int32_t>(id % nbc);
        }
        __syncthreads();
        if (threadIdx.x == blockDim.x - 1) carry_s = excl + f;
        __syncthreads();
    }
    if (threadIdx.x == 0) row_ptr[nbr] = carry_s;
}

// ---------------------------------------------------------------------------
// a1 + a3: pack. One workgroup per (block row, group), 64 rows per pass, four
// lanes per row with 32 weights each (eight 16-byte loads, one 16-byte store of
// codes into the tiled wq layout). The block row's CSR list is searched once, in
// parallel, for the two column blocks of the group; chosen blocks get their
// 16-byte residual rows written at their CSR position. W is read exactly once.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t pack8(const int* c) {
    uint32_t v = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) v |= static_cast<uint32_t>(c[i] & 15) << (4 * i);
    return v;
}

__global__ __launch_bounds__(256) void k_pack(const float* __restrict__ w, int64_t N, int64_t K, int bn,
                                              const int32_t* __restrict__ row_ptr,
                                              const int32_t* __restrict__ col_idx, int64_t nnz,
                                              uint8_t* __restrict__ wq, uint16_t* __restrict__ sw,
                                              uint8_t* __restrict__ rq) {
    __shared__ int pos[2];
    const int64_t br = blockIdx.x, g = blockIdx.y, G = K / kGroup, G4 = (G + 3) / 4;
    const int t = threadIdx.x, row = t >> 2, qd = t & 3;
    // first 64 rows' weights are requested before the list search, so the two
    // latencies overlap
    float wv0[32];
    {
        const float* src = w + (br * bn + row) * K + g * kGroup + qd * 32;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float4 u = *reinterpret_cast<const float4*>(src + 4 * i);
            wv0[4 * i] = u.x; wv0[4 * i + 1] = u.y; wv0[4 * i + 2] = u.z; wv0[4 * i + 3] = u.w;
        }
    }
    if (t < 2) pos[t] = -1;
    __syncthreads();
    if (nnz > 0) {
        const int lo = clampi(row_ptr[br], 0, static_cast<int>(nnz));
        const int hi = clampi(row_ptr[br + 1], lo, static_cast<int>(nnz));
        for (int i = lo + t; i < hi; i += blockDim.x) {
            const int e = col_idx[i];
            if (e == 2 * g) pos[0] = i;
            else if (e == 2 * g + 1) pos[1] = i;
        }
    }
    __syncthreads();
    const int p = pos[qd >> 1];
    for (int r0 = 0; r0 < bn; r0 += 64) {
        const int64_t n = br * bn + r0 + row;
        float wv[32];
        if (r0 == 0) {
#pragma unroll
            for (int i = 0; i < 32; ++i) wv[i] = wv0[i];
        } else {
            const float* src = w + n * K + g * kGroup + qd * 32;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float4 u = *reinterpret_cast<const float4*>(src + 4 * i);
                wv[4 * i] = u.x; wv[4 * i + 1] = u.y; wv[4 * i + 2] = u.z; wv[4 * i + 3] = u.w;
            }
        }
        float a = 0.0f;
#pragma unroll
        for (int i = 0; i < 32; ++i) a = fmaxf(a, fabsf(wv[i]));
        a = fmaxf(a, __shfl_xor(a, 1));
        a = fmaxf(a, __shfl_xor(a, 2));
        const uint16_t sb = f32_to_f16_bits(a / 7.0f);
        const GroupScale gs = group_scale(f16_bits_to_f32(sb));
        int qc[32], rc[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            const Elem o = quant_elem(wv[i], gs);
            qc[i] = static_cast<int>(o.q);
            rc[i] = static_cast<int>(o.r);
        }
        // tiled base codes: a wavefront's 16 rows x 4 quarters are one 1 KB tile
        *reinterpret_cast<uint4*>(wq + wq_byte(n, G, g, qd)) =
            make_uint4(pack8(qc), pack8(qc + 8), pack8(qc + 16), pack8(qc + 24));
        if (qd == 0) {
            sw[sw_index(n, G4, g)] = sb;
            if (g == G - 1)
                for (int64_t gp = G; gp < 4 * G4; ++gp) sw[sw_index(n, G4, gp)] = 0;   // padding slots
        }
        if (p >= 0)
            *reinterpret_cast<uint4*>(rq + (static_cast<int64_t>(p) * bn + r0 + row) * (kBk / 2) + (qd & 1) * 16) =
                make_uint4(pack8(rc), pack8(rc + 8), pack8(rc + 16), pack8(rc + 24));
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_hessian(const void* x, int bf16, int64_t M, int64_t K, float* h, hipStream_t st) {
    const int64_t blocks = (K + kHCh - 1) / kHCh;
    k_hessian<<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st>>>(x, bf16, M, K, h);
    return hipGetLastError();
}

hipError_t launch_quant_act(const void* x, int bf16, int64_t M, int64_t K, uint8_t* xq, float* sx,
                            hipStream_t st) {
    k_quant_act<<<dim3(static_cast<unsigned>(M)), dim3(256), 0, st>>>(x, bf16, M, K, xq, sx);
    return hipGetLastError();
}

hipError_t launch_select(const float* w, const float* h, int64_t N, int64_t K, int bn,
                         int64_t k_blocks, int32_t* row_ptr, int32_t* col_idx, double* delta,
                         hipStream_t st) {
    const int64_t nbr = N / bn, nbc = K / kBk, nb = nbr * nbc;
    int32_t* rank = nullptr;
    hipError_t err = hipMallocAsync(reinterpret_cast<void**>(&rank), static_cast<size_t>(nb) * sizeof(int32_t), st);
    if (err != hipSuccess) return err;
    k_delta<<<dim3(static_cast<unsigned>(nbr), static_cast<unsigned>((K / kGroup + 1) / 2)), dim3(256), 0, st>>>(
        w, h, K, bn, delta, rank);
    err = hipGetLastError();
    const unsigned nblk = static_cast<unsigned>((nb + 255) / 256);
    if (err == hipSuccess) {
        k_rank<<<dim3(nblk, static_cast<unsigned>((nb + kRankSlice - 1) / kRankSlice)), dim3(256), 0, st>>>(
            delta, nb, rank);
        err = hipGetLastError();
    }
    if (err == hipSuccess) {
        k_csr<<<dim3(1), dim3(1024), 0, st>>>(rank, nb, nbc, nbr, k_blocks, row_ptr, col_idx);
        err = hipGetLastError();
    }
    const hipError_t ferr = hipFreeAsync(rank, st);
    return err != hipSuccess ? err : ferr;
}

hipError_t launch_pack(const float* w, int64_t N, int64_t K, int bn, const int32_t* row_ptr,
                       const int32_t* col_idx, int64_t nnz, uint8_t* wq, uint16_t* sw, uint8_t* rq,
                       hipStream_t st) {
    k_pack<<<dim3(static_cast<unsigned>(N / bn), static_cast<unsigned>(K / kGroup)), dim3(256), 0, st>>>(
        w, N, K, bn, row_ptr, col_idx, nnz, wq, sw, rq);
    return hipGetLastError();
}

}  // namespace mq
