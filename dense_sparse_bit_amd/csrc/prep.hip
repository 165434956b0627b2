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
// a0: h_k = fp32( sum_{m ascending} x_mk^2 / M ). One thread per channel; a
// wavefront reads 64 consecutive channels of a token row per step (coalesced).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_hessian(const void* __restrict__ x, int bf16, int64_t M,
                                                 int64_t K, float* __restrict__ h) {
    const int64_t k = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (k >= K) return;
    double acc = 0.0;
    int64_t m = 0;
    // four independent loads in flight per step; the additions stay in order
    for (; m + 4 <= M; m += 4) {
        const double v0 = load_x(x, bf16, (m + 0) * K + k);
        const double v1 = load_x(x, bf16, (m + 1) * K + k);
        const double v2 = load_x(x, bf16, (m + 2) * K + k);
        const double v3 = load_x(x, bf16, (m + 3) * K + k);
        acc = acc + v0 * v0;
        acc = acc + v1 * v1;
        acc = acc + v2 * v2;
        acc = acc + v3 * v3;
    }
    for (; m < M; ++m) {
        const double v = load_x(x, bf16, m * K + k);
        acc = acc + v * v;
    }
    h[k] = static_cast<float>(acc / static_cast<double>(M));
}

// ---------------------------------------------------------------------------
// a4: per-token symmetric int4 quantization. One workgroup per token: an exact
// max-reduction of |x| (order-free), then each thread packs pairs of codes.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_quant_act(const void* __restrict__ x, int bf16, int64_t K,
                                                   uint8_t* __restrict__ xq, float* __restrict__ sx) {
    const int64_t m = blockIdx.x;
    __shared__ float red[4];
    float a = 0.0f;
    for (int64_t k = threadIdx.x; k < K; k += blockDim.x) a = fmaxf(a, fabsf(load_x(x, bf16, m * K + k)));
    for (int off = 32; off > 0; off >>= 1) a = fmaxf(a, __shfl_xor(a, off));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
    __syncthreads();
    a = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float s = a / 7.0f;
    if (threadIdx.x == 0) sx[m] = s;
    for (int64_t j = threadIdx.x; j < K / 2; j += blockDim.x) {
        const int q0 = rtn_code(load_x(x, bf16, m * K + 2 * j), s);
        const int q1 = rtn_code(load_x(x, bf16, m * K + 2 * j + 1), s);
        xq[m * (K / 2) + j] = static_cast<uint8_t>((q0 & 15) | ((q1 & 15) << 4));
    }
}

// ---------------------------------------------------------------------------
// a2 (part 1): Delta-score. One workgroup per (block row, group); the group's
// bn x 128 weights are staged in LDS once (coalesced rows of 512 B) and both
// 64-wide blocks of the group are scored from there:
//   row_sum(n) = sum_{k ascending} h_k * (E^2 - E'^2),  Delta = sum_{n ascending} row_sum(n)
// ---------------------------------------------------------------------------
constexpr int kTileStride = kGroup + 1;   // +1 float: consecutive rows start in different banks
constexpr int kTileRows = 64;             // rows staged per pass (bn = 128 takes two passes)

__global__ __launch_bounds__(256) void k_delta(const float* __restrict__ w, const float* __restrict__ h,
                                               int64_t K, int bn, double* __restrict__ delta) {
    __shared__ float tile[kTileRows * kTileStride];
    __shared__ float hs[kGroup];
    __shared__ double rowsum[2][128];
    const int64_t br = blockIdx.x, g = blockIdx.y;
    const int64_t nbc = K / kBk;
    if (threadIdx.x < kGroup) hs[threadIdx.x] = h[g * kGroup + threadIdx.x];
    for (int r0 = 0; r0 < bn; r0 += kTileRows) {
        const float* src = w + (br * bn + r0) * K + g * kGroup;
        __syncthreads();
        // stage 64 rows x 128 floats; each pass of the loop moves 8 rows of 32 float4
        for (int idx = threadIdx.x; idx < kTileRows * (kGroup / 4); idx += blockDim.x) {
            const int row = idx / (kGroup / 4), c4 = idx % (kGroup / 4);
            const float4 v = *reinterpret_cast<const float4*>(src + row * K + c4 * 4);
            float* d = tile + row * kTileStride + c4 * 4;
            d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
        }
        __syncthreads();
        // one chain per (row, block half)
        const int t = threadIdx.x;
        if (t < 2 * kTileRows) {
            const int row = t >> 1, half = t & 1;
            const float* r = tile + row * kTileStride;
            float a = 0.0f;
            for (int c = 0; c < kGroup; ++c) a = fmaxf(a, fabsf(r[c]));
            const float s = f16_bits_to_f32(f32_to_f16_bits(a / 7.0f));
            double acc = 0.0;
            for (int c = half * kBk; c < (half + 1) * kBk; ++c) {
                const Elem o = quant_elem(r[c], s);
                const double e = o.e, ep = o.ep;
                const double reduction = e * e - ep * ep;
                acc = acc + static_cast<double>(hs[c]) * reduction;
            }
            rowsum[half][r0 + row] = acc;
        }
    }
    __syncthreads();
    if (threadIdx.x < 2) {
        const int half = threadIdx.x;
        double total = 0.0;
        for (int row = 0; row < bn; ++row) total = total + rowsum[half][row];
        delta[br * nbc + 2 * g + half] = total;
    }
}

// ---------------------------------------------------------------------------
// a2 (part 2): rank of every block under (Delta descending, id ascending);
// chosen iff rank < k_blocks. Each thread compares its score with all NB scores,
// streamed through LDS in tiles. Exact for any ties; O(NB^2 / threads).
// ---------------------------------------------------------------------------
constexpr int kRankTile = 1024;

__global__ __launch_bounds__(256) void k_rank(const double* __restrict__ delta, int64_t nb,
                                              int64_t k_blocks, uint8_t* __restrict__ sel) {
    __shared__ double tile[kRankTile];
    const int64_t b = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const double d = b < nb ? delta[b] : 0.0;
    int64_t rank = 0;
    for (int64_t base = 0; base < nb; base += kRankTile) {
        __syncthreads();
        for (int i = threadIdx.x; i < kRankTile; i += blockDim.x)
            tile[i] = base + i < nb ? delta[base + i] : -1.0;    // scores are >= 0
        __syncthreads();
        const int lim = static_cast<int>(nb - base < kRankTile ? nb - base : kRankTile);
        int cnt = 0;
        for (int i = 0; i < lim; ++i) {
            const double o = tile[i];
            cnt += (o > d) || (o == d && base + i < b);
        }
        rank += cnt;
    }
    if (b < nb) sel[b] = rank < k_blocks ? 1 : 0;
}

// ---------------------------------------------------------------------------
// a2 (part 3): CSR of the chosen blocks in id order (= block row, then column
// block ascending). One workgroup scans the flags.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void k_csr(const uint8_t* __restrict__ sel, int64_t nb, int64_t nbc,
                                              int64_t nbr, int64_t k_blocks, int32_t* __restrict__ row_ptr,
                                              int32_t* __restrict__ col_idx) {
    __shared__ int wsum[16];
    __shared__ int carry_s;
    if (threadIdx.x == 0) carry_s = 0;
    __syncthreads();
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    for (int64_t base = 0; base < nb; base += blockDim.x) {
        const int64_t id = base + threadIdx.x;
        const int f = id < nb ? sel[id] : 0;
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
// a1 + a3: pack. One wavefront per (row n, group g): lane l holds k = 2l, 2l+1
// of the group. The wave writes 64 bytes of base codes and the fp16 scale; if a
// block of this (block row, group) is in the CSR list, the 32 lanes covering it
// write that row of its residual payload (32 bytes). W is read exactly once.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int find_block(const int32_t* __restrict__ col_idx, int lo, int hi, int kb) {
    // first index in [lo, hi) whose column block is >= kb (lists are ascending)
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (col_idx[mid] < kb) lo = mid + 1; else hi = mid;
    }
    return lo;
}

__global__ __launch_bounds__(256) void k_pack(const float* __restrict__ w, int64_t N, int64_t K, int bn,
                                              const int32_t* __restrict__ row_ptr,
                                              const int32_t* __restrict__ col_idx, int64_t nnz,
                                              uint8_t* __restrict__ wq, uint16_t* __restrict__ sw,
                                              uint8_t* __restrict__ rq) {
    const int64_t G = K / kGroup;
    const int64_t wave_id = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
    if (wave_id >= N * G) return;
    const int lane = threadIdx.x & 63;
    const int64_t n = wave_id / G, g = wave_id % G;
    const float2 v = *reinterpret_cast<const float2*>(w + n * K + g * kGroup + 2 * lane);
    float a = fmaxf(fabsf(v.x), fabsf(v.y));
    for (int off = 32; off > 0; off >>= 1) a = fmaxf(a, __shfl_xor(a, off));
    const uint16_t sb = f32_to_f16_bits(a / 7.0f);
    const float s = f16_bits_to_f32(sb);
    const Elem e0 = quant_elem(v.x, s), e1 = quant_elem(v.y, s);
    wq[n * (K / 2) + g * (kGroup / 2) + lane] = static_cast<uint8_t>((e0.q & 15) | ((e1.q & 15) << 4));
    if (lane == 0) sw[n * G + g] = sb;
    if (nnz == 0) return;
    const int64_t br = n / bn;
    const int lo = clampi(row_ptr[br], 0, static_cast<int>(nnz));
    const int hi = clampi(row_ptr[br + 1], lo, static_cast<int>(nnz));
    const int half = lane >> 5;
    const int kb = static_cast<int>(2 * g + half);
    const int p = find_block(col_idx, lo, hi, kb);
    if (p < hi && col_idx[p] == kb)
        rq[(static_cast<int64_t>(p) * bn + (n - br * bn)) * (kBk / 2) + (lane & 31)] =
            static_cast<uint8_t>((e0.r & 15) | ((e1.r & 15) << 4));
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_hessian(const void* x, int bf16, int64_t M, int64_t K, float* h, hipStream_t st) {
    const int64_t blocks = (K + 255) / 256;
    k_hessian<<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st>>>(x, bf16, M, K, h);
    return hipGetLastError();
}

hipError_t launch_quant_act(const void* x, int bf16, int64_t M, int64_t K, uint8_t* xq, float* sx,
                            hipStream_t st) {
    k_quant_act<<<dim3(static_cast<unsigned>(M)), dim3(256), 0, st>>>(x, bf16, K, xq, sx);
    return hipGetLastError();
}

hipError_t launch_select(const float* w, const float* h, int64_t N, int64_t K, int bn,
                         int64_t k_blocks, int32_t* row_ptr, int32_t* col_idx, double* delta,
                         hipStream_t st) {
    const int64_t nbr = N / bn, nbc = K / kBk, nb = nbr * nbc;
    k_delta<<<dim3(static_cast<unsigned>(nbr), static_cast<unsigned>(K / kGroup)), dim3(256), 0, st>>>(
        w, h, K, bn, delta);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    uint8_t* sel = nullptr;
    err = hipMallocAsync(reinterpret_cast<void**>(&sel), static_cast<size_t>(nb), st);
    if (err != hipSuccess) return err;
    k_rank<<<dim3(static_cast<unsigned>((nb + 255) / 256)), dim3(256), 0, st>>>(delta, nb, k_blocks, sel);
    err = hipGetLastError();
    if (err == hipSuccess) {
        k_csr<<<dim3(1), dim3(1024), 0, st>>>(sel, nb, nbc, nbr, k_blocks, row_ptr, col_idx);
        err = hipGetLastError();
    }
    const hipError_t ferr = hipFreeAsync(sel, st);
    return err != hipSuccess ? err : ferr;
}

hipError_t launch_pack(const float* w, int64_t N, int64_t K, int bn, const int32_t* row_ptr,
                       const int32_t* col_idx, int64_t nnz, uint8_t* wq, uint16_t* sw, uint8_t* rq,
                       hipStream_t st) {
    const int64_t waves = N * (K / kGroup);
    const int64_t blocks = (waves + 3) / 4;
    k_pack<<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st>>>(w, N, K, bn, row_ptr, col_idx, nnz,
                                                                      wq, sw, rq);
    return hipGetLastError();
}

}  // namespace mq
