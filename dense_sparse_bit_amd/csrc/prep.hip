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
#include <algorithm>

#include "mq_device.h"
#include "mq_internal.h"
#include "mq_quant.h"

namespace mq {

// native 4-float vector (HIP's float4 is a union struct, which keeps a
// loop-carried array of them in scratch memory)
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// a0: h_k = fp32( sum_{m ascending} x_mk^2 / M ). A workgroup owns 64 channels:
// all 256 threads stage 128-token slabs of those channels in LDS (every load of
// a slab in flight at once), then one thread per channel adds its column in
// token order.
// ---------------------------------------------------------------------------
constexpr int kHCh = 64, kHRows = 128;

__global__ __launch_bounds__(256) void k_hessian(const void* __restrict__ x, int bf16, int64_t M,
                                                 int64_t K, const float* __restrict__ colscale,
                                                 float* __restrict__ h) {
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
            // migrated activations x^ = fp32(x * r_k) (one rounding, as the definition)
            if (colscale && k0 + c < K) v[i] = v[i] * colscale[k0 + c];
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
// a4: per-token symmetric int4 quantization, one workgroup per token (the body
// is quant_act_row in mq_quant.h, shared with the GEMM that quantizes its own
// activations).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64 * kQaMaxWaves) void k_quant_act(const void* __restrict__ x, int bf16, int64_t M, int64_t K,
                                                   const float* __restrict__ colscale,
                                                   uint8_t* __restrict__ xq, float* __restrict__ sx) {
    __shared__ float red[kQaMaxWaves];
    quant_act_row(x, bf16, M, K, colscale, xq, sx, blockIdx.x, threadIdx.x, blockDim.x, red);
}

// ---------------------------------------------------------------------------
// a2 (part 1): Delta-score. A workgroup of two waves owns one group g and walks
// a strided set of block rows (about four workgroups per CU in total); each
// wave owns 32 rows of a block row per pass, and lane l runs the chain of row
// l % 32, column block l / 32 (64 terms h_k * (E^2 - E'^2) strictly in column
// order) after taking the group max with its partner lane (exact).
// The chains need 64 consecutive floats per lane, which direct loads would fetch
// as 64 scattered 16-byte pieces per wave instruction; instead the wave loads its
// 32 x 128 fp32 slab with 1 KB-contiguous instructions (two rows' group chunks)
// and stages it in LDS, swizzled (16-byte slot c of row r at c ^ (r & 7)) so that
// both the stores and the per-lane 16-byte reads are free of bank conflicts. The
// next pass's slab is loaded into registers while the current one is computed.
// A wave only reads rows it wrote itself and its LDS operations complete in issue
// order, so only the per-block row sum needs a workgroup barrier. Block score =
// sum of the block's row chains in ascending row order.
// ---------------------------------------------------------------------------
constexpr int kDeltaRows = 32;                 // rows per wave and pass

// (double)E^2 - (double)E'^2 of 8 elements through rtn_fast, computed stage by
// stage: every stage is 8 independent operations.
__device__ __forceinline__ void quant_reduction8(const float (&w)[8], const GroupScale& g, float& worst,
                                                 double (&red)[8]) {
    float t[8], q[8], e[8], r[8], ep[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = w[i] * g.rs;
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = __builtin_rintf(t[i]);
#pragma unroll
    for (int i = 0; i < 8; ++i) worst = fmaxf(worst, fabsf(t[i] - q[i]));
#pragma unroll
    for (int i = 0; i < 8; ++i) e[i] = __builtin_fmaf(-g.s, fminf(fmaxf(q[i], -7.0f), 7.0f), w[i]);
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = e[i] * g.rsr;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = __builtin_rintf(t[i]);
#pragma unroll
    for (int i = 0; i < 8; ++i) worst = fmaxf(worst, fabsf(t[i] - r[i]));
#pragma unroll
    for (int i = 0; i < 8; ++i) ep[i] = __builtin_fmaf(-g.sr, fminf(fmaxf(r[i], -7.0f), 7.0f), e[i]);
    double de[8], dp[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) de[i] = static_cast<double>(e[i]);
#pragma unroll
    for (int i = 0; i < 8; ++i) dp[i] = static_cast<double>(ep[i]);
#pragma unroll
    for (int i = 0; i < 8; ++i) de[i] = de[i] * de[i];
#pragma unroll
    for (int i = 0; i < 8; ++i) dp[i] = dp[i] * dp[i];
#pragma unroll
    for (int i = 0; i < 8; ++i) red[i] = de[i] - dp[i];
}

__device__ __forceinline__ void delta_load(f32x4 (&v)[kDeltaRows / 2], const float* __restrict__ w, int64_t K,
                                           int64_t row0, int64_t g, int lane) {
#pragma unroll
    for (int i = 0; i < kDeltaRows / 2; ++i) {
        const int r = 2 * i + (lane >> 5);
        v[i] = *reinterpret_cast<const f32x4*>(w + (row0 + r) * K + g * kGroup + (lane & 31) * 4);
    }
}

// LDS allows four workgroups (8 waves) per CU, so 2 waves per SIMD is the real
// occupancy; the attribute lets the prefetched slab stay in registers
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(1, 2)))
void k_delta(const float* __restrict__ w, const float* __restrict__ h,
                                               int64_t K, int bn, int nbr, double* __restrict__ delta,
                                               int32_t* __restrict__ rank) {
    __shared__ __align__(16) f32x4 slab[2][kDeltaRows][32];    // [wave][row][16-byte slot]
    __shared__ double hs[kGroup];
    __shared__ double rowsum[2][128];                          // [column block][row of the block]
    __shared__ double fixbuf[2][kBk];                          // per-wave terms of a repaired chain
    const int64_t nbc = K / kBk;
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const int64_t g = blockIdx.y;
    const int P = gridDim.x, br0 = blockIdx.x;
    hs[t] = static_cast<double>(h[g * kGroup + t]);
    __syncthreads();
    const int crow = lane & 31, half = lane >> 5;              // this lane's chain
    const double* hrow = hs + half * kBk;
    f32x4 (*mine)[32] = slab[wv];
    const int ppu = bn / (2 * kDeltaRows);                     // passes per block row
    const int units = br0 < nbr ? (nbr - br0 + P - 1) / P : 0;
    const int passes = units * ppu;
    // first row of this wave's 32 rows in pass ps
#define MQ_PASS_ROW0(ps) \
    ((br0 + static_cast<int64_t>((ps) / ppu) * P) * bn + ((ps) % ppu) * (2 * kDeltaRows) + wv * kDeltaRows)
    f32x4 v[kDeltaRows / 2];
    if (passes > 0) delta_load(v, w, K, MQ_PASS_ROW0(0), g, lane);
    for (int ps = 0; ps < passes; ++ps) {
#pragma unroll
        for (int i = 0; i < kDeltaRows / 2; ++i) {
            const int r = 2 * i + (lane >> 5);
            mine[r][(lane & 31) ^ (r & 7)] = v[i];
        }
        __builtin_amdgcn_wave_barrier();
        // next pass's slab in flight meanwhile (the last pass reloads its own rows)
        const int nxt = ps + 1 < passes ? ps + 1 : ps;
        delta_load(v, w, K, MQ_PASS_ROW0(nxt), g, lane);
        // two passes over the row in LDS: the group max, then the chain in chunks
        // of 8 values (keeps the registers for the prefetched slab free)
        float a = 0.0f;
#pragma unroll
        for (int j = 0; j < kBk / 4; ++j) {
            const f32x4 u = mine[crow][(half * 16 + j) ^ (crow & 7)];
            a = fmaxf(a, fmaxf(fmaxf(fabsf(u.x), fabsf(u.y)), fmaxf(fabsf(u.z), fabsf(u.w))));
        }
        a = fmaxf(a, __shfl_xor(a, 32));
        const GroupScale gs = group_scale(f16_bits_to_f32(f32_to_f16_bits(a / 7.0f)));
        // branch-free chain; a lane whose quotients came within 4e-6 of a rounding
        // boundary (rare) redoes it with the exact quantizer afterwards
        double acc = 0.0;
        float worst = 0.0f;
#pragma unroll
        for (int i0 = 0; i0 < kBk; i0 += 8) {
            // bounded scheduling window: keeps the live range of the per-element
            // temporaries short (no spills)
            __builtin_amdgcn_sched_barrier(0);
            const f32x4 u0 = mine[crow][(half * 16 + i0 / 4) ^ (crow & 7)];
            const f32x4 u1 = mine[crow][(half * 16 + i0 / 4 + 1) ^ (crow & 7)];
            const float wc[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
            // stage by stage over the 8 elements, so their independent work
            // interleaves (one element at a time is a single dependency chain)
            double red[8];
            quant_reduction8(wc, gs, worst, red);
#pragma unroll
            for (int i = 0; i < 8; ++i) acc = acc + hrow[i0 + i] * red[i];
        }
        const bool redo = !(worst < kFastMargin) || !fast_ok(gs);
        // Rare repair, done by the whole wave: for each flagged chain (lane L) every
        // lane requantizes one of its 64 elements exactly, and lane L adds the 64
        // terms in column order. Same operations and order as the chain itself,
        // so the result is bit-identical; a lane redoing its own chain serially
        // would put ~20k dependent cycles on the workgroup's critical path.
        uint64_t flagged = __ballot(redo);
        while (flagged) {
            const int L = __builtin_ctzll(flagged);
            flagged &= flagged - 1;
            const int lrow = L & 31, lhalf = L >> 5;
            const float ls = __shfl(gs.s, L);
            const GroupScale lg = group_scale(ls);
            const f32x4 u = mine[lrow][(lhalf * 16 + (lane >> 2)) ^ (lrow & 7)];
            const float x = (lane & 3) == 0 ? u.x : (lane & 3) == 1 ? u.y : (lane & 3) == 2 ? u.z : u.w;
            const Elem o = quant_elem(x, lg);
            const double e = o.e, ep = o.ep;
            fixbuf[wv][lane] = hs[lhalf * kBk + lane] * (e * e - ep * ep);
            __builtin_amdgcn_wave_barrier();
            if (lane == L) {
                double a2 = 0.0;
                for (int i = 0; i < kBk; ++i) a2 = a2 + fixbuf[wv][i];
                acc = a2;
            }
            __builtin_amdgcn_wave_barrier();
        }
        __builtin_amdgcn_wave_barrier();
        rowsum[half][(ps % ppu) * (2 * kDeltaRows) + wv * kDeltaRows + crow] = acc;
        if ((ps + 1) % ppu == 0) {
            __syncthreads();
            if (t < 2) {
                const int64_t br = br0 + static_cast<int64_t>(ps / ppu) * P;
                double total = 0.0;
                for (int r = 0; r < bn; ++r) total = total + rowsum[t][r];
                delta[br * nbc + 2 * g + t] = total;
                rank[br * nbc + 2 * g + t] = 0;     // counters for the ranking pass
            }
            __syncthreads();
        }
    }
#undef MQ_PASS_ROW0
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
// row, then column block ascending. One workgroup; each thread owns a contiguous
// run of ids, so one block-wide exclusive scan of the per-thread counts gives
// every chosen block its CSR position.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void k_csr(const int32_t* __restrict__ rank, int nb, int nbc, int nbr,
                                              int k_blocks, int32_t* __restrict__ row_ptr,
                                              int32_t* __restrict__ col_idx) {
    __shared__ int wsum[16];
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const int per = (nb + 1023) / 1024;
    const int id0 = min(t * per, nb), id1 = min(id0 + per, nb);
    int cnt = 0;
    for (int id = id0; id < id1; ++id) cnt += rank[id] < k_blocks;
    int v = cnt;                                          // inclusive scan in the wavefront
    for (int off = 1; off < 64; off <<= 1) {
        const int u = __shfl_up(v, off);
        if (lane >= off) v += u;
    }
    if (lane == 63) wsum[wv] = v;
    __syncthreads();
    int pos = v - cnt;
    for (int i = 0; i < wv; ++i) pos += wsum[i];
    int row = id0 / nbc, col = id0 - row * nbc;
    for (int id = id0; id < id1; ++id) {
        if (col == 0) row_ptr[row] = pos;
        if (rank[id] < k_blocks) {
            // ranks form a permutation, so exactly k_blocks flags are set; the
            // bound only matters for non-finite scores (unsupported inputs)
            if (pos < k_blocks) col_idx[pos] = col;
            ++pos;
        }
        if (++col == nbc) {
            col = 0;
            ++row;
        }
    }
    if (t == 1023) row_ptr[nbr] = pos;                    // the last thread ends at the total
}

// ---------------------------------------------------------------------------
// a1 + a3: pack. One workgroup per (block row, group), 64 rows per pass, four
// lanes per row with 32 weights each (eight 16-byte loads, one 16-byte store of
// codes into the tiled wq layout). The block row's CSR list is searched once, in
// parallel, for the two column blocks of the group; chosen blocks get their
// 16-byte residual rows written at their CSR position. W is read exactly once.
// ---------------------------------------------------------------------------

// 8 codes as two's-complement nibbles (code i in bits 4i..4i+3), the input of code_word
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
    __shared__ uint8_t fix[4][64];                 // per-wave codes of a repaired lane
    const int64_t br = blockIdx.x, g = blockIdx.y, G = K / kGroup, G4 = (G + 3) / 4;
    const int t = threadIdx.x, row = t >> 2, qd = t & 3, lane = t & 63, wave = t >> 6;
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
        float worst = 0.0f;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            const Elem o = quant_elem_fast(wv[i], gs, worst);
            qc[i] = static_cast<int>(o.q);
            rc[i] = static_cast<int>(o.r);
        }
        uint4 cq = make_uint4(code_word(pack8(qc)), code_word(pack8(qc + 8)), code_word(pack8(qc + 16)),
                              code_word(pack8(qc + 24)));
        uint4 cr = make_uint4(code_word(pack8(rc)), code_word(pack8(rc + 8)), code_word(pack8(rc + 16)),
                              code_word(pack8(rc + 24)));
        // Rare: a quotient within 4e-6 of a rounding boundary. The wave repairs each
        // flagged lane L together: lane i < 32 requantizes weight i of L's 32 with
        // the exact quantizer, and L gathers the codes through LDS.
        const bool redo = !(worst < kFastMargin) || !fast_ok(gs);
        uint64_t flagged = __ballot(redo);
        while (flagged) {
            const int L = __builtin_ctzll(flagged);
            flagged &= flagged - 1;
            const int64_t nL = __shfl(static_cast<int>(n), L);
            const int qdL = L & 3;
            const GroupScale lg = group_scale(__shfl(gs.s, L));
            if (lane < 32) {
                const Elem o = quant_elem(w[nL * K + g * kGroup + qdL * 32 + lane], lg);
                fix[wave][lane] = static_cast<uint8_t>(static_cast<int>(o.q) & 15);
                fix[wave][32 + lane] = static_cast<uint8_t>(static_cast<int>(o.r) & 15);
            }
            __builtin_amdgcn_wave_barrier();
            if (lane == L) {
                uint32_t q4[4] = {0, 0, 0, 0}, r4[4] = {0, 0, 0, 0};
#pragma unroll
                for (int i = 0; i < 32; ++i) {
                    q4[i >> 3] |= static_cast<uint32_t>(fix[wave][i]) << (4 * (i & 7));
                    r4[i >> 3] |= static_cast<uint32_t>(fix[wave][32 + i]) << (4 * (i & 7));
                }
                cq = make_uint4(code_word(q4[0]), code_word(q4[1]), code_word(q4[2]), code_word(q4[3]));
                cr = make_uint4(code_word(r4[0]), code_word(r4[1]), code_word(r4[2]), code_word(r4[3]));
            }
            __builtin_amdgcn_wave_barrier();
        }
        // tiled base codes: a wavefront's 16 rows x 4 quarters are one 1 KB tile
        *reinterpret_cast<uint4*>(wq + wq_byte(n, G, g, qd)) = cq;
        if (qd == 0) {
            sw[sw_index(n, G4, g)] = sb;
            if (g == G - 1)
                for (int64_t gp = G; gp < 4 * G4; ++gp) sw[sw_index(n, G4, gp)] = 0;   // padding slots
        }
        if (p >= 0)
            *reinterpret_cast<uint4*>(rq + (static_cast<int64_t>(p) * bn + r0 + row) * (kBk / 2) + (qd & 1) * 16) = cr;
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// The dense block map of a CSR selection: one workgroup per block row writes -1
// over the row, then each CSR entry p of the row writes p at its column block.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_block_map(const int32_t* __restrict__ row_ptr,
                                                   const int32_t* __restrict__ col_idx, int nnz, int nkb,
                                                   int32_t* __restrict__ rmap) {
    const int br = blockIdx.x;
    int32_t* row = rmap + static_cast<int64_t>(br) * nkb;
    for (int i = threadIdx.x; i < nkb; i += blockDim.x) row[i] = -1;
    __syncthreads();
    const int lo = min(max(row_ptr[br], 0), nnz);
    const int hi = min(max(row_ptr[br + 1], lo), nnz);
    for (int p = lo + static_cast<int>(threadIdx.x); p < hi; p += blockDim.x) {
        const int kb = col_idx[p];
        if (kb >= 0 && kb < nkb) row[kb] = p;
    }
}

hipError_t launch_block_map(const int32_t* row_ptr, const int32_t* col_idx, int64_t nnz, int64_t N, int64_t K,
                            int bn, int32_t* rmap, hipStream_t st) {
    k_block_map<<<dim3(static_cast<unsigned>(N / bn)), dim3(256), 0, st>>>(row_ptr, col_idx, static_cast<int>(nnz),
                                                                          static_cast<int>(K / kBk), rmap);
    return hipGetLastError();
}

hipError_t launch_hessian(const void* x, int bf16, int64_t M, int64_t K, const float* colscale, float* h,
                          hipStream_t st) {
    const int64_t blocks = (K + kHCh - 1) / kHCh;
    k_hessian<<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st>>>(x, bf16, M, K, colscale, h);
    return hipGetLastError();
}

// Threads per token. Few tokens (M <= 256): enough to hold the whole row in
// registers (kQaWords words of 8 inputs each), at least 256 and at most 1024, so
// that each thread's chain of loads is short. Many tokens: 256 (the grid alone
// fills the chip, and wider workgroups only cost). Measured on MI355X (us per
// call at 128 / 256 / 512 / 1024 threads): M=16, K=4096 3.80 / 3.46 / 3.46 / 4.50;
// M=32, K=14336 12.13 / 7.00 / 5.10 / 5.26; M=2048, K=5120 8.70 / 8.95 / 13.22 /
// 25.59. The width does not change the result: every thread's words are the same
// whichever of them it holds in registers.
int quant_act_threads(int64_t M, int64_t K) {
    if (M > 256) return 256;
    const int64_t words = K / 8;
    const int64_t nt = ((words + kQaWords - 1) / kQaWords + 63) / 64 * 64;
    return static_cast<int>(std::min<int64_t>(64 * kQaMaxWaves, std::max<int64_t>(256, nt)));
}

hipError_t launch_quant_act(const void* x, int bf16, int64_t M, int64_t K, const float* colscale, uint8_t* xq,
                            float* sx, hipStream_t st) {
    k_quant_act<<<dim3(static_cast<unsigned>(M)), dim3(quant_act_threads(M, K)), 0, st>>>(x, bf16, M, K, colscale,
                                                                                      xq, sx);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// a0' (offline): migration factors of the equivalent per-channel transform
// (Methodology 1): s_k = sqrt(a_k) / sqrt(b_k) with a_k = max_m |x_mk|,
// b_k = max_n |w_nk| (fp32, correctly rounded square roots and division),
// s_k = 1 for a dead channel; r_k = 1 / s_k. A workgroup owns 64 channels; its
// four row lanes take every fourth row of X and of W (max is exact in any order).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_smooth(const void* __restrict__ x, int bf16, int64_t M, int64_t K,
                                                const float* __restrict__ w, int64_t N, float* __restrict__ s,
                                                float* __restrict__ r) {
    __shared__ float red[2][4][64];
    const int t = threadIdx.x, c = t & 63, lane_row = t >> 6;
    const int64_t k = static_cast<int64_t>(blockIdx.x) * 64 + c;
    float a = 0.0f, b = 0.0f;
    if (k < K) {
        for (int64_t m = lane_row; m < M; m += 4) a = fmaxf(a, fabsf(load_x(x, bf16, m * K + k)));
        for (int64_t n = lane_row; n < N; n += 4) b = fmaxf(b, fabsf(w[n * K + k]));
    }
    red[0][lane_row][c] = a;
    red[1][lane_row][c] = b;
    __syncthreads();
    if (t < 64 && k < K) {
        a = fmaxf(fmaxf(red[0][0][c], red[0][1][c]), fmaxf(red[0][2][c], red[0][3][c]));
        b = fmaxf(fmaxf(red[1][0][c], red[1][1][c]), fmaxf(red[1][2][c], red[1][3][c]));
        const float sk = (a > 0.0f && b > 0.0f) ? sqrtf(a) / sqrtf(b) : 1.0f;
        s[k] = sk;
        r[k] = 1.0f / sk;
    }
}

// out[i][k] = fp32(in[i][k] * c[k]): the migrated weights W^ = W diag(s)
__global__ __launch_bounds__(256) void k_scale_cols(const float* __restrict__ in, int64_t rows, int64_t K,
                                                    const float* __restrict__ c, float* __restrict__ out) {
    const int64_t n4 = rows * K / 4;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n4;
         i += static_cast<int64_t>(gridDim.x) * 256) {
        const float4 v = reinterpret_cast<const float4*>(in)[i];
        const int64_t k = (i * 4) % K;
        const float4 f = *reinterpret_cast<const float4*>(c + k);
        reinterpret_cast<float4*>(out)[i] = make_float4(v.x * f.x, v.y * f.y, v.z * f.z, v.w * f.w);
    }
}

hipError_t launch_smooth(const void* x, int bf16, int64_t M, int64_t K, const float* w, int64_t N, float* s,
                         float* r, hipStream_t st) {
    k_smooth<<<dim3(static_cast<unsigned>((K + 63) / 64)), dim3(256), 0, st>>>(x, bf16, M, K, w, N, s, r);
    return hipGetLastError();
}

hipError_t launch_scale_cols(const float* in, int64_t rows, int64_t K, const float* c, float* out, hipStream_t st) {
    const int64_t n4 = rows * K / 4;
    const unsigned blocks = static_cast<unsigned>(std::min<int64_t>((n4 + 255) / 256, 8192));
    if (blocks) k_scale_cols<<<dim3(blocks), dim3(256), 0, st>>>(in, rows, K, c, out);
    return hipGetLastError();
}

hipError_t launch_select(const float* w, const float* h, int64_t N, int64_t K, int bn,
                         int64_t k_blocks, int32_t* row_ptr, int32_t* col_idx, double* delta,
                         void* scratch, hipStream_t st) {
    const int64_t nbr = N / bn, nbc = K / kBk, nb = nbr * nbc;
    void* buf = scratch;
    hipError_t err = hipSuccess;
    if (!buf) {
        err = hipMallocAsync(&buf, select_scratch_bytes(nb, delta == nullptr), st);
        if (err != hipSuccess) return err;
    }
    int32_t* rank = static_cast<int32_t*>(buf);
    double* score = delta ? delta
                          : reinterpret_cast<double*>(static_cast<char*>(buf) + select_scratch_bytes(nb, false));
    // about four workgroups per CU: each walks nbr / P block rows of one group
    const int64_t G = K / kGroup;
    const int64_t P = std::max<int64_t>(1, std::min<int64_t>(nbr, (1024 + G - 1) / G));
    k_delta<<<dim3(static_cast<unsigned>(P), static_cast<unsigned>(G)), dim3(128), 0, st>>>(
        w, h, K, bn, static_cast<int>(nbr), score, rank);
    err = hipGetLastError();
    const unsigned nblk = static_cast<unsigned>((nb + 255) / 256);
    if (err == hipSuccess) {
        k_rank<<<dim3(nblk, static_cast<unsigned>((nb + kRankSlice - 1) / kRankSlice)), dim3(256), 0, st>>>(
            score, nb, rank);
        err = hipGetLastError();
    }
    if (err == hipSuccess) {
        k_csr<<<dim3(1), dim3(1024), 0, st>>>(rank, static_cast<int>(nb), static_cast<int>(nbc),
                                              static_cast<int>(nbr), static_cast<int>(k_blocks), row_ptr, col_idx);
        err = hipGetLastError();
    }
    if (scratch) return err;
    const hipError_t ferr = hipFreeAsync(buf, st);
    return err != hipSuccess ? err : ferr;
}

hipError_t launch_pack(const float* w, int64_t N, int64_t K, int bn, const int32_t* row_ptr,
                       const int32_t* col_idx, int64_t nnz, uint8_t* wq, uint16_t* sw, uint8_t* rq,
                       hipStream_t st) {
    k_pack<<<dim3(static_cast<unsigned>(N / bn), static_cast<unsigned>(K / kGroup)), dim3(256), 0, st>>>(
        w, N, K, bn, row_ptr, col_idx, nnz, wq, sw, rq);
    return hipGetLastError();
}

// A plain streaming read of n16 16-byte words: the HBM read rate a kernel reaches
// at a given byte count (what the decode GEMM, which streams its weights once, is
// held against). Each lane keeps four loads in flight; each workgroup writes one
// word (the XOR of what it read) so the loads stay live.
__global__ __launch_bounds__(256) void k_read_probe(const uint4* __restrict__ p, int64_t n16,
                                                    uint32_t* __restrict__ out) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
    int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const uint4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
        acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
    }
    for (; i < n16; i += stride) {
        const uint4 a = p[i];
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off);
    __shared__ uint32_t w[4];
    if ((threadIdx.x & 63) == 0) w[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) out[blockIdx.x] = w[0] ^ w[1] ^ w[2] ^ w[3];
}

int read_probe_blocks(int64_t bytes) {
    const int64_t n16 = bytes / 16;
    return static_cast<int>(std::max<int64_t>(1, std::min<int64_t>((n16 + 1023) / 1024, kReadProbeMaxBlocks)));
}

hipError_t launch_read_probe(const void* p, int64_t bytes, uint32_t* out, hipStream_t st) {
    k_read_probe<<<dim3(static_cast<unsigned>(read_probe_blocks(bytes))), dim3(256), 0, st>>>(
        static_cast<const uint4*>(p), bytes / 16, out);
    return hipGetLastError();
}

}  // namespace mq
