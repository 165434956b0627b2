// ZipperEngine on gfx950: the fused dense + sparse-residual W4A4 GEMM.
//
// MosaicQuant technical summary (gist.science), Methodology 3 "ZipperEngine":
// the sparse-residual product is computed inside the dense 4-bit GEMM kernel, in
// a tiled pipeline, so activations are not reloaded and partial outputs are not
// merged by a second kernel. Methodology 1 fixes both parts at 4 bits.
//
// Data flow per 128-wide K group g (the weight scale group):
//   * base nibbles wq and activation nibbles xq arrive as 16-byte vector loads;
//   * both are widened to int8 operands of v_mfma_i32_16x16x64_i8 (gfx950 has no
//     int4 MFMA); the activation operand is staged once per tile and reused by
//     every product that needs it;
//   * the output rows' CSR list of residual blocks is walked in step with g (the
//     "zipper"); in a group holding a chosen block the weight operand becomes
//     14*q + r per element, so the residual rides in the same MFMAs and the same
//     int32 accumulator, which then holds T = 14*P + Pr exactly;
//   * at the end of the group the exact int32 sum is dequantized into fp32:
//     acc += s/256 * (256 P)      (dense group, both operands carry a x16 factor)
//     acc += s_r/16 * (16 T)      (residual group, s_r = fp32(s/14))
//   * the epilogue multiplies by the token scale sx and stores bf16 or fp32.
#include "mq_device.h"
#include "mq_internal.h"

namespace mq {

// The zipper: CSR positions of the residual blocks of one block row, for the
// column blocks a wave walks, gathered into an LDS table in one parallel pass
// (lane i reads list entry lo + i), so the K loop finds each group's blocks
// with an LDS read instead of a chain of dependent loads.
__device__ __forceinline__ void zip_table(const GemmArgs& a, int br, int kb0, int nkb, int* tab,
                                          int lane, int nlanes) {
    const int lo = clampi(a.row_ptr[br], 0, a.nnz);
    const int hi = clampi(a.row_ptr[br + 1], lo, a.nnz);
    for (int i = lo + lane; i < hi; i += nlanes) {
        const int rel = a.col_idx[i] - kb0;
        if (rel >= 0 && rel < nkb) tab[rel] = i;
    }
}

__device__ __forceinline__ void store_out(const GemmArgs& a, int OUTMODE, int m, int n, float v) {
    const int64_t idx = static_cast<int64_t>(m) * a.N + n;
    if (OUTMODE == 1) {
        a.ws[idx] = v;
    } else {
        v *= a.sx[m];
        if (a.y_bf16) static_cast<uint16_t*>(a.y)[idx] = f32_to_bf16_bits(v);
        else static_cast<float*>(a.y)[idx] = v;
    }
}

// ===========================================================================
// Skinny kernel, M <= 32 (decode). A workgroup owns 16 output columns and all
// tokens; its waves split the K groups and reduce through LDS in a fixed order.
// Every weight byte is read by exactly one lane, with 16-byte loads; each lane
// covers 32 consecutive K of one output row per group. A wave requests one
// chunk of groups at a time; the bytes in flight per CU come from the many
// workgroups that fit side by side (the kernel is kept small in registers).
// ===========================================================================
constexpr int kChunk = 4;      // groups per load batch
constexpr int kMaxWaves = 8;
constexpr int kMaxWaveKb = 64; // column blocks one wave may walk (32 groups)

template <int MT>
struct SkinnyChunk {
    uint4 bw[kChunk], rw[kChunk];
    uint4 aw[kChunk][MT];
    float sc[kChunk];
    int rg;   // bit u: group gc + u holds a chosen block in this row
};

template <int MT, bool RES, bool DUMP, int OUTMODE>
__global__ __launch_bounds__(512) void k_gemm_skinny(GemmArgs a) {
    __shared__ float red[kMaxWaves * MT * 256];
    __shared__ int jtab[RES ? kMaxWaves * kMaxWaveKb : 1];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    const int li = lane & 15, kg = lane >> 4;
    const int G = a.K / kGroup;
    const int n0 = blockIdx.x * 16, n = n0 + li;
    const int g0 = (wave * G) / nw, g1 = ((wave + 1) * G) / nw;
    const int64_t Kh = a.K / 2;
    const uint8_t* wrow = a.wq + static_cast<int64_t>(n) * Kh + kg * 16;
    const uint8_t* xrow[MT];
    bool xv[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        const int m = t * 16 + li;
        xv[t] = m < a.M;
        xrow[t] = a.xq + static_cast<int64_t>(xv[t] ? m : 0) * Kh + kg * 16;
    }
    const uint16_t* srow = a.sw + static_cast<int64_t>(n) * G;
    const int br = n0 / a.bn, rrow = n - br * a.bn;
    int* tab = jtab + (RES ? wave * kMaxWaveKb : 0);

    auto load_base = [&](int gc, SkinnyChunk<MT>& c) {
#pragma unroll
        for (int u = 0; u < kChunk; ++u) {
            const int g = gc + u;
            const bool ok = g < g1;
            c.bw[u] = ok ? ldg16(wrow + g * 64) : make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int t = 0; t < MT; ++t) c.aw[u][t] = (ok && xv[t]) ? ldg16(xrow[t] + g * 64) : make_uint4(0, 0, 0, 0);
            c.sc[u] = ok ? f16_bits_to_f32(srow[g]) : 0.0f;
        }
    };
    auto load_res = [&](int gc, SkinnyChunk<MT>& c) {
        c.rg = 0;
#pragma unroll
        for (int u = 0; u < kChunk; ++u) {
            const int g = gc + u;
            c.rw[u] = make_uint4(0, 0, 0, 0);
            if (RES && g < g1) {
                const int j0 = tab[2 * (g - g0)], j1 = tab[2 * (g - g0) + 1];
                if (j0 >= 0 || j1 >= 0) c.rg |= 1 << u;
                const int j = kg < 2 ? j0 : j1;
                if (j >= 0) c.rw[u] = ldg16(a.rq + (static_cast<int64_t>(j) * a.bn + rrow) * 32 + (kg & 1) * 16);
            }
        }
    };

    SkinnyChunk<MT> cur;
    load_base(g0, cur);
    if (RES) {
        tab[lane] = -1;
        zip_table(a, br, 2 * g0, 2 * (g1 - g0), tab, lane, 64);
        __syncthreads();
        load_res(g0, cur);
    } else {
        cur.rg = 0;
    }

    float acc[MT][4];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[t][r] = 0.0f;

    for (int gc = g0; gc < g1; gc += kChunk) {
        if (gc != g0) {
            load_base(gc, cur);
            if (RES) load_res(gc, cur);
        }
#pragma unroll
        for (int u = 0; u < kChunk; ++u) {
            const int g = gc + u;
            if (g >= g1) break;
            const bool res = RES && ((cur.rg >> u) & 1);
            v4i b0, b1;
            float scale;
            if (res) {
                unpack_comb(cur.bw[u], cur.rw[u], b0, b1);
                scale = (cur.sc[u] / 14.0f) * 0.0625f;
            } else {
                unpack16(cur.bw[u], b0, b1);
                scale = cur.sc[u] * 0.00390625f;
            }
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                v4i a0, a1;
                unpack16(cur.aw[u][t], a0, a1);
                v4i c = v4i{0, 0, 0, 0};
                c = mfma_i8(a0, b0, c);
                c = mfma_i8(a1, b1, c);
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[t][r] += scale * static_cast<float>(c[r]);
                if (DUMP) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int m = t * 16 + kg * 4 + r;
                        if (m < a.M)
                            a.acc_dump[(static_cast<int64_t>(m) * a.N + n) * G + g] =
                                res ? (c[r] >> 4) : 14 * (c[r] >> 8);
                    }
                }
            }
        }
    }

    // fixed-order reduction of the waves' partial tiles
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[((wave * MT + t) * 4 + r) * 64 + lane] = acc[t][r];
    __syncthreads();
    for (int o = threadIdx.x; o < MT * 256; o += blockDim.x) {
        const int t = o >> 8, r = (o >> 6) & 3, l = o & 63;
        float s = 0.0f;
        for (int w = 0; w < nw; ++w) s += red[((w * MT + t) * 4 + r) * 64 + l];
        const int m = t * 16 + (l >> 4) * 4 + r;
        if (m < a.M) store_out(a, OUTMODE, m, n0 + (l & 15), s);
    }
}

// ===========================================================================
// Tiled kernel, M > 32 (prefill). 128 x 128 output tile per workgroup, four
// waves of 64 x 64, one K group per step. The activation and base-weight tiles
// of the next group, and the residual rows it needs, are fetched into registers
// while the current group's tiles are consumed from LDS (double buffer, one
// barrier per group).
// ===========================================================================
constexpr int kBM = 128, kBN = 128;
constexpr int kRowB = 80;          // LDS bytes per tile row: 64 data + 16 pad (conflict-free b128 reads)
constexpr int kMaxKb = 1024;       // column blocks per row the LDS zipper table holds (K <= 65536)

template <bool RES, bool DUMP, int OUTMODE>
__global__ __launch_bounds__(256) void k_gemm_tiled(GemmArgs a) {
    __shared__ __align__(16) uint8_t As[2][kBM * kRowB];
    __shared__ __align__(16) uint8_t Bs[2][kBN * kRowB];
    __shared__ int jtab[RES ? 2 * kMaxKb : 1];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, kg = lane >> 4;
    const int wm = wave >> 1, wn = wave & 1;
    const int tiles_n = (a.N + kBN - 1) / kBN;
    const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
    const int m0 = tm * kBM, n0 = tn * kBN;
    const int G = a.K / kGroup, nbc = a.K / kBk;
    const int64_t Kh = a.K / 2;

    // global -> LDS assignment: 512 16-byte chunks per operand tile, two per thread
    int ld_row[2], ld_part[2];
    const uint8_t* ga[2];
    const uint8_t* gb[2];
    bool va[2], vb[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int c = tid + 256 * i;
        ld_row[i] = c >> 2;
        ld_part[i] = c & 3;
        const int m = m0 + ld_row[i], nn = n0 + ld_row[i];
        va[i] = m < a.M;
        vb[i] = nn < a.N;
        ga[i] = a.xq + static_cast<int64_t>(va[i] ? m : 0) * Kh + ld_part[i] * 16;
        gb[i] = a.wq + static_cast<int64_t>(vb[i] ? nn : 0) * Kh + ld_part[i] * 16;
    }
    const int nw0 = n0 + wn * 64;                 // this wave's first output column
    const bool wave_cols = nw0 < a.N;
    const int br = nw0 / a.bn, rbase = nw0 - br * a.bn;
    const int* tab = jtab + (RES ? wn * kMaxKb : 0);

    uint4 ra[2], rb[2], rr[4];
    float sn[4];
    int rgrp_next = 0;
    auto fetch = [&](int g) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            ra[i] = va[i] ? ldg16(ga[i] + g * 64) : make_uint4(0, 0, 0, 0);
            rb[i] = vb[i] ? ldg16(gb[i] + g * 64) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int nn = nw0 + j * 16 + li;
            sn[j] = nn < a.N ? f16_bits_to_f32(a.sw[static_cast<int64_t>(nn) * G + g]) : 0.0f;
        }
        if (RES) {
            const int j0 = wave_cols ? tab[2 * g] : -1, j1 = wave_cols ? tab[2 * g + 1] : -1;
            rgrp_next = (j0 >= 0) || (j1 >= 0);
            const int jb = kg < 2 ? j0 : j1;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int nn = nw0 + j * 16 + li;
                rr[j] = (jb >= 0 && nn < a.N)
                            ? ldg16(a.rq + (static_cast<int64_t>(jb) * a.bn + rbase + j * 16 + li) * 32 + (kg & 1) * 16)
                            : make_uint4(0, 0, 0, 0);
            }
        }
    };
    auto stash = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            *reinterpret_cast<uint4*>(&As[buf][ld_row[i] * kRowB + ld_part[i] * 16]) = ra[i];
            *reinterpret_cast<uint4*>(&Bs[buf][ld_row[i] * kRowB + ld_part[i] * 16]) = rb[i];
        }
    };

    if (RES) {
        for (int i = tid; i < 2 * nbc; i += 256) jtab[(i / nbc) * kMaxKb + i % nbc] = -1;
        __syncthreads();
        // both wave columns' block rows (the same row when bn == 128)
        const int brow0 = n0 / a.bn, brow1 = (n0 + 64) / a.bn;
        if (n0 < a.N) zip_table(a, brow0, 0, nbc, jtab, tid, 256);
        if (n0 + 64 < a.N) zip_table(a, brow1, 0, nbc, jtab + kMaxKb, tid, 256);
        __syncthreads();
    }

    float acc[4][4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.0f;

    fetch(0);
    stash(0);
    uint4 rw[4] = {rr[0], rr[1], rr[2], rr[3]};
    float sc[4] = {sn[0], sn[1], sn[2], sn[3]};
    int rgrp = rgrp_next;
    __syncthreads();
    for (int g = 0; g < G; ++g) {
        const int buf = g & 1;
        if (g + 1 < G) fetch(g + 1);
        v4i a0[4], a1[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 w = *reinterpret_cast<const uint4*>(&As[buf][(wm * 64 + i * 16 + li) * kRowB + kg * 16]);
            unpack16(w, a0[i], a1[i]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint4 w = *reinterpret_cast<const uint4*>(&Bs[buf][(wn * 64 + j * 16 + li) * kRowB + kg * 16]);
            v4i b0, b1;
            float scale;
            if (RES && rgrp) {
                unpack_comb(w, rw[j], b0, b1);
                scale = (sc[j] / 14.0f) * 0.0625f;
            } else {
                unpack16(w, b0, b1);
                scale = sc[j] * 0.00390625f;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v4i c = v4i{0, 0, 0, 0};
                c = mfma_i8(a0[i], b0, c);
                c = mfma_i8(a1[i], b1, c);
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[i][j][r] += scale * static_cast<float>(c[r]);
                if (DUMP) {
                    const int nn = nw0 + j * 16 + li;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int m = m0 + wm * 64 + i * 16 + kg * 4 + r;
                        if (m < a.M && nn < a.N)
                            a.acc_dump[(static_cast<int64_t>(m) * a.N + nn) * G + g] =
                                (RES && rgrp) ? (c[r] >> 4) : 14 * (c[r] >> 8);
                    }
                }
            }
        }
        if (g + 1 < G) {
            stash(buf ^ 1);
#pragma unroll
            for (int j = 0; j < 4; ++j) sc[j] = sn[j];
            if (RES) {
#pragma unroll
                for (int j = 0; j < 4; ++j) rw[j] = rr[j];
                rgrp = rgrp_next;
            }
        }
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int nn = nw0 + j * 16 + li;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + wm * 64 + i * 16 + kg * 4 + r;
                if (m < a.M && nn < a.N) store_out(a, OUTMODE, m, nn, acc[i][j][r]);
            }
        }
}

// ===========================================================================
// Second kernel of the separate-kernel alternative: re-reads the activations,
// computes each chosen block's residual product, adds it to the dense partial
// outputs in `ws` and writes y. One workgroup per 16 output columns.
// ===========================================================================
__global__ __launch_bounds__(256) void k_residual_merge(GemmArgs a) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    const int li = lane & 15, kg = lane >> 4;
    const int G = a.K / kGroup, nbc = a.K / kBk;
    const int n0 = blockIdx.x * 16, n = n0 + li;
    const int br = n0 / a.bn, rrow = n - br * a.bn;
    const int64_t Kh = a.K / 2;
    const int lo = clampi(a.row_ptr[br], 0, a.nnz);
    const int hi = clampi(a.row_ptr[br + 1], lo, a.nnz);
    const int mtiles = (a.M + 15) / 16;
    for (int t = wave; t < mtiles; t += nw) {
        const int ma = t * 16 + li;
        float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int p = lo; p < hi; ++p) {
            const int kb = a.col_idx[p];
            if (kb < 0 || kb >= nbc) continue;
            const int g = kb >> 1;
            uint2 av = make_uint2(0, 0);
            if (ma < a.M) av = *reinterpret_cast<const uint2*>(a.xq + static_cast<int64_t>(ma) * Kh + kb * 32 + kg * 8);
            const uint2 rv =
                *reinterpret_cast<const uint2*>(a.rq + (static_cast<int64_t>(p) * a.bn + rrow) * 32 + kg * 8);
            const v4i aop = v4i{(int)nib16_even(av.x), (int)nib16_odd(av.x), (int)nib16_even(av.y), (int)nib16_odd(av.y)};
            const v4i bop = v4i{(int)nib16_even(rv.x), (int)nib16_odd(rv.x), (int)nib16_even(rv.y), (int)nib16_odd(rv.y)};
            const v4i c = mfma_i8(aop, bop, v4i{0, 0, 0, 0});
            const float sr = f16_bits_to_f32(a.sw[static_cast<int64_t>(n) * G + g]) / 14.0f;
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] += (sr * 0.00390625f) * static_cast<float>(c[r]);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = t * 16 + kg * 4 + r;
            if (m < a.M) {
                const int64_t idx = static_cast<int64_t>(m) * a.N + n;
                const float v = (a.ws[idx] + acc[r]) * a.sx[m];
                if (a.y_bf16) static_cast<uint16_t*>(a.y)[idx] = f32_to_bf16_bits(v);
                else static_cast<float*>(a.y)[idx] = v;
            }
        }
    }
}

// ===========================================================================
// launch selection
// ===========================================================================
template <int MT, bool RES, bool DUMP, int OUT>
static hipError_t go_skinny(const GemmArgs& a, hipStream_t st) {
    const int G = a.K / kGroup;
    int nw = (G + 3) / 4;
    nw = nw < 1 ? 1 : (nw > kMaxWaves ? kMaxWaves : nw);
    k_gemm_skinny<MT, RES, DUMP, OUT><<<dim3(a.N / 16), dim3(64 * nw), 0, st>>>(a);
    return hipGetLastError();
}

template <bool RES, bool DUMP, int OUT>
static hipError_t go_tiled(const GemmArgs& a, hipStream_t st) {
    const int tiles = ((a.M + kBM - 1) / kBM) * ((a.N + kBN - 1) / kBN);
    k_gemm_tiled<RES, DUMP, OUT><<<dim3(tiles), dim3(256), 0, st>>>(a);
    return hipGetLastError();
}

template <bool RES, bool DUMP, int OUT>
static hipError_t go(const GemmArgs& a, hipStream_t st) {
    if (a.M <= 16) return go_skinny<1, RES, DUMP, OUT>(a, st);
    if (a.M <= 32) return go_skinny<2, RES, DUMP, OUT>(a, st);
    return go_tiled<RES, DUMP, OUT>(a, st);
}

hipError_t launch_gemm(const GemmArgs& a, GemmKind kind, hipStream_t st) {
    const bool dump = a.acc_dump != nullptr;
    switch (kind) {
        case GemmKind::Fused:
            return dump ? go<true, true, 0>(a, st) : go<true, false, 0>(a, st);
        case GemmKind::Dense:
            return dump ? go<false, true, 0>(a, st) : go<false, false, 0>(a, st);
        case GemmKind::DenseToWorkspace:
            return go<false, false, 1>(a, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_residual_merge(const GemmArgs& a, hipStream_t st) {
    k_residual_merge<<<dim3(a.N / 16), dim3(256), 0, st>>>(a);
    return hipGetLastError();
}

}  // namespace mq
