// ZipperEngine on gfx950: the fused dense + sparse-residual W4A4 GEMM.
//
// MosaicQuant technical summary (gist.science), Methodology 3 "ZipperEngine":
// the sparse-residual product is computed inside the dense 4-bit GEMM kernel, in
// a tiled pipeline, so activations are not reloaded and partial outputs are not
// merged by a second kernel. Methodology 1 fixes both parts at 4 bits.
//
// Data flow per 128-wide K group g (the weight scale group):
//   * base nibbles wq and activation nibbles xq arrive as 16-byte vector loads,
//     each wavefront load one contiguous 1 KB run (tiled wq, group-major xq);
//   * both are widened to int8 operands of v_mfma_i32_16x16x64_i8 (gfx950 has no
//     int4 MFMA);
//   * the output rows' CSR list of residual blocks is walked in step with g (the
//     "zipper"); in a group holding a chosen block the weight operand becomes
//     14*q + r per element, so the residual rides in the same MFMAs and the same
//     int32 accumulator, which then holds T = 14*P + Pr exactly;
//   * at the end of the group the exact int32 sum is dequantized into fp32:
//     acc += s/256 * (256 P)      (dense group, both operands carry a x16 factor)
//     acc += s_r/16 * (16 T)      (residual group, s_r = fp32(s/14))
//   * the epilogue multiplies by the token scale sx and stores bf16 or fp32.
#include <algorithm>
#include <cmath>

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
// Decode kernel, M <= 32: one workgroup per 16 output columns, its waves split
// K into runs of 4-group quads (a quad's four scales are one 8-byte load per
// lane). Each wave streams its tiles with the next quad's loads (weights,
// activations, residual rows, scales) in flight while the current quad is
// multiplied, then the waves' partial tiles are summed through LDS in wave
// order, so results do not depend on timing. The vector memory pipeline, not
// HBM, limits this shape class: every load instruction counts, hence 1 KB per
// instruction for weights and activations and one scale load per quad.
// ===========================================================================
constexpr int kMaxDecodeWaves = 8;
constexpr int kMaxGroups = 512;    // K <= 65536

// One pipeline step: QS consecutive groups (QS = 4 for one row tile of tokens,
// 2 for two, which keeps two steps' registers within three waves per SIMD).
template <int MT, int QS>
struct DecStep {
    uint4 w[QS];         // base nibbles of the step's groups
    uint4 x[MT][QS];     // activation nibbles
    uint4 r[QS];         // residual nibbles (zero where no chosen block)
    uint32_t s[(QS + 1) / 2];   // the row's fp16 group scales, two per word
    int rg;              // bit u: group g0+u holds a chosen block in this block row
};

// Per-wave buffer resources and lane offsets of the decode operands.
struct DecSrc {
    __amdgpu_buffer_rsrc_t w, x, s, r;   // this subtile's tiles, all activations, this subtile's
                                         // scales, this block row's residual payload
    uint32_t xrow[2];                    // lane's activation row offset per row tile
    uint32_t xstride;                    // bytes per group of activations (M * 64)
    int lo;                              // first CSR position of the block row
};

// base tiles, activations and scales of the step starting at group g0 (groups
// past the last read zero through the range check)
template <int MT, int QS>
__device__ __forceinline__ void dec_fetch_main(DecStep<MT, QS>& st, const DecSrc& src, int g0, int lane) {
#pragma unroll
    for (int u = 0; u < QS; ++u) {
        const uint32_t g = g0 + u;
        st.w[u] = buf_load16(src.w, g * 1024u + lane * 16u);
#pragma unroll
        for (int t = 0; t < MT; ++t) st.x[t][u] = buf_load16(src.x, g * src.xstride + src.xrow[t]);
    }
    const uint32_t so = (g0 >> 2) * 128u + (lane & 15) * 8u + (g0 & 3) * 2u;
    if (QS == 4) {
        const uint2 v = buf_load8(src.s, so);
        st.s[0] = v.x;
        st.s[(QS + 1) / 2 - 1] = v.y;
    } else if (QS == 2) {
        st.s[0] = buf_load4(src.s, so);
    } else {
        st.s[0] = __builtin_amdgcn_raw_buffer_load_b16(src.s, so, 0, 0);
    }
}

// residual rows of the step: the zipper table gives each column block's CSR
// position (or -1); lanes 0-31 take the group's first block, 32-63 the second
template <int MT, int QS, bool RES>
__device__ __forceinline__ void dec_fetch_res(DecStep<MT, QS>& st, const GemmArgs& a, const DecSrc& src,
                                              const int* tab, int rrow, int G, int g0, int lane) {
    const int kg = lane >> 4;
    st.rg = 0;
#pragma unroll
    for (int u = 0; u < QS; ++u) {
        const int g = g0 + u;
        st.r[u] = make_uint4(0, 0, 0, 0);
        if (RES && g < G) {
            // the table entry is the same for the whole wave: make that visible to
            // the compiler, so the residual branch in dec_compute is a scalar one
            const int j0 = __builtin_amdgcn_readfirstlane(tab[2 * g]);
            const int j1 = __builtin_amdgcn_readfirstlane(tab[2 * g + 1]);
            if (j0 >= 0 || j1 >= 0) {
                st.rg |= 1 << u;
                const int j = kg < 2 ? j0 : j1;
                // no block: an offset past the range reads zero
                const uint32_t off = j >= 0 ? ((j - src.lo) * a.bn + rrow) * 32u + (kg & 1) * 16u : 0xFFFFFFF0u;
                st.r[u] = buf_load16(src.r, off);
            }
        }
    }
}

// One fp8 MFMA per group and row tile gives P * 2^-18 exactly; a group with a
// chosen block in this block row adds the residual product Pr the same way and
// forms T = 14 P + Pr (exact in fp32), dequantized with s_r = fp32(s / 14).
template <int MT, int QS, bool RES, bool DUMP>
__device__ __forceinline__ void dec_compute(const DecStep<MT, QS>& st, const GemmArgs& a, int n, int G, int g0,
                                            int lane, float (&acc)[MT][4]) {
    const int kg = lane >> 4;
#pragma unroll
    for (int u = 0; u < QS; ++u) {
        const int g = g0 + u;
        if (g >= G) break;
        const float sc = f16_bits_to_f32(static_cast<uint16_t>(st.s[u >> 1] >> (16 * (u & 1))));
        const bool res = RES && ((st.rg >> u) & 1);
        if (res) {
            // the base products of both row tiles first, then the residual MFMAs
            // accumulating onto 14 P (T = 14 P + Pr, exact): the base and the
            // residual operands are never live together
            const float fr = (sc / 14.0f) * kF8Unit;
            v4f tv[MT];
            {
                const v8i b = f8_operand(st.w[u]);
#pragma unroll
                for (int t = 0; t < MT; ++t) tv[t] = mfma_f8(f8_operand(st.x[t][u]), b, v4f{0.0f, 0.0f, 0.0f, 0.0f}) * 14.0f;
            }
            const v8i rb = f8_operand(st.r[u]);
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                tv[t] = mfma_f8(f8_operand(st.x[t][u]), rb, tv[t]);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    acc[t][r] = fmaf(fr, tv[t][r], acc[t][r]);
                    if (DUMP) {
                        const int m = t * 16 + kg * 4 + r;
                        if (m < a.M)
                            a.acc_dump[(static_cast<int64_t>(m) * a.N + n) * G + g] = static_cast<int>(tv[t][r] * kF8Unit);
                    }
                }
            }
        } else {
            const float f = sc * kF8Unit;
            const v8i b = f8_operand(st.w[u]);
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const v4f p = mfma_f8(f8_operand(st.x[t][u]), b, v4f{0.0f, 0.0f, 0.0f, 0.0f});
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    acc[t][r] = fmaf(f, p[r], acc[t][r]);
                    if (DUMP) {
                        const int m = t * 16 + kg * 4 + r;
                        if (m < a.M)
                            a.acc_dump[(static_cast<int64_t>(m) * a.N + n) * G + g] = 14 * static_cast<int>(p[r] * kF8Unit);
                    }
                }
            }
        }
    }
}

template <int MT, bool RES, bool DUMP, int OUTMODE>
__global__ __launch_bounds__(64 * kMaxDecodeWaves) void k_gemm_decode(GemmArgs a) {
    // two groups per step; one for the residual variant with two row tiles,
    // which keeps its registers within four waves per SIMD
    constexpr int QS = (RES && MT == 2) ? 1 : 2;
    __shared__ float red[kMaxDecodeWaves * MT * 256];
    __shared__ int tab[RES ? 8 * (kMaxGroups / 4) : 1];   // column block -> CSR position
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
    const int G = a.K / kGroup, G4 = (G + 3) / 4;
    const int nt = blockIdx.x, n0 = nt * 16, n = n0 + (lane & 15);
    const int br = n0 / a.bn, rrow = n - br * a.bn;
    const int q0 = wave * G4 / nw, q1 = (wave + 1) * G4 / nw;       // this wave's quads
    const int gb = 4 * q0, ge = min(4 * q1, G);                      // and groups
    float acc[MT][4];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[t][r] = 0.0f;

    const int lo = RES ? clampi(a.row_ptr[br], 0, a.nnz) : 0;
    const int hi = RES ? clampi(a.row_ptr[br + 1], lo, a.nnz) : 0;
    DecSrc src;
    src.w = buf_rsrc(a.wq + wq_tile(nt, G, 0), static_cast<uint32_t>(G) * 1024u);
    src.x = buf_rsrc(a.xq, static_cast<uint32_t>(a.M) * static_cast<uint32_t>(a.K / 2));
    src.s = buf_rsrc(a.sw + static_cast<int64_t>(nt) * G4 * 64, static_cast<uint32_t>(G4) * 128u);
    src.r = buf_rsrc(RES && hi > lo ? a.rq + static_cast<int64_t>(lo) * a.bn * 32 : a.wq,
                     RES ? static_cast<uint32_t>(hi - lo) * static_cast<uint32_t>(a.bn) * 32u : 0u);
    src.xstride = static_cast<uint32_t>(a.M) * 64u;
#pragma unroll
    for (int t = 0; t < 2; ++t)
        src.xrow[t] = static_cast<uint32_t>(min(t * 16 + (lane & 15), a.M - 1)) * 64u + (lane >> 4) * 16u;
    src.lo = lo;

    // two steps in flight: step i+1 is fetched while step i is multiplied
    // (ping-pong buffers, so no register copy waits on the prefetch)
    DecStep<MT, QS> s0, s1;
    if (gb < ge) dec_fetch_main<MT, QS>(s0, src, gb, lane);
    if (RES) {
        // The zipper table of this wave's column blocks [2 gb, 2 ge), built by the
        // wave alone while its first loads are in flight: no workgroup barrier.
        // A wavefront's LDS operations complete in issue order, so the -1 fill,
        // the CSR positions and the later reads need no wait between lanes.
        const int kb0 = 2 * gb, kb1 = 2 * ge;
        for (int i = kb0 + lane; i < kb1; i += 64) tab[i] = -1;
        __builtin_amdgcn_wave_barrier();
        for (int i = lo + lane; i < hi; i += 64) {
            const int kb = a.col_idx[i];
            if (kb >= kb0 && kb < kb1) tab[kb] = i;
        }
        __builtin_amdgcn_wave_barrier();
        if (gb < ge) dec_fetch_res<MT, QS, RES>(s0, a, src, tab, rrow, G, gb, lane);
    }
    for (int g = gb; g < ge; g += 2 * QS) {
        if (g + QS < ge) {
            dec_fetch_main<MT, QS>(s1, src, g + QS, lane);
            if (RES) dec_fetch_res<MT, QS, RES>(s1, a, src, tab, rrow, G, g + QS, lane);
        }
        dec_compute<MT, QS, RES, DUMP>(s0, a, n, G, g, lane, acc);
        if (g + QS >= ge) break;
        if (g + 2 * QS < ge) {
            dec_fetch_main<MT, QS>(s0, src, g + 2 * QS, lane);
            if (RES) dec_fetch_res<MT, QS, RES>(s0, a, src, tab, rrow, G, g + 2 * QS, lane);
        }
        dec_compute<MT, QS, RES, DUMP>(s1, a, n, G, g + QS, lane, acc);
    }

#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[((wave * MT + t) * 4 + r) * 64 + lane] = acc[t][r];
    __syncthreads();
    for (int o = tid; o < MT * 256; o += blockDim.x) {
        const int t = o >> 8, r = (o >> 6) & 3, l = o & 63;
        float v = 0.0f;
        for (int w = 0; w < nw; ++w) v += red[((w * MT + t) * 4 + r) * 64 + l];
        const int m = t * 16 + (l >> 4) * 4 + r;
        if (m < a.M) store_out(a, OUTMODE, m, n0 + (l & 15), v);
    }
}

// ===========================================================================
// Prefill kernel, M > 32: 128 x 128 output tile per workgroup, four waves of
// 64 x 64, one K group (one fp8 MFMA deep) per step, two LDS stages.
//   * Operand tiles move from memory to LDS without passing through registers
//     (global_load_lds, 16 bytes per lane): each 16-row subtile of a group is one
//     1 KB load, placed in LDS in MFMA lane order (lane 16 kc + r holds row r,
//     codes 32 kc .. 32 kc + 31). The packed weight tiles already have that
//     order; activation rows are gathered into it. No staging registers, no LDS
//     store instructions, half the LDS bytes of fp8 operands, and every LDS read
//     is one conflict-free 1 KB access.
//   * Each wave widens its operands to fp8 after its LDS read (three operations
//     per 8 codes) and dequantizes each group's exact products with the
//     column's factor s * 2^18 (or fp32(s / 14) * 2^18 in a residual group).
//   * Residual blocks: a wave's 64 columns lie in one block row, so whether a
//     group holds a chosen block is the same for the whole wave (a scalar
//     branch). Such a group takes a second MFMA per subtile on the residual
//     codes, which the wave loads from memory one group ahead (zero for a
//     half-group without a chosen block); the MFMA accumulates them onto 14 P,
//     giving T = 14 P + Pr exactly, before the dequant.
//   * The loads of group g+1 are issued right after group g's LDS reads and
//     complete during its MFMAs: one wait and one barrier per group.
// ===========================================================================
constexpr int kPM = 128, kPN = 128;
typedef __attribute__((address_space(3))) void lds_void_t;

template <bool RES, bool DUMP, int OUTMODE>
__global__ __launch_bounds__(256, DUMP ? 1 : 2) void k_gemm_prefill(GemmArgs a) {
    __shared__ __align__(16) uint8_t tiles[2][2][8][1024];          // [stage][A, B][subtile][lane * 16]
    __shared__ int tab[RES ? 2 * 2 * kMaxGroups : 1];                // [2 block rows][2G]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, kg = lane >> 4;
    const int wm = wave >> 1, wn = wave & 1;
    const int tiles_n = (a.N + kPN - 1) / kPN;
    const int m0 = (blockIdx.x / tiles_n) * kPM, n0 = (blockIdx.x % tiles_n) * kPN;
    const int G = a.K / kGroup, G4 = (G + 3) / 4, nbc = 2 * G;
    const int br0 = n0 / a.bn;

    // zipper tables of the tile's block rows (one or two), gathered once
    if (RES) {
        for (int i = tid; i < 2 * nbc; i += 256) tab[i] = -1;
        __syncthreads();
        zip_table(a, br0, 0, nbc, tab, tid, 256);
        if ((n0 + kPN - 1) / a.bn != br0 && n0 + 64 < a.N) zip_table(a, br0 + 1, 0, nbc, tab + nbc, tid, 256);
        __syncthreads();
    }

    // Loads go through buffer resources with a per-group base: 32-bit lane offsets
    // stay small, and rows past M or subtiles past N fall outside the range and
    // read zero (their outputs are never stored). Wave w loads subtiles 2w and
    // 2w+1 of both operands.
    const int nsub = min(a.N / 16 - n0 / 16, 8);                    // column subtiles of this tile
    const uint32_t a_range = static_cast<uint32_t>(min(a.M - m0, kPM)) * 64u;
    const uint32_t b_range = static_cast<uint32_t>(nsub - 1) * static_cast<uint32_t>(G) * 1024u + 1024u;
    uint32_t aoff[2], boff[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int st = 2 * wave + u;
        aoff[u] = static_cast<uint32_t>(16 * st + li) * 64u + kg * 16u;
        boff[u] = static_cast<uint32_t>(st) * static_cast<uint32_t>(G) * 1024u + lane * 16u;
    }
    auto issue = [&](int g, int stage) {
        const __amdgpu_buffer_rsrc_t ra = buf_rsrc(a.xq + (static_cast<int64_t>(g) * a.M + m0) * 64, a_range);
        const __amdgpu_buffer_rsrc_t rb = buf_rsrc(a.wq + wq_tile(n0 >> 4, G, g), b_range);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int st = 2 * wave + u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void_t*)&tiles[stage][0][st][0], 16, aoff[u], 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void_t*)&tiles[stage][1][st][0], 16, boff[u], 0, 0, 0);
        }
    };
    // the lane's four column scales of group g: one 16-bit load each
    const __amdgpu_buffer_rsrc_t rs =
        buf_rsrc(a.sw + static_cast<int64_t>(n0 >> 4) * G4 * 64, static_cast<uint32_t>(nsub) * static_cast<uint32_t>(G4) * 128u);
    const uint32_t soff = (static_cast<uint32_t>(wn * 4) * static_cast<uint32_t>(G4) * 64u + li * 4u) * 2u;
    auto scales = [&](int g, uint16_t (&sc)[4]) {
        const int gs = ((g >> 2) * 64 + (g & 3)) * 2;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            sc[j] = __builtin_amdgcn_raw_buffer_load_b16(rs, soff + static_cast<uint32_t>(j) * static_cast<uint32_t>(G4) * 128u, gs, 0);
    };

    // this wave's residual payload: its 64 columns' block row, as a buffer range
    // (offsets past it read zero), and the lane's row in it for column subtile j
    __amdgpu_buffer_rsrc_t rsrc = buf_rsrc(a.wq, 0u);
    int wtab = 0, wlo = 0;
    uint32_t rrow0 = 0;
    if (RES) {
        const int wc0 = n0 + wn * 64;
        if (wc0 < a.N) {
            const int brw = wc0 / a.bn;
            wtab = (brw - br0) * nbc;
            wlo = clampi(a.row_ptr[brw], 0, a.nnz);
            const int whi = clampi(a.row_ptr[brw + 1], wlo, a.nnz);
            rsrc = buf_rsrc(whi > wlo ? a.rq + static_cast<int64_t>(wlo) * a.bn * 32 : a.wq,
                            static_cast<uint32_t>(whi - wlo) * static_cast<uint32_t>(a.bn) * 32u);
        }
        rrow0 = static_cast<uint32_t>((wc0 + li) % a.bn);
    }
    // residual codes of group g for this wave's columns; returns whether the wave
    // has a chosen block in the group (the same in every lane)
    auto fetch_res = [&](int g, uint4 (&rr)[4]) -> bool {
        const int j0 = __builtin_amdgcn_readfirstlane(tab[wtab + 2 * g]);
        const int j1 = __builtin_amdgcn_readfirstlane(tab[wtab + 2 * g + 1]);
        if (j0 < 0 && j1 < 0) return false;
        const int jb = kg < 2 ? j0 : j1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t off = jb >= 0 ? ((jb - wlo) * static_cast<uint32_t>(a.bn) + rrow0 + 16 * j) * 32u + (kg & 1) * 16u
                                         : 0xFFFFFFF0u;
            rr[j] = buf_load16(rsrc, off);
        }
        return true;
    };

    float acc[4][4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.0f;
    auto dump = [&](int g, int i, int j, int r, int T) {
        const int m = m0 + wm * 64 + i * 16 + kg * 4 + r;
        const int nn = n0 + wn * 64 + j * 16 + li;
        if (m < a.M && nn < a.N) a.acc_dump[(static_cast<int64_t>(m) * a.N + nn) * G + g] = T;
    };

    uint16_t sc[4];
    uint4 rr[4];
    bool res_cur = false;
    issue(0, 0);
    scales(0, sc);
    if (RES) res_cur = fetch_res(0, rr);
    __builtin_amdgcn_s_waitcnt(0);   // all counters: the direct loads are not tracked by the barrier's fence
    __syncthreads();
    for (int g = 0; g < G; ++g) {
        const int stage = g & 1;
        uint4 araw[4], braw[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) araw[i] = *reinterpret_cast<const uint4*>(&tiles[stage][0][wm * 4 + i][lane * 16]);
#pragma unroll
        for (int j = 0; j < 4; ++j) braw[j] = *reinterpret_cast<const uint4*>(&tiles[stage][1][wn * 4 + j][lane * 16]);
        const bool res = RES && res_cur;
        float f[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float s = f16_bits_to_f32(sc[j]);
            f[j] = res ? (s / 14.0f) * kF8Unit : s * kF8Unit;
        }
        // the next group's loads (the last step re-loads group G-1 into the idle stage)
        const int gn = min(g + 1, G - 1);
        issue(gn, stage ^ 1);
        scales(gn, sc);
        // next group's residual codes: now if this group does not use the
        // registers, else after its residual MFMAs
        bool res_next = false;
        if (RES && !res && g + 1 < G) res_next = fetch_res(g + 1, rr);
        v8i av[4], bv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) av[i] = f8_operand(araw[i]);
#pragma unroll
        for (int j = 0; j < 4; ++j) bv[j] = f8_operand(braw[j]);
        if (res) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const v8i rv = f8_operand(rr[j]);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const v4f p = mfma_f8(av[i], bv[j], v4f{0.0f, 0.0f, 0.0f, 0.0f});
                    // T = 14 P + Pr: the residual MFMA accumulates onto 14 P (exact:
                    // every partial sum is a multiple of 2^-18 far below 2^6)
                    const v4f t = mfma_f8(av[i], rv, p * 14.0f);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        acc[i][j][r] = fmaf(f[j], t[r], acc[i][j][r]);
                        if (DUMP) dump(g, i, j, r, static_cast<int>(t[r] * kF8Unit));
                    }
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const v4f p = mfma_f8(av[i], bv[j], v4f{0.0f, 0.0f, 0.0f, 0.0f});
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        acc[i][j][r] = fmaf(f[j], p[r], acc[i][j][r]);
                        if (DUMP) dump(g, i, j, r, 14 * static_cast<int>(p[r] * kF8Unit));
                    }
                }
        }
        if (RES && res && g + 1 < G) res_next = fetch_res(g + 1, rr);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        res_cur = res_next;
    }

#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int nn = n0 + wn * 64 + j * 16 + li;
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
    const int G = a.K / kGroup, G4 = (G + 3) / 4, nbc = a.K / kBk;
    const int n0 = blockIdx.x * 16, n = n0 + li;
    const int br = n0 / a.bn, rrow = n - br * a.bn;
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
            if (ma < a.M) av = *reinterpret_cast<const uint2*>(a.xq + xq_row(g, a.M, ma) + (kb & 1) * 32 + kg * 8);
            const uint2 rv =
                *reinterpret_cast<const uint2*>(a.rq + (static_cast<int64_t>(p) * a.bn + rrow) * 32 + kg * 8);
            // a block is 64 inputs: each lane's 16 codes fill half of the fp8
            // operand, the other half is zero in both operands
            const v8i aop = v8i{(int)f8_even(av.x), (int)f8_odd(av.x), (int)f8_even(av.y), (int)f8_odd(av.y), 0, 0, 0, 0};
            const v8i bop = v8i{(int)f8_even(rv.x), (int)f8_odd(rv.x), (int)f8_even(rv.y), (int)f8_odd(rv.y), 0, 0, 0, 0};
            const v4f c = mfma_f8(aop, bop, v4f{0.0f, 0.0f, 0.0f, 0.0f});
            const float sr = f16_bits_to_f32(a.sw[sw_index(n, G4, g)]) / 14.0f;
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] = fmaf(sr * kF8Unit, c[r], acc[r]);
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
static hipError_t go_decode(const GemmArgs& a, hipStream_t st) {
    const DecodePlan p = plan_decode(a.M, a.N, a.K);
    k_gemm_decode<MT, RES, DUMP, OUT><<<dim3(a.N / 16), dim3(64 * p.nw), 0, st>>>(a);
    return hipGetLastError();
}

template <bool RES, bool DUMP, int OUT>
static hipError_t go_prefill(const GemmArgs& a, hipStream_t st) {
    const int tiles = ((a.M + kPM - 1) / kPM) * ((a.N + kPN - 1) / kPN);
    k_gemm_prefill<RES, DUMP, OUT><<<dim3(tiles), dim3(256), 0, st>>>(a);
    return hipGetLastError();
}

template <bool RES, bool DUMP, int OUT>
static hipError_t go(const GemmArgs& a, hipStream_t st) {
    if (a.M <= 16) return go_decode<1, RES, DUMP, OUT>(a, st);
    if (a.M <= 32) return go_decode<2, RES, DUMP, OUT>(a, st);
    return go_prefill<RES, DUMP, OUT>(a, st);
}

// ---------------------------------------------------------------------------
// Decode plan: waves per workgroup. The grid has one workgroup per 16 columns;
// about 2048 waves in total keep enough loads in flight on all 256 CUs, with at
// least one quad per wave. The plan depends on (M, N, K) only, so the fused and
// the dense-only kernels of a shape sum in the same order.
// ---------------------------------------------------------------------------
DecodePlan plan_decode(int M, int N, int K) {
    (void)M;
    const int G4 = (K / kGroup + 3) / 4, subtiles = N / 16;
    int nw = subtiles > 0 ? (2048 + subtiles - 1) / subtiles : 1;
    nw = std::max(1, std::min(nw, std::min(kMaxDecodeWaves, G4)));
    return DecodePlan{nw};
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
