// ZipperEngine on gfx950: the fused dense + sparse-residual W4A4 GEMM.
//
// MosaicQuant technical summary (gist.science), Methodology 3 "ZipperEngine":
// the sparse-residual product is computed inside the dense 4-bit GEMM kernel, in
// a tiled pipeline, so activations are not reloaded and partial outputs are not
// merged by a second kernel. Methodology 1 fixes both parts at 4 bits.
//
// Arithmetic per 128-wide K group g (the weight scale group):
//   * base nibbles wq and activation nibbles xq arrive as 16-byte vector loads
//     (tiled wq and group-major xq: one contiguous 1 KB run per wavefront load);
//   * two masks turn a packed code word into fp8 (e4m3) MFMA operand bytes: code
//     c in [-7, 7] is the subnormal c * 2^-9 (see mq_device.h). gfx950 has no
//     int4 MFMA; the fp8 ones take 128 (16 x 16) or 64 (32 x 32) inputs per
//     instruction at the int8 rate and return fp32;
//   * every product is a multiple of 2^-18 and a group sum is at most
//     128 * 49 = 6272 units in magnitude (T = 14 P + Pr at most 15 * 6272), far
//     below 2^24, so the fp32 MFMA result is the exact integer sum times 2^-18;
//   * the chosen residual blocks are found from the dense block map (one
//     coalesced load of a wave's entries, issued ahead of its operand loads in
//     the decode kernel) or by walking the block row's CSR list; a chosen 64-wide
//     block costs one more MFMA per output tile, giving Pr exactly. The decode
//     kernel walks them in step with g (the "zipper"), on the same activation
//     operands; the prefill kernel multiplies them after all groups;
//   * each group is dequantized into an fp32 accumulator: acc += s * 2^18 * P,
//     and for a group with chosen blocks acc += fp32(s / 14) * 2^18 * (14 P + Pr)
//     (decode kernel); the prefill kernel adds acc += fp32(s / 14) * 2^18 * Pr per
//     chosen block once every group's dense part is in;
//   * the epilogue multiplies by the token scale sx and stores bf16 (RNE) or fp32.
// The debug build (acc_dump) writes every group's exact T = 14 P + Pr.
#include <algorithm>
#include <cmath>

#include "mq_device.h"
#include "mq_internal.h"
#include "mq_quant.h"

namespace mq {

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
// K into runs of 4-group quads (16 waves per workgroup on layers of at most 4096
// columns, else about 2048 waves per launch; see plan_decode). Each wave streams
// its groups in steps of two (one for the two-row-tile residual variant) with the
// next step's loads (weights, activations, residual rows, scales) in flight while
// the current step is multiplied, then the waves' partial tiles are summed through
// LDS in wave order, so results do not depend on timing. Load latency and the
// vector memory pipeline, not HBM bytes, limit this shape class: every load
// instruction counts, hence 1 KB per instruction for weights and activations.
// ===========================================================================
constexpr int kMaxDecodeWaves = 16;
static_assert(kMaxDecodeWaves <= kQaMaxWaves, "the quantizing workgroups run with the decode block size");
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

// Added to every offset of a step past the wave's groups: the loads fall outside
// their buffers and read zero without touching memory. The step after the last is
// fetched that way rather than skipped, so that no load depends on a branch: the
// loads of a wave complete in issue order, and a load issued on one path only
// would make the compiler wait for all of them before the next step's products.
constexpr uint32_t kDeadStep = 0x80000000u;

// activations of the step starting at group g0 (groups past the last read zero
// through the range check)
template <int MT, int QS>
__device__ __forceinline__ void dec_fetch_x(DecStep<MT, QS>& st, const DecSrc& src, int g0, uint32_t dead) {
#pragma unroll
    for (int u = 0; u < QS; ++u)
#pragma unroll
        for (int t = 0; t < MT; ++t) st.x[t][u] = buf_load16(src.x, ((g0 + u) * src.xstride + src.xrow[t]) | dead);
}

// base tiles, activations and scales of the step starting at group g0; X = false
// leaves the activations to a later dec_fetch_x
template <int MT, int QS, bool X = true>
__device__ __forceinline__ void dec_fetch_main(DecStep<MT, QS>& st, const DecSrc& src, int g0, int lane,
                                               uint32_t dead) {
#pragma unroll
    for (int u = 0; u < QS; ++u) {
        const uint32_t g = g0 + u;
        st.w[u] = buf_load16(src.w, (g * 1024u + lane * 16u) | dead);
        if (X) {
#pragma unroll
            for (int t = 0; t < MT; ++t) st.x[t][u] = buf_load16(src.x, (g * src.xstride + src.xrow[t]) | dead);
        }
    }
    const uint32_t so = ((g0 >> 2) * 128u + (lane & 15) * 8u + (g0 & 3) * 2u) | dead;
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
// position (or -1); lanes 0-31 take the group's first block, 32-63 the second.
// Groups from ge on (past the wave's own) fetch none.
template <int MT, int QS, bool RES>
__device__ __forceinline__ void dec_fetch_res(DecStep<MT, QS>& st, const GemmArgs& a, const DecSrc& src,
                                              const int* tab, int rrow, int ge, int g0, int lane) {
    const int kg = lane >> 4;
    st.rg = 0;
#pragma unroll
    for (int u = 0; u < QS; ++u) {
        const int g = g0 + u;
        st.r[u] = make_uint4(0, 0, 0, 0);
        if (RES && g < ge) {
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
__device__ __forceinline__ void dec_compute(const DecStep<MT, QS>& st, const GemmArgs& a, int n, int G, int ge,
                                            int g0, int lane, float (&acc)[MT][4]) {
    const int kg = lane >> 4;
#pragma unroll
    for (int u = 0; u < QS; ++u) {
        const int g = g0 + u;
        if (g >= ge) break;
        const float sc = f16_bits_to_f32(static_cast<uint16_t>(st.s[u >> 1] >> (16 * (u & 1))));
        const bool res = RES && ((st.rg >> u) & 1);
        if (res) {
            // the base products of both row tiles first, then the residual MFMAs
            // accumulating onto 14 P (T = 14 P + Pr, exact): the base and the
            // residual operands are never live together
            const float fr = div14(sc) * kF8Unit;
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

// The variant that quantizes its own activations (QX): the first M workgroups each
// quantize one token (the same arithmetic as the stand-alone kernel) into xq / sx
// and then count themselves done; the column workgroups wait for that count
// before their first activation load (their first weights, scales, residual rows
// and zipper table are already on the way). Workgroups are dispatched in index
// order, so the quantizing ones always start first and finish without waiting on
// anything: the wait ends. (It is also bounded: after well under a few seconds a
// flag is raised in sync[2] and the workgroup goes on.)
// Each XCD has its own L2, which may hold lines of xq / sx that are not yet
// current, so a reader must acquire at device scope; that acquire invalidates the
// whole L2 of its XCD, and one per column workgroup (hundreds per call) costs more
// than the GEMM. So only the first L = min(16, C) of the C column workgroups
// (the leaders, dispatched before the rest) take it, once the count is complete;
// each then raises the ready flag of its own XCD (XCC id from the hardware) and
// checks in. Any other workgroup goes on once its XCD's flag is up; if every
// leader has checked in and none ran on its XCD, it takes the acquire itself (so
// the result does not depend on how workgroups are spread over XCDs). No
// workgroup of the launch loads xq / sx before that point and the launch starts
// with invalidated L1s, so an L1 can hold of them only bytes its own CU's
// quantizing workgroup stored (already final), and every other line any CU loads
// is filled after an invalidation of its L2 that followed the count.
// Atomics that return a value keep their workgroup resident until memory answers,
// which under a full HBM queue is microseconds per workgroup, so the column
// workgroups use none: waits are plain polling loads, and at the end each adds
// one to a done count (one of 16, each on its own 128-byte line) without waiting
// for it or for its output stores. The last column workgroup waits for the other
// C - 1 counts and then resets the counts and flags, so every completed call
// leaves the words zero. Every workgroup's reads and stores of the words are
// complete before its done count is sent, so the reset cannot be seen by any of
// them.
constexpr int kSpinLimit = 1 << 20;
constexpr int kSyncLine = 32;      // int32 words per 128-byte line
constexpr int kSyncSlots = 16;     // XCC ids 0..15; also the number of leaders
// line 0: [0] quantized tokens, [2] give-up flag, [3] leaders checked in;
// line 1 + i: slot i's ready flag and done count
enum { kSyncCount = 0, kSyncGaveUp = 2, kSyncLeaders = 3, kSyncReady = 0, kSyncDone = 1 };
static_assert(kSyncLine * (1 + kSyncSlots) == kSyncWords, "sync word layout");

__device__ __forceinline__ int* sync_slot(int* sync, int xcc) { return sync + kSyncLine * (1 + xcc); }

__device__ __forceinline__ void wait_all_memory() { __builtin_amdgcn_s_waitcnt(0xF70); }   // vmcnt(0)

__device__ __forceinline__ bool spin_until(const int* p, int target, int* gave_up) {
    for (int it = 0; __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target; ++it) {
        if (it >= kSpinLimit) {
            __hip_atomic_store(gave_up, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return false;
        }
        __builtin_amdgcn_s_sleep(8);
    }
    return true;
}

// The protocol's three parts.
// Producer: the calling workgroup (every thread) quantizes token tok and counts it.
__device__ __forceinline__ void qx_produce(const GemmArgs& a, int tok, int tid, float* qred) {
    quant_act_row(a.x, a.x_bf16, a.M, a.K, nullptr, a.xq_w, a.sx_w, tok, tid, blockDim.x, qred);
    // each wave's stores have reached its XCD's L2 before the barrier; the count's
    // device-scope release then writes that L2 back
    wait_all_memory();
    __syncthreads();
    if (tid == 0) __hip_atomic_fetch_add(&a.sync[kSyncCount], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// Column workgroup ci (dispatch order) of C, thread 0 only: returns once every
// token is counted and this XCD's L2 holds no stale activations. The caller then
// holds the workgroup at a barrier before its first activation load.
__device__ __forceinline__ void qx_wait(int* sy, int M, int ci, int C) {
    int* const gave_up = &sy[kSyncGaveUp];
    const int L = min(kSyncSlots, C);
    // XCC id: hardware register 20, bits 3:0 (uniform over the workgroup)
    const int xcc = static_cast<int>(__builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20)) & (kSyncSlots - 1);
    int* const ready = &sync_slot(sy, xcc)[kSyncReady];
    if (ci < L) {
        spin_until(&sy[kSyncCount], M, gave_up);
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");   // this XCD's L2 holds no stale activations
        __hip_atomic_store(ready, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        wait_all_memory();   // the flag is up before the check-in
        __hip_atomic_fetch_add(&sy[kSyncLeaders], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    } else {
        bool up = false;
        for (int it = 0;; ++it) {
            if (__hip_atomic_load(ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) { up = true; break; }
            if (__hip_atomic_load(&sy[kSyncLeaders], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= L) break;
            if (it >= kSpinLimit) {
                __hip_atomic_store(gave_up, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            __builtin_amdgcn_s_sleep(8);
        }
        // every leader has checked in, so every flag that will be raised is up
        if (!up && !__hip_atomic_load(ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");   // no leader ran on this XCD
    }
}

// Column workgroup ci of C, thread 0 only, after its last use of the counters:
// counts itself done; the last one waits for the others and clears the words.
__device__ __forceinline__ void qx_done(int* sy, int ci, int C) {
    // A follower's accesses to the words were loads whose values it has used, so
    // they are complete; a leader's check-in must land before its done count, so
    // it waits (for its output stores too: 16 workgroups only).
    if (ci < min(kSyncSlots, C)) wait_all_memory();
    if (ci < C - 1) {
        __hip_atomic_fetch_add(&sync_slot(sy, ci & (kSyncSlots - 1))[kSyncDone], 1, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    } else {
        // the last column workgroup: every other one was dispatched before it and
        // waits on nothing it holds, so their done counts all arrive
        for (int it = 0;; ++it) {
            int total = 0;
            for (int i = 0; i < kSyncSlots; ++i)
                total += __hip_atomic_load(&sync_slot(sy, i)[kSyncDone], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (total >= C - 1) break;
            if (it >= kSpinLimit) {
                __hip_atomic_store(&sy[kSyncGaveUp], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            __builtin_amdgcn_s_sleep(1);   // the launch ends with this wait: poll closely
        }
        for (int i = 0; i < kSyncSlots; ++i) {
            __hip_atomic_store(&sync_slot(sy, i)[kSyncReady], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&sync_slot(sy, i)[kSyncDone], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __hip_atomic_store(&sy[kSyncLeaders], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&sy[kSyncCount], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

template <int MT, bool RES, bool DUMP, int OUTMODE, bool QX = false>
__global__ __launch_bounds__(64 * kMaxDecodeWaves) void k_gemm_decode(GemmArgs a) {
    // two groups per step; one for the residual variant with two row tiles,
    // which keeps its registers within four waves per SIMD
    constexpr int QS = (RES && MT == 2) ? 1 : 2;
    // per-wave partial sums for the final reduction: nw * MT * 256 floats, sized at
    // launch so that a plan with few waves does not pay LDS (occupancy) for many
    extern __shared__ float red[];
    __shared__ int tab[RES ? 8 * (kMaxGroups / 4) : 1];   // column block -> CSR position
    // the wave index as a scalar: the group loop's bounds and exits are then
    // wave-uniform branches, not exec masks (a masked exit merges into the loop
    // header and makes every load of the previous step look outstanding there)
    const int tid = threadIdx.x, lane = tid & 63, nw = blockDim.x >> 6;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (QX) {
        __shared__ float qred[kQaMaxWaves];
        if (static_cast<int>(blockIdx.x) < a.M) {
            qx_produce(a, blockIdx.x, tid, qred);
            return;
        }
    }
    const int G = a.K / kGroup, G4 = (G + 3) / 4;
    const int nt = blockIdx.x - (QX ? a.M : 0), n0 = nt * 16, n = n0 + (lane & 15);
    const int br = n0 / a.bn, rrow = n - br * a.bn;
    const int q0 = wave * G4 / nw, q1 = (wave + 1) * G4 / nw;       // this wave's quads
    const int gb = 4 * q0, ge = min(4 * q1, G);                      // and groups
    float acc[MT][4];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[t][r] = 0.0f;

    // block positions come from the dense block map when there is one (then the
    // payload is addressed from its start), else from the block row's CSR list
    const bool map = a.rmap != nullptr;
    const int lo = RES && !map ? clampi(a.row_ptr[br], 0, a.nnz) : 0;
    const int hi = RES ? (map ? a.nnz : clampi(a.row_ptr[br + 1], lo, a.nnz)) : 0;
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
    if (gb < ge) {
        // The zipper table of this wave's column blocks [2 gb, 2 ge), built by the
        // wave alone: no workgroup barrier. A wavefront's LDS operations complete in
        // issue order, so the fills and the later reads need no wait between lanes.
        // With a block map the wave's first 64 entries are requested before its
        // operands: loads return in issue order, so the table (and the residual
        // fetch that needs it) waits for that one load, not for the operands. The
        // index is clamped into the wave's range, so every lane loads a map entry.
        // (Everything stays inside this branch: a load left in flight across the
        // join would make the compiler drain every load before reusing its register.)
        const int kb0 = 2 * gb, kb1 = 2 * ge;
        int map0 = -1;
        if (RES && map) map0 = a.rmap[static_cast<int64_t>(br) * (2 * G) + min(kb0 + lane, kb1 - 1)];
        dec_fetch_main<MT, QS, !QX>(s0, src, gb, lane, 0u);
        if (RES) {
            if (map) {
                // out-of-range positions read as "no block"
                if (kb0 + lane < kb1) tab[kb0 + lane] = (map0 >= 0 && map0 < a.nnz) ? map0 : -1;
                for (int i = kb0 + lane + 64; i < kb1; i += 64) {
                    const int v = a.rmap[static_cast<int64_t>(br) * (2 * G) + i];
                    tab[i] = (v >= 0 && v < a.nnz) ? v : -1;
                }
                __builtin_amdgcn_wave_barrier();
            } else {
                // from the block row's CSR list: -1 everywhere, then the positions
                for (int i = kb0 + lane; i < kb1; i += 64) tab[i] = -1;
                __builtin_amdgcn_wave_barrier();
                for (int i = lo + lane; i < hi; i += 64) {
                    const int kb = a.col_idx[i];
                    if (kb >= kb0 && kb < kb1) tab[kb] = i;
                }
                __builtin_amdgcn_wave_barrier();
            }
            dec_fetch_res<MT, QS, RES>(s0, a, src, tab, rrow, ge, gb, lane);
        }
    }
    const int C = QX ? static_cast<int>(gridDim.x) - a.M : 0;   // column workgroups
    if (QX) {
        // the second step's weights, scales and residual rows go out before the wait too
        if (gb < ge) {
            const uint32_t d1 = gb + QS < ge ? 0u : kDeadStep;
            dec_fetch_main<MT, QS, false>(s1, src, gb + QS, lane, d1);
            if (RES) dec_fetch_res<MT, QS, RES>(s1, a, src, tab, rrow, ge, gb + QS, lane);
        }
        if (tid == 0) qx_wait(a.sync, a.M, nt, C);
        __syncthreads();
        if (gb < ge) {
            dec_fetch_x<MT, QS>(s0, src, gb, 0u);
            dec_fetch_x<MT, QS>(s1, src, gb + QS, gb + QS < ge ? 0u : kDeadStep);
        }
    }
    // Every fetch of the steady loop is for a step of the wave's own: no load is
    // left to a branch inside it, and the loop has its one exit at the top (an
    // exit between the halves would give the loop header a path on which the
    // second half's loads were never issued). The last one or two steps follow
    // it. s0 holds step g on entry to both.
    int g = gb;
    auto steady = [&]() {
        for (; g + 2 * QS < ge; g += 2 * QS) {
            dec_fetch_main<MT, QS>(s1, src, g + QS, lane, 0u);
            if (RES) dec_fetch_res<MT, QS, RES>(s1, a, src, tab, rrow, ge, g + QS, lane);
            dec_compute<MT, QS, RES, DUMP>(s0, a, n, G, ge, g, lane, acc);
            dec_fetch_main<MT, QS>(s0, src, g + 2 * QS, lane, 0u);
            if (RES) dec_fetch_res<MT, QS, RES>(s0, a, src, tab, rrow, ge, g + 2 * QS, lane);
            // The residual kernel with two row tiles takes every load in before the
            // second step of each pair (s_waitcnt vmcnt(0), expcnt and lgkmcnt left
            // at their maxima): one step in flight at all times measured slower on
            // the layers whose chosen blocks cluster in a few block rows.
            if constexpr (RES && MT == 2) __builtin_amdgcn_s_waitcnt(0x0F70);
            dec_compute<MT, QS, RES, DUMP>(s1, a, n, G, ge, g + QS, lane, acc);
        }
        if (g + QS < ge) {
            dec_fetch_main<MT, QS>(s1, src, g + QS, lane, 0u);
            if (RES) dec_fetch_res<MT, QS, RES>(s1, a, src, tab, rrow, ge, g + QS, lane);
            dec_compute<MT, QS, RES, DUMP>(s0, a, n, G, ge, g, lane, acc);
            dec_compute<MT, QS, RES, DUMP>(s1, a, n, G, ge, g + QS, lane, acc);
        } else if (g < ge) {
            dec_compute<MT, QS, RES, DUMP>(s0, a, n, G, ge, g, lane, acc);
        }
    };
    if (!QX) {
        steady();
    } else if (g + 2 * QS < ge) {
        // step 1 was fetched before the wait: the first two steps, then the loop
        // (entered only here, so its header never sees step 1 unconsumed)
        dec_compute<MT, QS, RES, DUMP>(s0, a, n, G, ge, g, lane, acc);
        dec_fetch_main<MT, QS>(s0, src, g + 2 * QS, lane, 0u);
        if (RES) dec_fetch_res<MT, QS, RES>(s0, a, src, tab, rrow, ge, g + 2 * QS, lane);
        dec_compute<MT, QS, RES, DUMP>(s1, a, n, G, ge, g + QS, lane, acc);
        g += 2 * QS;
        steady();
    } else if (g < ge) {
        dec_compute<MT, QS, RES, DUMP>(s0, a, n, G, ge, g, lane, acc);
        dec_compute<MT, QS, RES, DUMP>(s1, a, n, G, ge, g + QS, lane, acc);   // (nothing past ge)
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
    if (QX && tid == 0) qx_done(a.sync, nt, C);
}

typedef float v16f __attribute__((ext_vector_type(16)));

__device__ __forceinline__ v16f mfma32_f8(v8i a, v8i b, v16f c) {
    // format selectors 0/0 (e4m3 both operands), no block scales
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Workgroup b of a grid of T runs on XCD b % 8 (the dispatcher deals workgroups
// round-robin over the eight XCDs). Give XCD x the contiguous tile range
// [x q + min(x, r), ...) of q + (x < r) tiles (q = T / 8, r = T % 8), walked in
// order: a bijection of [0, T) that keeps neighbouring tiles on one L2.
__device__ __forceinline__ int xcd_tile(int b, int T) {
    const int q = T >> 3, r = T & 7, x = b & 7, l = b >> 3;
    return x * q + min(x, r) + l;
}

// ===========================================================================
// Wide prefill kernel, M > 32: a workgroup of NWN waves owns 96 tokens x 64 NWN
// output columns (32 x 64 NWN for the mid-size tile), and each wave all of its
// tokens for its own 64 columns (3 x 2 tiles of 32 x 32, 32 x 32 x 64 fp8 MFMAs),
// one 128-wide K group per step.
//   * Every weight tile is loaded and widened to fp8 by exactly one wave (straight
//     from memory into registers, a group ahead of its use).
//   * Every activation tile is loaded and widened once per workgroup: the waves
//     split the group's 96 x 64-byte run, widen their part and store it in LDS in
//     MFMA lane order; each operand read is then two conflict-free 1 KB LDS reads.
//     One barrier per group.
//   * Per group and tile: P from two MFMAs (one per 64-input half), then
//     acc += fp32(s) * 2^18 * P.
//   * The chosen blocks of the wave's block row (a wave's 64 columns lie in one
//     block row) are multiplied after the last group, one MFMA per tile on
//     activations the wave loads and widens itself: acc += fp32(s / 14) * 2^18 * Pr.
//     Done inside the K loop, they made every wave wait at each group's barrier for
//     the wave with the most chosen blocks in that group (the waves of a workgroup
//     cover several block rows); after it, that imbalance costs once per tile.
// Per group and wave the VALU work is the 96 dequantizing FMAs, the widening of
// 4 KB of weight nibbles and 1/NWN of the activation widening, against 12 MFMAs:
// close to balanced, so two waves per SIMD keep the MFMA pipe fed. 96 rows (not
// 128) leave the registers for the prefetched operands without spilling.
// ===========================================================================
constexpr int kWideRowTiles = 3;    // 32-row MFMA tiles per wave in the prefill tile
constexpr int kMidRowTiles = 1;     // ... in the mid-size tile (32 < M <= kMidMaxM)
constexpr int kMidMaxM = 384;       // measured on the LLaMA3-8B MLP up layer: the mid
                                    // tile 2.3x faster at M = 64, 1.5x at 384, equal at 512
constexpr int kMidWaves = 2;


template <int NWN, int MTW, bool RES, bool DUMP, int OUTMODE>
__global__ __launch_bounds__(64 * NWN, DUMP ? 1 : 2) void k_gemm_wide(GemmArgs a, int n_begin, int tiles_n) {
    constexpr int kMT = MTW;            // 32-row MFMA tiles per wave
    constexpr int kWM = 32 * kMT;       // tokens per workgroup tile
    constexpr int kRuns = kWM / 16;                   // 1 KB activation runs per group
    constexpr int kXU = (kRuns + NWN - 1) / NWN;      // runs per wave (run wave + NWN u)
    constexpr int kStages = 2;
    // [stage][32-row tile][half 2][part 2][lane 64][16 B]
    __shared__ __align__(16) uint8_t xs[kStages][kMT][2][2][1024];
    __shared__ __align__(16) uint8_t xspare[(kXU * NWN > kRuns) ? 2048 : 16];
    __shared__ int tab[RES ? NWN * 2 * kMaxGroups : 1];     // per wave: column block -> CSR position
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lc = lane & 31, lh = lane >> 5;
    // Tile order: workgroup b runs on XCD b % 8, and each XCD takes a contiguous
    // range of tiles ordered column-tile-major, so the workgroups an XCD runs at
    // one time share column tiles (weights) and all token tiles (activations) in
    // that XCD's L2.
    const int tiles_m = (a.M + kWM - 1) / kWM;
    const int t = xcd_tile(static_cast<int>(blockIdx.x), tiles_m * tiles_n);
    const int m0 = (t % tiles_m) * kWM;
    const int n0 = n_begin + (t / tiles_m) * (64 * NWN);
    const int G = a.K / kGroup, G4 = (G + 3) / 4, nbc = 2 * G;
    const int wc0 = n0 + wave * 64;                                   // the wave's first column

    // weights of the wave's 64 columns: four 16-row tiles; tiles past N read zero
    // (one resource per pair of tiles, so that the range check, which covers the
    // per-lane offset, alone decides which lanes read zeros)
    const int wtiles = max(0, min(4, (a.N - wc0) / 16));
    __amdgpu_buffer_rsrc_t rb[2], rs[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int t = max(0, min(2, wtiles - 2 * j));
        rb[j] = buf_rsrc_uniform(a.wq + static_cast<int64_t>((wc0 >> 4) + 2 * j) * G * 1024,
                                 static_cast<uint32_t>(t) * G * 1024u);
        rs[j] = buf_rsrc_uniform(a.sw + static_cast<int64_t>((wc0 >> 4) + 2 * j) * G4 * 64,
                                 static_cast<uint32_t>(t) * G4 * 128u);
    }
    // lane's offset for column tile j, half h of group g: tile 2j + lc/16, row lc%16,
    // chunk 2h + lh, i.e. a per-lane part plus a wave-uniform part (scalar offset)
    const uint32_t bvo = static_cast<uint32_t>(lc >> 4) * G * 1024u + static_cast<uint32_t>((lh * 16 + (lc & 15)) * 16);
    // the lane's fp16 group scale of column tile j: element (tile, g/4, row, g%4)
    const uint32_t svo = (static_cast<uint32_t>(lc >> 4) * G4 * 64u + (lc & 15) * 4u) * 2u;
    auto load_scale = [&](int g, int j) __attribute__((always_inline)) -> uint32_t {
        const uint32_t gc = static_cast<uint32_t>(min(g, G - 1));
        return __builtin_amdgcn_raw_buffer_load_b16(rs[j], svo, (gc >> 2) * 128u + (gc & 3) * 2u, 0);
    };

    // the wave's zipper table (its 64 columns lie in one block row), built by the
    // wave alone: a wavefront's LDS operations complete in issue order
    int* wt = tab + (RES ? wave * nbc : 0);
    __amdgpu_buffer_rsrc_t rr = buf_rsrc_uniform(a.wq, 0u);
    const __amdgpu_buffer_rsrc_t rnull = buf_rsrc_uniform(a.wq, 0u);   // reads zeros
    int wlo = 0, rbase = 0;
    if (RES) {
        const bool map = a.rmap != nullptr;
        const int brw = min(wc0, a.N - 1) / a.bn;
        for (int i = lane; i < nbc; i += 64) {
            int v = -1;
            if (map && wc0 < a.N) {
                v = a.rmap[static_cast<int64_t>(brw) * nbc + i];
                v = (v >= 0 && v < a.nnz) ? v : -1;
            }
            wt[i] = v;
        }
        __builtin_amdgcn_wave_barrier();
        if (wc0 < a.N) {
            wlo = map ? 0 : clampi(a.row_ptr[brw], 0, a.nnz);
            const int whi = map ? a.nnz : clampi(a.row_ptr[brw + 1], wlo, a.nnz);
            for (int i = map ? whi : wlo + lane; i < whi; i += 64) {
                const int kb = a.col_idx[i];
                if (kb >= 0 && kb < nbc) wt[kb] = i;
            }
            rr = buf_rsrc_uniform(whi > wlo ? a.rq + static_cast<int64_t>(wlo) * a.bn * 32 : a.wq,
                                  static_cast<uint32_t>(whi - wlo) * static_cast<uint32_t>(a.bn) * 32u);
            rbase = wc0 % a.bn;   // the wave's first row inside its block
        }
        __builtin_amdgcn_wave_barrier();
    }

    // activation fill: the wave's 1 KB runs of a group (rows R0 + 16 u + lane % 16,
    // 16-byte chunk lane / 16), stored widened at their MFMA operand positions
    // row of run r: 16 r + lane % 16, chunk kc = lane / 16; destination: 32-row
    // tile row / 32, half kc / 2, operand lane row % 32 + 32 (kc % 2)
    const uint32_t xvo = static_cast<uint32_t>(lane & 15) * 64u + static_cast<uint32_t>(lane >> 4) * 16u;
    const int kc = lane >> 4;
    const int xdl = ((kc >> 1) * 2 * 64 + (lane & 15) + 32 * (kc & 1)) * 16;   // per-lane part
    auto xdst = [&](int u) __attribute__((always_inline)) {
        const int row = 16 * (wave + NWN * u);                   // wave-uniform part of the row
        return xdl + ((row >> 5) * 4 * 64 + (row & 31)) * 16;
    };
    auto load_x = [&](int g, uint4 (&L)[kXU]) __attribute__((always_inline)) {
        const int gc = min(g, G - 1);
#pragma unroll
        for (int u = 0; u < kXU; ++u) {
            // this run's 16 rows (rows past M, and runs past the tile, read zero)
            const int r0 = 16 * (wave + NWN * u);
            const __amdgpu_buffer_rsrc_t rx = buf_rsrc_uniform(
                a.xq + (static_cast<int64_t>(gc) * a.M + m0 + r0) * 64,
                static_cast<uint32_t>(r0 < kWM ? max(0, min(a.M - m0 - r0, 16)) : 0) * 64u);
            L[u] = buf_load16(rx, xvo);
        }
    };
    auto store_x = [&](const uint4 (&L)[kXU], int st) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < kXU; ++u) {
            // a run past the tile (zeros) is written to a spare area: no branch
            const v8i v = f8_operand(L[u]);
            uint8_t* d = wave + NWN * u < kRuns ? &xs[st][0][0][0][0] + xdst(u) : &xspare[lane * 16];
            *reinterpret_cast<v4i*>(d) = v4i{v[0], v[1], v[2], v[3]};
            *reinterpret_cast<v4i*>(d + 1024) = v4i{v[4], v[5], v[6], v[7]};
        }
    };
    auto load_w = [&](int g, uint4 (&B)[2][2]) __attribute__((always_inline)) {
        const uint32_t gc = static_cast<uint32_t>(min(g, G - 1));
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int h = 0; h < 2; ++h) B[j][h] = buf_load16s(rb[j], bvo, h * 512u + gc * 1024u);
    };
    // the codes of column tile j of block jb: row rbase + 32 j + lc of the block, bytes
    // 16 lh .. 16 lh + 15 (a per-lane part and a wave-uniform part); no block reads zeros
    const uint32_t rvo = static_cast<uint32_t>(lc * 32 + lh * 16);
    auto load_codes = [&](int jb, int j) __attribute__((always_inline)) {
        const uint32_t so = static_cast<uint32_t>(((jb - wlo) * a.bn + rbase + 32 * j) * 32);
        return buf_load16s(jb >= 0 ? rr : rnull, rvo, jb >= 0 ? so : 0u);
    };
    auto a_operand = [&](int st, int i, int h) __attribute__((always_inline)) {
        const uint8_t* base = &xs[st][i][h][0][0];
        const v4i lo = *reinterpret_cast<const v4i*>(base + lane * 16);
        const v4i hi = *reinterpret_cast<const v4i*>(base + 1024 + lane * 16);
        return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    auto dump_idx = [&](int i, int j, int r, int g) __attribute__((always_inline)) -> int64_t {
        const int m = m0 + i * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
        const int nn = wc0 + j * 32 + lc;
        return (m < a.M && nn < a.N) ? (static_cast<int64_t>(m) * a.N + nn) * G + g : -1;
    };

    v16f acc[kMT][2];
#pragma unroll
    for (int i = 0; i < kMT; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // base pass of group g: operands of stage st, weight nibbles Bn, scale bits sb
    auto compute = [&](int g, int st, const uint4 (&Bn)[2][2], const uint32_t (&sb)[2]) __attribute__((always_inline)) {
        float fs[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) fs[j] = f16_bits_to_f32(static_cast<uint16_t>(sb[j])) * kF8Unit;
        v8i bop[2][2];
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int h = 0; h < 2; ++h) bop[j][h] = f8_operand(Bn[j][h]);
#pragma unroll
        for (int i = 0; i < kMT; ++i) {
            const v8i a0 = a_operand(st, i, 0), a1 = a_operand(st, i, 1);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const v16f z = {};
                v16f p = mfma32_f8(a0, bop[j][0], z);
                p = mfma32_f8(a1, bop[j][1], p);
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = fmaf(fs[j], p[r], acc[i][j][r]);
                if (DUMP) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int64_t d = dump_idx(i, j, r, g);
                        if (d >= 0) a.acc_dump[d] = 14 * static_cast<int>(p[r] * kF8Unit);
                    }
                }
            }
        }
    };
    // Residual blocks, after every group's dense part: the wave's chosen blocks (its
    // 64 columns lie in one block row), each one MFMA per 32 x 32 tile on
    // activations the wave loads itself (16 bytes per lane and row tile, from L2)
    // and widens: acc += fp32(s / 14) * 2^18 * Pr. No barrier follows, so a wave
    // with more chosen blocks than the others delays no one. A chosen entry is
    // packed as (CSR position - wlo) << 11 | column block: a list position is below
    // the block row's 2 G column blocks, a map position below 2^20 (the payload
    // offset check), a column block below 2^11.
    struct TailOps {
        uint32_t s[2];      // fp16 group scale bits, column tiles 0 and 1
        uint4 c[2];         // residual codes, column tiles 0 and 1
        uint4 x[kMT];       // activation codes, row tiles
        int kb;             // column block
    };
    // the activation codes of row tile i, half h of group g for this lane's operand
    // slot: row m0 + 32 i + lc (rows past M read zero), 16-byte chunk 2 h + lh
    auto load_res_x = [&](int g, int h, int i) __attribute__((always_inline)) {
        const int r0 = m0 + 32 * i;
        const __amdgpu_buffer_rsrc_t rx = buf_rsrc_uniform(
            a.xq + (static_cast<int64_t>(g) * a.M + r0) * 64, static_cast<uint32_t>(max(0, min(32, a.M - r0))) * 64u);
        return buf_load16(rx, static_cast<uint32_t>(lc * 64 + (2 * h + lh) * 16));
    };
    // e: (CSR position - wlo) << 11 | column block
    auto tail_fetch = [&](int e, TailOps& T) __attribute__((always_inline)) {
        const int kb = e & 2047, jb = wlo + (e >> 11), g = kb >> 1, h = kb & 1;
        T.kb = kb;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            T.s[j] = load_scale(g, j);
            T.c[j] = load_codes(jb, j);
        }
#pragma unroll
        for (int i = 0; i < kMT; ++i) T.x[i] = load_res_x(g, h, i);
    };
    auto tail_mul = [&](const TailOps& T) __attribute__((always_inline)) {
        const int g = T.kb >> 1;
        float fr[2];
        v8i ra[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            fr[j] = div14(f16_bits_to_f32(static_cast<uint16_t>(T.s[j]))) * kF8Unit;
            ra[j] = f8_operand(T.c[j]);
        }
#pragma unroll
        for (int i = 0; i < kMT; ++i) {
            const v8i aa = f8_operand(T.x[i]);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const v16f z = {};
                const v16f pr = mfma32_f8(aa, ra[j], z);
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = fmaf(fr[j], pr[r], acc[i][j][r]);
                if (DUMP) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int64_t d = dump_idx(i, j, r, g);
                        if (d >= 0) a.acc_dump[d] += static_cast<int>(pr[r] * kF8Unit);
                    }
                }
            }
            // keep the scheduler from hoisting every tile's MFMA (and its 16 result
            // registers) above the dequantization of the earlier tiles
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto residual_blocks = [&]() __attribute__((always_inline)) {
        if constexpr (kMT == 1) {
            // one row tile: the table is compacted in place into the list of chosen
            // entries (every lane reads its entry of a 64-entry chunk before any lane
            // writes, and an entry moves only to an index no later than its own), which
            // is walked with the next block's operands fetched while one is multiplied
            int n = 0;
            for (int c0 = 0; c0 < nbc; c0 += 64) {
                const int v = c0 + lane < nbc ? wt[c0 + lane] : -1;
                const uint64_t chosen = __ballot(v >= 0);
                __builtin_amdgcn_wave_barrier();
                if (v >= 0) {
                    const int below = __builtin_popcountll(chosen & ((uint64_t(1) << lane) - 1));
                    wt[n + below] = ((v - wlo) << 11) | (c0 + lane);
                }
                __builtin_amdgcn_wave_barrier();
                n += __builtin_popcountll(chosen);
            }
            // (the fetch is unconditional, of the last entry again past the end: a
            // fetch under a branch would leave the compiler unsure how many loads are
            // in flight at the join, and it would wait for all of them)
            TailOps t0, t1;
            if (n > 0) {
                tail_fetch(__builtin_amdgcn_readfirstlane(wt[0]), t0);
                for (int q = 0;; q += 2) {
                    tail_fetch(__builtin_amdgcn_readfirstlane(wt[min(q + 1, n - 1)]), t1);
                    tail_mul(t0);
                    if (q + 1 >= n) break;
                    tail_fetch(__builtin_amdgcn_readfirstlane(wt[min(q + 2, n - 1)]), t0);
                    tail_mul(t1);
                    if (q + 2 >= n) break;
                }
            }
        } else {
            // three row tiles: the next block's operands fetched while one is
            // multiplied measured no faster here (206.9 against 207.2 us on the
            // Qwen3-14B prefill shape; a wave's walk overlaps the other workgroup's K
            // loop), so each block's scales and codes go first and each row tile's
            // activations just before its MFMAs; the chosen entries of each 64-entry
            // chunk come from one ballot
            for (int c0 = 0; c0 < nbc; c0 += 64) {
                const int v = c0 + lane < nbc ? wt[c0 + lane] : -1;
                uint64_t chosen = __ballot(v >= 0);
                while (chosen) {
                    const int bit = __builtin_ctzll(chosen);
                    chosen &= chosen - 1;
                    const int jb = __builtin_amdgcn_readlane(v, bit);
                    const int kb = c0 + bit, g = kb >> 1, h = kb & 1;
                    float fr[2];
                    v8i ra[2];
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        fr[j] = div14(f16_bits_to_f32(static_cast<uint16_t>(load_scale(g, j)))) * kF8Unit;
                        ra[j] = f8_operand(load_codes(jb, j));
                    }
#pragma unroll
                    for (int i = 0; i < kMT; ++i) {
                        const v8i aa = f8_operand(load_res_x(g, h, i));
#pragma unroll
                        for (int j = 0; j < 2; ++j) {
                            const v16f z = {};
                            const v16f pr = mfma32_f8(aa, ra[j], z);
#pragma unroll
                            for (int r = 0; r < 16; ++r) acc[i][j][r] = fmaf(fr[j], pr[r], acc[i][j][r]);
                            if (DUMP) {
#pragma unroll
                                for (int r = 0; r < 16; ++r) {
                                    const int64_t d = dump_idx(i, j, r, g);
                                    if (d >= 0) a.acc_dump[d] += static_cast<int>(pr[r] * kF8Unit);
                                }
                            }
                        }
                    }
                }
            }
        }
    };

    // Instruction order of a step's base pass (the scheduler otherwise issues all
    // MFMAs back to back and all dequantizing FMAs after them, so the VALU and the
    // MFMA pipe of a wave take turns): the next group's loads first, then the
    // weight widening, then each row of tiles' LDS reads and MFMAs with VALU work
    // between the MFMAs (the widening of column tile 1 and of the next group's
    // activations under row 0, the previous row's FMAs under the later rows).
    auto schedule_step = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_sched_group_barrier(0x0020, 6, 0);       // loads of group g + 1
        __builtin_amdgcn_sched_group_barrier(0x0002, 24, 0);      // widen column tile 0
        __builtin_amdgcn_sched_group_barrier(0x0100, 4, 0);       // row 0 operands
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x0002, 12, 0);
        }
#pragma unroll
        for (int i = 1; i < kMT; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x0100, 4, 0);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x0002, 8, 0);
            }
        }
        __builtin_amdgcn_sched_group_barrier(0x0002, 40, 0);      // the last row's FMAs
        __builtin_amdgcn_sched_group_barrier(0x0200, 2 * kXU, 0); // activation stores
        __builtin_amdgcn_sched_group_barrier(0x0020, kXU, 0);     // loads of group g + 2
    };

    // Pipeline: step g (stage g % kStages) fetches group g + 2's weights and scales,
    // multiplies group g with the weights fetched during step g - 2, widens group
    // g + 1's activations (fetched during step g - 1) into the other stage and
    // fetches group g + 2's. Unrolled by three so that the weight and scale
    // registers rotate without copies.
    uint4 B0[2][2], B1[2][2], B2[2][2], X[kXU];
    uint32_t S0[2], S1[2], S2[2];
    load_x(0, X);
    load_w(0, B0);
    load_w(1, B1);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        S0[j] = load_scale(0, j);
        S1[j] = load_scale(1, j);
    }
    store_x(X, 0);
    load_x(1, X);
    __syncthreads();
    // step g: weights and scales of group g in Bc/Sc (fetched two steps earlier);
    // group g + 2's go to Bn/Sn, which held group g - 1's
    auto step = [&](int g, const uint4 (&Bc)[2][2], uint4 (&Bn)[2][2], const uint32_t (&Sc)[2],
                    uint32_t (&Sn)[2]) __attribute__((always_inline)) {
        const int st = g % kStages;
        // Each SIMD runs two of these waves. While one issues its MFMAs it takes
        // issue priority over the other, which is then in its loads, widening or
        // barrier: the MFMA pipe idles less (measured: dense 190 -> 179 us on the
        // Qwen3-14B prefill shape).
        __builtin_amdgcn_s_setprio(1);
        load_w(g + 2, Bn);
#pragma unroll
        for (int j = 0; j < 2; ++j) Sn[j] = load_scale(g + 2, j);
        compute(g, st, Bc, Sc);
        __builtin_amdgcn_s_setprio(0);
        store_x(X, (g + 1) % kStages);
        load_x(g + 2, X);
        schedule_step();
        __syncthreads();
    };
    if constexpr (RES || kMT == 1) {
        // one exit, at the top (an exit between steps would give the loop header a
        // path on which the later steps' loads were never issued, and the compiler
        // would wait there for every load in flight); the last one or two steps follow
        int g = 0;
        for (; g + 3 <= G; g += 3) {
            step(g, B0, B2, S0, S2);
            step(g + 1, B1, B0, S1, S0);
            step(g + 2, B2, B1, S2, S1);
        }
        if (g < G) {
            step(g, B0, B2, S0, S2);
            if (g + 1 < G) step(g + 1, B1, B0, S1, S0);
        }
    } else {
        // the dense-only wide tile: the two peeled steps above make it spill
        for (int g = 0; g < G; g += 3) {
            step(g, B0, B2, S0, S2);
            if (g + 1 >= G) break;
            step(g + 1, B1, B0, S1, S0);
            if (g + 2 >= G) break;
            step(g + 2, B2, B1, S2, S1);
        }
    }
    if (RES) residual_blocks();

    // Epilogue: y = acc * sx, bf16 or fp32 (rows past M and columns past N skipped)
    const __amdgpu_buffer_rsrc_t rsx = buf_rsrc_uniform(a.sx + m0, static_cast<uint32_t>(max(0, min(kWM, a.M - m0))) * 4u);
#pragma unroll
    for (int i = 0; i < kMT; ++i) {
        float sxi[16];
        if (OUTMODE == 0) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
                sxi[r] = __builtin_bit_cast(float, buf_load4(rsx, static_cast<uint32_t>(i * 32 + 8 * (r >> 2) + 4 * lh + (r & 3)) * 4u));
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int nn = wc0 + j * 32 + lc;
            if (nn >= a.N) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + i * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
                if (m >= a.M) continue;
                const int64_t idx = static_cast<int64_t>(m) * a.N + nn;
                if (OUTMODE == 1) a.ws[idx] = acc[i][j][r];
                else if (a.y_bf16) static_cast<uint16_t*>(a.y)[idx] = f32_to_bf16_bits(acc[i][j][r] * sxi[r]);
                else static_cast<float*>(a.y)[idx] = acc[i][j][r] * sxi[r];
            }
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
            const float sr = div14(f16_bits_to_f32(a.sw[sw_index(n, G4, g)]));
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
template <int MT>
static size_t decode_red_bytes(const DecodePlan& p) {
    return static_cast<size_t>(p.nw) * MT * 256 * sizeof(float);
}

template <int MT, bool RES, bool DUMP, int OUT>
static hipError_t go_decode(const GemmArgs& a, hipStream_t st) {
    const DecodePlan p = plan_decode(a.M, a.N, a.K);
    k_gemm_decode<MT, RES, DUMP, OUT><<<dim3(a.N / 16), dim3(64 * p.nw), decode_red_bytes<MT>(p), st>>>(a);
    return hipGetLastError();
}

template <bool RES, bool DUMP, int OUT>
static hipError_t go_wide(const GemmArgs& a, hipStream_t st) {
    // four waves (256 columns) per workgroup for both kernels (at eight the
    // dense-only loop, which the fused kernel now shares, measured 193.7 against
    // 179.7 us on the Qwen3-14B prefill shape). Every output is summed by one wave
    // in group order in both, so they agree bit for bit on an empty residual.
    if (a.M <= kMidMaxM) {
        // 32 < M <= 384: one 32-row tile per wave and two waves (128 columns) per
        // workgroup, so that the grid has enough workgroups (96 x 512 tiles give 28
        // for M = 64, N = 14336; 32 x 128 tiles give 224)
        constexpr int NWN = kMidWaves, MTW = kMidRowTiles;
        const int tiles_n = (a.N + 64 * NWN - 1) / (64 * NWN);
        const int tiles = ((a.M + 32 * MTW - 1) / (32 * MTW)) * tiles_n;
        k_gemm_wide<NWN, MTW, RES, DUMP, OUT><<<dim3(tiles), dim3(64 * NWN), 0, st>>>(a, 0, tiles_n);
        return hipGetLastError();
    }
    constexpr int NWN = 4, MTW = kWideRowTiles;
    const int tiles_n = (a.N + 64 * NWN - 1) / (64 * NWN);
    const int tiles = ((a.M + 32 * MTW - 1) / (32 * MTW)) * tiles_n;
    k_gemm_wide<NWN, MTW, RES, DUMP, OUT><<<dim3(tiles), dim3(64 * NWN), 0, st>>>(a, 0, tiles_n);
    return hipGetLastError();
}

// one launch: M quantizing workgroups, then the column workgroups (M <= 32)
template <int MT>
static hipError_t go_decode_qx(const GemmArgs& a, hipStream_t st) {
    const DecodePlan p = plan_decode(a.M, a.N, a.K);
    k_gemm_decode<MT, true, false, 0, true><<<dim3(a.M + a.N / 16), dim3(64 * p.nw), decode_red_bytes<MT>(p), st>>>(a);
    return hipGetLastError();
}

template <bool RES, bool DUMP, int OUT>
static hipError_t go(const GemmArgs& a, hipStream_t st) {
    if (a.M <= 16) return go_decode<1, RES, DUMP, OUT>(a, st);
    if (a.M <= 32) return go_decode<2, RES, DUMP, OUT>(a, st);
    return go_wide<RES, DUMP, OUT>(a, st);
}

// ---------------------------------------------------------------------------
// Decode plan: waves per workgroup. The grid has one workgroup per 16 columns,
// and each wave keeps two steps of loads in flight, so the time is about the
// steps per wave over two, times the load latency, as long as every workgroup is
// resident at once. With at most 256 column workgroups (one per CU or fewer) a
// workgroup takes 16 waves, so each wave's share of K is short (measured on the
// 4096-column shapes: 11-15% faster than 8 waves). With more, about 2048 waves in
// total: more waves there gave slower launches (measured at 14336 and 25600
// columns). Each wave gets at least one quad. The plan depends on (M, N, K) only,
// so the fused and the dense-only kernels of a shape sum in the same order.
// ---------------------------------------------------------------------------
DecodePlan plan_decode(int M, int N, int K) {
    (void)M;
    const int G4 = (K / kGroup + 3) / 4, subtiles = N / 16;
    int nw = subtiles <= 256 ? kMaxDecodeWaves : (2048 + subtiles - 1) / subtiles;
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
        case GemmKind::FusedQuantAct:
            return a.M <= 16 ? go_decode_qx<1>(a, st) : go_decode_qx<2>(a, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_residual_merge(const GemmArgs& a, hipStream_t st) {
    k_residual_merge<<<dim3(a.N / 16), dim3(256), 0, st>>>(a);
    return hipGetLastError();
}

}  // namespace mq
