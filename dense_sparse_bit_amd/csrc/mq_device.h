// Device-side helpers shared by the MosaicQuant HIP kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mq {

constexpr int kGroup = 128;   // weight group along K
constexpr int kBk = 64;       // residual block width along K (two blocks per group)
constexpr int kQmax = 7;

typedef int v4i __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// binary16 bits <-> fp32 through the hardware conversions (round to nearest even;
// fp16 denormals are kept by the default float mode).
__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
    return static_cast<float>(__builtin_bit_cast(_Float16, b));
}
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

// fp32 -> bf16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float load_x(const void* x, bool bf16, int64_t i) {
    return bf16 ? bf16_bits_to_f32(static_cast<const uint16_t*>(x)[i])
                : static_cast<const float*>(x)[i];
}

// Symmetric RTN code on scale s: 0 when s == 0, else clamp(rint(v / s), -7, 7).
// fp32 division is the correctly rounded one (the library is built without
// fast-math), rint is round-half-even.
__device__ __forceinline__ int rtn_code(float v, float s) {
    if (s == 0.0f) return 0;
    float t = __builtin_rintf(v / s);
    t = fminf(fmaxf(t, -7.0f), 7.0f);
    return static_cast<int>(t);
}

// rint(fl(v / s)) for s > 0 without a per-element division, given rs = fl(1 / s).
// t = fl(v * rs) differs from the exact quotient by at most |v/s| * 2^-22.9, and
// fl(v/s) by at most |v/s| * 2^-24, so for |t| <= 8 the two lie within 1.5e-6 of
// each other. When t is farther than 4e-6 from every half-integer, no rounding
// boundary separates them and rint(t) == rint(fl(v/s)); otherwise (or for larger
// quotients) the correctly rounded quotient is formed. The result is therefore
// identical to rintf(v / s). (A non-finite t, from a reciprocal that overflowed
// for a subnormal s, fails both comparisons and also takes the exact path.)
__device__ __forceinline__ float rint_quot(float v, float s, float rs) {
    const float t = v * rs;
    const float q = __builtin_rintf(t);
    if (__builtin_expect(fabsf(t - q) < 0.5f - 4e-6f && fabsf(t) <= 8.0f, 1)) return q;
    return __builtin_rintf(v / s);
}

// Symmetric RTN code as a float: 0 when s == 0, else clamp(rint(v / s), -7, 7).
__device__ __forceinline__ float rtn_codef(float v, float s, float rs) {
    if (s == 0.0f) return 0.0f;
    return fminf(fmaxf(rint_quot(v, s, rs), -7.0f), 7.0f);
}

// Per-group constants of the decomposition W ~ s*q + s_r*r for an fp16 scale s.
struct GroupScale {
    float s, rs, sr, rsr;   // s, 1/s, s_r = s/14, 1/s_r (all correctly rounded)
};
__device__ __forceinline__ GroupScale group_scale(float s) {
    GroupScale g;
    g.s = s;
    g.sr = s / 14.0f;
    g.rs = s == 0.0f ? 0.0f : 1.0f / s;
    g.rsr = s == 0.0f ? 0.0f : 1.0f / g.sr;
    return g;
}

// One element: base code q, E = w - s*q, residual code r, E' = E - s_r*r.
struct Elem {
    float q, r;
    float e, ep;
};
__device__ __forceinline__ Elem quant_elem(float w, const GroupScale& g) {
    Elem o;
    o.q = rtn_codef(w, g.s, g.rs);
    o.e = __builtin_fmaf(-g.s, o.q, w);
    o.r = rtn_codef(o.e, g.sr, g.rsr);
    o.ep = __builtin_fmaf(-g.sr, o.r, o.e);
    return o;
}

// Branch-free form of rtn_codef for long runs of elements. Returns the code of
// rint(v * rs) clamped to [-7, 7] and raises `worst` to |t - rint(t)|. While the
// caller's worst stays below 0.5 - 4e-6 (and rs is finite), every code equals
// rtn_codef's: no half-integer lies between t and fl(v/s) when |t| <= 8, and for
// larger |t| both quotients clamp to the same +-7. Otherwise the caller redoes the
// run with rtn_codef. s == 0 needs no special case: rs = 0 gives t = 0, code 0.
__device__ __forceinline__ float rtn_fast(float v, float rs, float& worst) {
    const float t = v * rs;
    const float q = __builtin_rintf(t);
    worst = fmaxf(worst, fabsf(t - q));
    return fminf(fmaxf(q, -7.0f), 7.0f);
}
constexpr float kFastMargin = 0.5f - 4e-6f;

// quant_elem through rtn_fast (valid when the run's worst stays below kFastMargin)
__device__ __forceinline__ Elem quant_elem_fast(float w, const GroupScale& g, float& worst) {
    Elem o;
    o.q = rtn_fast(w, g.rs, worst);
    o.e = __builtin_fmaf(-g.s, o.q, w);
    o.r = rtn_fast(o.e, g.rsr, worst);
    o.ep = __builtin_fmaf(-g.sr, o.r, o.e);
    return o;
}
// the reciprocals are finite, so rtn_fast's t is finite for finite inputs
__device__ __forceinline__ bool fast_ok(const GroupScale& g) {
    return fabsf(g.rs) <= 3.0e38f && fabsf(g.rsr) <= 3.0e38f;
}

// ---- int4 -> int8 operand construction for the int8 MFMA ------------------
// A 32-bit word holds 8 two's-complement nibbles (k0 in bits 0-3). Placing a
// nibble in the high half of a byte gives the int8 value 16*v, so two masks
// turn 8 nibbles into 8 int8 operands (k even in one dword, k odd in the other);
// the same permutation of k is applied to both MFMA operands, which leaves the
// dot product unchanged.
__device__ __forceinline__ uint32_t nib16_even(uint32_t w) { return (w << 4) & 0xF0F0F0F0u; }
__device__ __forceinline__ uint32_t nib16_odd(uint32_t w) { return w & 0xF0F0F0F0u; }

// 16 bytes of nibbles (32 values) -> two MFMA operands of 16 int8 (values x16).
__device__ __forceinline__ void unpack16(const uint4 w, v4i& op0, v4i& op1) {
    op0 = v4i{(int)nib16_even(w.x), (int)nib16_odd(w.x), (int)nib16_even(w.y), (int)nib16_odd(w.y)};
    op1 = v4i{(int)nib16_even(w.z), (int)nib16_odd(w.z), (int)nib16_even(w.w), (int)nib16_odd(w.w)};
}

// Combined operand 14*q + r per byte (plain int8, |value| <= 105), from the base
// word wq and residual word wr. In offset form q' = q+8, r' = r+8 (nibble ^ 8)
// every byte of 14*q' + r' + 8 stays in [23, 233], so whole-word integer
// arithmetic produces each byte without carries; xor 0x80 then subtracts 128.
__device__ __forceinline__ uint32_t comb_even(uint32_t qo, uint32_t ro) {
    const uint32_t qe = qo & 0x0F0F0F0Fu, re = ro & 0x0F0F0F0Fu;
    return (((qe << 4) - (qe << 1)) + re + 0x08080808u) ^ 0x80808080u;
}
__device__ __forceinline__ uint32_t comb_odd(uint32_t qo, uint32_t ro) {
    const uint32_t q16 = qo & 0xF0F0F0F0u, rd = (ro >> 4) & 0x0F0F0F0Fu;
    return ((q16 - (q16 >> 3)) + rd + 0x08080808u) ^ 0x80808080u;
}
__device__ __forceinline__ void unpack_comb(const uint4 wq, const uint4 wr, v4i& op0, v4i& op1) {
    const uint32_t x = 0x88888888u;
    const uint32_t q0 = wq.x ^ x, q1 = wq.y ^ x, q2 = wq.z ^ x, q3 = wq.w ^ x;
    const uint32_t r0 = wr.x ^ x, r1 = wr.y ^ x, r2 = wr.z ^ x, r3 = wr.w ^ x;
    op0 = v4i{(int)comb_even(q0, r0), (int)comb_odd(q0, r0), (int)comb_even(q1, r1), (int)comb_odd(q1, r1)};
    op1 = v4i{(int)comb_even(q2, r2), (int)comb_odd(q2, r2), (int)comb_even(q3, r3), (int)comb_odd(q3, r3)};
}

__device__ __forceinline__ v4i mfma_i8(v4i a, v4i b, v4i c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint4 ldg16(const uint8_t* p) {
    return *reinterpret_cast<const uint4*>(p);
}

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// ---- raw buffer loads ------------------------------------------------------
// A buffer resource (base in scalar registers, byte range `bytes`) turns every
// 16-byte load into one instruction with a 32-bit per-lane offset: no 64-bit
// address arithmetic per load. The hardware range check covers the per-lane
// offset: a load at or past `bytes` returns zero, which also replaces the
// in-range test for a step that runs past the last group.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kBufferFlags = 0x00020000;   // dword 3 of a raw (untyped) gfx9 buffer resource

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                             static_cast<int>(bytes), kBufferFlags);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0);
}
__device__ __forceinline__ uint2 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
    const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, 0, 0);
    return make_uint2(v.x, v.y);
}

// ---- device layouts of the packed operands --------------------------------
// Every 64-lane load of a GEMM operand is 1 KB of contiguous memory in MFMA lane
// order, so each request the vector memory pipeline carries is fully used:
//   wq  [N/16][G][64][16 B]  tile (nt, g) holds rows 16nt..16nt+15 of group g;
//                            lane l = 16*kc + r owns row 16nt + r, bytes
//                            16kc..16kc+15 of that row's 64-byte group chunk
//   sw  [N/16][G4][16][4]    fp16 group scales, G4 = ceil(G/4): one 8-byte load
//                            gives a row the scales of four consecutive groups;
//                            slots of groups >= G hold zero
//   xq  [G][M][64 B]         group-major activations: a group's rows are
//                            contiguous, so 16 tokens x 128 inputs is one 1 KB run
__device__ __forceinline__ int64_t wq_tile(int64_t nt, int64_t G, int64_t g) { return (nt * G + g) * 1024; }
__device__ __forceinline__ int64_t wq_byte(int64_t n, int64_t G, int64_t g, int kc) {
    return wq_tile(n >> 4, G, g) + (kc * 16 + (n & 15)) * 16;
}
__device__ __forceinline__ int64_t sw_index(int64_t n, int64_t G4, int64_t g) {
    return (((n >> 4) * G4 + (g >> 2)) * 16 + (n & 15)) * 4 + (g & 3);
}
__device__ __forceinline__ int64_t xq_row(int64_t g, int64_t M, int64_t m) { return (g * M + m) * 64; }

}  // namespace mq
