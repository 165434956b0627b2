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

// fp32(s / 14) for an fp16 scale s without a division: a product by fl(1/14)
// and one fma correction. For every finite binary16 value s this equals the
// correctly rounded quotient (checked exhaustively on the host by the test suite),
// so the GEMM's residual grid is the same s_r = fp32(s / 14) as the packing's.
__device__ __forceinline__ float div14(float s) {
    constexpr float c = 1.0f / 14.0f;
    const float q = s * c;
    const float r = __builtin_fmaf(-q, 14.0f, s);
    return __builtin_fmaf(r, c, q);
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

// ---- packed int4 codes and the fp8 MFMA -----------------------------------
// gfx950 has no int4 MFMA, and the int8 one returns integers that need a
// conversion per output before the per-group scale applies. The fp8 (e4m3)
// MFMA v_mfma_f32_16x16x128_f8f6f4 covers a whole 128-input group in one
// instruction at the int8 rate and returns fp32 directly. A code c in [-7, 7]
// is the e4m3 subnormal with sign bit 7 and mantissa |c| (value c * 2^-9), so
// each product is an exact multiple of 2^-18 and every group sum (at most
// 128 * 49 units) is exact in fp32: the MFMA result is the exact integer dot
// product times 2^-18.
//
// The packed code word is chosen so that two masks make those bytes: a 32-bit
// word holds 8 consecutive codes c0..c7; nibble e (bits 4e..4e+3) holds |c_e|
// in its low three bits and, in its high bit, the sign of code (e - 1) mod 8.
// Then  word & 0x87878787  is the e4m3 bytes of c0, c2, c4, c6 and
// rotr(word, 4) & 0x87878787  those of c1, c3, c5, c7. The same k order is used
// for both MFMA operands, which leaves the dot product unchanged.
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr float kF8Unit = 262144.0f;   // 2^18: an MFMA result of 1.0 is 2^18 code products

__device__ __forceinline__ uint32_t f8_even(uint32_t w) { return w & 0x87878787u; }
__device__ __forceinline__ uint32_t f8_odd(uint32_t w) { return __builtin_rotateright32(w, 4) & 0x87878787u; }

// 16 packed bytes (32 codes) -> one fp8 MFMA operand
__device__ __forceinline__ v8i f8_operand(const uint4 w) {
    return v8i{(int)f8_even(w.x), (int)f8_odd(w.x), (int)f8_even(w.y), (int)f8_odd(w.y),
               (int)f8_even(w.z), (int)f8_odd(w.z), (int)f8_even(w.w), (int)f8_odd(w.w)};
}

// 8 two's-complement nibbles (code e in bits 4e..4e+3) -> the packed code word:
// sign bits s (bit 4e), magnitudes by a per-nibble negate (c ^ 15) + 1, and the
// signs rotated by 7 bits into the spare high bit of the next nibble
__device__ __forceinline__ uint32_t code_word(uint32_t t) {
    const uint32_t sgn = (t >> 3) & 0x11111111u;
    const uint32_t mag = (t ^ ((sgn << 4) - sgn)) + sgn;
    return mag | __builtin_rotateleft32(sgn, 7);
}

__device__ __forceinline__ v4f mfma_f8(v8i a, v8i b, v4f c) {
    // format selectors 0/0 (e4m3 both operands), no block scales
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
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
// The same resource from values the caller knows to be wave-uniform but the
// compiler may not (it would otherwise wrap every load in a per-lane loop).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc_uniform(const void* base, uint32_t bytes) {
    const uint64_t p = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p >> 32));
    return buf_rsrc(reinterpret_cast<const void*>((static_cast<uint64_t>(hi) << 32) | lo),
                    __builtin_amdgcn_readfirstlane(bytes));
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}
// the same with a wave-uniform byte offset added in the instruction (scalar operand)
__device__ __forceinline__ uint4 buf_load16s(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
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
