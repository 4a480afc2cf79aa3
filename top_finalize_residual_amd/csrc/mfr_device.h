// Device helpers for the fused MoE finalize + RMSNorm kernels (gfx950).
//
// bf16 handling: a 16-byte vector holds 8 bf16 values as 4 dwords; element
// 2i sits in the low half of dword i and element 2i+1 in the high half.
// Widening is exact (a shift or a mask). Narrowing uses the CDNA4 packed
// convert v_cvt_pk_bf16_f32, which rounds to nearest-even (the default mode),
// reached through clang's vector conversion to __bf16.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mfr {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

// Two fp32 values -> one dword of two bf16 (round to nearest-even).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2 v = {lo, hi};
    bf16x2 r = __builtin_convertvector(v, bf16x2);
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float vec_elem(const u32x4& v, int e) {
    // e is a compile-time constant after unrolling
    const uint32_t d = (e >> 1) == 0 ? v.x : (e >> 1) == 1 ? v.y : (e >> 1) == 2 ? v.z : v.w;
    return (e & 1) ? bf16_hi(d) : bf16_lo(d);
}

// Raw buffer access. A descriptor covers [base, base + nbytes); loads at or
// past nbytes return zero without a memory access and stores there are
// dropped, so a zero-record descriptor turns a whole row access into a no-op.
// Word 3 of a gfx9-family raw buffer descriptor selects 32-bit data format.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;
// Cache-policy bits of a buffer access on gfx950 (sc0 = 1, nt = 2, sc1 = 16).
constexpr int kAuxDefault = 0;
constexpr int kAuxStream = 2;  // nt: data touched once, do not keep it in cache
constexpr int kAuxSc1 = 16;    // sc1 on a store: system scope, written through the L2
// Policy per stream of the fused op (chosen by measurement on MI355X).
constexpr int kAuxRows = kAuxStream;        // gathered expert rows (read once)
constexpr int kAuxActIn = kAuxStream;       // shared and residual rows (read once)
constexpr int kAuxGamma = kAuxDefault;      // gamma (re-read by every workgroup)
constexpr int kAuxOut = kAuxDefault;        // outputs that fit in L2: write-back
constexpr int kAuxWriteThrough = kAuxSc1;   // outputs larger than L2: write-through
// Output encodings reachable only through the tuning interface (measured
// slower than the two above).
constexpr int kAuxOutNt = kAuxStream;
constexpr int kAuxOutNtWriteThrough = kAuxStream | kAuxSc1;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t nbytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                             static_cast<int>(nbytes), kRsrcWord3);
}

template <int AUX>
__device__ __forceinline__ u32x4 buf_load(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, AUX);
}

template <int AUX>
__device__ __forceinline__ void buf_store(u32x4 v, rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, static_cast<int>(off), 0, AUX);
}

template <int AUX>
__device__ __forceinline__ void buf_store_b64(u32x2 v, rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b64(v, r, static_cast<int>(off), 0, AUX);
}

template <int AUX>
__device__ __forceinline__ void buf_store_b32(float v, rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, static_cast<int>(off), 0, AUX);
}

template <int AUX>
__device__ __forceinline__ void buf_store_u32(uint32_t v, rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b32(v, r, static_cast<int>(off), 0, AUX);
}

// 1/448 rounded to fp32, and 1 - 2^-21 (exact in fp32).
constexpr float kInvE4m3Max = 1.0f / 448.0f;
constexpr float kE4m3Shrink = 1.0f - 0x1p-21f;

// 448 / m for m in [2^-90, 2^128] or +inf, made safe to scale by: the
// hardware reciprocal (v_rcp_f32, within 1 ulp) of m * RN(1/448), shrunk by
// 2^-21. Whatever the three roundings do (each within 2^-24 or 2^-23
// relative), m times the factor stays below 448 * (1 - 2^-23), and the factor
// is within 2^-20 of 448 / m. Rounding is monotone, so |x| <= m then gives
// |x * factor| <= 448 after rounding, the largest finite OCP E4M3 magnitude
// (the hardware conversion turns values above it into NaN). Over that range
// of m every intermediate is a normal number. m = +inf gives 0.
__device__ __forceinline__ float e4m3_factor(float m) {
    return __builtin_amdgcn_rcpf(m * kInvE4m3Max) * kE4m3Shrink;
}

// Eight fp32 values in [-448, 448] (or NaN) to eight OCP E4M3 codes in
// element order, through the CDNA4 packed conversion v_cvt_pk_fp8_f32, which
// rounds to nearest-even and maps NaN to the NaN code.
__device__ __forceinline__ u32x2 pack_e4m3x8(const float (&v)[8]) {
    int lo = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], lo, true);
    int hi = __builtin_amdgcn_cvt_pk_fp8_f32(v[4], v[5], 0, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(v[6], v[7], hi, true);
    return u32x2{static_cast<uint32_t>(lo), static_cast<uint32_t>(hi)};
}

// One DPP move of a float within a row of 16 lanes (every lane active).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over the 64 lanes of a wave, returned to every lane. Fixed tree:
// xor-1 and xor-2 within quads, half-mirror and mirror within rows of 16
// (DPP, so every lane of a row ends with the row sum), then the four row sums
// read as scalars and added as (r0 + r1) + (r2 + r3). Deterministic.
__device__ __forceinline__ float wave_sum(float x) {
    x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
    x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
    x += dpp<0x141>(x);  // row_half_mirror
    x += dpp<0x140>(x);  // row_mirror
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
    return (r0 + r1) + (r2 + r3);
}

// One DPP move of a double (its two halves moved alike).
template <int CTRL>
__device__ __forceinline__ double dpp64(double x) {
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    const uint32_t lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(u), CTRL, 0xF, 0xF, false);
    const uint32_t hi =
        __builtin_amdgcn_update_dpp(0, static_cast<int>(u >> 32), CTRL, 0xF, 0xF, false);
    return __builtin_bit_cast(double, (static_cast<uint64_t>(hi) << 32) | lo);
}

__device__ __forceinline__ double readlane64(double x, int lane) {
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    const uint32_t lo = __builtin_amdgcn_readlane(static_cast<int>(u), lane);
    const uint32_t hi = __builtin_amdgcn_readlane(static_cast<int>(u >> 32), lane);
    return __builtin_bit_cast(double, (static_cast<uint64_t>(hi) << 32) | lo);
}

// wave_sum in fp64: the same fixed tree, for the sum of squares taken when
// the fp32 one leaves the fp32 range.
__device__ __forceinline__ double wave_sum_f64(double x) {
    x += dpp64<0xB1>(x);
    x += dpp64<0x4E>(x);
    x += dpp64<0x141>(x);
    x += dpp64<0x140>(x);
    return (readlane64(x, 0) + readlane64(x, 16)) + (readlane64(x, 32) + readlane64(x, 48));
}

// Maximum over the 64 lanes of a wave, returned to every lane; the same DPP
// tree as wave_sum with max in place of add.
__device__ __forceinline__ float wave_max(float x) {
    x = __builtin_fmaxf(x, dpp<0xB1>(x));
    x = __builtin_fmaxf(x, dpp<0x4E>(x));
    x = __builtin_fmaxf(x, dpp<0x141>(x));
    x = __builtin_fmaxf(x, dpp<0x140>(x));
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
    return __builtin_fmaxf(__builtin_fmaxf(r0, r1), __builtin_fmaxf(r2, r3));
}

}  // namespace mfr
