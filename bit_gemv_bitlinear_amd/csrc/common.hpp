// common.hpp -- device-side helpers shared by the gfx950 kernels of the W2A8
// ternary linear layer.  Source page: "BitNet GPU 推理框架：从零构建 W2A8 的
// 2-bit 大模型 CUDA GEMV 内核" (blog.gitcode.com), cited as [W2A8].
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bl {

// Geometry of the packed layout: a tile is 16 rows x 256 K = 1024 bytes; its
// 16-byte slot q holds four 32-bit words, rows 4*(q/16) .. +3 of the 16-wide
// K chunk q%16.
constexpr int kTileRows = 16;
constexpr int kTileK = 256;
constexpr int kTileBytes = 1024;

// Table for v_perm_b32: byte c of this word is the int8 weight of 2-bit code
// c.  Code 1 -> -1 (0xFF), 2 -> 0, 3 -> +1; code 0 (padding) -> 0.
constexpr uint32_t kCodeToInt8 = 0x0100FF00u;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));

// A pointer into the global address space.  Kernels that read their pointers
// from a record in memory (not from kernel arguments) cast them with global()
// so that the compiler emits global rather than flat loads and stores.
template <class T>
using global_ptr = __attribute__((address_space(1))) T*;
template <class T>
__device__ __forceinline__ global_ptr<T> global(T* p) {
    return (global_ptr<T>)(p);
}

__device__ __forceinline__ float bf16_to_float(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// bf16 rounding (nearest, ties to even) of an fp64 value in two hardware
// steps: to fp32 rounded to odd, then fp32 to bf16 with ties to even.  An
// intermediate format with at least two more significant bits than the
// target makes that pair equal to one direct rounding (Boldo and Melquiond,
// "Emulation of FMA and correctly rounded sums: proved algorithms using
// rounding to odd", IEEE Trans. Computers 57(4), 2008); fp32 carries 24 bits
// against bf16's 8, also among the subnormals (quantum 2^-149 against
// 2^-133), and shares bf16's exponent range, so a value beyond it lands on
// fp32's largest finite value, which rounds on to infinity as it should.
// Rounding to odd: the nearest fp32 (the conversion's own rounding, ties to
// even, with fp32 subnormals kept), and when that is inexact and even, its
// neighbour on the other side of the value, which is odd.  NaN gives the
// quiet NaN 0x7FC0.  About ten instructions, no 64-bit shifts: the exact
// paths of the epilogues below are short, which matters because they run
// rarely and their code is cold.
__device__ __forceinline__ uint32_t bf16_rne_f64(double d) {
    const float f = static_cast<float>(d);
    uint32_t u = __float_as_uint(f);
    const double back = static_cast<double>(f);
    if (back != d && !(u & 1u)) u += fabs(back) > fabs(d) ? 0xFFFFFFFFu : 1u;
    u = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
    return d != d ? 0x7FC0u : u;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 values to packed bf16 (a in the low half), nearest with ties to
// even: v_cvt_pk_bf16_f32 in the default rounding mode.
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
    const f32x2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// The epilogue of [W2A8] §5.3 under the reading y = acc * ws / s: the
// activation scale s = 127/amax multiplied x on the way in, so it divides
// here.  The result is bf16_rne(fl64(acc * ws) / s) -- the product is exact,
// the quotient is rounded once to fp64, then once to bf16.
__device__ __forceinline__ uint16_t epilogue_bf16(int32_t acc, float ws, float s) {
    const double v = (static_cast<double>(acc) * static_cast<double>(ws)) / static_cast<double>(s);
    return static_cast<uint16_t>(bf16_rne_f64(v));
}

// The same value as epilogue_bf16 without a division on the common path.
// cs = fl64(ws * fl64(1/s)) is formed once per kernel; v = fl64(acc * cs)
// carries three roundings and lies within 2^-51 (relative) of the quotient.
// v goes to bf16 through fp32 (one conversion, then v_cvt_pk_bf16_f32):
// every bf16 midpoint is an fp32 number, and a midpoint lying between v and
// the quotient, or one the fp64 quotient rounds onto, is so close to v that
// v's nearest fp32 is that midpoint -- among fp32 subnormals too, which keep
// 16 more bits than bf16's.  So the two roundings give the exact path's
// value unless the fp32 value is a midpoint (low 16 bits 0x8000, about one
// output in 65536) or NaN; then every active lane of the wavefront takes the
// exact path, in one uniform branch.
__device__ __forceinline__ uint16_t epilogue_bf16_scaled(int32_t acc, double cs, float ws,
                                                         float s) {
    const float f = static_cast<float>(static_cast<double>(acc) * cs);
    uint16_t out = static_cast<uint16_t>(cvt_pk_bf16(f, 0.0f));
    const bool redo = ((__float_as_uint(f) & 0xFFFFu) == 0x8000u) || __builtin_isnan(f);
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(redo) != 0, 0)) {
        asm volatile("");   // kept a branch: if-converted it would cost every output its division
        out = epilogue_bf16(acc, ws, s);
    }
    return out;
}

// y = bf16(fl64(acc * ws) / s), the §5.3 epilogue, for a group of four
// outputs, without a division on the common path.  v = fl64(acc * cs) with
// cs = fl64(ws * fl64(1 / s)) lies within 2^-51 (relative) of the quotient.
// It goes to bf16 through fp32 (one conversion to fp32, then
// v_cvt_pk_bf16_f32): every bf16 midpoint is an fp32 number, and a midpoint
// lying between v and the quotient, or one the fp64 quotient rounds onto, is
// so close to v that v's nearest fp32 is that midpoint -- among fp32
// subnormals too, which keep 16 more bits than bf16's.  So the two
// roundings give the exact path's bf16 unless the fp32 value is a midpoint
// (low 16 bits 0x8000), about one output in 65536, or NaN; a group holding
// one is redone exactly, by the whole wavefront in one uniform branch.
__device__ __forceinline__ uint2 epilogue4(const int (&acc)[4], const float (&ws)[4],
                                           const double (&cs)[4], float s) {
    float f[4];
    uint64_t redo = 0;   // lanes with a midpoint, one ballot per compare
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        f[v] = static_cast<float>(static_cast<double>(acc[v]) * cs[v]);
        redo |= __builtin_amdgcn_ballot_w64((__float_as_uint(f[v]) & 0xFFFFu) == 0x8000u);
    }
    redo |= __builtin_amdgcn_ballot_w64(__builtin_isunordered(f[0], f[1]) ||
                                        __builtin_isunordered(f[2], f[3]));
    uint2 o{cvt_pk_bf16(f[0], f[1]), cvt_pk_bf16(f[2], f[3])};
    if (__builtin_expect(redo != 0, 0)) {
        asm volatile("");   // kept a branch: if-converted it would cost every group its divisions
        o.x = epilogue_bf16(acc[0], ws[0], s) | (static_cast<uint32_t>(epilogue_bf16(acc[1], ws[1], s)) << 16);
        o.y = epilogue_bf16(acc[2], ws[2], s) | (static_cast<uint32_t>(epilogue_bf16(acc[3], ws[3], s)) << 16);
    }
    return o;
}

// Per-activation quantisation of [W2A8] §六 item 3: q = clamp(round half
// to even of fl32(x * s), -128, 127), for finite x and s = 127 / amax with
// |x| <= amax.  Then |fl32(x * s)| <= 127 * (1 + 2^-24)^2 < 127.5, so the
// clamp never binds, and adding 1.5 * 2^23 rounds the product to an integer
// (ties to even, the default rounding) in the low mantissa bits: the low
// byte of the sum's encoding is q in two's complement.  The multiply and
// the add must stay two roundings: fused into one FMA, a product such as
// -63.4999997 (fp32: -63.5, so q = -64) would give -63.
__device__ __forceinline__ uint32_t quant_byte(float x, float s) {
#pragma clang fp contract(off)
    const float p = x * s;
    return __float_as_uint(p + 12582912.0f);
}

// Four quantised values packed into an int8x4 word, value a in byte 0.
__device__ __forceinline__ uint32_t quant4(float a, float b, float c, float d, float s) {
    const uint32_t ab = __builtin_amdgcn_perm(quant_byte(b, s), quant_byte(a, s), 0x0C0C0400u);
    const uint32_t cd = __builtin_amdgcn_perm(quant_byte(d, s), quant_byte(c, s), 0x0C0C0400u);
    return __builtin_amdgcn_perm(cd, ab, 0x05040100u);
}

// Signed int8x4 dot product with int32 accumulate, no saturation (v_dot4_i32_i8).
__device__ __forceinline__ int dot4(int a, int b, int c) {
    return __builtin_amdgcn_sdot4(a, b, c, false);
}

// Wave-wide reductions over the 64 lanes, for uniform control flow (every
// lane active).  Inside each row of 16 lanes the values are combined with DPP
// moves (swap within pairs, then within quads, then rotations by 4 and 8
// lanes), which leaves the row's total in each of its lanes; the four row
// totals are then read into scalar registers and combined there.  The result
// is the same in every lane.
template <int CTRL>
__device__ __forceinline__ int dpp_row(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
constexpr int kDppQuadXor1 = 0xB1;   // quad_perm(1, 0, 3, 2)
constexpr int kDppQuadXor2 = 0x4E;   // quad_perm(2, 3, 0, 1)
constexpr int kDppRowRor4 = 0x124;   // lane i <- lane (i + 4) % 16 inside each 16 lanes
constexpr int kDppRowRor8 = 0x128;   // lane i <- lane (i + 8) % 16
constexpr int kDppRowHalfMirror = 0x141;   // lane i <- lane 7 - i inside each 8 lanes

__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, __int_as_float(dpp_row<kDppQuadXor1>(__float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_row<kDppQuadXor2>(__float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_row<kDppRowRor4>(__float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_row<kDppRowRor8>(__float_as_int(v))));
    const int b = __float_as_int(v);
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(b, 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(b, 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(b, 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(b, 48));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

__device__ __forceinline__ int wave_sum(int v) {
    v += dpp_row<kDppQuadXor1>(v);
    v += dpp_row<kDppQuadXor2>(v);
    v += dpp_row<kDppRowRor4>(v);
    v += dpp_row<kDppRowRor8>(v);
    return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) +
           __builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48);
}

}  // namespace bl
