// gemv_core.hpp -- pieces of the M = 1 GEMV shared by its kernels
// (gemv.hip) and by the projection with its glue (gemv_norm.hip): the K-step
// dot products of the packed 16 x 256 tiles, the weight loads, the row
// reduction, the bf16 quantisation helpers and the launch geometry's
// constants.  Source page: "BitNet GPU 推理框架：从零构建 W2A8 的 2-bit 大模型
// CUDA GEMV 内核" (blog.gitcode.com), cited as [W2A8] (§5.2 codes and words,
// §5.3 dot products, §六 item 3 the per-token quantisation).
#pragma once

#include "common.hpp"

namespace bl {

constexpr int kMaxWaves = 16;   // wavefronts per workgroup, at most

struct RowAcc {
    int a1[4], a4[4], a16[4];
};

// Dot of one packed word (16 K of one row) with its four activation words.
__device__ __forceinline__ void dot_word(uint32_t w, const int4& x, int& a1, int& a4, int& a16) {
    a1 = dot4(static_cast<int>(w & 0x03030303u), x.x, a1);
    a4 = dot4(static_cast<int>(w & 0x0C0C0C0Cu), x.y, a4);
    a16 = dot4(static_cast<int>(w & 0x30303030u), x.z, a16);
    a1 = dot4(static_cast<int>((w >> 6) & 0x03030303u), x.w, a1);
}

// One K step of a lane: the four words of its slot are four rows of the same
// 16-wide K chunk, all dotted with the same 16 activation bytes.
__device__ __forceinline__ void dot_slot(const v4u& wv, const int4& x, RowAcc& r) {
    dot_word(wv.x, x, r.a1[0], r.a4[0], r.a16[0]);
    dot_word(wv.y, x, r.a1[1], r.a4[1], r.a16[1]);
    dot_word(wv.z, x, r.a1[2], r.a4[2], r.a16[2]);
    dot_word(wv.w, x, r.a1[3], r.a4[3], r.a16[3]);
}

// The same sums by v_dot8 on 4-bit lanes.  Masked with 0x33333333, a packed
// word keeps fields 0 and 2 in the low bits of its nibbles: nibble k holds the
// code (0..3) of element k / 2 for even k and of element 8 + k / 2 for odd k
// (element e sits at bit 8 (e % 4) + 2 (e / 4)); shifted down by 2 first, it
// keeps fields 1 and 3, elements 4 + k / 2 and 12 + k / 2.  An int8 activation
// is 16 h + l with l its low nibble (0..15) and h its high nibble as a signed
// 4-bit number (-8..7), so sum c x = sum c l + 16 sum c h: one unsigned and
// one signed v_dot8 per masked word and activation order, 7 VALU per packed
// word against 9 for the four v_dot4 of dot_word.
struct NibAcc {
    uint32_t lo[4];
    int hi[4];
};

// A 16-byte activation chunk rearranged for dot_word_nib: the low nibbles of
// elements 0, 8, 1, 9, 2, 10, 3, 11, their high nibbles, then the same for
// elements 4, 12, 5, 13, 6, 14, 7, 15 (dwords 0 / 2 of the chunk hold elements
// 0..3 / 8..11, dwords 1 / 3 elements 4..7 / 12..15).
__device__ __forceinline__ int4 nibble_split(const int4& x) {
    constexpr uint32_t kLo = 0x0F0F0F0Fu;
    const uint32_t x0 = x.x, x1 = x.y, x2 = x.z, x3 = x.w;
    int4 r;
    r.x = static_cast<int>((x0 & kLo) | ((x2 << 4) & ~kLo));
    r.y = static_cast<int>(((x0 >> 4) & kLo) | (x2 & ~kLo));
    r.z = static_cast<int>((x1 & kLo) | ((x3 << 4) & ~kLo));
    r.w = static_cast<int>(((x1 >> 4) & kLo) | (x3 & ~kLo));
    return r;
}

__device__ __forceinline__ void dot_word_nib(uint32_t w, const int4& xn, uint32_t& lo, int& hi) {
    const uint32_t a = w & 0x33333333u;
    const uint32_t b = (w >> 2) & 0x33333333u;
    lo = __builtin_amdgcn_udot8(a, static_cast<uint32_t>(xn.x), lo, false);
    hi = __builtin_amdgcn_sdot8(static_cast<int>(a), xn.y, hi, false);
    lo = __builtin_amdgcn_udot8(b, static_cast<uint32_t>(xn.z), lo, false);
    hi = __builtin_amdgcn_sdot8(static_cast<int>(b), xn.w, hi, false);
}

// One K step of a lane on a chunk split by nibble_split.
__device__ __forceinline__ void dot_slot_nib(const v4u& wv, const int4& xn, NibAcc& r) {
    dot_word_nib(wv.x, xn, r.lo[0], r.hi[0]);
    dot_word_nib(wv.y, xn, r.lo[1], r.hi[1]);
    dot_word_nib(wv.z, xn, r.lo[2], r.hi[2]);
    dot_word_nib(wv.w, xn, r.lo[3], r.hi[3]);
}

// Ptr: const v4u*, or a pointer into the global address space (kernels that
// read their pointers from memory rather than kernel arguments cast them, so
// that the loads are global rather than flat loads).
template <int P, class Ptr>
__device__ __forceinline__ void load_steps(Ptr __restrict__ tiles, int s0, int s_last,
                                           v4u (&w)[P]) {
#pragma unroll
    for (int u = 0; u < P; ++u) {
        const int st = min(s0 + u, s_last);
        w[u] = __builtin_nontemporal_load(tiles + static_cast<size_t>(st) * 64);
    }
}

// load_steps with the loads kept in step order (a scheduling barrier after
// each): the waits for step u then count only the loads of steps u + 1 ..,
// so each step can start as soon as its own tile has landed.
template <int P, class Ptr>
__device__ __forceinline__ void load_steps_ordered(Ptr __restrict__ tiles, int s0, int s_last,
                                                   v4u (&w)[P]) {
#pragma unroll
    for (int u = 0; u < P; ++u) {
        const int st = min(s0 + u, s_last);
        w[u] = __builtin_nontemporal_load(tiles + static_cast<size_t>(st) * 64);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Each lane holds partial sums of the four rows of its 16-lane group (over
// its own K chunk).  Afterwards lane l holds the full sum, over the 16 lanes,
// of row l % 4 of the group: a reduce-scatter inside each quad, then a sum
// over the four quads by rotations that keep l % 4.
__device__ __forceinline__ int row_group_reduce(const int (&v)[4], int lane) {
    const bool b = (lane >> 1) & 1;
    const int send0 = b ? v[0] : v[2];
    const int send1 = b ? v[1] : v[3];
    int keep0 = b ? v[2] : v[0];
    int keep1 = b ? v[3] : v[1];
    keep0 += dpp_row<kDppQuadXor2>(send0);
    keep1 += dpp_row<kDppQuadXor2>(send1);
    const bool a = lane & 1;
    const int send = a ? keep0 : keep1;
    int keep = a ? keep1 : keep0;
    keep += dpp_row<kDppQuadXor1>(send);     // row 2b + a = lane % 4, summed over the quad
    keep += dpp_row<kDppRowRor4>(keep);
    keep += dpp_row<kDppRowRor8>(keep);       // summed over the four quads
    return keep;
}

__device__ __forceinline__ float absmax8_bf16(const uint4& v, float m) {
    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j)
        m = fmaxf(m, fmaxf(fabsf(__uint_as_float(d[j] << 16)),
                           fabsf(__uint_as_float(d[j] & 0xFFFF0000u))));
    return m;
}

__device__ __forceinline__ uint2 quant8_bf16(const uint4& v, float sm) {
    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
    uint2 o;
    o.x = quant4(__uint_as_float(d[0] << 16), __uint_as_float(d[0] & 0xFFFF0000u),
                 __uint_as_float(d[1] << 16), __uint_as_float(d[1] & 0xFFFF0000u), sm);
    o.y = quant4(__uint_as_float(d[2] << 16), __uint_as_float(d[2] & 0xFFFF0000u),
                 __uint_as_float(d[3] << 16), __uint_as_float(d[3] & 0xFFFF0000u), sm);
    return o;
}

__device__ __forceinline__ int sum_i8x4(uint32_t d, int acc) {
    return dot4(static_cast<int>(d), 0x01010101, acc);
}

constexpr int kMinGroups = 200;     // workgroups wanted in flight (256 CUs)
// K steps per wavefront aimed at.  A narrow matrix (fewer than kNarrowBands
// bands: fewer single-band workgroups than about 1.5 per CU) leaves most
// SIMDs with one wavefront, whose dot products after the last tile arrives
// set the tail, so it takes shorter runs.  Measured same-box: at 2560 x 2560,
// 3840 x 2560 and 2560 x 6912 the shorter runs gain 0.05-0.27 us; at
// 13824 x 2560 they lose 0.5 us.  Wide matrices take runs of up to 10 (a
// whole K = 2560 row per wavefront, half the wavefronts of runs of 5):
// 0.05 us faster at 13824 x 2560.
constexpr int kTargetSteps = 10;
constexpr int kTargetStepsNarrow = 4;
constexpr int kNarrowBands = 400;
// The M = 1 GEMV adds a middle tier and a cap (gemv_shape; a same-box sweep
// of the wavefronts per band over 16 shapes, int8 and bf16 input).  Between
// kNarrowBands and kWideBands bands, runs of at most 5: with one wavefront
// per band too few are in flight (6912 x 2560: 3.00 -> 2.87 us int8, 3.64 ->
// 3.13 us bf16).  And at most kBandWaves wavefronts per band while their
// runs stay within the kernels' steps: a band's 16 wavefronts cost more in
// their reduction than their shorter runs save (2560 x 13824: 4.77 -> 3.89
// us int8, 5.80 -> 4.88 bf16; 3200 x 10240: 4.12 -> 3.46, 5.25 -> 3.86;
// 5120 x 13824: 6.76 -> 6.06, 8.75 -> 7.73).
constexpr int kTargetStepsMedium = 5;
constexpr int kWideBands = 768;
constexpr int kBandWaves = 8;

}  // namespace bl
