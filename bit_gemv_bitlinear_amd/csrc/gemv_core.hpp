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
