// gemv.hip -- the M = 1 decode GEMV of the W2A8 ternary linear layer on gfx950.
//
// Source page: "BitNet GPU 推理框架：从零构建 W2A8 的 2-bit 大模型 CUDA GEMV 内核"
// (blog.gitcode.com), cited as [W2A8]: §5.2 (codes w + 2, interleaved 32-bit
// words decoded by shift and mask), §5.3 (int8 dot products into an int32
// accumulator, then out = acc * scales with ws[n / (N / ws_num)]), §六 item 3
// (per-token activation quantisation, fused here for bf16 input).
//
// Mapping (this library's design; the page's sm_80 kernel is prior art):
//   * a band is 16 output rows; a workgroup takes B = 1, 2 or 4 consecutive
//     bands (more for wide matrices, so that each activation staging serves
//     more rows; fewer for narrow ones, so that there are enough workgroups);
//     the Wb wavefronts of a band split its S K-steps (256 K = one 1 KiB
//     tile each), P consecutive steps per wavefront, (B, Wb, P) picked per
//     shape by gemv_shape();
//   * a wavefront's load of a tile is one coalesced 16-byte-per-lane load of
//     1 KiB; lane l's slot holds rows 4*(l/16) .. +3 of K chunk l%16, so each
//     lane needs one 16-byte run of activations per step;
//   * every weight load of the wavefront is issued up front (P is a template
//     argument, so the loads are unconditional and the compiler counts them
//     exactly), right after the lane's weight scale and its share of the
//     activation row, and nothing is scheduled above them; the weight scale's
//     row-to-segment division is a multiply and shift with host-made
//     constants, so no division delays the loads;
//   * the activation row is staged once per workgroup in LDS (zero-padded to
//     Wb*P steps; steps past the band's end re-read its last tile and meet
//     zero activations), read back as one 16-byte LDS load per step;
//   * decoding keeps the unsigned codes c = w + 2 and never shifts them into
//     place: field i of a word is masked in place (factor 4^i, i < 3) and
//     dotted with activation word i into one of three accumulators; field 3
//     is shifted down once.  acc = a1 + a4/4 + a16/16 - 2 * sum(x), the last
//     term removing the +2 offset (padding code 0 contributes nothing);
//   * the 16 lanes sharing four rows add their partial sums with DPP row
//     operations; the Wb wavefronts of a band are added through LDS;
//   * the fused bf16 path quantises in the workgroup: absmax by DPP within
//     each wavefront and LDS across them, then round-to-int by the 1.5 * 2^23
//     addition (two roundings, as the definition has them);
//   * the epilogue multiplies by a precomputed fp64 ws/s and rounds once to
//     bf16, dividing only when the product lies next to a rounding boundary
//     (so the result is that of the exact fp64 division); wavefront 0 forms
//     ws/s and the code offset before its main loop, so the tail after the
//     last barrier is one multiply, the rounding and the store.
#include <algorithm>
#include <array>
#include <utility>

#include "common.hpp"
#include "kernels.hpp"

namespace bl {

namespace {

constexpr int kMaxWaves = 16;
// C = 16-byte activation chunks per thread loaded ahead of the weights and
// kept in registers (1, 2 or 4, a template argument chosen per shape).
// Chunks beyond them are loaded after the weights, and since the waits count
// loads in issue order, using them waits for every weight; so C covers the
// row wherever it can (bf16 rows have twice the chunks of int8 rows: 2560 x
// 2 B over 128 threads for qkv and o, 6912 x 2 B over 256 threads for down).
// Chunks a thread does not need cost code on the path to the main loop, so C
// is no larger than the row needs.
constexpr int kMaxCached = 4;

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

template <int P>
__device__ __forceinline__ void load_steps(const v4u* __restrict__ tiles, int s0, int s_last,
                                           v4u (&w)[P]) {
#pragma unroll
    for (int u = 0; u < P; ++u) {
        const int st = min(s0 + u, s_last);
        w[u] = __builtin_nontemporal_load(tiles + static_cast<size_t>(st) * 64);
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

// Row n's weight scale is ws[n / seg], seg = N / ws_num, found as
// (n * seg_mul) >> seg_shift (see seg_divisor()).  B bands per workgroup, 2^lw
// wavefronts per band (blockDim.x = 64 * B * 2^lw), P K-steps per wavefront.
// FUSED = false: xin is int8 activations with scale s_in[0].
// FUSED = true:  xin is bf16; the workgroup quantises it (per-token absmax,
//                [W2A8] §六 item 3); workgroup 0 writes q_out / s_out if given.
template <int P, bool FUSED, int C>
__global__ __launch_bounds__(kMaxWaves * 64) void gemv_kernel(
    const void* __restrict__ xin, const v4u* __restrict__ packed, const float* __restrict__ s_in,
    const uint16_t* __restrict__ ws, uint32_t seg_mul, int seg_shift, uint16_t* __restrict__ y,
    int32_t* __restrict__ acc, int8_t* __restrict__ q_out, float* __restrict__ s_out, int N,
    int K, int B, int lw) {
    extern __shared__ int4 act[];   // Wb*P*16 16-byte chunks: the int8 row, zero-padded
    __shared__ int part_sh[kMaxWaves][64];
    __shared__ int xsum_sh[kMaxWaves];
    __shared__ float amax_sh[kMaxWaves];
    const int Wb = 1 << lw;
    const int W = B << lw;
    const int nthreads = W * 64;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nbands = (N + kTileRows - 1) / kTileRows;
    const int band = min(static_cast<int>(blockIdx.x) * B + (wave >> lw), nbands - 1);
    const int S = (K + kTileK - 1) / kTileK;
    const int s0 = (wave & (Wb - 1)) * P;
    const int n16 = K >> 4;        // 16-byte chunks of int8 activations
    const int padded16 = Wb * P * 16;

    // 1. The activation row and the weight scale of this thread's output row
    //    first (so that waiting for them does not wait for the weights), then
    //    every weight load of this wavefront.
    const int n_out = static_cast<int>(blockIdx.x) * B * kTileRows + tid;   // tid < 16*B writes
    const uint32_t n_ws = static_cast<uint32_t>(min(n_out, N - 1));
    // unconditional: no branch, no early wait
    const uint16_t wsb = ws[(static_cast<uint64_t>(n_ws) * seg_mul) >> seg_shift];
    constexpr int kCached = C;
    uint4 xv[kCached];
    const int n_in = FUSED ? (K >> 3) : n16;   // 16-byte input chunks
    const uint4* x16 = reinterpret_cast<const uint4*>(xin);
#pragma unroll
    for (int c = 0; c < kCached; ++c) {
        const int idx = tid + c * nthreads;
        xv[c] = make_uint4(0, 0, 0, 0);
        if (idx < n_in) xv[c] = x16[idx];
    }
    const v4u* tiles = packed + static_cast<size_t>(band) * S * 64 + lane;
    v4u w[P];
    load_steps<P>(tiles, s0, S - 1, w);
    // Nothing may be scheduled above this point: otherwise the compiler may
    // start on the activations first, and the wait for them would hold back
    // the remaining weight loads by a full memory latency.
    __builtin_amdgcn_sched_barrier(0);

    // 2. Stage the int8 row in LDS and sum it (for the +2 code offset).
    int xs = 0;
    float sm = 0.0f;
    if (!FUSED) {
        sm = s_in[0];
#pragma unroll
        for (int c = 0; c < kCached; ++c) {
            const int idx = tid + c * nthreads;
            if (idx < n_in) {
                act[idx] = make_int4(xv[c].x, xv[c].y, xv[c].z, xv[c].w);
                xs = sum_i8x4(xv[c].x, sum_i8x4(xv[c].y, sum_i8x4(xv[c].z, sum_i8x4(xv[c].w, xs))));
            }
        }
        for (int idx = tid + kCached * nthreads; idx < n_in; idx += nthreads) {
            const uint4 v = x16[idx];
            act[idx] = make_int4(v.x, v.y, v.z, v.w);
            xs = sum_i8x4(v.x, sum_i8x4(v.y, sum_i8x4(v.z, sum_i8x4(v.w, xs))));
        }
    } else {
        float amax = 0.0f;
#pragma unroll
        for (int c = 0; c < kCached; ++c)
            if (tid + c * nthreads < n_in) amax = absmax8_bf16(xv[c], amax);
        for (int idx = tid + kCached * nthreads; idx < n_in; idx += nthreads)
            amax = absmax8_bf16(x16[idx], amax);
        amax = wave_max(amax);
        if (lane == 0) amax_sh[wave] = amax;
        __syncthreads();
        amax = amax_sh[0];
        for (int i = 1; i < W; ++i) amax = fmaxf(amax, amax_sh[i]);
        sm = 127.0f / fmaxf(amax, 1e-5f);
        uint2* act8 = reinterpret_cast<uint2*>(act);
        const bool write_q = (blockIdx.x == 0) && (q_out != nullptr);
#pragma unroll
        for (int c = 0; c < kCached; ++c) {
            const int idx = tid + c * nthreads;
            if (idx < n_in) {
                const uint2 o = quant8_bf16(xv[c], sm);
                act8[idx] = o;
                xs = sum_i8x4(o.x, sum_i8x4(o.y, xs));
                if (write_q) reinterpret_cast<uint2*>(q_out)[idx] = o;
            }
        }
        for (int idx = tid + kCached * nthreads; idx < n_in; idx += nthreads) {
            const uint2 o = quant8_bf16(x16[idx], sm);
            act8[idx] = o;
            xs = sum_i8x4(o.x, sum_i8x4(o.y, xs));
            if (write_q) reinterpret_cast<uint2*>(q_out)[idx] = o;
        }
        if (blockIdx.x == 0 && s_out != nullptr && tid == 0) s_out[0] = sm;
    }
    for (int i = n16 + tid; i < padded16; i += nthreads) act[i] = make_int4(0, 0, 0, 0);
    xs = wave_sum(xs);
    if (lane == 0) xsum_sh[wave] = xs;
    __syncthreads();
    // Wavefront 0 alone needs the epilogue's factors: the scale ws / s (as
    // fl64(ws * fl64(1/s))) and the code offset correction -2 * sum(x).  It
    // forms them here, while the weights are still in flight, rather than
    // after the last barrier; the empty asm statement keeps the compiler from
    // sinking them past the barrier to their use.
    double cs = 0.0;
    int offset = 0;
    if (wave == 0) {
        cs = static_cast<double>(bf16_to_float(wsb)) * (1.0 / static_cast<double>(sm));
        for (int i = 0; i < W; ++i) offset -= 2 * xsum_sh[i];
        asm volatile("" : "+v"(cs), "+v"(offset));
    }

    // 3. P steps of 4 rows x 16 K per lane.
    RowAcc r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r.a1[i] = r.a4[i] = r.a16[i] = 0;
    const int kc = lane & 15;
#pragma unroll
    for (int u = 0; u < P; ++u) dot_slot(w[u], act[(s0 + u) * 16 + kc], r);
    int v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = r.a1[i] + (r.a4[i] >> 2) + (r.a16[i] >> 4);   // exact
    // lane l now holds row 4*(l/16) + l%4 of its band (replicated over l/4 % 4)
    part_sh[wave][lane] = row_group_reduce(v, lane);
    __syncthreads();

    // 4. Wavefront 0, lane l < 16*B: row l % 16 of band l / 16 -- add the
    //    Wb wavefronts' sums, remove the code offset, epilogue.
    if (wave == 0) {
        const int bw = lane >> 4;
        const int rw = lane & 15;
        const int slot = 16 * (rw >> 2) + (rw & 3);
        const int first = min(bw, B - 1) << lw;   // in range for every lane
        int total = offset;
        for (int j = 0; j < Wb; ++j) total += part_sh[first + j][slot];
        if (bw < B && n_out < N) {
            y[n_out] = epilogue_bf16_scaled(total, cs, bf16_to_float(wsb), sm);
            if (acc) acc[n_out] = total;
        }
    }
}

// The bf16-input layer with the activations kept wave-local (no staged row).
// Lane (rg = l/16, kc = l%16) of a wavefront covers, at step u, the 16-wide K
// chunk kc of tile s0 + u for the four rows of its slot.  It loads the 4 bf16
// values 4*rg .. +3 of that chunk, so the wavefront's 64 lanes cover its K
// range once; the absmax is exchanged across the workgroup (one barrier),
// each lane quantises its 4 values into one int8x4 word and writes it to a
// wavefront-private LDS slot, and reads back the chunk's 16 bytes (the words
// of lanes rg = 0..3) -- within a wavefront no barrier is needed.  The code
// offset -2 * sum(x) is taken per lane over its chunks and folded into its
// four rows before the row reduction.  Workgroup 0's first band writes
// q_out / s_out when given.
//
// Against the staged kernel this saves a barrier and the row copy, but every
// band of a workgroup loads its own copy of the row.  Measured same-box over
// bf16 shapes, it is faster (by about 0.3 us) only with one band per
// workgroup, at most 4 wavefronts and at most 256 workgroups -- 1024, 2560
// and 3840 rows at K = 2560 -- and slower elsewhere (5120 x 2560, 6912 x 2560,
// K >= 5120, 13824 x 2560); launch() uses it only there.
template <int P>
__global__ __launch_bounds__(kMaxWaves * 64) void gemv_local_kernel(
    const void* __restrict__ xin, const v4u* __restrict__ packed, const float* __restrict__ s_in,
    const uint16_t* __restrict__ ws, uint32_t seg_mul, int seg_shift, uint16_t* __restrict__ y,
    int32_t* __restrict__ acc, int8_t* __restrict__ q_out, float* __restrict__ s_out, int N,
    int K, int B, int lw) {
    extern __shared__ uint32_t actw[];   // W * P * 64 quantised words
    __shared__ int part_sh[kMaxWaves][64];
    __shared__ float amax_sh[kMaxWaves];
    const int Wb = 1 << lw;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nbands = (N + kTileRows - 1) / kTileRows;
    const int band = min(static_cast<int>(blockIdx.x) * B + (wave >> lw), nbands - 1);
    const int S = (K + kTileK - 1) / kTileK;
    const int s0 = (wave & (Wb - 1)) * P;
    const int kc = lane & 15;
    const int rg = lane >> 4;

    const int n_out = static_cast<int>(blockIdx.x) * B * kTileRows + tid;   // tid < 16*B writes
    const uint32_t n_ws = static_cast<uint32_t>(min(n_out, N - 1));
    const uint16_t wsb = ws[(static_cast<uint64_t>(n_ws) * seg_mul) >> seg_shift];
    // this lane's 4 activations per step, from clamped addresses (unconditional loads)
    uint2 xb[P];
#pragma unroll
    for (int u = 0; u < P; ++u) {
        const int kk = min((s0 + u) * kTileK + 16 * kc + 4 * rg, K - 4);
        xb[u] = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(xin) + kk);
    }
    const v4u* tiles = packed + static_cast<size_t>(band) * S * 64 + lane;
    v4u w[P];
    load_steps<P>(tiles, s0, S - 1, w);
    __builtin_amdgcn_sched_barrier(0);

    int4 xq[P];
    float sm;
    {
        float amax = 0.0f;
#pragma unroll
        for (int u = 0; u < P; ++u) {
            const bool live = (s0 + u) * kTileK + 16 * kc < K;
            const uint32_t lo = live ? xb[u].x : 0u;
            const uint32_t hi = live ? xb[u].y : 0u;
            xb[u] = uint2{lo, hi};
            amax = fmaxf(amax, fmaxf(fmaxf(fabsf(__uint_as_float(lo << 16)),
                                           fabsf(__uint_as_float(lo & 0xFFFF0000u))),
                                     fmaxf(fabsf(__uint_as_float(hi << 16)),
                                           fabsf(__uint_as_float(hi & 0xFFFF0000u)))));
        }
        amax = wave_max(amax);
        if (lane == 0) amax_sh[wave] = amax;
        __syncthreads();
        // the Wb wavefronts of this band cover the whole row
        const int first = (wave >> lw) << lw;
        amax = amax_sh[first];
        for (int j = 1; j < Wb; ++j) amax = fmaxf(amax, amax_sh[first + j]);
        sm = 127.0f / fmaxf(amax, 1e-5f);
        uint32_t* mine = actw + static_cast<size_t>(wave) * P * 64;
        const bool write_q = q_out != nullptr && blockIdx.x == 0 && (wave >> lw) == 0;
#pragma unroll
        for (int u = 0; u < P; ++u) {
            const uint32_t word = quant4(__uint_as_float(xb[u].x << 16),
                                         __uint_as_float(xb[u].x & 0xFFFF0000u),
                                         __uint_as_float(xb[u].y << 16),
                                         __uint_as_float(xb[u].y & 0xFFFF0000u), sm);
            mine[u * 64 + 4 * kc + rg] = word;   // word rg of chunk kc
            const int k = (s0 + u) * kTileK + 16 * kc + 4 * rg;
            if (write_q && k < K) *reinterpret_cast<uint32_t*>(q_out + k) = word;
        }
        // Within one wavefront LDS operations complete in order; the fence
        // keeps the compiler from moving the reads above the writes.
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int u = 0; u < P; ++u) xq[u] = *reinterpret_cast<const int4*>(mine + u * 64 + 4 * kc);
        if (s_out != nullptr && blockIdx.x == 0 && tid == 0) s_out[0] = sm;
    }
    double cs = 0.0;
    if (wave == 0) {
        cs = static_cast<double>(bf16_to_float(wsb)) * (1.0 / static_cast<double>(sm));
        asm volatile("" : "+v"(cs));
    }

    RowAcc r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r.a1[i] = r.a4[i] = r.a16[i] = 0;
    int xs = 0;
#pragma unroll
    for (int u = 0; u < P; ++u) {
        dot_slot(w[u], xq[u], r);
        xs = sum_i8x4(xq[u].x, sum_i8x4(xq[u].y, sum_i8x4(xq[u].z, sum_i8x4(xq[u].w, xs))));
    }
    int v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = r.a1[i] + (r.a4[i] >> 2) + (r.a16[i] >> 4) - 2 * xs;
    part_sh[wave][lane] = row_group_reduce(v, lane);
    __syncthreads();

    if (wave == 0) {
        const int bw = lane >> 4;
        const int rw = lane & 15;
        const int slot = 16 * (rw >> 2) + (rw & 3);
        const int first = min(bw, B - 1) << lw;
        int total = 0;
        for (int j = 0; j < Wb; ++j) total += part_sh[first + j][slot];
        if (bw < B && n_out < N) {
            y[n_out] = epilogue_bf16_scaled(total, cs, bf16_to_float(wsb), sm);
            if (acc) acc[n_out] = total;
        }
    }
}

// ---------------------------------------------------------------------------
// The projection of a decode step with its glue ([W2A8] §4.1 names the
// model's norms attention_norm / ffn_norm / attn_sub_norm / ffn_sub_norm and
// its fused projections wqkv / wo / w13 / w2; the formulas are readings):
//   m  = x, or bf16(max(x, 0)^2 * x_up) for the MLP's down projection
//        (x = the gate half and x_up = the up half of w13's output);
//   xn = bf16( fl64(m * gamma) * fl64(1 / sqrt(sum(m^2) / K + eps)) );
//   per-token absmax int8 quantisation of xn, the ternary layer, and
//   y = bf16(acc * ws / s), or bf16(residual + that) when a residual is given.
// The glue runs in the prologue of every workgroup (the row is at most a few
// thousand elements, read from L2 by each): no kernel of its own, so a chained
// decode step launches one kernel per projection.  Everything else is the
// staged kernel above: the weight loads are all issued before the first wait.
// ---------------------------------------------------------------------------

// Sum of a double over the 64 lanes: the two 32-bit halves move together
// through the DPP steps of wave_sum (pairs, quads, rotations by 4 and 8 inside
// each row of 16), then the four row totals are read out and added.  The
// result is the same in every lane.
template <int CTRL>
__device__ __forceinline__ double dpp_row_f64(double v) {
    const int lo = __builtin_amdgcn_mov_dpp(__double2loint(v), CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_mov_dpp(__double2hiint(v), CTRL, 0xF, 0xF, false);
    return __hiloint2double(hi, lo);
}
__device__ __forceinline__ double readlane_f64(double v, int l) {
    return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), l),
                            __builtin_amdgcn_readlane(__double2loint(v), l));
}
__device__ __forceinline__ double wave_sum_f64(double v) {
    v += dpp_row_f64<kDppQuadXor1>(v);
    v += dpp_row_f64<kDppQuadXor2>(v);
    v += dpp_row_f64<kDppRowRor4>(v);
    v += dpp_row_f64<kDppRowRor8>(v);
    return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}

// Unsigned maximum over the 64 lanes, by the same steps.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_row_u32(uint32_t v) {
    return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, dpp_row_u32<kDppQuadXor1>(v));
    v = max(v, dpp_row_u32<kDppQuadXor2>(v));
    v = max(v, dpp_row_u32<kDppRowRor4>(v));
    v = max(v, dpp_row_u32<kDppRowRor8>(v));
    const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
    const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
    return max(max(r0, r1), max(r2, r3));
}

__device__ __forceinline__ uint32_t bf16_lo(uint32_t w) { return w & 0xFFFFu; }
__device__ __forceinline__ uint32_t bf16_hi(uint32_t w) { return w >> 16; }
__device__ __forceinline__ double bf16_f64(uint32_t b) {
    return static_cast<double>(__uint_as_float(b << 16));
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
// quiet NaN 0x7FC0.
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

// Eight fp64 values to bf16 (nearest, ties to even) by way of fp32: one
// conversion to fp32, one to bf16.  Every bf16 midpoint is an fp32 number,
// so the first rounding can land on one but never step across one: the two
// roundings differ from one direct rounding only where the fp32 value is a
// bf16 midpoint (low 16 bits 0x8000).  Such chunks, and NaN, are rounded
// again by bf16_rne_f64.
__device__ __forceinline__ uint4 bf16x8_from_f64(const double (&d)[8]) {
    uint32_t o[4];
    bool redo = false;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float f0 = static_cast<float>(d[2 * j]), f1 = static_cast<float>(d[2 * j + 1]);
        redo = redo | ((__float_as_uint(f0) & 0xFFFFu) == 0x8000u);
        redo = redo | ((__float_as_uint(f1) & 0xFFFFu) == 0x8000u);
        redo = redo | __builtin_isunordered(f0, f1);
        o[j] = cvt_pk_bf16(f0, f1);
    }
    // a wave-uniform branch, taken by a wavefront when any of its lanes needs
    // it (rarely); the empty volatile statement keeps the compiler from
    // if-converting it, which would pay its work on every chunk
    if (__builtin_amdgcn_ballot_w64(redo) != 0) {
        asm volatile("");
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = bf16_rne_f64(d[2 * j]) | (bf16_rne_f64(d[2 * j + 1]) << 16);
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
}

// Chunk of 8 bf16: relu2-GLU, exact in fp64 (at most 24 significant bits),
// rounded once, into m.
__device__ __forceinline__ uint4 glu8(const uint4& g, const uint4& u) {
    const uint32_t gd[4] = {g.x, g.y, g.z, g.w};
    const uint32_t ud[4] = {u.x, u.y, u.z, u.w};
    double m[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float a0 = __uint_as_float(gd[j] << 16), a1 = __uint_as_float(gd[j] & 0xFFFF0000u);
        const double g0 = a0 > 0.0f ? static_cast<double>(a0) : 0.0;
        const double g1 = a1 > 0.0f ? static_cast<double>(a1) : 0.0;
        m[2 * j] = g0 * g0 * bf16_f64(bf16_lo(ud[j]));
        m[2 * j + 1] = g1 * g1 * bf16_f64(bf16_hi(ud[j]));
    }
    return bf16x8_from_f64(m);
}

// p = m * gamma (exact in fp64) for a chunk of 8, with the running sum of
// m^2 and the running maximum of |p| as the high word of its encoding: p has
// at most 16 significant bits, all in that word (the low word is zero), so
// comparing high words of magnitudes as integers compares the magnitudes.
__device__ __forceinline__ void products8(const uint4& m, const uint4& g, double (&p)[8],
                                          double& ssq, uint32_t& pm) {
    const uint32_t md[4] = {m.x, m.y, m.z, m.w};
    const uint32_t gd[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const double a = bf16_f64(bf16_lo(md[j])), b = bf16_f64(bf16_hi(md[j]));
        p[2 * j] = a * bf16_f64(bf16_lo(gd[j]));
        p[2 * j + 1] = b * bf16_f64(bf16_hi(gd[j]));
        ssq += a * a;
        ssq += b * b;
        pm = max(pm, max(static_cast<uint32_t>(__double2hiint(p[2 * j])) & 0x7FFFFFFFu,
                         static_cast<uint32_t>(__double2hiint(p[2 * j + 1])) & 0x7FFFFFFFu));
    }
}

// xn = bf16(p * inv) for a chunk of 8 (NaN where inv is infinite and p zero:
// a zero row with eps = 0).
__device__ __forceinline__ uint4 norm8(const double (&p)[8], double inv) {
    double v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = p[e] * inv;
    return bf16x8_from_f64(v);
}

// A row of K bf16 values as a raw buffer (16-byte loads by chunk index).
using RowBuf = __amdgpu_buffer_rsrc_t;
constexpr int kRawBufferFlags = 0x00020000;   // word 3 of the descriptor: 32-bit data format
__device__ __forceinline__ RowBuf row_buffer(const uint16_t* p, int K) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p), 0, 2 * K, kRawBufferFlags);
}
__device__ __forceinline__ uint4 row_load(RowBuf r, int chunk) {
    const v4u v = __builtin_amdgcn_raw_buffer_load_b128(r, chunk * 16, 0, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// At most kNormMaxWaves wavefronts per workgroup: the registers that hold
// the row's exact products (two per value) need the larger per-wavefront
// budget.
constexpr int kNormMaxWaves = 8;

template <int P, int C, bool GLU>
__global__ __launch_bounds__(kNormMaxWaves * 64) void gemv_norm_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ x_up,
    const uint16_t* __restrict__ gamma, double eps, const v4u* __restrict__ packed,
    const uint16_t* __restrict__ ws, uint32_t seg_mul, int seg_shift,
    const uint16_t* __restrict__ residual, uint16_t* __restrict__ y, int32_t* __restrict__ acc,
    int8_t* __restrict__ q_out, float* __restrict__ s_out, uint16_t* __restrict__ xn_out, int N,
    int K, int B, int lw) {
    extern __shared__ int4 act[];   // Wb*P*16 16-byte chunks: the int8 row, zero-padded
    __shared__ int part_sh[kNormMaxWaves][64];
    __shared__ int xsum_sh[kNormMaxWaves];
    __shared__ double ssq_sh[kNormMaxWaves];
    __shared__ uint32_t pm_sh[kNormMaxWaves];
    const int Wb = 1 << lw;
    const int W = B << lw;
    const int nthreads = W * 64;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nbands = (N + kTileRows - 1) / kTileRows;
    const int band = min(static_cast<int>(blockIdx.x) * B + (wave >> lw), nbands - 1);
    const int S = (K + kTileK - 1) / kTileK;
    const int s0 = (wave & (Wb - 1)) * P;
    const int n16 = K >> 4;
    const int padded16 = Wb * P * 16;
    const int n_in = K >> 3;        // 16-byte chunks of bf16

    // 1. The inputs of this thread's output row (weight scale, residual),
    //    the cached chunks of the row (x, x_up, gamma), then every weight load.
    const int n_out = static_cast<int>(blockIdx.x) * B * kTileRows + tid;   // tid < 16*B writes
    const uint32_t n_c = static_cast<uint32_t>(min(n_out, N - 1));
    const uint16_t wsb = ws[(static_cast<uint64_t>(n_c) * seg_mul) >> seg_shift];
    // unconditional (a branch would end in a wait for this load); the weight
    // scales stand in as a source when there is no residual
    const uint16_t resb = (residual ? residual : ws)[residual ? n_c : 0u];
    const uint4* x16 = reinterpret_cast<const uint4*>(x);
    const uint4* u16 = reinterpret_cast<const uint4*>(x_up);
    const uint4* g16 = reinterpret_cast<const uint4*>(gamma);
    // The cached chunks come through buffer loads: the compiler treats plain
    // loads of these read-only rows as free to sink to their first use,
    // past the weight loads, and a wait there would wait for every one.
    const RowBuf rx = row_buffer(x, K), ru = row_buffer(x_up, K), rg = row_buffer(gamma, K);
    // A chunk past the row's end reads as zeros (the buffer's range check),
    // which add nothing to the sum of squares or the maximum.
    uint4 xv[C], uv[GLU ? C : 1], gv[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int idx = tid + c * nthreads;
        xv[c] = row_load(rx, idx);
        if constexpr (GLU) uv[c] = row_load(ru, idx);
        gv[c] = row_load(rg, idx);
    }
    const v4u* tiles = packed + static_cast<size_t>(band) * S * 64 + lane;
    v4u w[P];
    load_steps<P>(tiles, s0, S - 1, w);
    // No load may move below this point (a row load sunk past the weight
    // loads would wait for all of them: the waits count loads in issue
    // order), and nothing may be scheduled above it.
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);

    // 2. m (GLU); p = m * gamma, exact in fp64 and kept for step 4; the sum
    //    of m^2 and the largest |p|.  Chunks beyond the C cached ones (rows
    //    longer than C x 8 x threads) are re-read from L2, here and in step 4.
    auto m_chunk = [&](int c, int idx) -> uint4 {
        if (c < C) {
            if constexpr (GLU) return glu8(xv[c], uv[c]);
            return xv[c];
        }
        if constexpr (GLU) return glu8(x16[idx], u16[idx]);
        return x16[idx];
    };
    double ssq = 0.0;
    uint32_t pm = 0;   // high word of the largest |p|
    double pv[C][8];
#pragma unroll
    for (int c = 0; c < C; ++c) products8(m_chunk(c, tid + c * nthreads), gv[c], pv[c], ssq, pm);
    for (int idx = tid + C * nthreads; idx < n_in; idx += nthreads) {
        double pt[8];
        products8(m_chunk(C, idx), g16[idx], pt, ssq, pm);
    }
    ssq = wave_sum_f64(ssq);
    pm = wave_max_u32(pm);
    if (lane == 0) {
        ssq_sh[wave] = ssq;
        pm_sh[wave] = pm;
    }
    __syncthreads();

    // 3. The inverse RMS and the activation scale.  Rounding is monotone and
    //    inv > 0, so the largest |xn| is the bf16 rounding of pmax * inv: the
    //    absmax needs no pass over xn.  The partial sums are added in wave
    //    order; all eight slots are read at once and the unused ones dropped.
    double total_sq = 0.0;
    pm = 0;
#pragma unroll
    for (int i = 0; i < kNormMaxWaves; ++i) {
        const double v = ssq_sh[i];
        const uint32_t u = pm_sh[i];
        total_sq += i < W ? v : 0.0;
        pm = max(pm, i < W ? u : 0u);
    }
    const double inv = 1.0 / sqrt(total_sq / static_cast<double>(K) + eps);
    const double pmax = __hiloint2double(static_cast<int>(pm), 0);
    const float amax = __uint_as_float(bf16_rne_f64(pmax * inv) << 16);
    const float sm = 127.0f / fmaxf(amax, 1e-5f);

    // 4. Quantise xn into LDS (workgroup 0 also writes xn, q and s when asked).
    uint2* act8 = reinterpret_cast<uint2*>(act);
    const bool first = blockIdx.x == 0;
    int xs = 0;
    auto put = [&](int idx, const uint4& v) {
        const uint2 o = quant8_bf16(v, sm);
        act8[idx] = o;
        xs = sum_i8x4(o.x, sum_i8x4(o.y, xs));
        if (first && q_out) reinterpret_cast<uint2*>(q_out)[idx] = o;
        if (first && xn_out) reinterpret_cast<uint4*>(xn_out)[idx] = v;
    };
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int idx = tid + c * nthreads;
        if (idx < n_in) put(idx, norm8(pv[c], inv));
    }
    for (int idx = tid + C * nthreads; idx < n_in; idx += nthreads) {
        double pt[8];
        products8(m_chunk(C, idx), g16[idx], pt, ssq, pm);
        put(idx, norm8(pt, inv));
    }
    if (first && s_out != nullptr && tid == 0) s_out[0] = sm;
    for (int i = n16 + tid; i < padded16; i += nthreads) act[i] = make_int4(0, 0, 0, 0);
    xs = wave_sum(xs);
    if (lane == 0) xsum_sh[wave] = xs;
    __syncthreads();
    double cs = 0.0;
    int offset = 0;
    if (wave == 0) {
        cs = static_cast<double>(bf16_to_float(wsb)) * (1.0 / static_cast<double>(sm));
        for (int i = 0; i < W; ++i) offset -= 2 * xsum_sh[i];
        asm volatile("" : "+v"(cs), "+v"(offset));
    }

    // 5. P steps of 4 rows x 16 K per lane, reduction, epilogue (+ residual).
    RowAcc r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r.a1[i] = r.a4[i] = r.a16[i] = 0;
    const int kc = lane & 15;
#pragma unroll
    for (int u = 0; u < P; ++u) dot_slot(w[u], act[(s0 + u) * 16 + kc], r);
    int v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = r.a1[i] + (r.a4[i] >> 2) + (r.a16[i] >> 4);
    part_sh[wave][lane] = row_group_reduce(v, lane);
    __syncthreads();
    if (wave == 0) {
        const int bw = lane >> 4;
        const int rw = lane & 15;
        const int slot = 16 * (rw >> 2) + (rw & 3);
        const int firstw = min(bw, B - 1) << lw;
        int total = offset;
        for (int j = 0; j < Wb; ++j) total += part_sh[firstw + j][slot];
        if (bw < B && n_out < N) {
            uint16_t o = epilogue_bf16_scaled(total, cs, bf16_to_float(wsb), sm);
            if (residual)   // the fp64 sum of two bf16 values rounds to bf16 as the exact sum does
                o = static_cast<uint16_t>(bf16_rne_f64(static_cast<double>(bf16_to_float(resb)) +
                                                       static_cast<double>(bf16_to_float(o))));
            y[n_out] = o;
            if (acc) acc[n_out] = total;
        }
    }
}

constexpr int kMaxSteps = 20;
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

using GemvFn = void (*)(const void*, const v4u*, const float*, const uint16_t*, uint32_t, int,
                        uint16_t*, int32_t*, int8_t*, float*, int, int, int, int);

template <bool FUSED, int C, int... Ps>
constexpr std::array<GemvFn, sizeof...(Ps)> kernel_table(std::integer_sequence<int, Ps...>) {
    return {{&gemv_kernel<Ps + 1, FUSED, C>...}};
}

template <int... Ps>
constexpr std::array<GemvFn, sizeof...(Ps)> local_table(std::integer_sequence<int, Ps...>) {
    return {{&gemv_local_kernel<Ps + 1>...}};
}

using KernelRow = std::array<GemvFn, kMaxSteps>;
// The wave-local bf16 kernel, P = 1 .. kLocalMaxSteps (beyond that its
// registers, 8 per step, would not fit a 16-wavefront workgroup).
constexpr int kLocalMaxSteps = 12;
const std::array<GemvFn, kLocalMaxSteps> kLocalKernels =
    local_table(std::make_integer_sequence<int, kLocalMaxSteps>{});
// [fused][log2 C][P - 1]
const std::array<std::array<KernelRow, 3>, 2> kKernels = {{
    {{kernel_table<false, 1>(std::make_integer_sequence<int, kMaxSteps>{}),
      kernel_table<false, 2>(std::make_integer_sequence<int, kMaxSteps>{}),
      kernel_table<false, 4>(std::make_integer_sequence<int, kMaxSteps>{})}},
    {{kernel_table<true, 1>(std::make_integer_sequence<int, kMaxSteps>{}),
      kernel_table<true, 2>(std::make_integer_sequence<int, kMaxSteps>{}),
      kernel_table<true, 4>(std::make_integer_sequence<int, kMaxSteps>{})}},
}};

using GemvNormFn = void (*)(const uint16_t*, const uint16_t*, const uint16_t*, double, const v4u*,
                            const uint16_t*, uint32_t, int, const uint16_t*, uint16_t*, int32_t*,
                            int8_t*, float*, uint16_t*, int, int, int, int);
template <int C, bool GLU, int... Ps>
constexpr std::array<GemvNormFn, sizeof...(Ps)> norm_table(std::integer_sequence<int, Ps...>) {
    return {{&gemv_norm_kernel<Ps + 1, C, GLU>...}};
}
// P = 1 .. kNormMaxSteps (rows up to kNormMaxK over at most kNormMaxWaves
// wavefronts per band) and C = 1 or 2 cached chunks per thread; the loop over
// uncached chunks serves longer rows.
constexpr int kNormMaxSteps = 16;
using NormRow = std::array<GemvNormFn, kNormMaxSteps>;
// [glu][C - 1][P - 1]
const std::array<std::array<NormRow, 2>, 2> kNormKernels = {{
    {{norm_table<1, false>(std::make_integer_sequence<int, kNormMaxSteps>{}),
      norm_table<2, false>(std::make_integer_sequence<int, kNormMaxSteps>{})}},
    {{norm_table<1, true>(std::make_integer_sequence<int, kNormMaxSteps>{}),
      norm_table<2, true>(std::make_integer_sequence<int, kNormMaxSteps>{})}},
}};

// The geometry of gemv_shape with at most kNormMaxWaves wavefronts per
// workgroup: fewer wavefronts per band (longer runs) or fewer bands.
GemvShape norm_shape(int N, int K) {
    const int S = (K + kTileK - 1) / kTileK;
    const int nbands = (N + kTileRows - 1) / kTileRows;
    const int target = nbands < kNarrowBands ? kTargetStepsNarrow : kTargetSteps;
    int Wb = 1;
    while (Wb < kNormMaxWaves && (S + Wb - 1) / Wb > target) Wb <<= 1;
    const int P = (S + Wb - 1) / Wb;
    if (P > kNormMaxSteps) return GemvShape{0, 0, 0};
    int B = 4;
    while (B > 1 && (nbands / B < kMinGroups || B * Wb > kNormMaxWaves)) B >>= 1;
    return GemvShape{B * Wb, P, B};
}

hipError_t launch(bool fused, const void* x, const uint8_t* packed, const float* s,
                  const uint16_t* ws, int ws_num, uint16_t* y, int32_t* acc, int8_t* q_out,
                  float* s_out, int N, int K, hipStream_t stream) {
    const GemvShape g = gemv_shape(N, K);
    if (g.waves == 0) return hipErrorInvalidValue;
    const int nbands = (N + kTileRows - 1) / kTileRows;
    const unsigned groups = static_cast<unsigned>((nbands + g.bands - 1) / g.bands);
    const int wb = g.waves / g.bands;
    int lw = 0;
    while ((1 << lw) < wb) ++lw;
    const size_t lds = static_cast<size_t>(wb) * g.steps * kTileK;
    // chunks of the activation row per thread, rounded up to 1, 2 or 4
    const int chunks = fused ? K / 8 : K / 16;
    const int threads = g.waves * 64;
    const int need = (chunks + threads - 1) / threads;
    const int lc = need <= 1 ? 0 : need <= 2 ? 1 : 2;
    GemvFn fn = kKernels[fused ? 1 : 0][lc][g.steps - 1];
    size_t lds_bytes = lds;
    // the wave-local bf16 kernel where it measured faster (see its comment)
    if (fused && g.bands == 1 && g.waves <= 4 && groups <= 256 && g.steps <= kLocalMaxSteps) {
        fn = kLocalKernels[g.steps - 1];
        lds_bytes = static_cast<size_t>(g.waves) * g.steps * 64 * 4;
    }
    uint32_t seg_mul;
    int seg_shift;
    seg_divisor(N / ws_num, seg_mul, seg_shift);
    fn<<<groups, g.waves * 64, lds_bytes, stream>>>(x, reinterpret_cast<const v4u*>(packed), s, ws,
                                             seg_mul, seg_shift, y, acc, q_out, s_out, N, K,
                                             g.bands, lw);
    return hipGetLastError();
}

}  // namespace

// n / d == (n * mul) >> shift for every 0 <= n < 2^24 (N <= 2^24): with
// l = ceil(log2 d), shift = 24 + l and mul = ceil(2^shift / d), the excess
// mul * d - 2^shift is at most d - 1 <= 2^l = 2^(shift - 24), the condition
// under which the product gives exact quotients of 24-bit numerators
// (Granlund and Montgomery, "Division by invariant integers using
// multiplication", 1994).  mul < 2^25, so n * mul < 2^49.
void seg_divisor(int d, uint32_t& mul, int& shift) {
    int l = 0;
    while ((1 << l) < d) ++l;
    shift = 24 + l;
    mul = static_cast<uint32_t>(((1ull << shift) + static_cast<uint64_t>(d) - 1) / d);
}

GemvShape gemv_shape(int N, int K) {
    const int S = (K + kTileK - 1) / kTileK;
    const int nbands = (N + kTileRows - 1) / kTileRows;
    // Wavefronts per band: the smallest power of two (the kernel splits by
    // shifts) that leaves at most the target number of steps per wavefront.
    const int target = nbands < kNarrowBands ? kTargetStepsNarrow : kTargetSteps;
    int Wb = 1;
    while (Wb < kMaxWaves && (S + Wb - 1) / Wb > target) Wb <<= 1;
    const int P = (S + Wb - 1) / Wb;
    if (P > kMaxSteps) return GemvShape{0, 0, 0};
    // Bands per workgroup: as many as keep >= kMinGroups workgroups in flight.
    int B = 4;
    while (B > 1 && (nbands / B < kMinGroups || B * Wb > kMaxWaves)) B >>= 1;
    return GemvShape{B * Wb, P, B};
}

hipError_t launch_gemv_i8(const int8_t* xq, const uint8_t* packed, const float* s,
                          const uint16_t* ws, int ws_num, uint16_t* y, int32_t* acc, int N, int K,
                          hipStream_t stream) {
    return launch(false, xq, packed, s, ws, ws_num, y, acc, nullptr, nullptr, N, K, stream);
}

hipError_t launch_gemv_norm(const uint16_t* x, const uint16_t* x_up, const uint16_t* gamma,
                            float eps, const uint8_t* packed, const uint16_t* ws, int ws_num,
                            const uint16_t* residual, uint16_t* y, uint16_t* xn_out,
                            int8_t* q_out, float* s_out, int32_t* acc, int N, int K,
                            hipStream_t stream) {
    const GemvShape g = norm_shape(N, K);
    if (g.waves == 0 || K > kNormMaxK) return hipErrorInvalidValue;
    const int nbands = (N + kTileRows - 1) / kTileRows;
    const unsigned groups = static_cast<unsigned>((nbands + g.bands - 1) / g.bands);
    const int wb = g.waves / g.bands;
    int lw = 0;
    while ((1 << lw) < wb) ++lw;
    const size_t lds = static_cast<size_t>(wb) * g.steps * kTileK;
    const int threads = g.waves * 64;
    const int need = (K / 8 + threads - 1) / threads;
    const GemvNormFn fn = kNormKernels[x_up ? 1 : 0][need <= 1 ? 0 : 1][g.steps - 1];
    uint32_t seg_mul;
    int seg_shift;
    seg_divisor(N / ws_num, seg_mul, seg_shift);
    fn<<<groups, threads, lds, stream>>>(x, x_up, gamma, static_cast<double>(eps),
                                         reinterpret_cast<const v4u*>(packed), ws, seg_mul,
                                         seg_shift, residual, y, acc, q_out, s_out, xn_out, N, K,
                                         g.bands, lw);
    return hipGetLastError();
}

hipError_t launch_gemv_bf16_fused(const uint16_t* x, const uint8_t* packed, const uint16_t* ws,
                                  int ws_num, uint16_t* y, int8_t* q_out, float* s_out,
                                  int32_t* acc, int N, int K, hipStream_t stream) {
    return launch(true, x, packed, nullptr, ws, ws_num, y, acc, q_out, s_out, N, K, stream);
}

}  // namespace bl
