// gemv.hip -- the M = 1 decode GEMV of the W2A8 ternary linear layer on gfx950.
//
// Source page: "BitNet GPU 推理框架：从零构建 W2A8 的 2-bit 大模型 CUDA GEMV 内核"
// (blog.gitcode.com), cited as [W2A8]: §5.2 (codes w + 2, interleaved 32-bit
// words decoded by shift and mask), §5.3 (int8 dot products into an int32
// accumulator, then out = acc * scales with ws[n / (N / ws_num)]), §六 item 3
// (per-token activation quantisation, fused here for bf16 input).
//
// Mapping (this library's design; the page's sm_80 kernel is prior art):
//   * one workgroup per band of 64 output rows, 8 wavefronts;
//   * lane r of every wavefront owns row 64*band + r; the K steps of the band
//     (64 K = one 1 KiB tile each) are split between the 8 wavefronts, so a
//     wavefront's load of a tile is one coalesced 16-byte-per-lane load of
//     1 KiB and there is no cross-lane reduction at all;
//   * every lane of a wavefront needs the same 64 activation bytes per step:
//     for int8 input they are read with scalar loads into SGPRs (no LDS, no
//     VGPRs); for bf16 input the workgroup quantises the row into LDS first
//     and the lanes read it back as a broadcast;
//   * decoding keeps the unsigned codes c = w + 2 and never shifts them into
//     place: field i of a word is masked in place (factor 4^i, i < 3) and
//     dotted with activation word i, into one of three accumulators; field 3
//     is shifted down once.  acc = a1 + a4/4 + a16/16 - 2 * sum(x), the last
//     term removing the +2 offset (padding code 0 contributes nothing);
//   * the 8 partial sums of a row are added through LDS; the epilogue runs in
//     fp64 and rounds once to bf16.
#include "common.hpp"
#include "kernels.hpp"

namespace bl {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kBatch = 8;   // tiles in flight per wavefront per batch

// Dot of one packed word (16 K) with its four activation words.
__device__ __forceinline__ void dot_word(uint32_t w, int x0, int x1, int x2, int x3, int& a1,
                                         int& a4, int& a16) {
    a1 = dot4(static_cast<int>(w & 0x03030303u), x0, a1);
    a4 = dot4(static_cast<int>(w & 0x0C0C0C0Cu), x1, a4);
    a16 = dot4(static_cast<int>(w & 0x30303030u), x2, a16);
    a1 = dot4(static_cast<int>((w >> 6) & 0x03030303u), x3, a1);
}

__device__ __forceinline__ void dot_tile(const v4u& wv, const int (&xa)[16], int& a1, int& a4,
                                         int& a16) {
    dot_word(wv.x, xa[0], xa[1], xa[2], xa[3], a1, a4, a16);
    dot_word(wv.y, xa[4], xa[5], xa[6], xa[7], a1, a4, a16);
    dot_word(wv.z, xa[8], xa[9], xa[10], xa[11], a1, a4, a16);
    dot_word(wv.w, xa[12], xa[13], xa[14], xa[15], a1, a4, a16);
}

// Activations of one K step from global memory (int8 input): uniform
// addresses, so the compiler issues scalar loads.  Kw = K / 4 words; words
// past K read as zero (K % 16 == 0, so a step is 0, 4, 8, 12 or 16 words).
struct GlobalAct {
    const int* __restrict__ xw;
    int Kw;
    __device__ __forceinline__ void fetch(int st, int (&xa)[16]) const {
        const int base = st * 16;
        if (base + 16 <= Kw) {
#pragma unroll
            for (int j = 0; j < 16; ++j) xa[j] = xw[base + j];
        } else {
#pragma unroll
            for (int j = 0; j < 16; ++j) xa[j] = (base + j < Kw) ? xw[base + j] : 0;
        }
    }
};

// Activations of one K step from LDS (bf16 input quantised by the
// workgroup); the LDS copy is zero-padded to a whole number of steps.
struct LdsAct {
    const int4* qa;
    __device__ __forceinline__ void fetch(int st, int (&xa)[16]) const {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int4 v = qa[st * 4 + j];
            xa[4 * j] = v.x;
            xa[4 * j + 1] = v.y;
            xa[4 * j + 2] = v.z;
            xa[4 * j + 3] = v.w;
        }
    }
};

// The band's partial sum for this lane's row over steps [s0, s1): batches of
// kBatch 16-byte non-temporal loads issued back to back, then consumed.
template <class Act>
__device__ __forceinline__ int band_partial(const v4u* __restrict__ tiles, int s0, int s1,
                                            const Act& act) {
    int a1 = 0, a4 = 0, a16 = 0;
    for (int st = s0; st < s1; st += kBatch) {
        v4u wv[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
            if (st + u < s1) wv[u] = __builtin_nontemporal_load(tiles + static_cast<size_t>(st + u) * 64);
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            if (st + u < s1) {
                int xa[16];
                act.fetch(st + u, xa);
                dot_tile(wv[u], xa, a1, a4, a16);
            }
        }
    }
    // a4 and a16 are exact multiples of 4 and 16: the shifts divide exactly.
    return a1 + (a4 >> 2) + (a16 >> 4);
}

__device__ __forceinline__ void write_row(int32_t total, int n, int N, const uint16_t* ws,
                                          int ws_num, float s, uint16_t* y, int32_t* acc) {
    if (n >= N) return;
    const float wsv = bf16_to_float(ws[n / (N / ws_num)]);
    y[n] = epilogue_bf16(total, wsv, s);
    if (acc) acc[n] = total;
}

__global__ __launch_bounds__(kThreads) void gemv_i8_kernel(
    const int8_t* __restrict__ xq, const v4u* __restrict__ packed, const float* __restrict__ s,
    const uint16_t* __restrict__ ws, int ws_num, uint16_t* __restrict__ y,
    int32_t* __restrict__ acc, int N, int K) {
    __shared__ int part_sh[kWaves][64];
    __shared__ int xsum_sh[kWaves];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int band = blockIdx.x;
    const int S = (K + kTileK - 1) / kTileK;
    const int s0 = (S * wave) / kWaves;
    const int s1 = (S * (wave + 1)) / kWaves;
    const int* xw = reinterpret_cast<const int*>(xq);
    const int Kw = K >> 2;

    const v4u* tiles = packed + static_cast<size_t>(band) * S * 64 + lane;
    const int part = band_partial(tiles, s0, s1, GlobalAct{xw, Kw});

    // sum(x) for the +2 code offset, spread over the workgroup.
    int xs = 0;
    for (int j = threadIdx.x; j < Kw; j += kThreads) xs = dot4(xw[j], 0x01010101, xs);
    xs = wave_sum(xs);

    part_sh[wave][lane] = part;
    if (lane == 0) xsum_sh[wave] = xs;
    __syncthreads();
    if (wave == 0) {
        int total = 0, xsum = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            total += part_sh[w][lane];
            xsum += xsum_sh[w];
        }
        total -= 2 * xsum;
        write_row(total, band * 64 + lane, N, ws, ws_num, s[0], y, acc);
    }
}

// Fused: bf16 row -> per-token int8 quantisation into LDS -> GEMV.  Each
// workgroup quantises the whole row (it is small and L2-resident); the max
// is order-independent and the arithmetic is the quantiser's, so every
// workgroup gets identical int8 activations and scale.  Workgroup 0 also
// writes them out when asked.
constexpr int kCached = 4;   // 8-element chunks per thread kept in registers

__global__ __launch_bounds__(kThreads) void gemv_bf16_fused_kernel(
    const uint16_t* __restrict__ x, const v4u* __restrict__ packed,
    const uint16_t* __restrict__ ws, int ws_num, uint16_t* __restrict__ y,
    int8_t* __restrict__ q_out, float* __restrict__ s_out, int32_t* __restrict__ acc, int N,
    int K) {
    extern __shared__ int4 q_lds[];   // S * 64 bytes: the quantised row, zero-padded
    __shared__ int part_sh[kWaves][64];
    __shared__ int xsum_sh[kWaves];
    __shared__ float amax_sh[kWaves];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int band = blockIdx.x;
    const int S = (K + kTileK - 1) / kTileK;
    const int s0 = (S * wave) / kWaves;
    const int s1 = (S * (wave + 1)) / kWaves;
    const int chunks = K >> 3;
    const uint4* x8 = reinterpret_cast<const uint4*>(x);

    // Pass 1: max|x| over the row.
    uint4 xv[kCached];
    float amax = 0.0f;
#pragma unroll
    for (int c = 0; c < kCached; ++c) {
        const int idx = threadIdx.x + c * kThreads;
        xv[c] = make_uint4(0, 0, 0, 0);
        if (idx < chunks) xv[c] = x8[idx];
    }
    for (int idx = threadIdx.x + kCached * kThreads; idx < chunks; idx += kThreads) {
        const uint4 v = x8[idx];
        const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j)
            amax = fmaxf(amax, fmaxf(fabsf(__uint_as_float(d[j] << 16)),
                                     fabsf(__uint_as_float(d[j] & 0xFFFF0000u))));
    }
#pragma unroll
    for (int c = 0; c < kCached; ++c) {
        const uint32_t d[4] = {xv[c].x, xv[c].y, xv[c].z, xv[c].w};
#pragma unroll
        for (int j = 0; j < 4; ++j)
            amax = fmaxf(amax, fmaxf(fabsf(__uint_as_float(d[j] << 16)),
                                     fabsf(__uint_as_float(d[j] & 0xFFFF0000u))));
    }
    amax = wave_max(amax);
    if (lane == 0) amax_sh[wave] = amax;
    __syncthreads();
    amax = amax_sh[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) amax = fmaxf(amax, amax_sh[w]);
    const float sm = 127.0f / fmaxf(amax, 1e-5f);

    // Pass 2: quantise into LDS, sum the int8 values.
    uint2* q_lds2 = reinterpret_cast<uint2*>(q_lds);
    const bool write_q = (band == 0) && (q_out != nullptr);
    int xs = 0;
    auto quant_chunk = [&](int idx, const uint4& v) {
        const uint32_t d[4] = {v.x, v.y, v.z, v.w};
        uint2 o;
        o.x = pack4_i8(quant_one(__uint_as_float(d[0] << 16), sm),
                       quant_one(__uint_as_float(d[0] & 0xFFFF0000u), sm),
                       quant_one(__uint_as_float(d[1] << 16), sm),
                       quant_one(__uint_as_float(d[1] & 0xFFFF0000u), sm));
        o.y = pack4_i8(quant_one(__uint_as_float(d[2] << 16), sm),
                       quant_one(__uint_as_float(d[2] & 0xFFFF0000u), sm),
                       quant_one(__uint_as_float(d[3] << 16), sm),
                       quant_one(__uint_as_float(d[3] & 0xFFFF0000u), sm));
        q_lds2[idx] = o;
        xs = dot4(static_cast<int>(o.x), 0x01010101, xs);
        xs = dot4(static_cast<int>(o.y), 0x01010101, xs);
        if (write_q) reinterpret_cast<uint2*>(q_out)[idx] = o;
    };
#pragma unroll
    for (int c = 0; c < kCached; ++c) {
        const int idx = threadIdx.x + c * kThreads;
        if (idx < chunks) quant_chunk(idx, xv[c]);
    }
    for (int idx = threadIdx.x + kCached * kThreads; idx < chunks; idx += kThreads)
        quant_chunk(idx, x8[idx]);
    // zero the padding up to a whole number of steps (K % 16 == 0: whole int4s)
    for (int i = (K >> 4) + threadIdx.x; i < S * 4; i += kThreads) q_lds[i] = make_int4(0, 0, 0, 0);
    if (band == 0 && s_out != nullptr && threadIdx.x == 0) s_out[0] = sm;
    xs = wave_sum(xs);
    if (lane == 0) xsum_sh[wave] = xs;
    __syncthreads();

    const v4u* tiles = packed + static_cast<size_t>(band) * S * 64 + lane;
    const int part = band_partial(tiles, s0, s1, LdsAct{q_lds});
    part_sh[wave][lane] = part;
    __syncthreads();
    if (wave == 0) {
        int total = 0, xsum = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            total += part_sh[w][lane];
            xsum += xsum_sh[w];
        }
        total -= 2 * xsum;
        write_row(total, band * 64 + lane, N, ws, ws_num, sm, y, acc);
    }
}

}  // namespace

hipError_t launch_gemv_i8(const int8_t* xq, const uint8_t* packed, const float* s,
                          const uint16_t* ws, int ws_num, uint16_t* y, int32_t* acc, int N, int K,
                          hipStream_t stream) {
    const unsigned bands = static_cast<unsigned>((N + kTileRows - 1) / kTileRows);
    gemv_i8_kernel<<<bands, kThreads, 0, stream>>>(
        xq, reinterpret_cast<const v4u*>(packed), s, ws, ws_num, y, acc, N, K);
    return hipGetLastError();
}

hipError_t launch_gemv_bf16_fused(const uint16_t* x, const uint8_t* packed, const uint16_t* ws,
                                  int ws_num, uint16_t* y, int8_t* q_out, float* s_out,
                                  int32_t* acc, int N, int K, hipStream_t stream) {
    const unsigned bands = static_cast<unsigned>((N + kTileRows - 1) / kTileRows);
    const int S = (K + kTileK - 1) / kTileK;
    const size_t lds = static_cast<size_t>(S) * kTileK;
    gemv_bf16_fused_kernel<<<bands, kThreads, lds, stream>>>(
        x, reinterpret_cast<const v4u*>(packed), ws, ws_num, y, q_out, s_out, acc, N, K);
    return hipGetLastError();
}

}  // namespace bl
