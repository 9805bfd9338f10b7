// gemv_lut.hip -- the M = 1 ternary layer by table lookup: a second algorithm
// for the same exact int32 sums as the dot-product GEMV, kept as a
// cross-check.
//
// Source pages: "BitNet на микроконтроллерах: как устроен запуск 1.58-битной
// LLM на кластере ESP32-S3" (sarnas.ru), cited as [TL1]: its sections on the
// LUT compilation (lut_ctor: from the quantised activations of a block, a
// table of every sum of two activations' contributions under two ternary
// weights, so that a weight pair selects an entry instead of multiplying) and
// on the qgemm_lut kernel (4-bit indices split from the packed bytes, table
// lookups into 16-bit partial sums, widened to 32 bits).  "BitNet GPU
// 推理框架：从零构建 W2A8 的 2-bit 大模型 CUDA GEMV 内核" (blog.gitcode.com),
// cited as [W2A8]: the packed codes (§5.2) and the epilogue (§5.3).
//
// Mapping onto the packed 16 x 256 tiles (this library's design; the CPU
// page's NEON kernel is prior art):
//   * a nibble of a packed word holds the codes of two weights of one row: the
//     low nibble of byte b those of elements b and b + 4 of the word's 16-wide
//     K chunk, the high nibble those of elements b + 8 and b + 12; its value
//     c0 + 4 * c1 indexes that pair's table directly;
//   * the table of the activation pair (x0, x1) has 16 int16 entries,
//     entry c0 + 4 * c1 = (c0 - 2) * x0 + (c1 - 2) * x1 -- the +2 code offset
//     folded in, so no -2 * sum(x) term remains (code 0 occurs only at
//     padding, where x is zero or the row is discarded);
//   * the workgroup builds the tables of the whole row in LDS, eight pairs
//     per 16-K chunk, with packed 16-bit adds (8 per pair), chunk stride 272
//     bytes so that the 16 chunks a wavefront reads at once start on
//     different banks;
//   * Wb wavefronts per band of 16 rows split its S K steps, P each (all
//     loaded up front), B bands per workgroup sharing its tables; per K step
//     a lane looks up 8 entries for each of its 4 rows; then the row
//     reduction (across the Wb wavefronts through LDS) and the epilogue of
//     the dot-product kernel.  The lookups are VALU work in proportion to
//     the weights, so they are spread over many wavefronts (runs of at most
//     kLutTargetSteps), unlike the dot-product kernel's runs of up to 10.
// Bound: LDS lookups and VALU (8 lookups per packed word against 4 dot4 in
// the dot-product kernel); the weights stream from HBM as there.
#include <array>
#include <utility>

#include "gemv_core.hpp"
#include "kernels.hpp"

namespace bl {

namespace {

constexpr int kLutChunkStride = 272;   // 8 pair tables x 32 bytes + 16 bytes of bank offset
// 16-byte activation chunks a thread builds tables for: one.  Either every
// wavefront takes at most 4 steps, so S <= 4 Wb and the S * 16 chunks are no
// more than the band's 64 Wb threads; or the matrix is wide (at least
// 4 kMinGroups bands: 4 bands per workgroup, 256 threads) with at most
// kLutWideSteps steps (160 chunks).  The launcher checks it.
constexpr int kLutMaxX = 1;

typedef short s16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack16(int lo, int hi) {
    return (static_cast<uint32_t>(lo) & 0xFFFFu) | (static_cast<uint32_t>(hi) << 16);
}

__device__ __forceinline__ uint32_t add16x2(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t,
                              __builtin_bit_cast(s16x2, a) + __builtin_bit_cast(s16x2, b));
}

// The 16 entries of the table of activations (x0, x1) as 8 words, entry
// 2d in the low half of word d: entry c0 + 4 c1 = u(c0, x0) + u(c1, x1) with
// u(c, x) = (c - 2) x, so word d = (u(0 or 2), u(1 or 3) of x0) + u(d / 2, x1)
// twice.  Every entry fits int16 (|entry| <= 512), so the 16-bit adds are
// exact.
__device__ __forceinline__ void pair_table(int x0, int x1, uint32_t (&t)[8]) {
    const uint32_t even = pack16(-2 * x0, -x0);   // c0 = 0, 1
    const uint32_t odd = pack16(0, x0);            // c0 = 2, 3
    const uint32_t v0 = pack16(-2 * x1, -2 * x1);  // c1 = 0
    const uint32_t v1 = pack16(-x1, -x1);          // c1 = 1
    const uint32_t v3 = pack16(x1, x1);            // c1 = 3 (c1 = 2 adds nothing)
    t[0] = add16x2(even, v0);
    t[1] = add16x2(odd, v0);
    t[2] = add16x2(even, v1);
    t[3] = add16x2(odd, v1);
    t[4] = even;
    t[5] = odd;
    t[6] = add16x2(even, v3);
    t[7] = add16x2(odd, v3);
}

__device__ __forceinline__ int sbyte(uint32_t w, int b) {
    return __builtin_amdgcn_sbfe(static_cast<int>(w), 8 * b, 8);
}

// Lookups of one packed word (16 weights of one row) against the tables of
// its K chunk (at byte offset base).  Twice each nibble is formed for all
// four bytes at once (one shift and one mask per half), then selected byte by
// byte into the address.
__device__ __forceinline__ int lookup_word(const uint8_t* lut, int base, uint32_t w, int acc) {
    uint32_t lo2 = (w << 1) & 0x1E1E1E1Eu;   // 2 * low nibble of each byte: pairs 0..3
    uint32_t hi2 = (w >> 3) & 0x1E1E1E1Eu;   // 2 * high nibble: pairs 4..7
    // opaque to the compiler, which would otherwise fold the masks back into
    // a shift and a mask per nibble
    asm("" : "+v"(lo2), "+v"(hi2));
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const int ol = static_cast<int>((lo2 >> (8 * b)) & 0xFFu);
        const int oh = static_cast<int>((hi2 >> (8 * b)) & 0xFFu);
        acc += *reinterpret_cast<const int16_t*>(lut + base + b * 32 + ol);
        acc += *reinterpret_cast<const int16_t*>(lut + base + (b + 4) * 32 + oh);
    }
    return acc;
}

// B bands per workgroup, 2^lw wavefronts per band, P K steps per wavefront
// (steps past the row's S are skipped).
constexpr int kLutMaxWaves = 8;
template <int P>
__global__ __launch_bounds__(kLutMaxWaves * 64) void gemv_lut_kernel(
    const int8_t* __restrict__ xq, const v4u* __restrict__ packed, const float* __restrict__ s_in,
    const uint16_t* __restrict__ ws, uint32_t seg_mul, int seg_shift, uint16_t* __restrict__ y,
    int32_t* __restrict__ acc, int N, int K, int B, int lw) {
    extern __shared__ uint4 lut_sh[];
    __shared__ int part_sh[kLutMaxWaves][64];
    uint8_t* lut = reinterpret_cast<uint8_t*>(lut_sh);
    const int Wb = 1 << lw;
    const int nthreads = (B << lw) * 64;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nbands = (N + kTileRows - 1) / kTileRows;
    const int band_lin = static_cast<int>(blockIdx.x) * B + (wave >> lw);
    const int band = min(band_lin, nbands - 1);
    const int S = (K + kTileK - 1) / kTileK;
    const int s0 = (wave & (Wb - 1)) * P;
    const int chunks = S * 16;   // 16-K chunks of the padded row

    // 1. This lane's output row and weight scale, the activation chunks this
    //    thread builds tables for (buffer loads: zeros past the row's end),
    //    then every weight tile of this wavefront's steps.
    const int n_out = band_lin * kTileRows + 4 * (lane >> 4) + (lane & 3);
    const uint32_t n_ws = static_cast<uint32_t>(min(n_out, N - 1));
    const uint16_t wsb = ws[(static_cast<uint64_t>(n_ws) * seg_mul) >> seg_shift];
    const float s = s_in[0];
    const __amdgpu_buffer_rsrc_t rx =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(xq), 0, K, 0x00020000);
    const int nx = (chunks + nthreads - 1) / nthreads;
    v4u xv[kLutMaxX];
#pragma unroll
    for (int j = 0; j < kLutMaxX; ++j)
        if (j < nx) xv[j] = __builtin_amdgcn_raw_buffer_load_b128(rx, (tid + j * nthreads) * 16, 0, 0);
    const v4u* tiles = packed + static_cast<size_t>(band) * S * 64 + lane;
    v4u w[P];
    load_steps<P>(tiles, s0, S - 1, w);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);

    // 2. The tables: chunk c, pair p of elements e = (p % 4) + 8 (p / 4) and e + 4.
#pragma unroll
    for (int j = 0; j < kLutMaxX; ++j) {
        const int c = tid + j * nthreads;
        if (j < nx && c < chunks) {
            uint4* dst = reinterpret_cast<uint4*>(lut + c * kLutChunkStride);
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                const uint32_t lo = p < 4 ? xv[j].x : xv[j].z;
                const uint32_t hi = p < 4 ? xv[j].y : xv[j].w;
                uint32_t t[8];
                pair_table(sbyte(lo, p & 3), sbyte(hi, p & 3), t);
                dst[2 * p] = make_uint4(t[0], t[1], t[2], t[3]);
                dst[2 * p + 1] = make_uint4(t[4], t[5], t[6], t[7]);
            }
        }
    }
    // ws / s for this lane's row, formed while the weights are in flight
    const double cs = static_cast<double>(bf16_to_float(wsb)) * (1.0 / static_cast<double>(s));
    __syncthreads();

    // 3. Lookups: step s0 + u, K chunk (s0 + u) * 16 + lane % 16, the four
    //    rows of the slot; a step past the row's end is skipped (uniform).
    int v[4] = {0, 0, 0, 0};
    const int kc = lane & 15;
#pragma unroll
    for (int u = 0; u < P; ++u) {
        if (s0 + u < S) {
            const int base = ((s0 + u) * 16 + kc) * kLutChunkStride;
            v[0] = lookup_word(lut, base, w[u].x, v[0]);
            v[1] = lookup_word(lut, base, w[u].y, v[1]);
            v[2] = lookup_word(lut, base, w[u].z, v[2]);
            v[3] = lookup_word(lut, base, w[u].w, v[3]);
        }
    }
    // 4. Row reduction (lane l with (l / 4) % 4 == 0 holds row 4 (l / 16) + l % 4),
    //    then the band's first wavefront adds its Wb partial sums and writes.
    int total = row_group_reduce(v, lane);
    if (Wb > 1) {
        part_sh[wave][lane] = total;
        __syncthreads();
        if ((wave & (Wb - 1)) != 0) return;
        for (int j = 1; j < Wb; ++j) total += part_sh[wave + j][lane];
    }
    if (((lane >> 2) & 3) == 0 && band_lin < nbands && n_out < N) {
        y[n_out] = epilogue_bf16_scaled(total, cs, bf16_to_float(wsb), s);
        if (acc) acc[n_out] = total;
    }
}

using LutFn = void (*)(const int8_t*, const v4u*, const float*, const uint16_t*, uint32_t, int,
                       uint16_t*, int32_t*, int, int, int, int);

template <int... Ps>
constexpr std::array<LutFn, sizeof...(Ps)> lut_table(std::integer_sequence<int, Ps...>) {
    return {{&gemv_lut_kernel<Ps + 1>...}};
}

// K steps per wavefront aimed at: the smallest power of two of wavefronts
// per band that leaves at most this many, then as many bands per workgroup
// (at most kLutMaxWaves wavefronts in all) as keep kMinGroups workgroups.
// K <= kLutMaxK is at most 32 steps: P <= 4 with 8 wavefronts.  Against one
// wavefront per band (same box): 3840 x 2560 5.80 -> 3.50 us, 2560 x 6912
// 11.88 -> 6.00, 6912 x 2560 5.52 -> 4.70, 20480 x 3200 12.11 -> 10.30, but
// 13824 x 2560 6.30 -> 6.58 (16 wavefronts per workgroup there: 7.08).
constexpr int kLutTargetSteps = 4;
// Wide matrices (at least 4 kMinGroups bands, already about one wavefront
// per SIMD) with rows of at most kLutWideSteps steps keep one wavefront per
// band: 13824 x 2560 6.59 -> 6.00 us, 12816 x 2320 6.47 -> 5.96; at
// 20480 x 3200 (13 steps) the split wins.
constexpr int kLutWideSteps = 10;
constexpr int kLutMaxSteps = kLutWideSteps;
const std::array<LutFn, kLutMaxSteps> kLutKernels =
    lut_table(std::make_integer_sequence<int, kLutMaxSteps>{});

}  // namespace

hipError_t launch_gemv_lut(const int8_t* xq, const uint8_t* packed, const float* s,
                           const uint16_t* ws, int ws_num, uint16_t* y, int32_t* acc, int N, int K,
                           hipStream_t stream) {
    const int S = (K + kTileK - 1) / kTileK;
    if (K > kLutMaxK || S < 1) return hipErrorInvalidValue;
    const int nbands = (N + kTileRows - 1) / kTileRows;
    int Wb = 1;
    if (nbands < 4 * kMinGroups || S > kLutWideSteps)
        while (Wb < kLutMaxWaves && (S + Wb - 1) / Wb > kLutTargetSteps) Wb <<= 1;
    const int P = (S + Wb - 1) / Wb;
    if (P > kLutMaxSteps) return hipErrorInvalidValue;
    int lw = 0;
    while ((1 << lw) < Wb) ++lw;
    int B = 4;
    while (B > 1 && (nbands / B < kMinGroups || B * Wb > kLutMaxWaves)) B >>= 1;
    if (S * 16 > B * Wb * 64 * kLutMaxX) return hipErrorInvalidValue;
    const unsigned groups = static_cast<unsigned>((nbands + B - 1) / B);
    const size_t lds = static_cast<size_t>(S) * 16 * kLutChunkStride;
    // Tables beyond 64 KiB (K > 3840) need the kernel's dynamic-LDS limit
    // raised (to the largest table), once per kernel and device.
    if (lds > 65536) {
        const hipError_t attr =
            raise_lds_limit(reinterpret_cast<const void*>(kLutKernels[P - 1]),
                            static_cast<int>(kLutMaxK / kTileK * 16 * kLutChunkStride));
        if (attr != hipSuccess) return attr;
    }
    uint32_t seg_mul;
    int seg_shift;
    seg_divisor(N / ws_num, seg_mul, seg_shift);
    kLutKernels[P - 1]<<<groups, B * Wb * 64, lds, stream>>>(
        xq, reinterpret_cast<const v4u*>(packed), s, ws, seg_mul, seg_shift, y, acc, N, K, B, lw);
    return hipGetLastError();
}

}  // namespace bl
