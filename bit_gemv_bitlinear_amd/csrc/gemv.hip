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
//   * decoding keeps the unsigned codes c = w + 2 and removes the +2 offset
//     once, as -2 * sum(x) (padding code 0 contributes nothing).  int8 rows
//     are staged split into nibbles (nibble_split), and a word masked two
//     ways (0x33333333, and after a shift by 2) feeds one unsigned v_dot8 for
//     the low nibbles and one signed v_dot8 for the high ones per mask: 7
//     VALU per word.  Rows quantised in the kernel (bf16 input) are staged
//     whole: field i of a word is masked in place (factor 4^i, i < 3) and
//     dotted with activation word i by v_dot4 into one of three accumulators,
//     field 3 shifted down once (9 VALU per word);
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

#include "gemv_core.hpp"
#include "kernels.hpp"

namespace bl {

namespace {

// C = 16-element activation chunks per thread (16 bytes of int8, 32 of bf16)
// loaded ahead of the weights and kept in registers (1, 2 or 4, a template
// argument chosen per shape).  Chunks beyond them are loaded after the
// weights, and since the waits count loads in issue order, using them waits
// for every weight; so C covers the row wherever it can (2560 / 16 = 160
// chunks over 128 threads for qkv and o, 6912 / 16 = 432 over 256 threads
// for down).  Chunks a thread does not need cost code on the path to the
// main loop, so C is no larger than the row needs.
//
// Row n's weight scale is ws[n / seg], seg = N / ws_num, found as
// (n * seg_mul) >> seg_shift (see seg_divisor()).  B bands per workgroup, 2^lw
// wavefronts per band (blockDim.x = 64 * B * 2^lw), P K-steps per wavefront.
// FUSED = false: xin is int8 activations with scale s_in[0].
// FUSED = true:  xin is bf16; the workgroup quantises it (per-token absmax,
//                [W2A8] §六 item 3); workgroup 0 writes q_out / s_out if given.
template <int P, bool FUSED, int C, bool OWN>
__global__ __launch_bounds__(kMaxWaves * 64) void gemv_kernel(
    int N, int K, int B, int lw, uint32_t seg_mul, int seg_shift, const v4u* __restrict__ packed,
    const void* __restrict__ xin, const uint16_t* __restrict__ ws, const float* __restrict__ s_in,
    uint16_t* __restrict__ y, int32_t* __restrict__ acc, int8_t* __restrict__ q_out,
    float* __restrict__ s_out) {
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
    // OWN (one wavefront per band, Wb = 1): each wavefront finishes its own
    // band, without the last barrier: lane l with (l / 4) % 4 == 0 writes row
    // 4 * (l / 16) + l % 4, where the row reduction leaves that row's sum.
    // Otherwise wavefront 0 writes row tid of the workgroup's bands after a
    // barrier.  Measured same-box at 13824 x 2560 with int8 input: 3.60 ->
    // 3.41 us.  With bf16 input every wavefront forms ws / s after the
    // quantisation, on its path to the main loop, and the gain shrinks to
    // 3.65 -> 3.62 us: not worth 45 more kernels, so only the int8 kernels
    // are compiled with OWN.
    constexpr bool own = OWN;
    const int band_lin = static_cast<int>(blockIdx.x) * B + (wave >> lw);
    const int n_out = own ? band_lin * kTileRows + 4 * (lane >> 4) + (lane & 3)
                          : static_cast<int>(blockIdx.x) * B * kTileRows + tid;
    const uint32_t n_ws = static_cast<uint32_t>(min(n_out, N - 1));
    // unconditional: no branch, no early wait
    const uint16_t wsb = ws[(static_cast<uint64_t>(n_ws) * seg_mul) >> seg_shift];
    // C 16-element chunks of the row per thread: 16 bytes of int8, or 32
    // bytes (two adjacent 16-byte loads) of bf16, so that a thread quantises
    // whole chunks and can stage them split into nibbles.
    constexpr int kCached = C;
    constexpr int kLoads = FUSED ? 2 * C : C;
    uint4 xv[kLoads];
    const uint4* x16 = reinterpret_cast<const uint4*>(xin);
#pragma unroll
    for (int c = 0; c < kCached; ++c) {
        const int q = tid + c * nthreads;
        if constexpr (FUSED) {
            xv[2 * c] = xv[2 * c + 1] = make_uint4(0, 0, 0, 0);
            if (q < n16) {
                xv[2 * c] = x16[2 * q];
                xv[2 * c + 1] = x16[2 * q + 1];
            }
        } else {
            xv[c] = make_uint4(0, 0, 0, 0);
            if (q < n16) xv[c] = x16[q];
        }
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
            if (idx < n16) {
                act[idx] = nibble_split(make_int4(xv[c].x, xv[c].y, xv[c].z, xv[c].w));
                xs = sum_i8x4(xv[c].x, sum_i8x4(xv[c].y, sum_i8x4(xv[c].z, sum_i8x4(xv[c].w, xs))));
            }
        }
        for (int idx = tid + kCached * nthreads; idx < n16; idx += nthreads) {
            const uint4 v = x16[idx];
            act[idx] = nibble_split(make_int4(v.x, v.y, v.z, v.w));
            xs = sum_i8x4(v.x, sum_i8x4(v.y, sum_i8x4(v.z, sum_i8x4(v.w, xs))));
        }
    } else {
        float amax = 0.0f;
#pragma unroll
        for (int c = 0; c < kCached; ++c)
            if (tid + c * nthreads < n16)
                amax = absmax8_bf16(xv[2 * c], absmax8_bf16(xv[2 * c + 1], amax));
        for (int q = tid + kCached * nthreads; q < n16; q += nthreads)
            amax = absmax8_bf16(x16[2 * q], absmax8_bf16(x16[2 * q + 1], amax));
        amax = wave_max(amax);
        if (lane == 0) amax_sh[wave] = amax;
        __syncthreads();
        amax = amax_sh[0];
        for (int i = 1; i < W; ++i) amax = fmaxf(amax, amax_sh[i]);
        sm = 127.0f / fmaxf(amax, 1e-5f);
        const bool write_q = (blockIdx.x == 0) && (q_out != nullptr);
        // quantise a whole chunk (two 8-element halves), stage it split
        auto put = [&](int q, const uint4& lo, const uint4& hi) {
            const uint2 o0 = quant8_bf16(lo, sm), o1 = quant8_bf16(hi, sm);
            const int4 ch = make_int4(o0.x, o0.y, o1.x, o1.y);
            act[q] = nibble_split(ch);
            xs = sum_i8x4(o0.x, sum_i8x4(o0.y, sum_i8x4(o1.x, sum_i8x4(o1.y, xs))));
            if (write_q) reinterpret_cast<int4*>(q_out)[q] = ch;
        };
#pragma unroll
        for (int c = 0; c < kCached; ++c) {
            const int q = tid + c * nthreads;
            if (q < n16) put(q, xv[2 * c], xv[2 * c + 1]);
        }
        for (int q = tid + kCached * nthreads; q < n16; q += nthreads) put(q, x16[2 * q], x16[2 * q + 1]);
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
    if (own || wave == 0) {
        cs = static_cast<double>(bf16_to_float(wsb)) * (1.0 / static_cast<double>(sm));
        for (int i = 0; i < W; ++i) offset -= 2 * xsum_sh[i];
        asm volatile("" : "+v"(cs), "+v"(offset));
    }

    // 3. P steps of 4 rows x 16 K per lane on the chunks staged split into
    //    nibbles (v_dot8, 7 VALU per packed word).
    const int kc = lane & 15;
    NibAcc r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r.lo[i] = 0, r.hi[i] = 0;
#pragma unroll
    for (int u = 0; u < P; ++u) dot_slot_nib(w[u], act[(s0 + u) * 16 + kc], r);
    int v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = static_cast<int>(r.lo[i]) + 16 * r.hi[i];   // exact
    // lane l now holds row 4*(l/16) + l%4 of its band (replicated over l/4 % 4)
    const int rsum = row_group_reduce(v, lane);
    if (own) {
        if (((lane >> 2) & 3) == 0 && n_out < N) {
            const int total = rsum + offset;
            y[n_out] = epilogue_bf16_scaled(total, cs, bf16_to_float(wsb), sm);
            if (acc) acc[n_out] = total;
        }
        return;
    }
    part_sh[wave][lane] = rsum;
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

// K <= kGemvMaxK = 61440 is at most 240 steps, which 16 wavefronts per band
// take in runs of at most 15.
constexpr int kMaxSteps = 15;

using GemvFn = void (*)(int, int, int, int, uint32_t, int, const v4u*, const void*,
                        const uint16_t*, const float*, uint16_t*, int32_t*, int8_t*, float*);

template <bool FUSED, int C, bool OWN, int... Ps>
constexpr std::array<GemvFn, sizeof...(Ps)> kernel_table(std::integer_sequence<int, Ps...>) {
    return {{&gemv_kernel<Ps + 1, FUSED, C, OWN>...}};
}

using KernelRow = std::array<GemvFn, kMaxSteps>;
// [fused][log2 C][P - 1]
const std::array<std::array<KernelRow, 3>, 2> kKernels = {{
    {{kernel_table<false, 1, false>(std::make_integer_sequence<int, kMaxSteps>{}),
      kernel_table<false, 2, false>(std::make_integer_sequence<int, kMaxSteps>{}),
      kernel_table<false, 4, false>(std::make_integer_sequence<int, kMaxSteps>{})}},
    // bf16 rows: at most 2 chunks (4 loads) per thread, the registers of
    // 4 int8 chunks; longer rows load the rest in the staging loop
    {{kernel_table<true, 1, false>(std::make_integer_sequence<int, kMaxSteps>{}),
      kernel_table<true, 2, false>(std::make_integer_sequence<int, kMaxSteps>{}),
      kernel_table<true, 2, false>(std::make_integer_sequence<int, kMaxSteps>{})}},
}};
// int8 input with one wavefront per band: [log2 C][P - 1]
const std::array<KernelRow, 3> kKernelsOwn = {{
    kernel_table<false, 1, true>(std::make_integer_sequence<int, kMaxSteps>{}),
    kernel_table<false, 2, true>(std::make_integer_sequence<int, kMaxSteps>{}),
    kernel_table<false, 4, true>(std::make_integer_sequence<int, kMaxSteps>{}),
}};

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
    const int chunks = K / 16;          // 16-element chunks (32 bytes of bf16)
    const int threads = g.waves * 64;
    const int need = (chunks + threads - 1) / threads;
    const int lc = need <= 1 ? 0 : need <= 2 ? 1 : 2;
    uint32_t seg_mul;
    int seg_shift;
    seg_divisor(N / ws_num, seg_mul, seg_shift);
    // the wave-local bf16 kernel where it measured faster (gemv_local.hip)
    if (fused && g.bands == 1 && g.waves <= 4 && groups <= 256 && g.steps <= kLocalMaxSteps)
        return launch_gemv_local(static_cast<const uint16_t*>(x), packed, ws, seg_mul, seg_shift,
                                 y, acc, q_out, s_out, N, K, groups, g.waves, g.steps, lw, stream);
    const GemvFn fn = (!fused && wb == 1) ? kKernelsOwn[lc][g.steps - 1]
                                          : kKernels[fused ? 1 : 0][lc][g.steps - 1];
    fn<<<groups, g.waves * 64, lds, stream>>>(N, K, g.bands, lw, seg_mul, seg_shift,
                                              reinterpret_cast<const v4u*>(packed), x, ws, s, y,
                                              acc, q_out, s_out);
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
    // shifts) that leaves at most the target number of steps per wavefront,
    // then no more than kBandWaves while the runs fit the kernels.
    const int target = nbands < kNarrowBands ? kTargetStepsNarrow
                       : nbands < kWideBands ? kTargetStepsMedium
                                             : kTargetSteps;
    int Wb = 1;
    while (Wb < kMaxWaves && (S + Wb - 1) / Wb > target) Wb <<= 1;
    while (Wb > kBandWaves && (S + Wb / 2 - 1) / (Wb / 2) <= kMaxSteps) Wb >>= 1;
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

hipError_t launch_gemv_bf16_fused(const uint16_t* x, const uint8_t* packed, const uint16_t* ws,
                                  int ws_num, uint16_t* y, int8_t* q_out, float* s_out,
                                  int32_t* acc, int N, int K, hipStream_t stream) {
    return launch(true, x, packed, nullptr, ws, ws_num, y, acc, q_out, s_out, N, K, stream);
}

}  // namespace bl
